"""Pins of the oracle's sliding-window mask (CPU only).

Reading: with a window of W > 0 tokens, the row at position p attends to
keys max(0, p - W + 1) .. p.  Pinned by an independently written brute force,
by the closed forms at both ends (W >= context: the plain causal result,
bit for bit; W = 1: the row's own V), and by truncation: attending with a
window equals attending, without one, to a re-paged copy of only the keys
in the window.
"""

import numpy as np
import pytest

import oracle.paged_attention as opa
from tests.bruteforce import brute_attention, page_requests

pytestmark = pytest.mark.cpu

SEQS = [(1, 1), (3, 17), (1, 33), (16, 16), (5, 40), (2, 70)]


def _case(seed, seqs, Hq=4, Hkv=2, D=8):
    rng = np.random.default_rng(seed)
    K = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for _, L in seqs]
    V = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for _, L in seqs]
    Q = [rng.standard_normal((n, Hq, D)).astype(np.float32) for n, _ in seqs]
    kp, vp, bt = page_requests(K, V, rng)
    cu = np.concatenate([[0], np.cumsum([n for n, _ in seqs])]).astype(np.int32)
    L = np.array([l for _, l in seqs], np.int32)
    return K, V, Q, np.concatenate(Q), kp, vp, bt, cu, L


@pytest.mark.parametrize("W", [1, 2, 5, 16, 17, 33])
def test_window_matches_bruteforce(W):
    K, V, Q, q, kp, vp, bt, cu, L = _case(1, SEQS)
    got = opa.oracle_attention_varlen(q, kp, vp, cu, L, bt, 0.3, 2, "f32", sliding_window=W)
    want = []
    for b in range(len(SEQS)):
        want += brute_attention(Q[b].tolist(), K[b].tolist(), V[b].tolist(), float(np.float32(0.3)), 2, window=W)
    assert np.allclose(got, np.array(want), rtol=1e-12, atol=1e-12)


def test_window_at_least_context_is_plain_causal():
    K, V, Q, q, kp, vp, bt, cu, L = _case(2, SEQS)
    plain = opa.oracle_attention_varlen(q, kp, vp, cu, L, bt, 0.3, 2, "f32")
    wide = opa.oracle_attention_varlen(q, kp, vp, cu, L, bt, 0.3, 2, "f32", sliding_window=int(L.max()))
    assert np.array_equal(plain, wide)


def test_window_one_returns_own_value():
    K, V, Q, q, kp, vp, bt, cu, L = _case(3, SEQS)
    got = opa.oracle_attention_varlen(q, kp, vp, cu, L, bt, 0.3, 2, "f32", sliding_window=1)
    for b, (n, Lb) in enumerate(SEQS):
        for j in range(n):
            pos = Lb - n + j
            for h in range(4):
                assert np.array_equal(got[cu[b] + j, h], V[b][pos, h // 2].astype(np.float64))


@pytest.mark.parametrize("W", [3, 16, 29])
def test_window_equals_truncated_context(W):
    """Decode rows: a window of W over context L equals no window over a
    fresh request holding only keys L-W .. L-1."""
    seqs = [(1, 50), (1, 20), (1, 3)]
    K, V, Q, q, kp, vp, bt, cu, L = _case(4, seqs)
    got = opa.oracle_attention_varlen(q, kp, vp, cu, L, bt, 0.3, 2, "f32", sliding_window=W)
    Kt = [k[max(0, len(k) - W):] for k in K]
    Vt = [v[max(0, len(v) - W):] for v in V]
    kp2, vp2, bt2 = page_requests(Kt, Vt, np.random.default_rng(5))
    L2 = np.array([len(k) for k in Kt], np.int32)
    want = opa.oracle_attention_varlen(q, kp2, vp2, cu, L2, bt2, 0.3, 2, "f32")
    assert np.allclose(got, want, rtol=1e-13, atol=1e-13)


def test_first_visible_key():
    assert opa.first_visible_key(10, 1, 0) == 0
    assert opa.first_visible_key(10, 1, 0, 4) == 6
    assert opa.first_visible_key(10, 3, 0, 4) == 4     # row 0 sits at position 7
    assert opa.first_visible_key(10, 3, 2, 100) == 0


def test_planted_off_by_one_window_is_caught(monkeypatch):
    """A window one key too wide fails the brute-force pin."""
    orig = opa.first_visible_key
    monkeypatch.setattr(opa, "first_visible_key", lambda L, n, j, W=0: max(0, orig(L, n, j, W) - (1 if W else 0)))
    K, V, Q, q, kp, vp, bt, cu, L = _case(1, SEQS)
    got = opa.oracle_attention_varlen(q, kp, vp, cu, L, bt, 0.3, 2, "f32", sliding_window=5)
    want = []
    for b in range(len(SEQS)):
        want += brute_attention(Q[b].tolist(), K[b].tolist(), V[b].tolist(), float(np.float32(0.3)), 2, window=5)
    assert not np.allclose(got, np.array(want), rtol=1e-12, atol=1e-12)
