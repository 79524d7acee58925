"""Pins of the CPU oracle against things other than itself (CPU only).

Each pin is chosen so that a plausible slip in the oracle (a wrong address
rule, a dropped scale, a transposed GQA mapping, an off-by-one causal mask,
K used in place of V) fails at least one test; ``test_planted_*`` plant such
slips in the oracle and check that a pin catches them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.paged_attention as opa
from oracle import (
    OracleError,
    gather_request_kv,
    oracle_attention_varlen,
    oracle_cache_write,
    physical_location,
)
from tests.bruteforce import brute_attention, page_requests

pytestmark = pytest.mark.cpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# helpers


def _tiny(rng, seqs, Hq, Hkv, D):
    """Contiguous per-request K/V/Q (float32 values) for [(n, L), ...]."""
    K = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for n, L in seqs]
    V = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for n, L in seqs]
    Q = [rng.standard_normal((n, Hq, D)).astype(np.float32) for n, L in seqs]
    return K, V, Q


def _run_oracle(K, V, Q, seqs, Hkv, scale, rng, block_size=16):
    k_pool, v_pool, tables = page_requests(K, V, rng, block_size)
    cu = np.concatenate([[0], np.cumsum([n for n, _ in seqs])]).astype(np.int32)
    L = np.array([l for _, l in seqs], np.int32)
    q = np.concatenate(Q, axis=0) if Q else np.zeros((0, 1, 1), np.float32)
    out = opa.oracle_attention_varlen(q, k_pool, v_pool, cu, L, tables, scale, Hkv, "f32", block_size)
    return out, (k_pool, v_pool, tables, cu, L, q)


def _brute_all(K, V, Q, seqs, scale, group):
    res = []
    for b in range(len(seqs)):
        res.extend(brute_attention(Q[b].tolist(), K[b].tolist(), V[b].tolist(), float(np.float32(scale)), group))
    return np.array(res, np.float64)


SEQS_MIXED = [(1, 1), (3, 17), (1, 33), (16, 16), (5, 40), (0, 7)]


# ---------------------------------------------------------------------------
# worked example of the address rule (quant67 §3.3)


def test_worked_example_address_rule():
    ex = json.load(open(os.path.join(GOLDEN, "block_table_worked_example.json")))
    bs = ex["block_size"]
    a = ex["seq_a"]
    assert physical_location(np.array(a["block_table"]), a["token"], bs) == (a["physical_block"], a["offset"])
    assert a["physical_block"] * bs + a["offset"] == a["slot"]
    for tok in ex["seq_b"]["tokens"]:
        blk, off = physical_location(np.array(ex["seq_b"]["block_table"]), tok["token"], bs)
        assert (blk, off) == (tok["physical_block"], tok["offset"])
        assert blk * bs + off == tok["slot"]
    for ntok, nblk in ex["blocks_for_tokens"]:
        assert -(-ntok // bs) == nblk


def test_worked_example_cache_write_and_gather():
    """Token 18 of table [17, 42] is written by slot 674 and read back by the gather."""
    ex = json.load(open(os.path.join(GOLDEN, "block_table_worked_example.json")))
    a = ex["seq_a"]
    NB, Hkv, D = 48, 2, 4
    k = np.zeros((NB, Hkv, 16, D), np.float32)
    v = np.zeros((NB, Hkv, 16, D), np.float32)
    new = np.arange(Hkv * D, dtype=np.float32).reshape(1, Hkv, D) + 1
    k2, v2 = oracle_cache_write(k, v, new, -new, np.array([a["slot"]]))
    assert (k2[42, :, 2, :] == new[0]).all() and (v2[42, :, 2, :] == -new[0]).all()
    assert np.count_nonzero(k2) == Hkv * D
    got = gather_request_kv(k2, np.array(a["block_table"]), a["num_tokens"], "f32")
    assert (got[a["token"]] == new[0]).all()
    assert np.count_nonzero(got) == Hkv * D


# ---------------------------------------------------------------------------
# cache write by brute force


def test_cache_write_bruteforce_bits():
    rng = np.random.default_rng(1)
    NB, Hkv, D, N = 9, 3, 8, 40
    k = rng.integers(0, 65535, (NB, Hkv, 16, D), dtype=np.uint16)
    v = rng.integers(0, 65535, (NB, Hkv, 16, D), dtype=np.uint16)
    kn = rng.integers(0, 65535, (N, Hkv, D), dtype=np.uint16)
    vn = rng.integers(0, 65535, (N, Hkv, D), dtype=np.uint16)
    slots = rng.choice(NB * 16, N, replace=False).astype(np.int64)
    slots[::7] = -1
    k2, v2 = oracle_cache_write(k, v, kn, vn, slots)
    written = set()
    for i, s in enumerate(slots):
        if s < 0:
            continue
        written.add(int(s))
        for h in range(Hkv):
            assert (k2[s // 16, h, s % 16] == kn[i, h]).all()
            assert (v2[s // 16, h, s % 16] == vn[i, h]).all()
    for s in range(NB * 16):
        if s not in written:
            assert (k2[s // 16, :, s % 16] == k[s // 16, :, s % 16]).all()
            assert (v2[s // 16, :, s % 16] == v[s // 16, :, s % 16]).all()
    # inputs untouched
    assert not np.shares_memory(k2, k)


@pytest.mark.parametrize("bs", [8, 32])
def test_cache_write_bruteforce_bits_other_block_sizes(bs):
    """Block sizes 8 and 32 (quant67 §3.7 lists 8/16/32): slot s lands in block
    s // bs at offset s % bs, every other slot keeps its bits."""
    rng = np.random.default_rng(bs)
    NB, Hkv, D, N = 7, 2, 4, 30
    k = rng.integers(0, 65535, (NB, Hkv, bs, D), dtype=np.uint16)
    kn = rng.integers(0, 65535, (N, Hkv, D), dtype=np.uint16)
    slots = rng.choice(NB * bs, N, replace=False).astype(np.int64)
    slots[::5] = -1
    k2, _ = oracle_cache_write(k, k.copy(), kn, kn, slots, block_size=bs)
    expect = k.copy()
    for i, s in enumerate(slots):
        if s >= 0:
            for h in range(Hkv):
                expect[s // bs, h, s % bs] = kn[i, h]
    assert (k2 == expect).all()
    with pytest.raises(OracleError):
        oracle_cache_write(k, k, kn[:1], kn[:1], np.array([NB * bs]), block_size=bs)


def test_cache_write_rejects_duplicates_and_range():
    k = np.zeros((2, 1, 16, 4), np.float32)
    row = np.ones((2, 1, 4), np.float32)
    with pytest.raises(OracleError):
        oracle_cache_write(k, k, row, row, np.array([5, 5]))
    with pytest.raises(OracleError):
        oracle_cache_write(k, k, row[:1], row[:1], np.array([32]))
    k2, _ = oracle_cache_write(k, k, row, row, np.array([-1, -7]))
    assert (k2 == 0).all()


# ---------------------------------------------------------------------------
# attention against an unpaged brute force and a library routine


@pytest.mark.parametrize("Hq,Hkv,D", [(4, 4, 8), (4, 2, 8), (6, 1, 4), (8, 2, 16)])
def test_attention_matches_unpaged_bruteforce(Hq, Hkv, D):
    rng = np.random.default_rng(Hq * 100 + Hkv * 10 + D)
    K, V, Q = _tiny(rng, SEQS_MIXED, Hq, Hkv, D)
    scale = np.float32(1 / math.sqrt(D))
    out, _ = _run_oracle(K, V, Q, SEQS_MIXED, Hkv, scale, rng)
    ref = _brute_all(K, V, Q, SEQS_MIXED, scale, Hq // Hkv)
    assert out.shape == ref.shape
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("bs", [8, 32])
def test_attention_matches_unpaged_bruteforce_other_block_sizes(bs):
    """The paged result at block sizes 8 and 32 equals attention over the
    contiguous (never paged) K/V of each request."""
    rng = np.random.default_rng(300 + bs)
    Hq, Hkv, D = 4, 2, 8
    K, V, Q = _tiny(rng, SEQS_MIXED, Hq, Hkv, D)
    scale = np.float32(1 / math.sqrt(D))
    out, _ = _run_oracle(K, V, Q, SEQS_MIXED, Hkv, scale, rng, block_size=bs)
    ref = _brute_all(K, V, Q, SEQS_MIXED, scale, Hq // Hkv)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_attention_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(7)
    Hq, Hkv, D = 8, 2, 32
    seqs = [(1, 70), (9, 50), (33, 33), (2, 100)]
    K, V, Q = _tiny(rng, seqs, Hq, Hkv, D)
    scale = np.float32(0.125)
    out, _ = _run_oracle(K, V, Q, seqs, Hkv, scale, rng)
    rows = []
    for b, (n, L) in enumerate(seqs):
        q = torch.from_numpy(Q[b].astype(np.float64)).permute(1, 0, 2)          # [Hq, n, D]
        k = torch.from_numpy(K[b].astype(np.float64)).permute(1, 0, 2)
        v = torch.from_numpy(V[b].astype(np.float64)).permute(1, 0, 2)
        k = k.repeat_interleave(Hq // Hkv, dim=0)
        v = v.repeat_interleave(Hq // Hkv, dim=0)
        j = torch.arange(n)[:, None]
        t = torch.arange(L)[None, :]
        mask = t <= (L - n + j)
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=float(scale))
        rows.append(o.permute(1, 0, 2).numpy())
    np.testing.assert_allclose(out, np.concatenate(rows), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# closed forms


def test_context_length_one_returns_v_exactly():
    rng = np.random.default_rng(3)
    K, V, Q = _tiny(rng, [(1, 1), (1, 1)], 4, 2, 8)
    out, _ = _run_oracle(K, V, Q, [(1, 1), (1, 1)], 2, np.float32(0.3), rng)
    for b in range(2):
        for h in range(4):
            assert (out[b, h] == V[b][0, h // 2].astype(np.float64)).all()


def test_constant_v_gives_constant_output():
    rng = np.random.default_rng(4)
    seqs = [(1, 45), (7, 30)]
    K, V, Q = _tiny(rng, seqs, 4, 4, 8)
    c = rng.standard_normal((4, 8)).astype(np.float32)
    V = [np.broadcast_to(c, v.shape).copy() for v in V]
    out, _ = _run_oracle(K, V, Q, seqs, 4, np.float32(0.35), rng)
    np.testing.assert_allclose(out, np.broadcast_to(c, out.shape), rtol=0, atol=1e-14)


def test_identical_keys_give_mean_of_visible_values():
    rng = np.random.default_rng(5)
    seqs = [(4, 20), (1, 37)]
    K, V, Q = _tiny(rng, seqs, 2, 1, 8)
    K = [np.broadcast_to(k[:1], k.shape).copy() for k in K]
    out, _ = _run_oracle(K, V, Q, seqs, 1, np.float32(0.5), rng)
    r = 0
    for b, (n, L) in enumerate(seqs):
        for j in range(n):
            pos = L - n + j
            want = V[b][:pos + 1, 0].astype(np.float64).mean(axis=0)
            for h in range(2):
                np.testing.assert_allclose(out[r, h], want, rtol=0, atol=1e-14)
            r += 1


# ---------------------------------------------------------------------------
# invariances


def _case_arrays(seed, seqs, Hq, Hkv, D):
    rng = np.random.default_rng(seed)
    K, V, Q = _tiny(rng, seqs, Hq, Hkv, D)
    return K, V, Q, rng


def test_block_permutation_invariance_bitwise():
    K, V, Q, rng = _case_arrays(11, SEQS_MIXED, 4, 2, 8)
    scale = np.float32(0.3)
    out1, (kp, vp, bt, cu, L, q) = _run_oracle(K, V, Q, SEQS_MIXED, 2, scale, rng)
    perm = rng.permutation(kp.shape[0])          # new id of old block i is perm[i]
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[perm] = kp
    vp2[perm] = vp
    out2 = oracle_attention_varlen(q, kp2, vp2, cu, L, perm[bt], scale, 2, "f32")
    assert np.array_equal(out1, out2, equal_nan=True)


def test_shared_prefix_invariance_bitwise():
    """Requests with equal prefix contents: shared physical blocks == private copies."""
    rng = np.random.default_rng(12)
    Hq, Hkv, D, nsh = 4, 2, 8, 3
    prefix_k = rng.standard_normal((nsh * 16, Hkv, D)).astype(np.float32)
    prefix_v = rng.standard_normal((nsh * 16, Hkv, D)).astype(np.float32)
    tails = [0, 5, 21]
    K = [np.concatenate([prefix_k, rng.standard_normal((t, Hkv, D)).astype(np.float32)]) for t in tails]
    V = [np.concatenate([prefix_v, rng.standard_normal((t, Hkv, D)).astype(np.float32)]) for t in tails]
    seqs = [(1, len(k)) for k in K]
    Q = [rng.standard_normal((1, Hq, D)).astype(np.float32) for _ in seqs]
    out_private, (kp, vp, bt, cu, L, q) = _run_oracle(K, V, Q, seqs, Hkv, np.float32(0.3), rng)
    bt2 = bt.copy()
    bt2[1:, :nsh] = bt[0, :nsh]           # everyone points at request 0's prefix blocks
    out_shared = oracle_attention_varlen(q, kp, vp, cu, L, bt2, np.float32(0.3), Hkv, "f32")
    assert np.array_equal(out_private, out_shared)


def test_chunk_row_equals_decode_row():
    """Row j of a chunk with prior context P equals a decode row with context P + j + 1."""
    rng = np.random.default_rng(13)
    Hq, Hkv, D, P, n = 4, 2, 8, 19, 9
    K, V, Q = _tiny(rng, [(n, P + n)], Hq, Hkv, D)
    out_chunk, (kp, vp, bt, cu, L, q) = _run_oracle(K, V, Q, [(n, P + n)], Hkv, np.float32(0.3), rng)
    for j in range(n):
        one = oracle_attention_varlen(q[j:j + 1], kp, vp, np.array([0, 1], np.int32),
                                      np.array([P + j + 1], np.int32), bt, np.float32(0.3), Hkv, "f32")
        assert np.array_equal(one[0], out_chunk[j])


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (15, 3), (12, 2)])   # G = 4, 5 and 6
def test_gqa_equals_mha_with_repeated_heads(Hq, Hkv):
    rng = np.random.default_rng(14)
    D = 8
    seqs = [(1, 30), (4, 18)]
    K, V, Q = _tiny(rng, seqs, Hq, Hkv, D)
    out_gqa, _ = _run_oracle(K, V, Q, seqs, Hkv, np.float32(0.3), np.random.default_rng(1))
    G = Hq // Hkv
    Kx = [np.repeat(k, G, axis=1) for k in K]       # head h of the copy = KV head h // G
    Vx = [np.repeat(v, G, axis=1) for v in V]
    out_mha, _ = _run_oracle(Kx, Vx, Q, seqs, Hq, np.float32(0.3), np.random.default_rng(2))
    assert np.array_equal(out_gqa, out_mha)


def test_request_reorder_permutes_outputs():
    K, V, Q, rng = _case_arrays(15, SEQS_MIXED, 4, 2, 8)
    out, _ = _run_oracle(K, V, Q, SEQS_MIXED, 2, np.float32(0.3), rng)
    order = [3, 0, 5, 2, 1, 4]
    out2, _ = _run_oracle([K[i] for i in order], [V[i] for i in order], [Q[i] for i in order],
                          [SEQS_MIXED[i] for i in order], 2, np.float32(0.3), np.random.default_rng(99))
    cu = np.concatenate([[0], np.cumsum([n for n, _ in SEQS_MIXED])])
    expect = np.concatenate([out[cu[i]:cu[i + 1]] for i in order])
    assert np.array_equal(out2, expect)


def test_nan_outside_context_never_leaks():
    """Unowned slots and padding blocks hold NaN; outputs stay finite."""
    K, V, Q, rng = _case_arrays(16, SEQS_MIXED, 4, 2, 8)
    out, _ = _run_oracle(K, V, Q, SEQS_MIXED, 2, np.float32(0.3), rng)
    assert np.isfinite(out).all()


def test_bf16_widening_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F, 0x0000, 0x8000], np.uint16)
    want = [1.0, -1.0, 3.140625, 2.0 ** -133, 3.3895313892515355e38, 0.0, -0.0]
    got = oracle.widen(bits, "bf16")
    assert got.tolist() == want


def test_metadata_validation():
    bt = np.zeros((2, 2), np.int32)
    with pytest.raises(OracleError):
        oracle.validate_metadata([0, 2, 1], [3, 3], bt, 4)       # decreasing cu
    with pytest.raises(OracleError):
        oracle.validate_metadata([0, 4, 5], [3, 3], bt, 4)       # n > L
    with pytest.raises(OracleError):
        oracle.validate_metadata([0, 1, 2], [40, 3], bt, 4)      # table too narrow
    with pytest.raises(OracleError):
        oracle.validate_metadata([0, 1, 2], [3, 3], bt + 9, 4)   # id out of range
    oracle.validate_metadata([0, 1, 1], [3, 0], bt, 4)           # empty request is fine


def test_compare_outputs_bounds():
    z = np.zeros((20, 30))
    w = z.copy()
    w[0, 0] = 0.0199
    assert oracle.compare_outputs(w, z, "bf16")[2]
    w[0, 0] = 0.0201
    assert not oracle.compare_outputs(w, z, "bf16")[2]            # max bound
    assert oracle.compare_outputs(z + 0.0019, z, "bf16")[2]
    assert not oracle.compare_outputs(z + 0.0021, z, "bf16")[2]   # mean bound
    w[0, 0] = 0.0199
    assert oracle.compare_outputs(z + 9e-6, z, "f32")[2]
    assert not oracle.compare_outputs(z + 1.1e-5, z, "f32")[2]
    w[1, 1] = np.nan
    assert not oracle.compare_outputs(w, z, "bf16")[2]


# ---------------------------------------------------------------------------
# planted slips: each must be caught by a pin above


def _pin_vs_brute(Hq=4, Hkv=2, D=8, seqs=SEQS_MIXED, seed=21):
    rng = np.random.default_rng(seed)
    K, V, Q = _tiny(rng, seqs, Hq, Hkv, D)
    scale = np.float32(1 / math.sqrt(D))
    out, _ = _run_oracle(K, V, Q, seqs, Hkv, scale, rng)
    ref = _brute_all(K, V, Q, seqs, scale, Hq // Hkv)
    return np.nan_to_num(np.abs(out - ref), nan=np.inf).max()


@pytest.mark.parametrize("slip", ["gqa_mod", "causal_off_by_one", "address_swap", "no_scale", "k_for_v"])
def test_planted_slip_is_caught(monkeypatch, slip):
    assert _pin_vs_brute() < 1e-12
    if slip == "gqa_mod":
        monkeypatch.setattr(opa, "kv_head_of", lambda h, G: h % 2)
    elif slip == "causal_off_by_one":
        monkeypatch.setattr(opa, "last_visible_key", lambda L, n, j: L - n + j - 1 if L - n + j > 0 else 0)
    elif slip == "address_swap":
        # logical block index used as if it were the physical block
        monkeypatch.setattr(opa, "physical_location", lambda row, t, bs=16: (t // bs, t % bs))
    elif slip == "no_scale":
        orig = opa.oracle_attention_varlen
        monkeypatch.setattr(opa, "oracle_attention_varlen",
                            lambda q, k, v, cu, L, bt, scale, *a, **kw: orig(q, k, v, cu, L, bt, 1.0, *a, **kw))
    elif slip == "k_for_v":
        orig_g = opa.gather_request_kv
        state = {"k": None}

        def g(cache, row, L, dtype, bs=16):
            r = orig_g(cache, row, L, dtype, bs)
            if state["k"] is None:
                state["k"] = r
                return r
            out = state["k"]
            state["k"] = None
            return out
        monkeypatch.setattr(opa, "gather_request_kv", g)
    try:
        err = _pin_vs_brute()
    except (IndexError, OracleError, ValueError):
        err = np.inf
    assert err > 1e-6, f"slip {slip} not caught"
