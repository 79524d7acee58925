"""GPU parity on seeded random shapes: every dispatch path of the attention
call against the oracle in one sweep.

Each case draws a head dim (64, 128, 256), a group size (1 to 16; 4 to 32
in the large-group cases, where a KV head's heads span several work items), a block
size (8, 16, 32), a dtype (bf16 mostly, fp32 sometimes), a batch mixing
single-row requests with chunked-prefill and short multi-row requests, ragged
contexts (some a single token), an optional sliding window and an optional
explicit partition size.  Together the cases reach the fast decode kernel,
the MFMA kernel with and without split short requests, the generic kernel
for the shapes the others do not take, and the partition merges.  The bars
are the oracle comparison's (bf16 max-abs 2e-2 and mean-abs 2e-3, fp32
max-abs 1e-5), and the cache write must leave the pool bit-exact.
"""

import numpy as np
import pytest
import torch

from tests.gpu_util import run_and_compare, say
from workloads import build_case

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _draw(seed, large_groups=False):
    rng = np.random.default_rng(1000 + seed)
    dtype = "f32" if rng.random() < 0.2 else "bf16"
    D = int(rng.choice([64, 128, 256]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    if large_groups:   # several work items per KV head in the decode and MFMA kernels
        dtype = "bf16"
        G = int(rng.choice([16, 32])) if D < 256 else int(rng.choice([4, 8, 16]))
    Hkv = int(rng.choice([1, 2, 4]))
    bs = int(rng.choice([8, 16, 32]))
    B = int(rng.integers(1, 24))
    n = np.ones(B, np.int64)
    kind = rng.integers(0, 3)   # 0: decode only, 1: with chunked prefill, 2: with short multi-row requests
    if kind == 1:
        k = int(rng.integers(1, min(B, 3) + 1))
        n[rng.choice(B, k, replace=False)] = rng.integers(2, 300, k)
    elif kind == 2:
        k = int(rng.integers(1, B + 1))
        n[rng.choice(B, k, replace=False)] = rng.integers(2, 9, k)
    L = np.maximum(n, rng.integers(1, 3000, B))
    one = (rng.random(B) < 0.15) & (n == 1)
    L[one] = 1                                   # single-token contexts
    # bound the oracle's fp64 work (rows x query heads x keys x D) to about a second
    while int((n * L).sum()) * G * Hkv * D > 3e8:
        big = int(np.argmax(n * L))
        if n[big] > 2:
            n[big] = max(2, n[big] // 2)
        L[big] = max(int(n[big]), int(L[big]) // 2)
    window = int(rng.choice([0, 0, 0, int(rng.integers(1, 700))]))
    psize = int(rng.choice([0, 0, 16 * int(rng.integers(1, 40))]))
    return dict(dtype=dtype, D=D, G=G, Hkv=Hkv, bs=bs, n=n, L=L, window=window, psize=psize)


@pytest.mark.parametrize("seed", range(24))
def test_random_shape(seed):
    _check(seed, _draw(seed))


@pytest.mark.parametrize("seed", range(24, 32))
def test_random_shape_large_groups(seed):
    _check(seed, _draw(seed, large_groups=True))


@pytest.mark.parametrize("seed", range(1000, 1200))
def test_random_shape_sweep(seed):
    """A wider sweep of the same draw: every fourth case with large groups, and
    in every third no single-row request at all, so the MFMA prefill kernel
    runs alone (its 8-wave workgroups) and not beside the decode kernel."""
    s = _draw(seed, large_groups=(seed % 4 == 3))
    if seed % 3 == 0:
        s["n"] = np.maximum(s["n"], 2)
        s["L"] = np.maximum(s["L"], s["n"])
    _check(seed, s)


def _check(seed, s):
    c = build_case(f"rand{seed}", 300 + seed, s["dtype"], s["G"] * s["Hkv"], s["Hkv"], s["D"], s["n"], s["L"],
                   block_size=s["bs"])
    say(f"seed {seed}: {s['dtype']} D={s['D']} G={s['G']} Hkv={s['Hkv']} bs={s['bs']} B={len(s['n'])} "
        f"max n={int(s['n'].max())} max L={int(s['L'].max())} window={s['window']} psize={s['psize']}")
    mx, mean, ok, dc = run_and_compare(c, partition_size=s["psize"], sliding_window=s["window"])
    say(f"  max {mx:.3g} mean {mean:.3g}")
    assert ok, (mx, mean)
    # The count of single-row requests only schedules the kernels: without it
    # the result is the same bits.
    hinted = dc.out.clone()
    dc.attention(s["psize"], sliding_window=s["window"], decode_hint=False)
    torch.cuda.synchronize()
    bits = torch.int16 if c.dtype == "bf16" else torch.int32
    assert torch.equal(hinted.view(bits), dc.out.view(bits)), "the decode-row count changed bits"
