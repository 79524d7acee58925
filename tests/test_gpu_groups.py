"""GPU parity for query groups that are not a power of two (3, 5, 6, 7 and 9
to 15 query heads per KV head, D = 128): the decode and MFMA prefill kernels
serve them with work items of the next power of two (8 at most) whose extra
head slots are padding, never read from q and never written.

Decode batches, chunked prefill beside decode rows, split-K partitions, a
sliding window, 8- and 32-token blocks and 8-bit pools, each against the
oracle (bf16 max-abs 2e-2, mean-abs 2e-3), the pools bit-exact, and the same
bits with and without the count of single-row requests.  The oracle's head
mapping (query head h reads KV head h // G) is pinned on the CPU for any G.
Unused slots and padding blocks hold NaN, and q rows past the batch's last
head of the last row are not touched: the q buffer ends with the batch.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_371_amd as pa
from tests.gpu_util import run_and_compare, say, to_host
from tests.test_gpu_fp8 import Fp8Case
from workloads import build_case

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _mixed(G, Hkv, seed, chunks=True):
    rng = np.random.default_rng(seed)
    B = 20
    n = np.ones(B, np.int64)
    if chunks:
        n[:3] = [300, 65, 7]
    L = np.maximum(n, rng.integers(1, 2500, B))
    L[5] = 1
    return n, L


def _no_hint_same(c, dc, psize, window):
    hinted = dc.out.clone()
    dc.attention(psize, sliding_window=window, decode_hint=False)
    torch.cuda.synchronize()
    assert torch.equal(hinted.view(torch.int16), dc.out.view(torch.int16)), "the decode-row count changed bits"


@pytest.mark.parametrize("G", [3, 5, 6, 7, 12, 15])
@pytest.mark.parametrize("kind", ["decode", "mixed"])
def test_padded_group_bf16(G, kind):
    Hkv = 2 if G > 8 else 4
    n, L = _mixed(G, Hkv, 70 + G, chunks=kind == "mixed")
    c = build_case(f"grp{G}_{kind}", 80 + G, "bf16", G * Hkv, Hkv, 128, n, L)
    for psize in (0, 256):
        mx, mean, ok, dc = run_and_compare(c, partition_size=psize, check_pool=psize == 0)
        say(f"G={G} {kind} psize {psize}: max {mx:.3g} mean {mean:.3g}")
        assert ok, (psize, mx, mean)
        _no_hint_same(c, dc, psize, 0)


@pytest.mark.parametrize("G,bs,window", [(5, 8, 0), (6, 32, 0), (7, 16, 300), (3, 8, 100), (10, 16, 0)])
def test_padded_group_blocks_and_window(G, bs, window):
    Hkv = 2
    n, L = _mixed(G, Hkv, 90 + G)
    c = build_case(f"grpb{G}_{bs}", 95 + G, "bf16", G * Hkv, Hkv, 128, n, L, block_size=bs)
    mx, mean, ok, dc = run_and_compare(c, partition_size=0, sliding_window=window)
    say(f"G={G} bs={bs} window={window}: max {mx:.3g} mean {mean:.3g}")
    assert ok, (mx, mean)
    _no_hint_same(c, dc, 0, window)


@pytest.mark.parametrize("G", [5, 6, 12])
def test_padded_group_fp8(G):
    Hkv = 2
    n, L = _mixed(G, Hkv, 110 + G)
    c = build_case(f"grpf8{G}", 120 + G, "bf16", G * Hkv, Hkv, 128, n, L)
    fc = Fp8Case(c, 130 + G, 0.5, 0.25)
    fc.write_and_attend(0)
    mx, mean, ok = fc.compare()
    say(f"fp8 G={G}: max {mx:.3g} mean {mean:.3g}")
    assert ok, (mx, mean)


def test_padded_group_last_head_of_last_row():
    """The last KV head's item of the batch's last row: its padding slots would
    lie past the q buffer's end; q is an exact-size tensor here, so a read of a
    padding slot would fault or show as a wrong row, and the output rows past
    the batch are a guard that must stay untouched."""
    G, Hkv = 5, 3
    n = np.array([1, 40, 1], np.int64)
    L = np.array([700, 900, 33], np.int64)
    c = build_case("grp_last", 140, "bf16", G * Hkv, Hkv, 128, n, L)
    mx, mean, ok, dc = run_and_compare(c, partition_size=64)
    say(f"last head: max {mx:.3g} mean {mean:.3g}")
    assert ok, (mx, mean)
    out = torch.full((c.q.shape[0] + 1,) + tuple(c.q.shape[1:]), 0x7FC0, dtype=torch.int16, device="cuda:0")
    view = out[:-1].view(torch.bfloat16)
    pa.attention_varlen(view, dc.q, dc.k_cache, dc.v_cache, dc.cu, dc.seq_lens, dc.tables, float(c.scale),
                        c.max_query_len, c.max_seq_len, partition_size=64, num_decode_rows=2)
    torch.cuda.synchronize()
    assert torch.equal(view.view(torch.int16), dc.out.view(torch.int16))
    assert bool((out[-1] == 0x7FC0).all()), "a row past the batch was written"


@pytest.mark.parametrize("dtype,D,G", [("f32", 128, 5), ("f32", 64, 3), ("bf16", 64, 6), ("bf16", 256, 7),
                                       ("f32", 256, 5)])
def test_generic_kernel_groups(dtype, D, G):
    """Shapes the fast kernels do not build (fp32; bf16 at D = 64 and 256 with a
    group that is not a power of two) run on the generic split-K kernel, which
    takes every group of up to 8 heads: decode rows and chunked prefill rows,
    default and explicit partitions."""
    Hkv = 2
    n, L = _mixed(G, Hkv, 150 + G + D)
    n, L = n[:10], L[:10]
    c = build_case(f"grpgen_{dtype}{D}_{G}", 160 + G, dtype, G * Hkv, Hkv, D, n, L)
    for psize in (0, 128):
        mx, mean, ok, dc = run_and_compare(c, partition_size=psize, check_pool=psize == 0)
        say(f"generic {dtype} D={D} G={G} psize {psize}: max {mx:.3g} mean {mean:.3g}")
        assert ok, (psize, mx, mean)


@pytest.mark.parametrize("seed", range(40))
def test_random_shape_padded_groups(seed):
    """The random-shape draw (request mixes, windows, partitions, block sizes) with
    a group of 3, 5, 6, 7, 10, 12 or 15 heads at D = 128, bf16 pools: against the
    oracle, the pools bit-exact, and the same bits without the decode-row hint."""
    from tests.test_gpu_random_shapes import _draw

    s = _draw(seed)
    rng = np.random.default_rng(50000 + seed)
    G = int(rng.choice([3, 5, 6, 7, 10, 12, 15]))
    Hkv = int(rng.choice([1, 2, 4]))
    n, L = s["n"], s["L"]
    if seed % 3 == 0:   # no single-row request: the prefill kernel runs alone
        n = np.maximum(n, 2)
        L = np.maximum(L, n)
    while int((n * L).sum()) * G * Hkv * 128 > 3e8:   # the oracle's work, about a second
        big = int(np.argmax(n * L))
        if n[big] > 2:
            n[big] = max(2, n[big] // 2)
        L[big] = max(int(n[big]), int(L[big]) // 2)
    c = build_case(f"grprand{seed}", 900 + seed, "bf16", G * Hkv, Hkv, 128, n, L, block_size=s["bs"])
    say(f"seed {seed}: G={G} Hkv={Hkv} bs={s['bs']} B={len(n)} max n={int(n.max())} window={s['window']} "
        f"psize={s['psize']}")
    mx, mean, ok, dc = run_and_compare(c, partition_size=s["psize"], sliding_window=s["window"])
    assert ok, (mx, mean)
    _no_hint_same(c, dc, s["psize"], s["window"])
