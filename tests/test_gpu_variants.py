"""GPU parity of the block-size and head-dim variants against the oracle.

Block sizes 8 and 32 (the pages list 8, 16 and 32 as selectable, quant67
§3.7) run on the cache writes, on the fast decode kernel for bf16 D = 128
(its 16-token tiles paged onto two 8-token blocks or half a 32-token block)
and on the MFMA prefill kernel for multi-row requests (the same 16-key units
per wave), on the generic split-K kernel otherwise; D = 256 runs on the
generic kernel; D = 64 and 128 at block size 16 were covered before.  Bars: cache writes
bit-exact over the whole pool, attention within the fp32 / bf16 bounds of
the oracle, with poisoned (NaN) slots outside every context, ragged contexts
ending anywhere in a block, multi-row requests, partitions that start inside
a block, and a sliding window.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_371_amd as pa
from tests.gpu_util import DeviceCase, oracle_out, oracle_pools, run_and_compare, say, to_dev, to_host
from workloads import build_case

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


LENS = [1, 7, 8, 9, 31, 32, 33, 100, 700]


COMBOS = [("f32", 64, 8, 8), ("f32", 64, 32, 2), ("bf16", 128, 16, 4), ("bf16", 128, 32, 2), ("bf16", 256, 8, 8),
          ("bf16", 256, 16, 2), ("f32", 256, 16, 4)]


@pytest.mark.parametrize("bs", [8, 32])
@pytest.mark.parametrize("dtype,D,Hq,Hkv", COMBOS)
def test_decode_block_size_and_head_dim(bs, dtype, D, Hq, Hkv):
    c = build_case(f"bs{bs}_{dtype}_{D}", 70 + bs, dtype, Hq, Hkv, D, [1] * len(LENS), LENS, block_size=bs)
    for psize in (0, 48):
        mx, mean, ok, _ = run_and_compare(c, partition_size=psize)
        say(f"bs {bs} {dtype} D={D} {Hq}/{Hkv} psize {psize}: max {mx:.3g} mean {mean:.3g}")
        assert ok, (psize, mx, mean)


@pytest.mark.parametrize("bs", [8, 16, 32])
@pytest.mark.parametrize("dtype,D", [("bf16", 256), ("f32", 64), ("bf16", 64)])
def test_multi_row_block_size_and_head_dim(bs, dtype, D):
    """Chunked-prefill rows and decode rows on the generic kernel."""
    n = [5, 1, 17, 1, 2]
    L = [40, 9, 130, 300, 2]
    c = build_case(f"mr{bs}_{dtype}_{D}", 80 + bs, dtype, 16, 4, D, n, L, block_size=bs)
    mx, mean, ok, _ = run_and_compare(c, partition_size=64)
    say(f"multi-row bs {bs} {dtype} D={D}: max {mx:.3g} mean {mean:.3g}")
    assert ok, (mx, mean)


@pytest.mark.parametrize("bs", [8, 32])
def test_window_with_block_size(bs):
    c = build_case(f"wbs{bs}", 90 + bs, "bf16", 32, 8, 128, [1, 1, 3, 1], [50, 500, 77, 1000], block_size=bs)
    for W in (1, 9, 33, 200):
        mx, mean, ok, _ = run_and_compare(c, partition_size=64, sliding_window=W)
        say(f"window {W} bs {bs}: max {mx:.3g} mean {mean:.3g}")
        assert ok, (W, mx, mean)


@pytest.mark.parametrize("bs", [8, 32])
def test_fp8_cache_write_block_size(bs):
    c = build_case(f"f8bs{bs}", 95 + bs, "bf16", 8, 4, 256, [3, 1, 9], [3, 40, 75], block_size=bs)
    rng = np.random.default_rng(1)
    kc = rng.integers(0, 255, c.k_cache.shape, dtype=np.uint8)
    vc = rng.integers(0, 255, c.v_cache.shape, dtype=np.uint8)
    dk, dv = torch.from_numpy(kc).to("cuda:0"), torch.from_numpy(vc).to("cuda:0")
    slots = torch.from_numpy(c.slot_mapping).to("cuda:0")
    pa.cache_write_fp8(to_dev(c.k_new, "bf16"), to_dev(c.v_new, "bf16"), dk, dv, slots, 0.5, 0.125)
    torch.cuda.synchronize()
    wk, wv = oracle.oracle_cache_write(kc, vc, oracle.fp8_quantize_rows(c.k_new, 0.5),
                                       oracle.fp8_quantize_rows(c.v_new, 0.125), c.slot_mapping, bs)
    assert np.array_equal(dk.cpu().numpy(), wk) and np.array_equal(dv.cpu().numpy(), wv)


def test_validate_metadata_block_size():
    c = build_case("vbs", 99, "bf16", 8, 8, 64, [1, 1], [20, 9], block_size=8, poison=False)
    cu = torch.from_numpy(c.cu_seqlens).to("cuda:0")
    sl = torch.from_numpy(c.seq_lens).to("cuda:0")
    bt = torch.from_numpy(c.block_tables).to("cuda:0")
    assert pa.validate_metadata(cu, sl, bt, c.num_blocks, 1, 20, block_size=8) == 0
    narrow = torch.from_numpy(np.ascontiguousarray(c.block_tables[:, :2])).to("cuda:0")
    assert pa.validate_metadata(cu, sl, narrow, c.num_blocks, 1, 20, block_size=8) & pa.BAD_TABLE_WIDTH


FAST_LENS = [1, 7, 8, 9, 15, 16, 17, 24, 31, 32, 33, 47, 100, 700, 2049, 3000]


@pytest.mark.parametrize("bs", [8, 32])
@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (64, 8), (16, 4)])
def test_fast_decode_block_size(bs, Hq, Hkv):
    """The fast decode kernel on 8- and 32-token blocks: contexts ending at
    every offset class of a block, partitions of 16 and 48 tokens that start
    inside 32-token blocks, NaN in every slot and table entry past a context."""
    c = build_case(f"fbs{bs}_{Hq}_{Hkv}", 110 + bs, "bf16", Hq, Hkv, 128, [1] * len(FAST_LENS), FAST_LENS,
                   block_size=bs)
    for psize in (0, 16, 48, 256):
        mx, mean, ok, _ = run_and_compare(c, partition_size=psize, check_pool=psize == 0)
        say(f"fast bs {bs} {Hq}/{Hkv} psize {psize}: max {mx:.3g} mean {mean:.3g}")
        assert ok, (psize, mx, mean)


def _repage(pool_bits, tables, lens, bs, num_blocks, rng):
    """Lay each request's contiguous rows (read from a 16-token-block pool) out
    again on bs-token blocks in shuffled order; unused slots hold NaN (bf16
    bits, or the E4M3 NaN code for 8-bit pools)."""
    Hkv, D = pool_bits[0].shape[1], pool_bits[0].shape[3]
    perm = rng.permutation(num_blocks)
    width = max(-(-int(L) // bs) for L in lens)
    new_tables = np.full((len(lens), width), num_blocks - 1, np.int32)
    fill = 0x7F if pool_bits[0].dtype == np.uint8 else 0x7FC0
    pools = [np.full((num_blocks, Hkv, bs, D), fill, src.dtype) for src in pool_bits]
    nxt = 0
    for b, L in enumerate(lens):
        for j in range(-(-int(L) // bs)):
            new_tables[b, j] = perm[nxt]
            nxt += 1
        for t in range(int(L)):
            src_blk, src_off = tables[b, t // 16], t % 16
            for src, dst in zip(pool_bits, pools):
                dst[new_tables[b, t // bs], :, t % bs, :] = src[src_blk, :, src_off, :]
    return pools, new_tables


def _bitwise_across_block_sizes(name, seed, n, lens, Hq, Hkv, psize, D=128):
    """Outputs for the same logical K/V paged on 8-, 16- and 32-token blocks;
    asserts they are bitwise equal and match the oracle."""
    c = build_case(name, seed, "bf16", Hq, Hkv, D, n, lens)
    k16, v16 = oracle_pools(c)
    outs = {}
    rng = np.random.default_rng(seed)
    for bs in (16, 8, 32):
        if bs == 16:
            kp, vp, tables = k16, v16, c.block_tables
        else:
            nb = sum(-(-int(L) // bs) for L in lens) + 3
            (kp, vp), tables = _repage((k16, v16), c.block_tables, lens, bs, nb, rng)
        out = torch.empty_like(to_dev(c.q, "bf16"))
        pa.attention_varlen(out, to_dev(c.q, "bf16"), to_dev(kp, "bf16"), to_dev(vp, "bf16"),
                            torch.from_numpy(c.cu_seqlens).to("cuda:0"), torch.from_numpy(c.seq_lens).to("cuda:0"),
                            torch.from_numpy(np.ascontiguousarray(tables)).to("cuda:0"), float(c.scale),
                            c.max_query_len, c.max_seq_len, partition_size=psize)
        torch.cuda.synchronize()
        outs[bs] = to_host(out, "bf16")
    assert np.array_equal(outs[8], outs[16]) and np.array_equal(outs[32], outs[16])
    mx, mean, ok = oracle.compare_outputs(oracle.widen(outs[16], "bf16"), oracle_out(c, k16, v16), "bf16")
    say(f"{name}: bitwise equal across block sizes; max {mx:.3g} mean {mean:.3g}")
    assert ok


def test_fast_decode_bitwise_across_block_sizes():
    """Single-row requests: the fast decode kernel visits the same 16-token
    tiles in the same order at every block size, only their addresses change."""
    _bitwise_across_block_sizes("xbs", 120, [1] * len(FAST_LENS), FAST_LENS, 64, 8, 256)


@pytest.mark.parametrize("n,lens,Hq", [
    ([200, 1, 37, 1, 129, 5], [1000, 700, 37, 33, 700, 9], 32),   # chunked prefill, 128-pair tiles
    ([4, 1, 8, 2, 1, 3], [3000, 2049, 1500, 700, 5, 4100], 64),  # short requests split over partitions
])
def test_prefill_bitwise_across_block_sizes(n, lens, Hq):
    """Multi-row requests: the MFMA kernel's waves each stage one 16-key unit
    of every key tile, from one 16-token block, half a 32-token block or two
    8-token blocks; the staged tiles and so the results are the same."""
    _bitwise_across_block_sizes(f"xpbs{Hq}", 121, n, lens, Hq, 8, 0)


@pytest.mark.parametrize("bs", [8, 32])
@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (8, 8), (64, 8)])
def test_prefill_block_size(bs, Hq, Hkv):
    """Chunked-prefill rows with decode rows on 8- and 32-token blocks: prior
    contexts ending anywhere in a block, chunks of 1..200 rows, partitions of
    64 tokens, NaN in every unowned slot and table entry."""
    n = [200, 1, 37, 1, 5, 129, 1, 2]
    L = [1000, 700, 37, 33, 9, 700, 3000, 17]
    c = build_case(f"pbs{bs}_{Hq}_{Hkv}", 130 + bs, "bf16", Hq, Hkv, 128, n, L, block_size=bs)
    for psize in (0, 64):
        mx, mean, ok, _ = run_and_compare(c, partition_size=psize, check_pool=psize == 0)
        say(f"prefill bs {bs} {Hq}/{Hkv} psize {psize}: max {mx:.3g} mean {mean:.3g}")
        assert ok, (psize, mx, mean)


@pytest.mark.parametrize("bs", [8, 32])
def test_split_short_requests_block_size(bs):
    """Speculative-verify shape (2..8 rows, G = 8): short requests split over
    context partitions on the MFMA kernel, merged per row."""
    n = [4, 1, 8, 2, 1, 3, 7]
    L = [3000, 2049, 1500, 700, 5, 4100, 8]
    c = build_case(f"sbs{bs}", 140 + bs, "bf16", 64, 8, 128, n, L, block_size=bs)
    for psize in (0, 512):
        mx, mean, ok, _ = run_and_compare(c, partition_size=psize, check_pool=psize == 0)
        say(f"split bs {bs} psize {psize}: max {mx:.3g} mean {mean:.3g}")
        assert ok, (psize, mx, mean)


@pytest.mark.parametrize("bs", [8, 32])
def test_prefill_window_block_size(bs):
    c = build_case(f"pwbs{bs}", 150 + bs, "bf16", 32, 8, 128, [100, 1, 9], [900, 400, 60], block_size=bs)
    for W in (17, 300):
        mx, mean, ok, _ = run_and_compare(c, partition_size=64, sliding_window=W)
        say(f"prefill window {W} bs {bs}: max {mx:.3g} mean {mean:.3g}")
        assert ok, (W, mx, mean)


@pytest.mark.parametrize("bs", [8, 16, 32])
@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (16, 8), (32, 8), (64, 8)])
def test_fast_decode_head_dim_64(bs, Hq, Hkv):
    """The fast decode kernel at D = 64 (8 bytes of a row per lane, a ring
    twice as deep) for every group size and block size."""
    c = build_case(f"d64_{bs}_{Hq}", 160 + bs, "bf16", Hq, Hkv, 64, [1] * len(FAST_LENS), FAST_LENS, block_size=bs)
    for psize in (0, 48):
        mx, mean, ok, _ = run_and_compare(c, partition_size=psize, check_pool=psize == 0)
        say(f"D=64 bs {bs} {Hq}/{Hkv} psize {psize}: max {mx:.3g} mean {mean:.3g}")
        assert ok, (psize, mx, mean)


def test_fast_decode_head_dim_64_bitwise_across_block_sizes():
    _bitwise_across_block_sizes("xbs64", 123, [1] * len(FAST_LENS), FAST_LENS, 32, 8, 256, D=64)


@pytest.mark.parametrize("bs", [8, 16, 32])
@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (16, 8)])
def test_fast_decode_head_dim_256(bs, Hq, Hkv):
    """The fast decode kernel at D = 256 for G = 1 and 2 (32 bytes of a row per
    lane as two loads, two tiles in flight)."""
    c = build_case(f"d256_{bs}_{Hq}", 170 + bs, "bf16", Hq, Hkv, 256, [1] * len(FAST_LENS), FAST_LENS, block_size=bs)
    for psize in (0, 48):
        mx, mean, ok, _ = run_and_compare(c, partition_size=psize, check_pool=psize == 0)
        say(f"D=256 bs {bs} {Hq}/{Hkv} psize {psize}: max {mx:.3g} mean {mean:.3g}")
        assert ok, (psize, mx, mean)


def test_fast_decode_head_dim_256_bitwise_across_block_sizes():
    _bitwise_across_block_sizes("xbs256", 124, [1] * len(FAST_LENS), FAST_LENS, 16, 8, 256, D=256)


@pytest.mark.parametrize("bs", [8, 16, 32])
@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (32, 8), (64, 8)])
def test_prefill_head_dim_64(bs, Hq, Hkv):
    """The MFMA kernel at D = 64 (two 32-wide d steps, four output blocks; the
    unit's 8 d-chunks per key staged by half the lanes): chunked prefill with
    decode rows, prior contexts ending anywhere in a block."""
    n = [200, 1, 37, 1, 5, 129, 1, 2]
    L = [1000, 700, 37, 33, 9, 700, 3000, 17]
    c = build_case(f"p64_{bs}_{Hq}", 180 + bs, "bf16", Hq, Hkv, 64, n, L, block_size=bs)
    for psize in (0, 64):
        mx, mean, ok, _ = run_and_compare(c, partition_size=psize, check_pool=psize == 0)
        say(f"prefill D=64 bs {bs} {Hq}/{Hkv} psize {psize}: max {mx:.3g} mean {mean:.3g}")
        assert ok, (psize, mx, mean)


def test_split_short_requests_head_dim_64():
    n = [4, 1, 8, 2, 1, 3, 7]
    L = [3000, 2049, 1500, 700, 5, 4100, 8]
    c = build_case("s64", 190, "bf16", 64, 8, 64, n, L)
    for psize in (0, 512):
        mx, mean, ok, _ = run_and_compare(c, partition_size=psize, check_pool=psize == 0)
        say(f"split D=64 psize {psize}: max {mx:.3g} mean {mean:.3g}")
        assert ok, (psize, mx, mean)


def test_prefill_head_dim_64_bitwise_across_block_sizes():
    _bitwise_across_block_sizes("xpbs64", 125, [200, 1, 37, 1, 129, 5], [1000, 700, 37, 33, 700, 9], 32, 8, 0, D=64)


@pytest.mark.parametrize("bs", [8, 16, 32])
@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (16, 8), (64, 8)])
def test_prefill_head_dim_256(bs, Hq, Hkv):
    """The MFMA kernel at D = 256 (one 16-pair block per wave, 64-pair items;
    8 K chunks and two V chunk groups staged per lane)."""
    n = [200, 1, 37, 1, 5, 129, 1, 2]
    L = [1000, 700, 37, 33, 9, 700, 3000, 17]
    c = build_case(f"p256_{bs}_{Hq}", 200 + bs, "bf16", Hq, Hkv, 256, n, L, block_size=bs)
    for psize in (0, 64):
        mx, mean, ok, _ = run_and_compare(c, partition_size=psize, check_pool=psize == 0)
        say(f"prefill D=256 bs {bs} {Hq}/{Hkv} psize {psize}: max {mx:.3g} mean {mean:.3g}")
        assert ok, (psize, mx, mean)


def test_split_short_requests_head_dim_256():
    n = [4, 1, 8, 2, 1, 3, 7]
    L = [3000, 2049, 1500, 700, 5, 4100, 8]
    c = build_case("s256", 210, "bf16", 16, 8, 256, n, L)
    for psize in (0, 512):
        mx, mean, ok, _ = run_and_compare(c, partition_size=psize, check_pool=psize == 0)
        say(f"split D=256 psize {psize}: max {mx:.3g} mean {mean:.3g}")
        assert ok, (psize, mx, mean)


def test_prefill_head_dim_256_bitwise_across_block_sizes():
    _bitwise_across_block_sizes("xpbs256", 126, [200, 1, 37, 1, 129, 5], [1000, 700, 37, 33, 700, 9], 16, 8, 0, D=256)


@pytest.mark.parametrize("D,Hq,Hkv,bs", [(256, 32, 8, 16), (256, 64, 8, 8), (256, 16, 1, 32), (128, 64, 4, 16),
                                         (128, 32, 1, 32), (64, 128, 4, 16), (256, 64, 1, 8), (128, 128, 2, 16)])
def test_fast_decode_head_split(D, Hq, Hkv, bs):
    """A KV head with more query heads than one work item holds (G > 2 at
    D = 256, G > 8 otherwise) is served by several adjacent items of the fast
    kernel that read the same tiles; the plan's decode list is filled, so the
    fast kernel (not the generic one) ran."""
    c = build_case(f"hs{D}_{Hq}_{Hkv}_{bs}", 200 + Hq // Hkv + D, "bf16", Hq, Hkv, D, [1] * len(FAST_LENS), FAST_LENS,
                   block_size=bs)
    for psize in (0, 48):
        mx, mean, ok, dc = run_and_compare(c, partition_size=psize, check_pool=psize == 0)
        say(f"split heads D={D} {Hq}/{Hkv} bs {bs} psize {psize}: max {mx:.3g} mean {mean:.3g}")
        assert ok, (psize, mx, mean)
    p = pa.make_params(dc.q, dc.k_cache, dc.cu, dc.tables, Hkv, float(c.scale), c.max_query_len, c.max_seq_len,
                       out=dc.out)
    ws = torch.zeros(pa.workspace_size(p), dtype=torch.uint8, device="cuda:0")
    pa.attention_varlen(dc.out, dc.q, dc.k_cache, dc.v_cache, dc.cu, dc.seq_lens, dc.tables, float(c.scale),
                        c.max_query_len, c.max_seq_len, workspace=ws)
    torch.cuda.synchronize()
    hdr = ws[:64 * 4].view(torch.int32).cpu().numpy()
    P = pa.partition_size(p)
    assert hdr[8] == sum(-(-int(L) // P) for L in FAST_LENS), (hdr[8], P)
    assert hdr[11] == 0 and hdr[12] == 0


def test_fast_decode_head_split_bitwise_per_head():
    """Splitting a KV head's query heads over items does not change any head's
    result: a 64/8-head layer at D = 128 (one item of 8 heads per KV head)
    equals, head for head, the same heads served as a 128/8-head layer (two
    items of 8), at one explicit partition size."""
    c8 = build_case("hsb8", 240, "bf16", 64, 8, 128, [1] * len(FAST_LENS), FAST_LENS)
    dc = DeviceCase(c8)
    dc.cache_write()
    dc.attention(512)
    torch.cuda.synchronize()
    T = dc.q.shape[0]
    # heads 8j..8j+7 of KV head j, twice: 16 query heads per KV head
    q2 = dc.q.view(T, 8, 8, 128).repeat(1, 1, 2, 1).reshape(T, 128, 128).contiguous()
    out2 = torch.empty_like(q2)
    pa.attention_varlen(out2, q2, dc.k_cache, dc.v_cache, dc.cu, dc.seq_lens, dc.tables, float(c8.scale),
                        1, c8.max_seq_len, partition_size=512)
    torch.cuda.synchronize()
    o2 = out2.view(T, 8, 2, 8, 128)
    f = dc.out.view(T, 8, 8, 128)
    for half in range(2):
        assert torch.equal(o2[:, :, half].contiguous().view(torch.int16), f.contiguous().view(torch.int16)), half


@pytest.mark.parametrize("D,Hq,Hkv,bs", [(128, 64, 4, 16), (128, 128, 4, 8), (64, 128, 8, 32), (256, 32, 2, 16),
                                         (256, 64, 4, 8), (256, 64, 1, 8)])
def test_prefill_head_split(D, Hq, Hkv, bs):
    """Multi-row requests of a KV head with more than 8 query heads: the MFMA
    kernel serves the heads 8 at a time (adjacent items on the same K/V), with
    chunked prefill, decode rows and short requests in one batch; and a batch
    of short requests only, which takes the split-over-partitions path."""
    n = [200, 1, 37, 1, 5, 129, 1, 2]
    L = [1000, 700, 37, 33, 9, 700, 3000, 17]
    c = build_case(f"phs{D}_{Hq}_{Hkv}_{bs}", 260 + Hq // Hkv + D, "bf16", Hq, Hkv, D, n, L, block_size=bs)
    for psize in (0, 64):
        mx, mean, ok, _ = run_and_compare(c, partition_size=psize, check_pool=psize == 0)
        say(f"prefill split heads D={D} {Hq}/{Hkv} bs {bs} psize {psize}: max {mx:.3g} mean {mean:.3g}")
        assert ok, (psize, mx, mean)
    n = [4, 1, 3, 2, 1, 3, 2]
    L = [3000, 2049, 1500, 700, 5, 4100, 8]
    c = build_case(f"shs{D}_{Hq}_{Hkv}_{bs}", 270 + Hq // Hkv + D, "bf16", Hq, Hkv, D, n, L, block_size=bs)
    for psize in (0, 512):
        mx, mean, ok, _ = run_and_compare(c, partition_size=psize, check_pool=psize == 0)
        say(f"short split heads D={D} {Hq}/{Hkv} bs {bs} psize {psize}: max {mx:.3g} mean {mean:.3g}")
        assert ok, (psize, mx, mean)
