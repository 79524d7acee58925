"""GPU parity of the 8-bit (OCP FP8 E4M3) KV cache path against the oracle.

Bars: the quantising cache write is bit-exact over the whole pool (the
oracle divides by the scale in fp32 and encodes with ties to even and
saturation); attention over 8-bit pools is within the bf16 bounds (max-abs
2e-2, mean-abs 2e-3) of the fp64 oracle attending over decode(code) *
scale.  Slots that hold no token keep the NaN code, so a read outside a
context shows up in the output.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_371_amd as pa
from tests.gpu_util import oracle_pool, say, to_dev, to_host
from workloads import build_case, make_config

pytestmark = pytest.mark.gpu

NAN_CODE = 0x7F
BF16_NAN = 0x7FC0


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def fp8_pools(c, seed, max_exp=10):
    """8-bit pools shaped like the case's: random finite codes of magnitude
    below 2^(max_exp - 7), NaN codes wherever the case left a poisoned slot."""
    rng = np.random.default_rng(seed)
    pools = []
    for bf in (c.k_cache, c.v_cache):
        e = rng.integers(0, max_exp + 1, bf.shape)
        m = rng.integers(0, 8, bf.shape)
        s = rng.integers(0, 2, bf.shape)
        codes = ((s << 7) | (e << 3) | m).astype(np.uint8)
        codes[bf == BF16_NAN] = NAN_CODE
        pools.append(codes)
    return pools


def to_dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


class Fp8Case:
    def __init__(self, c, seed, k_scale, v_scale):
        self.c, self.k_scale, self.v_scale = c, k_scale, v_scale
        self.k_codes, self.v_codes = fp8_pools(c, seed)
        self.q = to_dev(c.q, "bf16")
        self.k_cache, self.v_cache = to_dev_u8(self.k_codes), to_dev_u8(self.v_codes)
        self.k_new, self.v_new = to_dev(c.k_new, "bf16"), to_dev(c.v_new, "bf16")
        self.slots = torch.from_numpy(c.slot_mapping).to("cuda:0")
        self.cu = torch.from_numpy(c.cu_seqlens).to("cuda:0")
        self.seq_lens = torch.from_numpy(c.seq_lens).to("cuda:0")
        self.tables = torch.from_numpy(c.block_tables).to("cuda:0")
        self.out = torch.empty_like(self.q)

    def oracle_pools(self):
        kq = oracle.fp8_quantize_rows(self.c.k_new, self.k_scale)
        vq = oracle.fp8_quantize_rows(self.c.v_new, self.v_scale)
        return oracle.oracle_cache_write(self.k_codes, self.v_codes, kq, vq, self.c.slot_mapping, self.c.block_size)

    def write_and_attend(self, partition_size=0):
        c = self.c
        pa.cache_write_fp8(self.k_new, self.v_new, self.k_cache, self.v_cache, self.slots, self.k_scale, self.v_scale)
        pa.attention_varlen(self.out, self.q, self.k_cache, self.v_cache, self.cu, self.seq_lens, self.tables,
                            float(c.scale), c.max_query_len, c.max_seq_len, partition_size=partition_size,
                            k_scale=self.k_scale, v_scale=self.v_scale)
        torch.cuda.synchronize()

    def compare(self, rows=None, check_pool=True, sharded=False):
        c = self.c
        kp, vp = self.oracle_pools()
        if check_pool:
            assert np.array_equal(self.k_cache.cpu().numpy(), kp), "K pool differs"
            assert np.array_equal(self.v_cache.cpu().numpy(), vp), "V pool differs"
        args = (c.q, kp, vp, c.cu_seqlens, c.seq_lens, c.block_tables, c.scale, c.num_kv_heads, "bf16", c.block_size)
        kw = dict(rows=rows, kv_dtype="fp8", k_scale=self.k_scale, v_scale=self.v_scale)
        if sharded:
            from oracle.sharded import oracle_attention_sharded

            want = oracle_attention_sharded(*args, pool=oracle_pool(), **kw)
        else:
            want = oracle.oracle_attention_varlen(*args, **kw)
        got = oracle.widen(to_host(self.out, "bf16"), "bf16")
        if rows is not None:
            idx = np.asarray(sorted(set(int(r) for r in rows)))
            got, want = got[idx], want[idx]
        return oracle.compare_outputs(got, want, "bf16")


@pytest.mark.parametrize("D", [128, 64])
def test_cache_write_fp8_bitexact(D):
    """Quantisation of new rows, including ties, saturation, tiny values and NaN."""
    c = build_case(f"cw8_{D}", 31, "bf16", 4, 2, D, [1, 16, 5, 1, 30], [1, 16, 40, 100, 33])
    c.slot_mapping[2] = -1
    rng = np.random.default_rng(2)
    special = np.array([0x4700, 0xC700, 0x3F88, 0x3F98, 0x3400, 0x2F80, 0x0001, BF16_NAN, 0x7F80, 0xFF80, 0x8000],
                       np.uint16)   # 32768, -32768, ties near 1, 2^-23, tiny, subnormal bf16, NaN, +-inf, -0
    for arr in (c.k_new, c.v_new):
        flat = arr.reshape(-1)
        pos = rng.choice(flat.size, special.size * 6, replace=False)
        flat[pos] = np.tile(special, 6)
    fc = Fp8Case(c, 7, 0.0625, 0.3)
    pa.cache_write_fp8(fc.k_new, fc.v_new, fc.k_cache, fc.v_cache, fc.slots, fc.k_scale, fc.v_scale)
    torch.cuda.synchronize()
    kp, vp = fc.oracle_pools()
    assert np.array_equal(fc.k_cache.cpu().numpy(), kp)
    assert np.array_equal(fc.v_cache.cpu().numpy(), vp)


LENS = [1, 2, 15, 16, 17, 63, 64, 65, 129, 500, 513, 1025, 3000]


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (16, 8), (16, 4), (64, 8)])
@pytest.mark.parametrize("psize", [0, 256])
def test_decode_fp8_edge_lengths(Hq, Hkv, psize):
    c = build_case(f"dec8_{Hq}_{Hkv}", 32, "bf16", Hq, Hkv, 128, [1] * len(LENS), LENS)
    fc = Fp8Case(c, 8, 0.5, 0.25)
    fc.write_and_attend(psize)
    mx, mean, ok = fc.compare()
    say(f"fp8 {Hq}/{Hkv} psize {psize}: max {mx:.3g} mean {mean:.3g}")
    assert ok, (mx, mean)


@pytest.mark.parametrize("bs", [8, 32])
@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (64, 8)])
def test_decode_fp8_block_sizes(bs, Hq, Hkv):
    """8-bit pools on 8- and 32-token blocks (the fast kernel's paging of
    16-token tiles onto two blocks, or onto half a block)."""
    c = build_case(f"dec8bs{bs}_{Hq}", 35 + bs, "bf16", Hq, Hkv, 128, [1] * len(LENS), LENS, block_size=bs)
    fc = Fp8Case(c, 9, 0.5, 0.25)
    for psize in (0, 48):
        fc.write_and_attend(psize)
        mx, mean, ok = fc.compare(check_pool=psize == 0)
        say(f"fp8 bs {bs} {Hq}/{Hkv} psize {psize}: max {mx:.3g} mean {mean:.3g}")
        assert ok, (psize, mx, mean)


@pytest.mark.parametrize("D,Hq,Hkv", [(64, 8, 8), (64, 32, 8), (64, 64, 8), (256, 8, 8), (256, 16, 8),
                                      (256, 64, 8), (128, 128, 8)])
def test_decode_fp8_head_dim_64(D, Hq, Hkv):
    """8-bit pools at D = 64 (4 codes of a row per lane) and D = 256 (16 codes),
    and KV heads served by several items (G = 8 at D = 256, G = 16 at D = 128)."""
    c = build_case(f"dec8d{D}_{Hq}", 37, "bf16", Hq, Hkv, D, [1] * len(LENS), LENS)
    fc = Fp8Case(c, 10, 0.5, 0.25)
    for psize in (0, 256):
        fc.write_and_attend(psize)
        mx, mean, ok = fc.compare(check_pool=psize == 0)
        say(f"fp8 D={D} {Hq}/{Hkv} psize {psize}: max {mx:.3g} mean {mean:.3g}")
        assert ok, (psize, mx, mean)


@pytest.mark.parametrize("Hq,Hkv,n,lens", [
    (64, 8, [1] * 10, [1, 8, 9, 16, 17, 33, 100, 700, 2049, 3000]),   # items of 8 heads
    (32, 8, [1] * 10, [1, 8, 9, 16, 17, 33, 100, 700, 2049, 3000]),   # items of 4 heads
    (32, 8, [40, 1, 7, 1], [1000, 700, 37, 33]),                       # chunked prefill with decode rows
])
def test_fp8_bitwise_across_block_sizes(Hq, Hkv, n, lens):
    """The same 8-bit K/V paged on 8-, 16- and 32-token blocks gives bitwise the
    same outputs (16-token tiles in the same order at every block size; with 8-
    token blocks a tile's two halves come from two blocks)."""
    from tests.test_gpu_variants import _repage

    c = build_case(f"f8xbs{Hq}", 150 + Hq, "bf16", Hq, Hkv, 128, n, lens)
    k16, v16 = Fp8Case(c, 15, 0.5, 0.25).oracle_pools()   # the pools after this step's (quantising) cache write
    rng = np.random.default_rng(16)
    outs = {}
    for bs in (16, 8, 32):
        if bs == 16:
            kp, vp, tables = k16, v16, c.block_tables
        else:
            nb = sum(-(-int(L) // bs) for L in lens) + 3
            (kp, vp), tables = _repage((k16, v16), c.block_tables, lens, bs, nb, rng)
        out = torch.empty_like(to_dev(c.q, "bf16"))
        pa.attention_varlen(out, to_dev(c.q, "bf16"), to_dev_u8(kp), to_dev_u8(vp),
                            torch.from_numpy(c.cu_seqlens).to("cuda:0"), torch.from_numpy(c.seq_lens).to("cuda:0"),
                            torch.from_numpy(np.ascontiguousarray(tables)).to("cuda:0"), float(c.scale),
                            c.max_query_len, c.max_seq_len, partition_size=256, k_scale=0.5, v_scale=0.25)
        torch.cuda.synchronize()
        outs[bs] = to_host(out, "bf16")
    assert np.array_equal(outs[8], outs[16]) and np.array_equal(outs[32], outs[16])
    want = oracle.oracle_attention_varlen(c.q, k16, v16, c.cu_seqlens, c.seq_lens, c.block_tables, c.scale,
                                          c.num_kv_heads, "bf16", 16, kv_dtype="fp8", k_scale=0.5, v_scale=0.25)
    mx, mean, ok = oracle.compare_outputs(oracle.widen(outs[16], "bf16"), want, "bf16")
    say(f"fp8 {Hq}/{Hkv}: bitwise equal across block sizes; max {mx:.3g} mean {mean:.3g}")
    assert ok, (mx, mean)


def test_decode_fp8_deterministic_bitwise():
    c = build_case("det8", 33, "bf16", 64, 8, 128, [1] * 6, [3000, 17, 900, 2049, 1, 4500])
    fc = Fp8Case(c, 9, 0.5, 0.25)
    fc.write_and_attend(0)
    a = fc.out.clone()
    pa.attention_varlen(fc.out, fc.q, fc.k_cache, fc.v_cache, fc.cu, fc.seq_lens, fc.tables, float(c.scale),
                        1, c.max_seq_len, k_scale=fc.k_scale, v_scale=fc.v_scale)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), fc.out.view(torch.int16))


def test_gqa_config_fp8_every_row():
    """The Llama-3-70B-shaped GQA decode layer with 8-bit pools, in the launch
    configuration the benchmark times (default partition): the whole pool bit
    for bit and every row against the oracle."""
    c = make_config("gqa_decode_bf16", 0)
    fc = Fp8Case(c, 10, 0.5, 0.25)
    fc.write_and_attend(0)
    mx, mean, ok = fc.compare(sharded=True)
    say(f"gqa fp8 every row: max {mx:.3g} mean {mean:.3g}")
    assert ok, (mx, mean)


@pytest.mark.parametrize("D,Hq,Hkv,bs", [(128, 32, 8, 16), (128, 8, 8, 16), (128, 64, 8, 16), (64, 16, 8, 16),
                                         (256, 16, 8, 16), (128, 32, 8, 8), (128, 32, 8, 32), (128, 128, 8, 16)])
def test_prefill_fp8_chunks(D, Hq, Hkv, bs):
    """Multi-row requests on 8-bit pools (the MFMA kernel widens the codes to
    bf16 when it stages them): chunks of 2, 17, 65 and 300 rows with and without
    a cached prefix, next to decode rows and an empty request."""
    n = [2, 17, 1, 65, 0, 300, 1]
    L = [2, 17 + 401, 900, 65 + 1000, 3, 300 + 77, 33]
    c = build_case(f"pf8_{D}_{Hq}_{bs}", 60 + D + bs, "bf16", Hq, Hkv, D, n, L, block_size=bs)
    fc = Fp8Case(c, 12, 0.5, 0.25)
    for psize in (0, 256):
        fc.write_and_attend(psize)
        mx, mean, ok = fc.compare(check_pool=psize == 0)
        say(f"fp8 prefill D={D} {Hq}/{Hkv} bs {bs} psize {psize}: max {mx:.3g} mean {mean:.3g}")
        assert ok, (psize, mx, mean)


@pytest.mark.parametrize("Hq,Hkv,maxn", [(64, 8, 8), (32, 8, 16)])
def test_fp8_short_multirow_split(Hq, Hkv, maxn):
    """Short multi-row requests on 8-bit pools whose contexts span several
    partitions: computed per partition by the MFMA kernel and merged."""
    n = [2, maxn, 3, 1, 5, maxn]
    L = [2049, 5000, 513, 3000, 1030, 2048 + maxn]
    c = build_case(f"split8_{Hq}_{maxn}", 70 + maxn, "bf16", Hq, Hkv, 128, n, L)
    fc = Fp8Case(c, 13, 0.5, 0.25)
    for psize in (0, 512):
        fc.write_and_attend(psize)
        mx, mean, ok = fc.compare(check_pool=psize == 0)
        say(f"fp8 split {Hq}/{Hkv} psize {psize}: max {mx:.3g} mean {mean:.3g}")
        assert ok, (psize, mx, mean)


def test_mixed_config_fp8_every_row():
    """The mixed chunked-prefill step (8 chunks of 512 rows with cached prefixes and
    248 decode rows, 32/8 heads) on 8-bit pools in the launch configuration the
    benchmark times: the whole pool bit for bit and every row against the oracle."""
    c = make_config("mixed_prefill_bf16", 0)
    fc = Fp8Case(c, 14, 0.5, 0.25)
    fc.write_and_attend(0)
    mx, mean, ok = fc.compare(sharded=True)
    say(f"mixed fp8 every row: max {mx:.3g} mean {mean:.3g}")
    assert ok, (mx, mean)


def test_fp8_multirow_needs_a_built_group():
    """Multi-row requests on 8-bit pools run on the MFMA kernel only; a group
    size it does not build (not a power of two, at D = 64) is refused."""
    c = build_case("mr8", 34, "bf16", 6, 2, 64, [3, 1], [20, 30])
    fc = Fp8Case(c, 11, 1.0, 1.0)
    with pytest.raises(pa.PAError) as e:
        fc.write_and_attend(0)
    assert e.value.status == -3


@pytest.mark.parametrize("seed", range(60))
def test_random_shape_fp8(seed):
    """The random-shape draw of the bf16 sweep (head dims, groups, block sizes,
    decode, chunked and short multi-row requests, windows, explicit partitions)
    on 8-bit pools at three scale pairs: the cache write bit for bit, the
    attention against the oracle, and the same bits without the count of
    single-row requests."""
    from tests.test_gpu_random_shapes import _draw

    s = _draw(seed, large_groups=(seed % 4 == 3))
    if seed % 3 == 0:
        s["n"] = np.maximum(s["n"], 2)
        s["L"] = np.maximum(s["L"], s["n"])
    c = build_case(f"f8rand{seed}", 500 + seed, "bf16", s["G"] * s["Hkv"], s["Hkv"], s["D"], s["n"], s["L"],
                   block_size=s["bs"])
    ks, vs = [(0.5, 0.25), (0.25, 0.125), (0.03, 0.07)][seed % 3]
    say(f"fp8 seed {seed}: D={s['D']} G={s['G']} Hkv={s['Hkv']} bs={s['bs']} B={len(s['n'])} "
        f"max n={int(s['n'].max())} window={s['window']} psize={s['psize']} scales {ks} {vs}")
    fc = Fp8Case(c, 700 + seed, ks, vs)
    pa.cache_write_fp8(fc.k_new, fc.v_new, fc.k_cache, fc.v_cache, fc.slots, ks, vs)
    outs = []
    for hint in (int((c.q_lens == 1).sum()), 0):
        o = torch.empty_like(fc.q)
        pa.attention_varlen(o, fc.q, fc.k_cache, fc.v_cache, fc.cu, fc.seq_lens, fc.tables, float(c.scale),
                            c.max_query_len, c.max_seq_len, partition_size=s["psize"], sliding_window=s["window"],
                            k_scale=ks, v_scale=vs, num_decode_rows=hint)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), "the decode-row count changed bits"
    kp, vp = fc.oracle_pools()
    assert np.array_equal(fc.k_cache.cpu().numpy(), kp), "K pool differs"
    assert np.array_equal(fc.v_cache.cpu().numpy(), vp), "V pool differs"
    want = oracle.oracle_attention_varlen(c.q, kp, vp, c.cu_seqlens, c.seq_lens, c.block_tables, c.scale,
                                          c.num_kv_heads, "bf16", c.block_size, kv_dtype="fp8", k_scale=ks,
                                          v_scale=vs, sliding_window=s["window"])
    got = oracle.widen(to_host(outs[0], "bf16"), "bf16")
    mx, mean, ok = oracle.compare_outputs(got, want, "bf16")
    say(f"  max {mx:.3g} mean {mean:.3g}")
    assert ok, (mx, mean)
