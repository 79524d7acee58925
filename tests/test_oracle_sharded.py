"""The process-pool driver of the oracle returns exactly the oracle's result."""

import numpy as np
import pytest

import oracle
from oracle.sharded import make_pool, oracle_attention_sharded, split_rows
from workloads import build_case


@pytest.fixture(scope="module")
def pool():
    ex = make_pool(3)
    yield ex
    ex.shutdown()


def test_split_rows_covers_each_wanted_row_once():
    cu = np.array([0, 1, 9, 9, 40, 41])
    L = np.array([30, 100, 5, 64, 2])
    pieces = split_rows(cu, L, pieces=7)
    got = sorted(int(cu[b]) + j for b, js in pieces for j in js)
    assert got == list(range(41))
    rows = [0, 3, 8, 20, 40]
    pieces = split_rows(cu, L, rows=rows, pieces=3, window=4)
    assert sorted(int(cu[b]) + j for b, js in pieces for j in js) == rows


@pytest.mark.parametrize("dtype,Hq,Hkv,bs,window", [("bf16", 8, 2, 16, 0), ("f32", 4, 4, 8, 0),
                                                     ("bf16", 16, 2, 32, 20)])
def test_sharded_equals_oracle_bitwise(pool, dtype, Hq, Hkv, bs, window):
    c = build_case("shard", 3, dtype, Hq, Hkv, 64, [1, 37, 0, 1, 5, 1], [90, 60, 3, 1, 200, 33], block_size=bs,
                   poison=True)
    kp, vp = oracle.oracle_cache_write(c.k_cache, c.v_cache, c.k_new, c.v_new, c.slot_mapping, bs)
    args = (c.q, kp, vp, c.cu_seqlens, c.seq_lens, c.block_tables, c.scale, c.num_kv_heads, dtype, bs)
    want = oracle.oracle_attention_varlen(*args, sliding_window=window)
    got = oracle_attention_sharded(*args, sliding_window=window, pool=pool)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(got[~np.isnan(want)], want[~np.isnan(want)])
    rows = [0, 5, 40, 43]
    want_r = oracle.oracle_attention_varlen(*args, rows=rows, sliding_window=window)
    got_r = oracle_attention_sharded(*args, rows=rows, sliding_window=window, pool=pool)
    assert np.array_equal(got_r[rows], want_r[rows])
    assert np.isnan(np.delete(got_r, rows, axis=0)).all()


def test_sharded_fp8_pools(pool):
    c = build_case("shard8", 4, "bf16", 8, 2, 64, [1, 1, 1], [50, 129, 7], poison=False)
    rng = np.random.default_rng(0)
    k8 = rng.integers(0, 0x78, c.k_cache.shape).astype(np.uint8)
    v8 = rng.integers(0, 0x78, c.v_cache.shape).astype(np.uint8)
    args = (c.q, k8, v8, c.cu_seqlens, c.seq_lens, c.block_tables, c.scale, c.num_kv_heads, "bf16", 16)
    kw = dict(kv_dtype="fp8", k_scale=0.5, v_scale=0.25)
    want = oracle.oracle_attention_varlen(*args, **kw)
    got = oracle_attention_sharded(*args, pool=pool, **kw)
    assert np.array_equal(got, want)
