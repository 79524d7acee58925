"""pa_attention_varlen_noalloc (the library's static per-GPU scratch instead of a
workspace) against pa_attention_varlen on the same inputs, through the C ABI:
two calls in a row, the second on a smaller batch, each bitwise equal to the
workspace entry point and within the bf16 bounds of the oracle."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_371_amd as pa
from tests.gpu_util import DeviceCase, oracle_out, oracle_pools, say, to_host
from workloads import build_case

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _both(c, psize=0):
    dc = DeviceCase(c)
    dc.cache_write()
    want = dc.attention(psize, out=torch.full_like(dc.q, float("nan")))
    got = torch.full_like(dc.q, float("nan"))
    pa.attention_varlen_noalloc(got, dc.q, dc.k_cache, dc.v_cache, dc.cu, dc.seq_lens, dc.tables, float(c.scale),
                                c.max_query_len, c.max_seq_len, partition_size=psize)
    torch.cuda.synchronize()
    return dc, want, got


def _check(c, psize=0):
    dc, want, got = _both(c, psize)
    assert torch.equal(got.view(torch.int16), want.view(torch.int16)), "differs from pa_attention_varlen"
    kp, vp = oracle_pools(c)
    mx, mean, ok = oracle.compare_outputs(oracle.widen(to_host(got, c.dtype), c.dtype), oracle_out(c, kp, vp),
                                          c.dtype)
    say(f"  {c.name}: max {mx:.3g} mean {mean:.3g}")
    assert ok, (mx, mean)


def test_noalloc_two_calls_second_smaller():
    """A GQA decode batch with multi-partition contexts, then a smaller batch of
    decode rows and a prefill chunk: the second call must not see the first
    call's lists or partials."""
    rng = np.random.default_rng(5)
    L = rng.integers(1, 6000, 40)
    big = build_case("noalloc_big", 5, "bf16", 64, 8, 128, [1] * 40, L)
    say("case", big.name)
    _check(big)
    small = build_case("noalloc_small", 6, "bf16", 32, 8, 128, [1, 70, 1, 0, 1], [3000, 900, 17, 4, 2500])
    say("case", small.name)
    _check(small)
    say("case", small.name, "partition 256")
    _check(small, 256)


def test_noalloc_fp32_generic_path():
    c = build_case("noalloc_f32", 7, "f32", 8, 8, 64, [1, 3, 1], [700, 40, 1])
    _check(c)


def test_noalloc_padded_group():
    """A group of 5 query heads per KV head (items with padding head slots):
    decode rows and a prefill chunk, default and 256-token partitions."""
    c = build_case("noalloc_g5", 9, "bf16", 40, 8, 128, [1, 90, 1, 1], [2600, 700, 33, 1900])
    _check(c)
    _check(c, 256)


def test_noalloc_rejects_beyond_scratch():
    """A batch whose workspace exceeds the scratch is refused before any launch."""
    c = build_case("noalloc_tiny", 8, "bf16", 64, 8, 128, [1], [64])
    dc = DeviceCase(c)
    with pytest.raises(pa.PAError) as e:
        # 60000 requests of 8192 tokens in 512-token partitions: far beyond 64 MiB of partials
        p = pa.make_params(dc.q, dc.k_cache, dc.cu, dc.tables, 8, float(c.scale), 1, 8192, partition_size=512)
        p.num_seqs, p.total_q, p.max_blocks_per_seq = 60000, 60000, 512
        assert pa.workspace_size(p) > pa.NOALLOC_SCRATCH_BYTES
        pa._check(pa.lib().pa_attention_varlen_noalloc(16, 16, 16, 16, 16, 16, 16, __import__("ctypes").byref(p),
                                                       None))
    assert e.value.status == -5
