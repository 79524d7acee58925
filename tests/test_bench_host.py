"""Host-side pieces of bench.py: the multi-row sub-batch that times the prefill
kernel on its own, the flop count, and reading a committed kernel summary."""

import types

import numpy as np
import torch

import bench


def _fake_batch():
    q_lens = np.array([3, 1, 2, 1, 4], np.int32)
    cu = np.zeros(6, np.int32)
    cu[1:] = np.cumsum(q_lens)
    seq_lens = np.array([40, 17, 9, 30, 64], np.int32)
    tables = np.arange(5 * 4, dtype=np.int32).reshape(5, 4)
    c = types.SimpleNamespace(q_lens=q_lens, cu_seqlens=cu, seq_lens=seq_lens, block_tables=tables, num_kv_heads=2,
                              num_q_heads=4, head_dim=8, scale=0.125, block_size=16, num_seqs=5,
                              total_q=int(cu[-1]), max_query_len=4, max_seq_len=64)
    q = torch.arange(int(cu[-1]) * 4 * 8, dtype=torch.float32).reshape(-1, 4, 8)
    dc = types.SimpleNamespace(c=c, pa=None, fp8=False, window=0, q=q, k_cache=torch.zeros(1), v_cache=torch.zeros(1))
    return c, dc


def test_multi_row_batch_selects_the_multi_row_requests():
    c, dc = _fake_batch()
    sub = bench._MultiRowBatch(dc, torch)
    want = [0, 2, 4]
    assert sub.c.num_seqs == 3 and sub.c.total_q == 9 and sub.c.max_query_len == 4
    assert sub.cu.tolist() == [0, 3, 5, 9]
    assert sub.seq_lens.tolist() == [40, 9, 64]
    assert sub.tables.tolist() == c.block_tables[want].tolist()
    rows = [r for b in want for r in range(c.cu_seqlens[b], c.cu_seqlens[b + 1])]
    assert torch.equal(sub.q, dc.q[rows])
    assert sub.k_cache is dc.k_cache and sub.v_cache is dc.v_cache


def test_flops_of_the_sub_batch_are_those_of_its_requests():
    c, dc = _fake_batch()
    sub = bench._MultiRowBatch(dc, torch)
    # row j of a request with n rows and context L sees L - n + j + 1 keys
    keys = sum(L - n + j + 1 for L, n in [(40, 3), (9, 2), (64, 4)] for j in range(n))
    assert bench.attention_flops(sub.c) == 4.0 * 8 * 4 * keys
    assert bench.attention_flops(c) == bench.attention_flops(sub.c) + 4.0 * 8 * 4 * (17 + 30)


def test_profiled_kernel_needs_the_current_digest(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    table = "| `pa::prefill_kernel<4, 4, 16, 128, false>` | 44 | 231.76 | 211.29 | 271.44 | 34.74 |\n"
    (tmp_path / "attention_call_w_kernels.md").write_text(table + "source_sha256: " + "0" * 64 + "\n")
    assert bench.profiled_kernel_us("w", "prefill_kernel") is None
    (tmp_path / "attention_call_w_kernels.md").write_text(table + "source_sha256: " + bench.kernel_source_digest()
                                                         + "\n")
    assert bench.profiled_kernel_us("w", "prefill_kernel") == 231.76
    assert bench.profiled_kernel_us("w", "decode_gqa_kernel") is None
    assert bench.profiled_kernel_us("missing", "prefill_kernel") is None
