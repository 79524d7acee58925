"""HIP graph capture of one step (cache write, then attention over the paged
cache): the hot calls only enqueue work on the caller's stream, with no host
synchronisation or allocation, so a scheduler can capture a step once and
replay it ([Q67] §3.3: the scheduler builds the step's metadata once; the
kernels read it).  A mixed batch with the decode-row hint also records the
library's fork to its side stream and the join back.

Each graph is replayed several times with fresh inputs written eagerly in
place between the replays, and every replay is compared bit for bit with an
eager call of the same step on the same inputs.  The persistent kernels'
claim counters are re-armed by the kernels themselves (no memset in the
captured work), which the replays exercise.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import paged_kv_cache_371_amd as pa
from tests.gpu_util import DeviceCase, say, to_dev
from workloads import build_case


def _case(kind):
    rng = np.random.default_rng(41)
    if kind == "decode":
        B, Hq, Hkv = 96, 32, 8
        n = np.ones(B, np.int64)
        L = rng.integers(1, 3000, B)
    else:   # decode rows plus prefill chunks
        B, Hq, Hkv = 48, 32, 8
        n = np.ones(B, np.int64)
        n[:3] = [200, 33, 5]
        L = np.maximum(n, rng.integers(1, 3000, B))
    return build_case(f"graph_{kind}", 42, "bf16", Hq, Hkv, 128, n, L, poison=False)


def _fresh(t: torch.Tensor, seed: int) -> np.ndarray:
    """bf16 N(0, 1) values of t's shape (RNE from fp32), as uint16 bits."""
    x = np.random.default_rng(seed).standard_normal(t.shape).astype(np.float32)
    u = x.view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.gpu
@pytest.mark.parametrize("kind", ["decode", "mixed"])
def test_graph_replays_match_eager(kind):
    c = _case(kind)
    dc = DeviceCase(c)
    hint = int((c.q_lens == 1).sum())
    p = pa.make_params(dc.q, dc.k_cache, dc.cu, dc.tables, c.num_kv_heads, float(c.scale), c.max_query_len,
                       c.max_seq_len, out=dc.out, num_decode_rows=hint)
    ws_graph = torch.empty(pa.workspace_size(p), dtype=torch.uint8, device="cuda:0")
    ws_eager = torch.empty_like(ws_graph)

    def step(out, ws):
        dc.cache_write()
        pa.attention_varlen(out, dc.q, dc.k_cache, dc.v_cache, dc.cu, dc.seq_lens, dc.tables, float(c.scale),
                            c.max_query_len, c.max_seq_len, workspace=ws, num_decode_rows=hint)

    out_graph = torch.empty_like(dc.q)
    step(out_graph, ws_graph)   # loads the kernels and creates the side stream before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out_graph, ws_graph)
    torch.cuda.synchronize()
    say(f"{kind}: captured; hint {hint}, rows {int(c.q_lens.sum())}")
    for r in range(4):
        dc.q.copy_(to_dev(_fresh(dc.q, 100 + r), "bf16"))
        dc.k_new.copy_(to_dev(_fresh(dc.k_new, 200 + r), "bf16"))
        dc.v_new.copy_(to_dev(_fresh(dc.v_new, 300 + r), "bf16"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out_graph.clone()
        out_eager = torch.empty_like(dc.q)
        step(out_eager, ws_eager)   # rewrites the same cache rows with the same values
        torch.cuda.synchronize()
        assert bool(torch.isfinite(got.float()).all())
        assert torch.equal(got.view(torch.int16), out_eager.view(torch.int16)), f"replay {r}"
        say(f"{kind}: replay {r} equals the eager step")
