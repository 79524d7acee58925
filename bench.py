"""Benchmark of the paged-attention step on one MI355X.

One step = the cache write of the batch's new K/V rows followed by paged
attention of its query rows, both through the C ABI on torch's current
stream.  Default workload: the Llama-3-70B-shaped GQA decode layer (256
requests, 64 query / 8 KV heads, D=128, bf16, log-normal contexts with median
1024 clipped to [16, 8192], shuffled 16-token blocks).

Prints one JSON line.  ``value`` is KV GB/s: the attention's algorithmic
K/V bytes per step divided by the step time (inputs resident in HBM), over
the K timed steps; before the W warm-up steps the step runs untimed for 50 ms
so the GPU's clocks settle (``settle_steps``), and the timed steps make the C
calls through the binding's prepared calls (checks and marshalling done once).
``roofline`` reports one layer's attention: pa_attention_run over the
step's work lists (the split-K decode kernel and the partition merge; the
prefill kernel too when the batch has multi-row requests), timed with HIP
events on the launch stream.  The work lists (pa_attention_plan, one small
kernel) depend only on the request lengths and are built once per step for
every layer; ``attention_plan_ms`` times that stage and
``call_frac_incl_plan`` the whole pa_attention_varlen call, and the whole
step behind ``value`` includes it.
Its ``traffic`` is the HBM bytes per call that rocprofv3's FETCH_SIZE and
WRITE_SIZE counters measured, scaled by the same counters' reading for a
plain copy of known size; it is read from the committed counter summary
under profiles/ and reported only while the kernel sources still hash to
the digest recorded there (null otherwise).  ``cpu_baseline`` times the fp64
CPU oracle on a bounded sample of the same requests.

``--calibrate-copy`` runs only a 1 GiB device-to-device copy (the counters'
calibration run).  By default a 1 GiB buffer is read before each timed plan
and run call (a read, so no dirty lines are left to be written back during
the call), so those times, and ``roofline``, start with no part of the batch
in the L2s or the Infinity Cache; the run stage is also timed back to back
(``attention_run_ms_unflushed``), and ``--no-flush-cache`` drops the flushed
timing.  For workloads with multi-row requests, ``prefill_kernel`` times the
call over those requests alone and reports the prefill kernel's TFLOP/s
against the bf16 matrix-core peak, and ``roofline.combined`` sets the run
stage against the step's HBM time and matrix-core time at peak: the larger of
the two (perfect overlap) and their sum (none).  ``--block-size 8|32`` builds the same workload on 8- or
32-token blocks.  ``--sliding-window W`` runs the workload with a sliding
window of W tokens (KV bytes then count only the keys in some row's window).  ``--op copy_blocks`` times copy-on-write block copies
(pa_copy_blocks) and ``--op swap_out`` / ``--op swap_in`` time swapping a
sequence's blocks to and from pinned host memory (pa_swap_blocks); see
``run_copy_blocks`` and ``run_swap`` for their workloads.  ``--kv-dtype fp8`` runs the same workload on 8-bit (OCP
E4M3) pools of random finite codes with per-tensor scales; KV bytes then
count one byte per element.  Parity of this exact
launch configuration against the oracle is the job of the GPU tests; the
oracle is used here only for the CPU baseline.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
HOST_LINK_PEAK_GBS = 64.0      # PCIe 5.0 x16, one direction
BF16_MFMA_PEAK_TFLOPS = 2500.0
CSRC = os.path.join(ROOT, "paged_kv_cache_371_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 1 << 30
SETTLE_S = 0.05   # seconds of untimed steps before the warm-up (clock settle)


# Sources that decide what one pa_attention_varlen call moves: its argument
# checks and launch configuration, the kernels it runs, their shared headers.
ATTENTION_SOURCES = ("decode.hip", "decode_gqa.hip", "pa_api.cpp", "pa_common.h", "pa_internal.h", "plan.hip",
                     "prefill.hip")


def kernel_source_digest(names=ATTENTION_SOURCES) -> str:
    """sha256 over the named library sources (file names and bytes, in sorted order)."""
    import hashlib

    h = hashlib.sha256()
    for name in sorted(names):
        h.update(name.encode())
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


BLOCK_COPY_SOURCES = ("block_copy.hip", "pa_common.h")


def measured_block_traffic(workload: str):
    """HBM bytes per block-copy launch from the committed counter summary, or
    None when there is none or the copy kernel changed since it was taken."""
    import re

    path = os.path.join(PROFILES, f"copy_blocks_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    dig = re.search(r"^source_sha256:\s*([0-9a-f]{64})", text, re.M)
    val = re.search(r"^traffic_bytes_per_launch:\s*(\d+)", text, re.M)
    if not dig or not val or dig.group(1) != kernel_source_digest(BLOCK_COPY_SOURCES):
        return None
    return int(val.group(1))


def measured_traffic(workload: str):
    """HBM bytes per attention call from the committed counter summary, or None
    when there is none or the kernels changed since it was taken."""
    import re

    path = os.path.join(PROFILES, f"attention_call_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    dig = re.search(r"^source_sha256:\s*([0-9a-f]{64})", text, re.M)
    val = re.search(r"^traffic_bytes_per_call:\s*(\d+)", text, re.M)
    if not dig or not val or dig.group(1) != kernel_source_digest():
        return None
    return int(val.group(1))


K_SCALE_FP8, V_SCALE_FP8 = 0.5, 0.25


def fp8_codes(shape, seed: int) -> np.ndarray:
    """Random finite OCP E4M3 codes of magnitude below 16 (the 8-bit pools' contents)."""
    rng = np.random.default_rng(seed)
    e = rng.integers(0, 11, shape)
    m = rng.integers(0, 8, shape)
    sgn = rng.integers(0, 2, shape)
    return ((sgn << 7) | (e << 3) | m).astype(np.uint8)


def algorithmic_bytes(c, kv_elem_bytes=None, window: int = 0) -> dict:
    """Bytes the attention must move for this batch (no re-reads, no partial-block over-read).

    With a sliding window only the keys some row of the request sees count:
    from its first row's window start to the end of its context."""
    s = 2 if c.dtype == "bf16" else 4
    kvs = s if kv_elem_bytes is None else kv_elem_bytes
    L = c.seq_lens.astype(np.int64)
    n = c.q_lens.astype(np.int64)
    keys = L if window <= 0 else L - np.maximum(0, L - n - window + 1)
    kv = int((keys * c.num_kv_heads * c.head_dim * 2 * kvs).sum())
    q = int(n.sum() * c.num_q_heads * c.head_dim * s)
    o = q
    tables = int(4 * (-(-keys // int(c.block_size))).sum())
    meta = 4 * (2 * c.num_seqs + 1)
    cw = int(2 * (s + kvs) * (c.slot_mapping >= 0).sum() * c.num_kv_heads * c.head_dim + 8 * c.total_q)
    return dict(kv=kv, q=q, o=o, tables=tables, meta=meta, attention=kv + q + o + tables + meta, cache_write=cw)


def unique_kv_bytes(c, kv_elem_bytes=None) -> int:
    """K/V bytes of the distinct physical blocks the batch reads (a block shared by
    several requests counted once, each with the most tokens any of them reads)."""
    s = 2 if c.dtype == "bf16" else 4
    kvs = s if kv_elem_bytes is None else kv_elem_bytes
    bs = int(c.block_size)
    tokens = {}
    for b, L in enumerate(c.seq_lens.astype(np.int64)):
        for j in range(-(-int(L) // bs)):
            blk = int(c.block_tables[b, j])
            tokens[blk] = max(tokens.get(blk, 0), min(bs, int(L) - j * bs))
    return int(sum(tokens.values()) * c.num_kv_heads * c.head_dim * 2 * kvs)


def attention_kernels(c) -> str:
    """The kernels one layer's pa_attention_run launches for this batch (bf16, D = 128, G <= 8)."""
    k = "pa_attention_run (one layer over the step's work lists): decode_gqa_kernel + merge_list_kernel"
    if c.max_query_len > 1:
        k += " + prefill_kernel"
    return k


def attention_flops(c, window: int = 0) -> float:
    """4 * D * Hq per (row, visible key)."""
    L = c.seq_lens.astype(np.int64)
    n = c.q_lens.astype(np.int64)
    keys = 0
    for Lb, nb in zip(L, n):
        for j in range(int(nb)):
            p = int(Lb) - int(nb) + j
            keys += p + 1 if window <= 0 else min(p + 1, window)
    return 4.0 * c.head_dim * c.num_q_heads * keys


def cpu_model() -> str:
    """The host CPU's model name (first 'model name' line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(c, budget_s: float = 12.0, fp8_pools=None, window: int = 0, pool=None) -> dict:
    """Time the fp64 oracle on the batch's rows, on one core and on all cores.

    The batch's rows are cut into pieces of about equal cost (a piece is some
    rows of one request; a decode request is one piece), taken in a fixed
    shuffled order.  Each piece is one call of the oracle over its request.
    One core: pieces in order, in passes over the batch, until half the
    budget is spent (one BLAS thread).  All cores (``pool``: one worker
    process per core, one BLAS thread each, the inputs memory-mapped from
    files written beforehand): the next pieces in the same order, as many as
    take about half the budget at the one-core rate times the workers.  KV
    bytes of a piece are its request's K/V bytes times its share of the
    request's rows.  With ``fp8_pools`` (K and V codes) the oracle attends
    over the 8-bit pools."""
    import oracle
    from oracle.sharded import SharedBatch, run_piece, run_pieces, split_rows

    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        limit = None
    meta = dict(scale=c.scale, num_kv_heads=c.num_kv_heads, dtype=c.dtype, block_size=c.block_size,
                sliding_window=window)
    if fp8_pools is None:
        kp, vp = oracle.oracle_cache_write(c.k_cache, c.v_cache, c.k_new, c.v_new, c.slot_mapping, c.block_size)
        s = 2 if c.dtype == "bf16" else 4
    else:
        kp, vp = oracle.oracle_cache_write(fp8_pools[0], fp8_pools[1],
                                           oracle.fp8_quantize_rows(c.k_new, K_SCALE_FP8),
                                           oracle.fp8_quantize_rows(c.v_new, V_SCALE_FP8), c.slot_mapping,
                                           c.block_size)
        meta.update(kv_dtype="fp8", k_scale=K_SCALE_FP8, v_scale=V_SCALE_FP8)
        s = 1

    def kv_of(b, rows):
        Lb, nb = int(c.seq_lens[b]), int(c.cu_seqlens[b + 1] - c.cu_seqlens[b])
        keys = Lb if window <= 0 else Lb - max(0, Lb - nb - window + 1)
        return keys * c.num_kv_heads * c.head_dim * 2 * s * rows / nb

    pieces = split_rows(c.cu_seqlens, c.seq_lens, pieces=max(1024, 4 * c.num_seqs), window=window)
    pieces = [pieces[i] for i in np.random.default_rng(1).permutation(len(pieces))]
    arrays = dict(q=c.q, k=kp, v=vp, cu=c.cu_seqlens, lens=c.seq_lens, tables=c.block_tables)
    one_budget = budget_s / 2 if pool is not None else budget_s
    done_rows = done_kv = done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < one_budget:
        b, js = pieces[done % len(pieces)]
        run_piece(arrays, meta, b, js)
        done_rows += len(js)
        done_kv += kv_of(b, len(js))
        done += 1
    dt = time.perf_counter() - t0
    if limit is not None and hasattr(limit, "unregister"):
        limit.unregister()
    model = cpu_model()
    one = {"value": done_kv / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"{done} pieces ({done_rows} query rows, {done_kv / 1e9:.3f} GB of KV) of the "
                     f"{c.num_seqs}-request batch in passes over it, in {dt:.1f} s, fp64 NumPy, one process, "
                     f"one BLAS thread",
           "query_tokens_per_s": done_rows / dt}
    if pool is None:
        one["cpu_model"] = model
        return one

    workers = pool._max_workers  # noqa: SLF001
    want_kv = one["value"] * 1e9 * workers * (budget_s / 2)
    sample, kv, rows = [], 0.0, 0
    i = 0
    while not sample or kv < want_kv:    # in passes over the batch, like the one-core leg
        b, js = pieces[(done + i) % len(pieces)]
        sample.append((b, js))
        kv += kv_of(b, len(js))
        rows += len(js)
        i += 1
    with SharedBatch(c.q, kp, vp, c.cu_seqlens, c.seq_lens, c.block_tables, **meta) as batch:
        t0 = time.perf_counter()
        run_pieces(batch, sample, pool)
        dt_all = time.perf_counter() - t0
    return {"value": kv / dt_all / 1e9, "unit": "GB/s", "cores": workers, "kind": "oracle",
            "sample": f"{len(sample)} pieces ({rows} query rows, {kv / 1e9:.3f} GB of KV) of the "
                      f"{c.num_seqs}-request batch in passes over it, in {dt_all:.1f} s wall on a pool of {workers} "
                      f"worker processes "
                      f"(one BLAS thread each, inputs memory-mapped), fp64 NumPy",
            "query_tokens_per_s": rows / dt_all,
            "cpu_model": model,
            "one_core": one}


def calibrate_copy() -> None:
    """One device-to-device copy of COPY_BYTES (the counter calibration run)."""
    import torch

    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": COPY_BYTES}), flush=True)


class _DeviceBatch:
    """The workload's arrays in HBM, and the two ABI calls of one step."""

    def __init__(self, c, torch, pa, fp8_pools=None, window=0):
        self.c, self.torch, self.pa = c, torch, pa
        self.fp8 = fp8_pools is not None
        self.window = window

        def dev(a):
            if c.dtype == "bf16":
                return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda:0").view(torch.bfloat16)
            return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")

        self.q = dev(c.q)
        if self.fp8:
            self.k_cache = torch.from_numpy(fp8_pools[0]).to("cuda:0")
            self.v_cache = torch.from_numpy(fp8_pools[1]).to("cuda:0")
        else:
            self.k_cache, self.v_cache = dev(c.k_cache), dev(c.v_cache)
        self.k_new, self.v_new = dev(c.k_new), dev(c.v_new)
        self.slots = torch.from_numpy(c.slot_mapping).to("cuda:0")
        self.cu = torch.from_numpy(c.cu_seqlens).to("cuda:0")
        self.seq_lens = torch.from_numpy(c.seq_lens).to("cuda:0")
        self.tables = torch.from_numpy(c.block_tables).to("cuda:0")
        self.out = torch.empty_like(self.q)
        self.ws = None
        self.partition_size = None
        self._fast = {}

    def prepare(self, partition_size):
        """Marshal the step's C calls once (after a checked call): the timed loops
        then make only the C calls, so the host's per-call Python work does not
        hold the GPU back (prepare_* of the binding)."""
        pa, c = self.pa, self.c
        if getattr(self, "k_new", None) is None:   # a batch without new rows (the multi-row sub-batch)
            pass
        elif self.fp8:
            self._fast["cw"] = pa.prepare_cache_write_fp8(self.k_new, self.v_new, self.k_cache, self.v_cache,
                                                          self.slots, K_SCALE_FP8, V_SCALE_FP8)
        else:
            self._fast["cw"] = pa.prepare_cache_write(self.k_new, self.v_new, self.k_cache, self.v_cache, self.slots)
        for stage in ("all", "plan", "run"):
            self._fast[stage] = pa.prepare_attention_varlen(
                self.out, self.q, self.k_cache, self.v_cache, self.cu, self.seq_lens, self.tables, float(c.scale),
                c.max_query_len, c.max_seq_len, workspace=self.ws, partition_size=partition_size,
                sliding_window=self.window, k_scale=K_SCALE_FP8 if self.fp8 else None,
                v_scale=V_SCALE_FP8 if self.fp8 else None, stage=stage, num_decode_rows=int((c.q_lens == 1).sum()))

    def cache_write(self):
        if "cw" in self._fast:
            self._fast["cw"]()
        elif self.fp8:
            self.pa.cache_write_fp8(self.k_new, self.v_new, self.k_cache, self.v_cache, self.slots, K_SCALE_FP8,
                                    V_SCALE_FP8)
        else:
            self.pa.cache_write(self.k_new, self.v_new, self.k_cache, self.v_cache, self.slots)

    def attention(self, partition_size, stage="all"):
        c = self.c
        if self.ws is None:
            p = self.pa.make_params(self.q, self.k_cache, self.cu, self.tables, c.num_kv_heads, float(c.scale),
                                    c.max_query_len, c.max_seq_len, out=self.out, partition_size=partition_size,
                                    sliding_window=self.window)
            self.ws = self.torch.empty(max(16, self.pa.workspace_size(p)), dtype=self.torch.uint8, device="cuda:0")
            self.partition_size = self.pa.partition_size(p)
        if stage in self._fast:
            self._fast[stage]()
            return
        self.pa.attention_varlen(self.out, self.q, self.k_cache, self.v_cache, self.cu, self.seq_lens, self.tables,
                                 float(c.scale), c.max_query_len, c.max_seq_len, workspace=self.ws,
                                 partition_size=partition_size, sliding_window=self.window,
                                 k_scale=K_SCALE_FP8 if self.fp8 else None,
                                 v_scale=V_SCALE_FP8 if self.fp8 else None, stage=stage,
                                 num_decode_rows=int((c.q_lens == 1).sum()))


class _MultiRowBatch:
    """The multi-row requests of a device batch as a batch of their own: their
    query rows copied out, the same pools and block-table rows, own workspace."""

    def __init__(self, dc, torch):
        c = dc.c
        idx = np.nonzero(c.q_lens > 1)[0]
        rows = np.concatenate([np.arange(c.cu_seqlens[b], c.cu_seqlens[b + 1]) for b in idx]).astype(np.int64)
        q_lens = c.q_lens[idx]
        cu = np.zeros(len(idx) + 1, dtype=c.cu_seqlens.dtype)
        cu[1:] = np.cumsum(q_lens)
        self.c = _SubConfig(c, idx, q_lens, cu)
        self.torch, self.pa, self.fp8, self.window = torch, dc.pa, dc.fp8, dc.window
        dev = dc.q.device
        self.q = dc.q[torch.from_numpy(rows).to(dev)].contiguous()
        self.k_cache, self.v_cache = dc.k_cache, dc.v_cache
        self.cu = torch.from_numpy(cu).to(dev)
        self.seq_lens = torch.from_numpy(np.ascontiguousarray(c.seq_lens[idx])).to(dev)
        self.tables = torch.from_numpy(np.ascontiguousarray(c.block_tables[idx])).to(dev)
        self.out = torch.empty_like(self.q)
        self.ws = None
        self.partition_size = None
        self._fast = {}

    attention = _DeviceBatch.attention
    prepare = _DeviceBatch.prepare


class _SubConfig:
    """The fields of a workload config that the attention call and the flop count read, for a subset of its requests."""

    def __init__(self, c, idx, q_lens, cu):
        self.num_kv_heads, self.num_q_heads, self.head_dim = c.num_kv_heads, c.num_q_heads, c.head_dim
        self.scale, self.block_size = c.scale, c.block_size
        self.q_lens, self.seq_lens, self.cu_seqlens = q_lens, c.seq_lens[idx], cu
        self.num_seqs, self.total_q = len(idx), int(q_lens.sum())
        self.max_query_len, self.max_seq_len = int(q_lens.max()), int(self.seq_lens.max())


def profiled_kernel_us(workload: str, kernel: str):
    """Average duration of a kernel in the committed kernel-trace summary of the
    workload, or None when there is none or the kernels changed since it was taken."""
    import re

    path = os.path.join(PROFILES, f"attention_call_{workload}_kernels.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    dig = re.search(r"^source_sha256:\s*([0-9a-f]{64})", text, re.M)
    row = re.search(r"^\| `pa::" + kernel + r"<[^`]*>` \| \d+ \| ([0-9.]+) \|", text, re.M)
    if not dig or not row or dig.group(1) != kernel_source_digest():
        return None
    return float(row.group(1))


def _timed_loop(torch, fn, steps, warmup, stream):
    """Warm up, then time `steps` calls of fn with HIP events on `stream` and the host clock."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall * 1e3 / steps, float(np.mean([a.elapsed_time(b) for a, b in ev]))


def _block_result(args, metric, value, ms_step, dtype, config, roofline, cpu):
    out = {
        "metric": metric, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dtype, "data": "synthetic", "config": config, "roofline": roofline,
    }
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


COW_BLOCKS, COW_PAIRS = 16384, 4096
LAYER_SHAPE = (8, 16, 128)      # Hkv, tokens per block, D of the Llama-3-70B-shaped GQA layer


def _oracle_block_rate(fn, block_bytes, pairs_per_call, budget_s):
    calls = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        fn()
        calls += 1
    dt = time.perf_counter() - t0
    return calls, dt, 2 * 2 * block_bytes * pairs_per_call * calls / dt / 1e9


def run_copy_blocks(args) -> None:
    """Copy-on-write copies of one parallel-sampling decode step: 4096 samples
    each copy their shared, partly filled last block (K and V, 32 KiB each in
    the GQA layer's bf16 pools of 16384 blocks) to a fresh block.  Moves
    2 x 4096 x 64 KiB = 512 MiB of HBM per call (every byte read once and
    written once)."""
    import torch

    import paged_kv_cache_371_amd as pa

    rng = np.random.default_rng(args.seed)
    perm = rng.permutation(COW_BLOCKS)
    pairs = np.stack([perm[:COW_PAIRS], perm[COW_PAIRS:2 * COW_PAIRS]], 1).astype(np.int64)
    shape = (COW_BLOCKS,) + LAYER_SHAPE
    k = torch.randn(shape, dtype=torch.bfloat16, device="cuda:0")
    v = torch.randn(shape, dtype=torch.bfloat16, device="cuda:0")
    dpairs = torch.from_numpy(pairs).to("cuda:0")
    L = pa.lib()
    block_bytes = k[0].numel() * k.element_size()
    stream = torch.cuda.current_stream()

    def call():
        pa._check(L.pa_copy_blocks(k.data_ptr(), v.data_ptr(), dpairs.data_ptr(), COW_PAIRS, block_bytes,
                                   COW_BLOCKS, stream.cuda_stream))

    call()
    torch.cuda.synchronize()
    src, dst = torch.from_numpy(pairs[:, 0]).to("cuda:0"), torch.from_numpy(pairs[:, 1]).to("cuda:0")
    if not (torch.equal(k[dst], k[src]) and torch.equal(v[dst], v[src])):
        raise SystemExit("block copy mismatch")
    ms_step, kern_ms = _timed_loop(torch, call, args.steps, args.warmup, stream)
    moved = 2 * 2 * COW_PAIRS * block_bytes
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        nb, npairs = 1024, 256
        hk = np.zeros((nb,) + LAYER_SHAPE, np.uint16)
        hv = np.zeros_like(hk)
        small = _small_pairs(nb, npairs)
        calls, dt, rate = _oracle_block_rate(lambda: oracle.oracle_copy_blocks(hk, hv, small), block_bytes, npairs,
                                             args.cpu_budget)
        cpu = {"value": round(rate, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{calls} calls of the oracle's block copy, {npairs} pairs over a {nb}-block pool of the "
                         f"same block shape, in {dt:.1f} s"}
    roof = {"bound": "hbm", "kernel": "pa::copy_blocks_kernel", "achieved": round(moved / (kern_ms * 1e-3) / 1e9, 2),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(moved / (kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": measured_block_traffic("cow_copy_gqa_layer"), "algorithmic_bytes_per_launch": moved}
    _block_result(args, "copy-on-write block copy GB/s (HBM read + write) at 1 MI355X", moved / (ms_step * 1e-3) / 1e9,
                  ms_step, "bf16",
                  {"workload": "cow_copy_gqa_layer", "num_blocks": COW_BLOCKS, "pairs_per_call": COW_PAIRS,
                   "block_shape": list(LAYER_SHAPE), "block_bytes_per_pool": block_bytes,
                   "step": "pa_copy_blocks (K and V)"}, roof, cpu)


def _small_pairs(nb, n):
    perm = np.random.default_rng(7).permutation(nb)
    return np.stack([perm[:n], perm[n:2 * n]], 1).astype(np.int64)


SWAP_LAYERS, SWAP_BLOCKS = 80, 512


def run_swap(args, direction: str) -> None:
    """Swap of one 8192-token sequence of an 80-layer Llama-3-70B-shaped cache
    (GQA, 8 KV heads, D=128, bf16): 512 blocks per layer, K and V, 32 KiB each
    -- 2.5 GiB per step, one pa_swap_blocks call per layer, between the
    device pools and a pinned host pool."""
    import torch

    import paged_kv_cache_371_amd as pa

    rng = np.random.default_rng(args.seed)
    nb_dev = 2 * SWAP_BLOCKS
    dshape = (SWAP_LAYERS, nb_dev) + LAYER_SHAPE
    hshape = (SWAP_LAYERS, SWAP_BLOCKS) + LAYER_SHAPE
    dk = torch.randn(dshape, dtype=torch.bfloat16, device="cuda:0")
    dv = torch.randn(dshape, dtype=torch.bfloat16, device="cuda:0")
    hk = torch.empty(hshape, dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty(hshape, dtype=torch.bfloat16, pin_memory=True)
    dev_blocks = rng.permutation(nb_dev)[:SWAP_BLOCKS]
    host_blocks = np.arange(SWAP_BLOCKS)
    if direction == "swap_out":
        pairs = np.stack([dev_blocks, host_blocks], 1).astype(np.int64)
        layers = [(hk[l], hv[l], dk[l], dv[l], SWAP_BLOCKS, nb_dev) for l in range(SWAP_LAYERS)]
    else:
        pairs = np.stack([host_blocks, dev_blocks], 1).astype(np.int64)
        layers = [(dk[l], dv[l], hk[l], hv[l], nb_dev, SWAP_BLOCKS) for l in range(SWAP_LAYERS)]
    if direction == "swap_in":
        hk.copy_(dk[:, dev_blocks].cpu())
        hv.copy_(dv[:, dev_blocks].cpu())
    dpairs = torch.from_numpy(pairs).to("cuda:0")
    L = pa.lib()
    block_bytes = dk[0, 0].numel() * dk.element_size()
    stream = torch.cuda.current_stream()

    def step():
        for dst_k, dst_v, src_k, src_v, ndst, nsrc in layers:
            pa._check(L.pa_swap_blocks(dst_k.data_ptr(), dst_v.data_ptr(), src_k.data_ptr(), src_v.data_ptr(),
                                       dpairs.data_ptr(), SWAP_BLOCKS, block_bytes, nsrc, ndst, stream.cuda_stream))

    step()
    torch.cuda.synchronize()
    idx = torch.from_numpy(dev_blocks).to("cuda:0")
    for l in (0, SWAP_LAYERS - 1):
        a = dk[l, idx].cpu()
        if not torch.equal(a.view(torch.int16), hk[l].view(torch.int16)):
            raise SystemExit("swap mismatch")
    ms_step, kern_ms = _timed_loop(torch, step, args.steps, args.warmup, stream)
    per_step = SWAP_LAYERS * 2 * SWAP_BLOCKS * block_bytes
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        h1k, h1v = np.zeros((SWAP_BLOCKS,) + LAYER_SHAPE, np.uint16), np.zeros((SWAP_BLOCKS,) + LAYER_SHAPE, np.uint16)
        d1k, d1v = np.zeros((nb_dev,) + LAYER_SHAPE, np.uint16), np.zeros((nb_dev,) + LAYER_SHAPE, np.uint16)
        calls, dt, rate = _oracle_block_rate(lambda: oracle.oracle_swap_blocks(h1k, h1v, d1k, d1v,
                                                                               np.stack([dev_blocks, host_blocks], 1)),
                                             block_bytes, SWAP_BLOCKS, args.cpu_budget)
        cpu = {"value": round(rate / 2, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{calls} calls of the oracle's block swap of one layer ({SWAP_BLOCKS} blocks, K and V) "
                         f"between host arrays, in {dt:.1f} s; bytes counted once"}
    achieved = per_step / SWAP_LAYERS / (kern_ms / SWAP_LAYERS * 1e-3) / 1e9
    roof = {"bound": "host_link", "kernel": "pa::copy_blocks_kernel", "achieved": round(achieved, 2),
            "peak": HOST_LINK_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HOST_LINK_PEAK_GBS, 4),
            "traffic": None, "algorithmic_bytes_per_launch": per_step // SWAP_LAYERS}
    _block_result(args, f"KV {direction.replace('_', '-')} GB/s over the host link at 1 MI355X",
                  per_step / (ms_step * 1e-3) / 1e9, ms_step, "bf16",
                  {"workload": f"{direction}_8k_seq_70b", "layers": SWAP_LAYERS, "blocks_per_layer": SWAP_BLOCKS,
                   "block_shape": list(LAYER_SHAPE), "bytes_per_step": per_step,
                   "step": f"{SWAP_LAYERS} x pa_swap_blocks (K and V)"}, roof, cpu)


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gqa_decode_bf16")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--partition-size", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of CPU baseline: half on one core, half on all cores")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="worker processes of the all-core CPU baseline (0: the host cores, at most 16; "
                         "1: one-core baseline only)")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--kv-dtype", choices=("bf16", "fp8"), default="bf16",
                    help="fp8: 8-bit (OCP E4M3) pools with per-tensor scales, bf16 q and out")
    ap.add_argument("--op", choices=("attention", "copy_blocks", "swap_out", "swap_in"), default="attention")
    ap.add_argument("--sliding-window", type=int, default=0,
                    help="W > 0: each row sees only the last W positions up to its own")
    ap.add_argument("--block-size", type=int, default=16, choices=(8, 16, 32),
                    help="tokens per physical block")
    ap.add_argument("--flush-cache", dest="flush_cache", action="store_true", default=True,
                    help="(default) before each timed plan/run call, read a 1 GiB buffer (outside the events) so "
                         "the L2s and the Infinity Cache hold none of the batch; the run stage is timed unflushed "
                         "as well and reported beside it")
    ap.add_argument("--no-flush-cache", dest="flush_cache", action="store_false",
                    help="time the plan/run calls back to back only")
    ap.add_argument("--multi-row-only", action="store_true",
                    help="the workload's multi-row requests alone, laid out as a batch of their own (the same "
                         "lengths, heads and block size; workload name + '_multirow')")
    ap.add_argument("--no-prefill-alone", action="store_true",
                    help="skip timing the call over the multi-row requests alone (profiler runs: its decode and "
                         "merge launches have empty lists and would enter those kernels' per-dispatch figures)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this framework runs the path on one GPU; --gpus must be 1 "
                                   "(sharding across GPUs is designed, not built)"}))
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.op == "copy_blocks":
        run_copy_blocks(args)
        return
    if args.op in ("swap_out", "swap_in"):
        run_swap(args, args.op)
        return

    # The CPU baseline's worker processes start before anything touches the GPU.
    cpu_pool = None
    if not args.no_cpu_baseline and args.cpu_workers != 1:
        from oracle.sharded import host_workers, make_pool

        cpu_pool = make_pool(args.cpu_workers or host_workers())

    import torch

    import paged_kv_cache_371_amd as pa
    from workloads import make_config

    c = make_config(args.workload, args.seed, poison=False, block_size=args.block_size)
    if args.multi_row_only:
        from workloads import build_case

        keep = c.q_lens > 1
        if not keep.any():
            raise SystemExit("the workload has no multi-row requests")
        c = build_case(c.name + "_multirow", args.seed, c.dtype, c.num_q_heads, c.num_kv_heads, c.head_dim,
                       c.q_lens[keep], c.seq_lens[keep], poison=False, block_size=c.block_size,
                       rescale_tables=c.block_size != 16)
    fp8 = args.kv_dtype == "fp8"
    if fp8 and c.dtype != "bf16":
        raise SystemExit("8-bit pools need a bf16 workload")
    pools8 = (fp8_codes(c.k_cache.shape, 1000 + args.seed), fp8_codes(c.v_cache.shape, 2000 + args.seed)) if fp8 \
        else None
    W = args.sliding_window
    dc = _DeviceBatch(c, torch, pa, pools8, W)
    ab = algorithmic_bytes(c, 1 if fp8 else None, W)
    flops = attention_flops(c, W)
    stream = torch.cuda.current_stream()

    def step():
        dc.cache_write()
        dc.attention(partition_size=args.partition_size)

    step()
    torch.cuda.synchronize()
    if not bool(torch.isfinite(dc.out.float()).all()):
        raise SystemExit("non-finite attention output")
    dc.prepare(args.partition_size)

    # Clock settle: the GPU reaches its sustained clocks only after some tens of
    # milliseconds of work (with 5 warm-up steps, ~1.5 ms, the timed steps ran
    # 3% slower than after 50).  The step runs untimed until SETTLE_S seconds
    # have passed, then the W warm-up steps, then the K timed ones.
    settle_steps = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < SETTLE_S:
        for _ in range(10):
            step()
        settle_steps += 10
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        dc.cache_write()
        ev[i][1].record(stream)
        dc.attention(partition_size=args.partition_size)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    cw_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    attn_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    ms_per_step = wall * 1e3 / args.steps

    # The two stages of the call on their own: the work lists (pa_attention_plan,
    # built once per step from the request lengths and shared by every layer)
    # and one layer's attention over them (pa_attention_run), each timed with
    # HIP events on the launch stream.
    flush_buf = torch.ones(COPY_BYTES // 4, dtype=torch.int32, device="cuda:0") if args.flush_cache else None

    def stage_ms(stage, flush, batch=dc):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i, (a_, b_) in enumerate(evs):
            if flush:   # a read of 1 GiB: evicts with clean lines, leaves nothing to write back
                flush_buf.sum()
            a_.record(stream)
            batch.attention(partition_size=args.partition_size, stage=stage)
            b_.record(stream)
        torch.cuda.synchronize()
        return np.array([a_.elapsed_time(b_) for a_, b_ in evs])

    flushed = flush_buf is not None
    plan_ms = float(stage_ms("plan", flushed).mean())
    run_unflushed = stage_ms("run", False)
    run_all = stage_ms("run", True) if flushed else run_unflushed
    run_ms = float(run_all.mean())

    # The prefill kernel on its own: the same call over the batch's multi-row
    # requests alone (same pools and table rows), whose run stage is the
    # prefill kernel plus the decode and merge launches with empty lists.
    prefill = None
    if c.max_query_len > 1 and not args.no_prefill_alone:
        sub = _MultiRowBatch(dc, torch)
        sub.attention(partition_size=args.partition_size, stage="plan")
        sub.prepare(args.partition_size)
        sub_run = stage_ms("run", flushed, batch=sub)
        sub_ms = float(sub_run.mean())
        sub_flops = attention_flops(sub.c, W)
        prefill = {
            "what": "pa_attention_run over the multi-row requests alone: prefill_kernel, plus the decode and "
                    "merge kernels launched with empty work lists",
            "requests": int(sub.c.num_seqs),
            "rows": int(sub.c.total_q),
            "run_ms": round(sub_ms, 5),
            "flops": sub_flops,
            "tflops": round(sub_flops / (sub_ms * 1e-3) / 1e12, 2),
            "peak_tflops": BF16_MFMA_PEAK_TFLOPS,
            "mfma_frac": round(sub_flops / (sub_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
            "profiled_prefill_kernel_us": (profiled_kernel_us(c.name + "_multirow", "prefill_kernel")
                                           if not fp8 and not W else None),
        }

    value = ab["kv"] / (ms_per_step * 1e-3) / 1e9
    achieved = ab["attention"] / (run_ms * 1e-3) / 1e9
    call_gbs = ab["attention"] / (attn_ms * 1e-3) / 1e9
    result = {
        "metric": "paged-attn decode KV GB/s (% of HBM peak) and query tokens/s at 1 MI355X",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle_steps,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c.dtype,
        "data": "synthetic",
        "config": {
            "workload": c.name,
            "seed": args.seed,
            "num_seqs": c.num_seqs,
            "total_q": c.total_q,
            "num_q_heads": c.num_q_heads,
            "num_kv_heads": c.num_kv_heads,
            "head_dim": c.head_dim,
            "block_size": c.block_size,
            "num_blocks": c.num_blocks,
            "mean_context": float(c.seq_lens.mean()),
            "partition_size": dc.partition_size,
            "kv_dtype": "fp8_e4m3" if fp8 else c.dtype,
            "sliding_window": W,
            "caches_flushed_before_each_run": bool(args.flush_cache),
            "step": "cache_write + attention_varlen",
        },
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "query_tokens_per_s": round(c.total_q / (ms_per_step * 1e-3), 1),
        "attention_ms": round(attn_ms, 5),
        "attention_run_ms": round(run_ms, 5),
        "attention_run_ms_p10_p50_p90": [round(float(x), 5) for x in np.percentile(run_all, [10, 50, 90])],
        "attention_run_ms_unflushed": round(float(run_unflushed.mean()), 5),
        "attention_run_frac_unflushed": round(ab["attention"] / (float(run_unflushed.mean()) * 1e-3) / 1e9
                                              / HBM_PEAK_GBS, 4),
        "attention_plan_ms": round(plan_ms, 5),
        "cache_write_ms": round(cw_ms, 5),
        "kv_bytes_per_step": ab["kv"],
        "kv_unique_bytes": unique_kv_bytes(c, 1 if fp8 else None),
        "unique_kv_gbs_run": round(unique_kv_bytes(c, 1 if fp8 else None) / (run_ms * 1e-3) / 1e9, 1),
        "roofline": {
            "bound": "hbm",
            "kernel": attention_kernels(c),
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "call_frac_incl_plan": round(call_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(c.name + ("_fp8kv" if fp8 else "") + (f"_w{W}" if W else "")
                                        + (f"_bs{c.block_size}" if c.block_size != 16 else "")),
            "algorithmic_bytes_per_launch": ab["attention"],
            "attention_tflops": round(flops / (attn_ms * 1e-3) / 1e12, 3),
        },
    }
    if c.max_query_len > 1:
        # A step with multi-row requests against its two bounds: the larger of
        # its HBM time and its matrix-core time (both overlapped perfectly), and
        # their sum (nothing overlapped).
        bytes_ms = ab["attention"] / (HBM_PEAK_GBS * 1e9) * 1e3
        flops_ms = flops / (BF16_MFMA_PEAK_TFLOPS * 1e12) * 1e3
        result["roofline"]["combined"] = {
            "hbm_ms": round(bytes_ms, 5),
            "mfma_ms": round(flops_ms, 5),
            "max_bound_ms": round(max(bytes_ms, flops_ms), 5),
            "frac_of_max_bound": round(max(bytes_ms, flops_ms) / run_ms, 4),
            "sum_bound_ms": round(bytes_ms + flops_ms, 5),
            "frac_of_sum_bound": round((bytes_ms + flops_ms) / run_ms, 4),
        }
    if prefill is not None:
        result["prefill_kernel"] = prefill
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(c, args.cpu_budget, pools8, W, pool=cpu_pool)
    if cpu_pool is not None:
        cpu_pool.shutdown()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
