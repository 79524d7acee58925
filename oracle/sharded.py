"""The attention oracle run over a pool of worker processes (test infrastructure).

Test infrastructure only: the product library never imports this module.

``oracle_attention_sharded`` returns exactly what ``oracle_attention_varlen``
returns for the same arguments, bit for bit: every output row is computed by
``oracle_attention_varlen`` itself, in a worker process, called on one
request at a time (its packed rows, its context length, its block-table row
and the whole pools).  A request's result depends only on that request, so
the rows come out the same as in one call over the batch.  What this module
adds is bookkeeping only: it writes the inputs once to memory-mapped files
(under /dev/shm when it exists) that every worker maps read-only, cuts the
wanted rows into pieces of about equal cost (a row costs its number of
visible keys), and puts the returned rows in place.  No attention arithmetic
happens here.

Workers are started with the ``spawn`` method, so each is a fresh
interpreter that imports only NumPy and this package; every worker uses one
BLAS thread.
"""

from __future__ import annotations

import multiprocessing as mp
import os
import shutil
import tempfile
from concurrent.futures import ProcessPoolExecutor

import numpy as np

from .paged_attention import first_visible_key, last_visible_key, oracle_attention_varlen


def host_workers(limit: int = 16) -> int:
    """Worker count: the host cores this process may run on, at most ``limit``."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(limit, n))


def _one_blas_thread() -> None:
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    try:
        from threadpoolctl import threadpool_limits

        threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        pass


def _noop(i):
    return i


def make_pool(workers: int | None = None) -> ProcessPoolExecutor:
    """A spawn-started process pool whose workers use one BLAS thread each.

    The workers are started before this returns (one trivial task each), so
    a caller can create the pool early and time only the work it submits."""
    n = workers or host_workers()
    ex = ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn"), initializer=_one_blas_thread)
    list(ex.map(_noop, range(n)))
    return ex


class SharedBatch:
    """A batch's oracle inputs as .npy files that workers map read-only.

    Arrays: q, k (pool), v (pool), cu, lens, tables.  ``meta`` holds the
    scalar arguments of oracle_attention_varlen.  Use as a context manager;
    the files are removed on exit."""

    def __init__(self, q, k_cache, v_cache, cu_seqlens, seq_lens, block_tables, **meta):
        base = "/dev/shm" if os.path.isdir("/dev/shm") and os.access("/dev/shm", os.W_OK) else None
        self.dir = tempfile.mkdtemp(prefix="pa_oracle_", dir=base)
        self.paths = {}
        arrays = dict(q=q, k=k_cache, v=v_cache, cu=cu_seqlens, lens=seq_lens, tables=block_tables)
        try:
            for name, arr in arrays.items():
                path = os.path.join(self.dir, name + ".npy")
                np.save(path, np.ascontiguousarray(arr), allow_pickle=False)
                self.paths[name] = path
        except BaseException:
            self.close()
            raise
        self.meta = meta
        self.cu = np.asarray(cu_seqlens, np.int64)
        self.lens = np.asarray(seq_lens, np.int64)
        self.shape = tuple(np.shape(q))

    def close(self):
        shutil.rmtree(self.dir, ignore_errors=True)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def handle(self):
        return (tuple(sorted(self.paths.items())), tuple(sorted(self.meta.items())))


def _arrays(paths) -> dict:
    """The batch's arrays mapped read-only (mapped per piece, so no mapping
    outlives the files once the batch is closed)."""
    return {name: np.load(path, mmap_mode="r", allow_pickle=False) for name, path in paths}


def run_piece(arrays: dict, meta: dict, b: int, js):
    """Rows js (indices within request b) of oracle_attention_varlen, computed
    by a call over request b alone; returns an fp64 [len(js), Hq, D] array."""
    cu = arrays["cu"]
    q0, q1 = int(cu[b]), int(cu[b + 1])
    out = oracle_attention_varlen(arrays["q"][q0:q1], arrays["k"], arrays["v"], np.array([0, q1 - q0], np.int64),
                                  arrays["lens"][b:b + 1], arrays["tables"][b:b + 1], rows=list(js), validate=False,
                                  **meta)
    return out[list(js)]


def _worker_piece(task):
    handle, b, js = task
    paths, meta = handle
    return run_piece(_arrays(paths), dict(meta), b, js)


def _row_cost(L: int, n: int, j: int, window: int) -> int:
    return last_visible_key(L, n, j) - first_visible_key(L, n, j, window) + 1


def split_rows(cu_seqlens, seq_lens, rows=None, pieces: int = 64, window: int = 0):
    """Pieces (request, [row indices within the request]) of about equal cost,
    largest first; every wanted row is in exactly one piece."""
    cu = np.asarray(cu_seqlens, np.int64)
    L_all = np.asarray(seq_lens, np.int64)
    want = None if rows is None else set(int(r) for r in rows)
    per_req = []
    total = 0
    for b in range(L_all.shape[0]):
        q0, q1 = int(cu[b]), int(cu[b + 1])
        n, L = q1 - q0, int(L_all[b])
        js = [r - q0 for r in range(q0, q1) if want is None or r in want]
        if not js:
            continue
        costs = [_row_cost(L, n, j, window) for j in js]
        per_req.append((b, js, costs))
        total += sum(costs)
    target = max(1, total // max(1, pieces))
    out = []
    for b, js, costs in per_req:
        cur, acc = [], 0
        for j, cst in zip(js, costs):
            cur.append(j)
            acc += cst
            if acc >= target:
                out.append((acc, b, cur))
                cur, acc = [], 0
        if cur:
            out.append((acc, b, cur))
    out.sort(key=lambda t: -t[0])
    return [(b, js) for _, b, js in out]


def run_pieces(batch: SharedBatch, pieces, pool: ProcessPoolExecutor) -> np.ndarray:
    """The pieces' rows on the pool; an fp64 [total_q, Hq, D] array, NaN elsewhere."""
    out = np.full(batch.shape, np.nan, np.float64)
    handle = batch.handle()
    nw = pool._max_workers  # noqa: SLF001 -- the pool's size
    inflight = []

    def place(item):
        q0, js, fut = item
        out[q0 + np.asarray(js, np.int64)] = fut.result()

    for b, js in pieces:
        inflight.append((int(batch.cu[b]), js, pool.submit(_worker_piece, (handle, b, tuple(js)))))
        while len(inflight) >= 4 * nw:
            place(inflight.pop(0))
    for item in inflight:
        place(item)
    return out


def oracle_attention_sharded(q, k_cache, v_cache, cu_seqlens, seq_lens, block_tables, scale, num_kv_heads: int,
                             dtype: str, block_size: int = 16, rows=None, kv_dtype: str | None = None,
                             k_scale: float = 1.0, v_scale: float = 1.0, sliding_window: int = 0,
                             pool: ProcessPoolExecutor | None = None, workers: int | None = None):
    """``oracle_attention_varlen`` (same arguments and result) computed by a process pool.

    ``pool``: an executor from ``make_pool`` to reuse; otherwise one is made
    for this call and shut down afterwards."""
    meta = dict(scale=scale, num_kv_heads=num_kv_heads, dtype=dtype, block_size=block_size, kv_dtype=kv_dtype,
                k_scale=k_scale, v_scale=v_scale, sliding_window=sliding_window)
    own = pool is None
    ex = make_pool(workers) if own else pool
    try:
        with SharedBatch(q, k_cache, v_cache, cu_seqlens, seq_lens, block_tables, **meta) as batch:
            pieces = split_rows(cu_seqlens, seq_lens, rows, pieces=8 * ex._max_workers,  # noqa: SLF001
                                window=sliding_window)
            return run_pieces(batch, pieces, ex)
    finally:
        if own:
            ex.shutdown()
