"""Python binding of the paged-attention C ABI (``include/pa.h``, ``include/pa_blocks.h``).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the computation runs in the HIP kernels of
``libpa.so``.  The library must be built first
(``python -m paged_kv_cache_371_amd.build``); nothing here falls back to
another implementation when it is missing.
"""

from __future__ import annotations

import ctypes
import os

__all__ = [
    "PAError",
    "AttnParams",
    "lib",
    "lib_path",
    "exported_symbols",
    "cache_write",
    "attention_varlen",
    "attention_varlen_noalloc",
    "make_params",
    "workspace_size",
    "validate_metadata",
    "copy_blocks",
    "swap_blocks",
    "BlockManager",
    "OutOfBlocks",
    "PA_F32",
    "PA_BF16",
]

PA_F32 = 0
PA_BF16 = 1
BLOCK_SIZE = 16

# Bits reported by validate_metadata (mirrors PA_BAD_* in pa.h).
BAD_CU_SEQLENS = 1
BAD_LENGTHS = 2
BAD_TABLE_WIDTH = 4
BAD_BLOCK_ID = 8
BAD_SLOT_RANGE = 16
BAD_SLOT_DUP = 32

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

# Every function pa.h declares, with its ctypes signature.
_SIGNATURES = {
    "pa_cache_write": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]),
    "pa_attention_workspace_size": (ctypes.c_size_t, [ctypes.c_void_p]),
    "pa_attention_partition_size": (ctypes.c_int32, [ctypes.c_void_p]),
    "pa_attention_varlen": (ctypes.c_int, [ctypes.c_void_p] * 7 + [ctypes.c_void_p, ctypes.c_void_p,
                                                                 ctypes.c_size_t, ctypes.c_void_p]),
    "pa_validate_metadata": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "pa_cache_write_fp8": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                          ctypes.c_float, ctypes.c_void_p]),
    "pa_attention_varlen_fp8": (ctypes.c_int, [ctypes.c_void_p] * 7 + [ctypes.c_void_p, ctypes.c_float, ctypes.c_float,
                                                                     ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "pa_attention_varlen_noalloc": (ctypes.c_int, [ctypes.c_void_p] * 9),
    "pa_attention_plan": (ctypes.c_int, [ctypes.c_void_p] * 4 + [ctypes.c_size_t, ctypes.c_void_p]),
    "pa_attention_run": (ctypes.c_int, [ctypes.c_void_p] * 7 + [ctypes.c_void_p, ctypes.c_void_p,
                                                              ctypes.c_size_t, ctypes.c_void_p]),
    "pa_attention_run_fp8": (ctypes.c_int, [ctypes.c_void_p] * 7 + [ctypes.c_void_p, ctypes.c_float, ctypes.c_float,
                                                                  ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "pa_copy_blocks": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]),
    "pa_swap_blocks": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 4 + [ctypes.c_void_p]),
    "pa_bm_create": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p]),
    "pa_bm_destroy": (None, [ctypes.c_void_p]),
    "pa_bm_add_sequence": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                          ctypes.c_void_p]),
    "pa_bm_fork": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64]),
    "pa_bm_append_slot": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p]),
    "pa_bm_free": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64]),
    "pa_bm_swap_out": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                      ctypes.c_void_p]),
    "pa_bm_swap_in": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.c_void_p]),
    "pa_bm_block_table": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_void_p]),
    "pa_bm_block_tables": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                          ctypes.c_int32, ctypes.c_void_p]),
    "pa_bm_slot_mapping": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_void_p]),
    "pa_bm_seq_info": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]),
    "pa_bm_refcount": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]),
    "pa_bm_stats": (ctypes.c_int, [ctypes.c_void_p] * 5),
    "pa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pa_abi_version": (ctypes.c_int32, []),
}


class PAError(RuntimeError):
    """A non-zero pa_status returned by the library."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class OutOfBlocks(PAError):
    """PA_ERR_NO_BLOCKS: the block manager lacks free blocks; nothing changed."""


ERR_NO_BLOCKS = -8
ERR_STATE = -9


class AttnParams(ctypes.Structure):
    """Mirror of ``pa_attn_params``."""

    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("total_q", ctypes.c_int64),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int64),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("max_query_len", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
        ("q_row_stride", ctypes.c_int64),
        ("o_row_stride", ctypes.c_int64),
        ("scale", ctypes.c_float),
        ("dtype", ctypes.c_int),
        ("partition_size", ctypes.c_int32),
        ("sliding_window", ctypes.c_int32),
        ("num_decode_rows", ctypes.c_int32),
    ]


def lib_path() -> str:
    return os.environ.get("PA_LIB", os.path.join(_HERE, "libpa.so"))


def lib() -> ctypes.CDLL:
    """Load libpa.so once; raise if it has not been built."""
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m paged_kv_cache_371_amd.build`")
        handle = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def exported_symbols():
    return tuple(_SIGNATURES)


def _check(status: int) -> None:
    if status != 0:
        msg = lib().pa_status_string(status)
        cls = OutOfBlocks if status == ERR_NO_BLOCKS else PAError
        raise cls(status, msg.decode() if msg else f"pa_status {status}")


def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _stream(stream) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t


def _call(fn, args, prepare: bool, keep=()):
    """Make the C call now, or (prepare) return a function of no arguments that
    makes exactly this call (the same pointers and stream) each time it is called."""
    if prepare:
        def call(_fn=fn, _args=args, _keep=keep):
            _check(_fn(*_args))
        return call
    _check(fn(*args))
    return None


def cache_write(k_new, v_new, k_cache, v_cache, slot_mapping, stream=None, _prepare: bool = False):
    """Scatter new K/V rows [N, Hkv, D] into pools [NB, Hkv, 16, D] via int64 slots."""
    torch = _torch()
    for t, nm in ((k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                  (slot_mapping, "slot_mapping")):
        _dev(t, nm)
    if slot_mapping.dtype != torch.int64 or not slot_mapping.is_contiguous():
        raise TypeError("slot_mapping must be a contiguous int64 tensor")
    if k_new.shape != v_new.shape or k_new.stride() != v_new.stride():
        raise ValueError("k_new and v_new must share shape and strides")
    if k_cache.shape != v_cache.shape or not (k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("pools must be contiguous [NB, Hkv, 16, D] tensors of one shape")
    if k_new.dtype != k_cache.dtype or v_new.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype:
        raise TypeError("all K/V tensors must share one dtype")
    N, Hkv, D = k_new.shape
    if k_new.stride(2) != 1 or k_new.stride(1) != D:
        raise ValueError("each new row must hold contiguous [Hkv, D]")
    if slot_mapping.shape[0] != N:
        raise ValueError("slot_mapping must have one entry per new row")
    NB, Hc, bs, Dc = k_cache.shape
    if Hc != Hkv or Dc != D:
        raise ValueError("pool heads/head_dim differ from the new rows")
    return _call(lib().pa_cache_write, (k_new.data_ptr(), v_new.data_ptr(), k_new.stride(0), k_cache.data_ptr(),
                                        v_cache.data_ptr(), slot_mapping.data_ptr(), N, Hkv, D, bs, NB,
                                        _dtype_code(k_cache), _stream(stream)), _prepare)


def cache_write_fp8(k_new, v_new, k_cache, v_cache, slot_mapping, k_scale: float, v_scale: float,
                    stream=None, _prepare: bool = False):
    """Quantise new bf16 K/V rows [N, Hkv, D] into 8-bit (OCP E4M3) pools
    [NB, Hkv, 16, D] (uint8 tensors) with per-pool scales."""
    torch = _torch()
    for t, nm in ((k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                  (slot_mapping, "slot_mapping")):
        _dev(t, nm)
    if slot_mapping.dtype != torch.int64 or not slot_mapping.is_contiguous():
        raise TypeError("slot_mapping must be a contiguous int64 tensor")
    if k_new.dtype != torch.bfloat16 or v_new.dtype != torch.bfloat16:
        raise TypeError("new rows must be bf16")
    if k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
        raise TypeError("8-bit pools must be uint8 tensors")
    if k_new.shape != v_new.shape or k_new.stride() != v_new.stride():
        raise ValueError("k_new and v_new must share shape and strides")
    if k_cache.shape != v_cache.shape or not (k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("pools must be contiguous [NB, Hkv, 16, D] tensors of one shape")
    N, Hkv, D = k_new.shape
    if k_new.stride(2) != 1 or k_new.stride(1) != D:
        raise ValueError("each new row must hold contiguous [Hkv, D]")
    if slot_mapping.shape[0] != N:
        raise ValueError("slot_mapping must have one entry per new row")
    NB, Hc, bs, Dc = k_cache.shape
    if Hc != Hkv or Dc != D:
        raise ValueError("pool heads/head_dim differ from the new rows")
    return _call(lib().pa_cache_write_fp8, (k_new.data_ptr(), v_new.data_ptr(), k_new.stride(0), k_cache.data_ptr(),
                                            v_cache.data_ptr(), slot_mapping.data_ptr(), N, Hkv, D, bs, NB,
                                            float(k_scale), float(v_scale), _stream(stream)), _prepare)


def make_params(q, k_cache, cu_seqlens, block_tables, num_kv_heads: int, scale: float, max_query_len: int,
                max_seq_len: int, out=None, partition_size: int = 0, sliding_window: int = 0,
                num_decode_rows: int = 0) -> AttnParams:
    total_q, Hq, D = q.shape
    p = AttnParams()
    p.num_seqs = int(cu_seqlens.shape[0]) - 1
    p.total_q = int(total_q)
    p.num_q_heads = int(Hq)
    p.num_kv_heads = int(num_kv_heads)
    p.head_dim = int(D)
    p.block_size = int(k_cache.shape[2])
    p.num_blocks = int(k_cache.shape[0])
    p.max_blocks_per_seq = int(block_tables.shape[1])
    p.max_query_len = int(max_query_len)
    p.max_seq_len = int(max_seq_len)
    p.q_row_stride = int(q.stride(0))
    p.o_row_stride = int(out.stride(0) if out is not None else Hq * D)
    p.scale = float(scale)
    p.dtype = _dtype_code(q)
    p.partition_size = int(partition_size)
    p.sliding_window = int(sliding_window)
    p.num_decode_rows = int(num_decode_rows)
    return p


def workspace_size(params: AttnParams) -> int:
    return int(lib().pa_attention_workspace_size(ctypes.byref(params)))


def partition_size(params: AttnParams) -> int:
    """Context-partition length the attention call uses for ``params`` (0 if they are invalid)."""
    return int(lib().pa_attention_partition_size(ctypes.byref(params)))


def attention_varlen(out, q, k_cache, v_cache, cu_seqlens, seq_lens, block_tables, scale: float,
                     max_query_len: int, max_seq_len: int, workspace=None, partition_size: int = 0,
                     stream=None, k_scale=None, v_scale=None, sliding_window: int = 0, stage: str = "all",
                     num_decode_rows: int = 0, _prepare: bool = False):
    """Paged causal attention of packed rows; writes ``out`` [total_q, Hq, D] and returns it.

    ``sliding_window`` W > 0 limits each row to the last W positions up to
    its own.  ``num_decode_rows``: the host's count of requests with one query
    row (0: none or unknown); scheduling only (pa_attn_params.num_decode_rows).  ``stage``: "all" (pa_attention_varlen), "plan" (only the work
    lists, pa_attention_plan: once per step, into ``workspace``) or "run" (one
    layer over the lists already in ``workspace``, pa_attention_run).

    ``workspace`` (a contiguous device tensor of any dtype, at least
    ``workspace_size`` bytes) is allocated here when not given.  uint8 pools
    hold 8-bit (OCP E4M3) codes: q and out are then bf16 and ``k_scale`` /
    ``v_scale`` give the pools' scales.
    """
    torch = _torch()
    for t, nm in ((out, "out"), (q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (cu_seqlens, "cu_seqlens"),
                  (seq_lens, "seq_lens"), (block_tables, "block_tables")):
        _dev(t, nm)
    for t, nm in ((cu_seqlens, "cu_seqlens"), (seq_lens, "seq_lens"), (block_tables, "block_tables")):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise TypeError(f"{nm} must be a contiguous int32 tensor")
    if q.dim() != 3 or out.shape != q.shape:
        raise ValueError("q and out must be [total_q, Hq, D]")
    if q.stride(2) != 1 or q.stride(1) != q.shape[2] or out.stride(2) != 1 or out.stride(1) != out.shape[2]:
        raise ValueError("q and out rows must hold contiguous [Hq, D]")
    if not (k_cache.is_contiguous() and v_cache.is_contiguous()) or k_cache.shape != v_cache.shape:
        raise ValueError("pools must be contiguous [NB, Hkv, 16, D] tensors of one shape")
    fp8 = k_cache.dtype == torch.uint8
    if fp8:
        if v_cache.dtype != torch.uint8 or q.dtype != torch.bfloat16 or out.dtype != torch.bfloat16:
            raise TypeError("8-bit pools need uint8 K and V pools and bf16 q and out")
        if k_scale is None or v_scale is None:
            raise ValueError("8-bit pools need k_scale and v_scale")
    elif len({q.dtype, out.dtype, k_cache.dtype, v_cache.dtype}) != 1:
        raise TypeError("q, out and the pools must share one dtype")
    if seq_lens.shape[0] != cu_seqlens.shape[0] - 1 or block_tables.shape[0] != seq_lens.shape[0]:
        raise ValueError("cu_seqlens [B+1], seq_lens [B] and block_tables [B, W] disagree on B")
    num_kv_heads = int(k_cache.shape[1])
    p = make_params(q, k_cache, cu_seqlens, block_tables, num_kv_heads, scale, max_query_len, max_seq_len,
                    out=out, partition_size=partition_size, sliding_window=sliding_window,
                    num_decode_rows=num_decode_rows)
    need = workspace_size(p)
    if workspace is None:
        if stage != "all":
            raise ValueError("the plan and run stages share a workspace: pass one")
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    ws_bytes = workspace.numel() * workspace.element_size()
    if stage not in ("all", "plan", "run"):
        raise ValueError("stage must be 'all', 'plan' or 'run'")
    keep = (p, workspace)
    if stage == "plan":
        call = _call(lib().pa_attention_plan, (cu_seqlens.data_ptr(), seq_lens.data_ptr(), ctypes.byref(p),
                                               workspace.data_ptr(), ws_bytes, _stream(stream)), _prepare, keep)
    elif fp8:
        fn = lib().pa_attention_run_fp8 if stage == "run" else lib().pa_attention_varlen_fp8
        call = _call(fn, (out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), cu_seqlens.data_ptr(),
                          seq_lens.data_ptr(), block_tables.data_ptr(), ctypes.byref(p), float(k_scale),
                          float(v_scale), workspace.data_ptr(), ws_bytes, _stream(stream)), _prepare, keep)
    else:
        fn = lib().pa_attention_run if stage == "run" else lib().pa_attention_varlen
        call = _call(fn, (out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), cu_seqlens.data_ptr(),
                          seq_lens.data_ptr(), block_tables.data_ptr(), ctypes.byref(p), workspace.data_ptr(),
                          ws_bytes, _stream(stream)), _prepare, keep)
    return call if _prepare else out


def prepare_cache_write(*args, **kwargs):
    """``cache_write`` with its checks and argument marshalling done once: returns
    a function of no arguments that makes only the C call (the same tensors and
    stream) each time -- for loops that repeat one step."""
    return cache_write(*args, _prepare=True, **kwargs)


def prepare_cache_write_fp8(*args, **kwargs):
    """``cache_write_fp8`` prepared the same way (see ``prepare_cache_write``)."""
    return cache_write_fp8(*args, _prepare=True, **kwargs)


def prepare_attention_varlen(*args, **kwargs):
    """``attention_varlen`` prepared the same way (see ``prepare_cache_write``); a
    workspace it allocates is kept alive by the returned function."""
    return attention_varlen(*args, _prepare=True, **kwargs)


NOALLOC_SCRATCH_BYTES = 64 << 20   # PA_NOALLOC_SCRATCH_BYTES


def attention_varlen_noalloc(out, q, k_cache, v_cache, cu_seqlens, seq_lens, block_tables, scale: float,
                             max_query_len: int, max_seq_len: int, partition_size: int = 0, stream=None,
                             sliding_window: int = 0, num_decode_rows: int = 0):
    """``attention_varlen`` through pa_attention_varlen_noalloc: no workspace, the
    library's static per-GPU scratch instead (bf16 or fp32 pools)."""
    torch = _torch()
    for t, nm in ((out, "out"), (q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (cu_seqlens, "cu_seqlens"),
                  (seq_lens, "seq_lens"), (block_tables, "block_tables")):
        _dev(t, nm)
    for t, nm in ((cu_seqlens, "cu_seqlens"), (seq_lens, "seq_lens"), (block_tables, "block_tables")):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise TypeError(f"{nm} must be a contiguous int32 tensor")
    if q.dim() != 3 or out.shape != q.shape:
        raise ValueError("q and out must be [total_q, Hq, D]")
    if q.stride(2) != 1 or q.stride(1) != q.shape[2] or out.stride(2) != 1 or out.stride(1) != out.shape[2]:
        raise ValueError("q and out rows must hold contiguous [Hq, D]")
    if not (k_cache.is_contiguous() and v_cache.is_contiguous()) or k_cache.shape != v_cache.shape:
        raise ValueError("pools must be contiguous [NB, Hkv, 16, D] tensors of one shape")
    if len({q.dtype, out.dtype, k_cache.dtype, v_cache.dtype}) != 1:
        raise TypeError("q, out and the pools must share one dtype")
    if seq_lens.shape[0] != cu_seqlens.shape[0] - 1 or block_tables.shape[0] != seq_lens.shape[0]:
        raise ValueError("cu_seqlens [B+1], seq_lens [B] and block_tables [B, W] disagree on B")
    p = make_params(q, k_cache, cu_seqlens, block_tables, int(k_cache.shape[1]), scale, max_query_len, max_seq_len,
                    out=out, partition_size=partition_size, sliding_window=sliding_window,
                    num_decode_rows=num_decode_rows)
    _check(lib().pa_attention_varlen_noalloc(out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                             cu_seqlens.data_ptr(), seq_lens.data_ptr(), block_tables.data_ptr(),
                                             ctypes.byref(p), _stream(stream)))
    return out


def validate_metadata(cu_seqlens, seq_lens, block_tables, num_blocks: int, max_query_len: int,
                      max_seq_len: int, slot_mapping=None, stream=None, block_size: int = BLOCK_SIZE) -> int:
    """Run the device checks and return the PA_BAD_* bitmask (0 = all pass).  Synchronises."""
    torch = _torch()
    p = AttnParams()
    p.num_seqs = int(seq_lens.shape[0])
    p.total_q = int(cu_seqlens[-1].item()) if p.num_seqs else 0
    p.num_blocks = int(num_blocks)
    p.block_size = int(block_size)
    p.max_blocks_per_seq = int(block_tables.shape[1])
    p.max_query_len = int(max_query_len)
    p.max_seq_len = int(max_seq_len)
    result = torch.empty(1, dtype=torch.int32, device=seq_lens.device)
    n_slots = int(slot_mapping.shape[0]) if slot_mapping is not None else 0
    _check(lib().pa_validate_metadata(cu_seqlens.data_ptr(), seq_lens.data_ptr(), block_tables.data_ptr(),
                                      slot_mapping.data_ptr() if slot_mapping is not None else None, n_slots,
                                      ctypes.byref(p), result.data_ptr(), _stream(stream)))
    return int(result.item())


# ---------------------------------------------------------------------------
# block copies and the host block manager (include/pa_blocks.h)


def _pairs_arg(pairs, device):
    """(src, dst) pairs as a contiguous int64 [n, 2] tensor on ``device``."""
    torch = _torch()
    if not torch.is_tensor(pairs):
        pairs = torch.as_tensor(pairs, dtype=torch.int64).reshape(-1, 2)
    if pairs.dtype != torch.int64:
        raise TypeError("block pairs must be int64")
    pairs = pairs.reshape(-1, 2)
    if pairs.device != device:
        pairs = pairs.to(device)
    return pairs.contiguous()


def _block_bytes(pool) -> int:
    if not pool.is_contiguous():
        raise ValueError("pools must be contiguous")
    return pool[0].numel() * pool.element_size()


def copy_blocks(k_cache, v_cache, pairs, stream=None) -> None:
    """Copy-on-write copies inside one layer's pools: block dst <- block src for
    every (src, dst) pair, K and V, bit for bit (any pool dtype)."""
    _dev(k_cache, "k_cache")
    _dev(v_cache, "v_cache")
    if k_cache.shape != v_cache.shape or k_cache.dtype != v_cache.dtype:
        raise ValueError("K and V pools must share shape and dtype")
    pairs = _pairs_arg(pairs, k_cache.device)
    _check(lib().pa_copy_blocks(k_cache.data_ptr(), v_cache.data_ptr(), pairs.data_ptr(), int(pairs.shape[0]),
                                _block_bytes(k_cache), int(k_cache.shape[0]), _stream(stream)))
    return pairs


def swap_blocks(dst_k, dst_v, src_k, src_v, pairs, stream=None):
    """dst[d] <- src[s] for every (s, d) pair between two pools of one block
    shape; one side is usually a pinned host pool (swap out or swap in).
    Returns the device copy of ``pairs``, which must stay alive until the
    stream has run the copy."""
    dev = next((t.device for t in (dst_k, src_k) if t.is_cuda), None)
    if dev is None:
        raise ValueError("one side of a swap must be a device pool")
    for t, nm in ((dst_k, "dst_k"), (dst_v, "dst_v"), (src_k, "src_k"), (src_v, "src_v")):
        if not t.is_cuda and not t.is_pinned():
            raise ValueError(f"{nm}: host pools must be pinned (pin_memory=True)")
    if dst_k.shape[1:] != src_k.shape[1:] or dst_k.dtype != src_k.dtype:
        raise ValueError("pools must share block shape and dtype")
    if dst_k.shape != dst_v.shape or src_k.shape != src_v.shape:
        raise ValueError("K and V pools must share shapes")
    pairs = _pairs_arg(pairs, dev)
    _check(lib().pa_swap_blocks(dst_k.data_ptr(), dst_v.data_ptr(), src_k.data_ptr(), src_v.data_ptr(),
                                pairs.data_ptr(), int(pairs.shape[0]), _block_bytes(dst_k), int(src_k.shape[0]),
                                int(dst_k.shape[0]), _stream(stream)))
    return pairs


def _i64(v=0):
    return ctypes.c_int64(v)


class BlockManager:
    """Host block manager (native): free pool, block tables, reference counts
    with copy-on-write, prefix keys with LRU eviction, host pool for swap."""

    def __init__(self, num_blocks: int, block_size: int = BLOCK_SIZE, num_host_blocks: int = 0,
                 prefix_caching: bool = True):
        h = ctypes.c_void_p()
        _check(lib().pa_bm_create(int(num_blocks), int(block_size), int(num_host_blocks), int(bool(prefix_caching)),
                                  ctypes.byref(h)))
        self._h = h
        self.block_size = int(block_size)
        self.num_blocks = int(num_blocks)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _LIB is not None:
            _LIB.pa_bm_destroy(h)
            self._h = None

    def add_sequence(self, seq_id: int, tokens) -> int:
        arr = (ctypes.c_int32 * len(tokens))(*[int(t) for t in tokens])
        cached = _i64()
        _check(lib().pa_bm_add_sequence(self._h, int(seq_id), arr, len(tokens), ctypes.byref(cached)))
        return cached.value

    def fork(self, parent: int, child: int) -> None:
        _check(lib().pa_bm_fork(self._h, int(parent), int(child)))

    def append_slot(self, seq_id: int, token: int):
        slot, src, dst = _i64(), _i64(), _i64()
        _check(lib().pa_bm_append_slot(self._h, int(seq_id), int(token), ctypes.byref(slot), ctypes.byref(src),
                                       ctypes.byref(dst)))
        return slot.value, src.value, dst.value

    def free(self, seq_id: int) -> None:
        _check(lib().pa_bm_free(self._h, int(seq_id)))

    def _swap(self, fn, seq_id):
        cap = len(self.table(seq_id))
        buf = (ctypes.c_int64 * (2 * max(cap, 1)))()
        n = _i64()
        _check(fn(self._h, int(seq_id), buf, cap, ctypes.byref(n)))
        return [(buf[2 * i], buf[2 * i + 1]) for i in range(n.value)]

    def swap_out(self, seq_id: int):
        return self._swap(lib().pa_bm_swap_out, seq_id)

    def swap_in(self, seq_id: int):
        return self._swap(lib().pa_bm_swap_in, seq_id)

    def table(self, seq_id: int):
        n = _i64()
        st = lib().pa_bm_block_table(self._h, int(seq_id), None, 0, ctypes.byref(n))
        if st not in (0, -2):
            _check(st)
        buf = (ctypes.c_int32 * max(n.value, 1))()
        _check(lib().pa_bm_block_table(self._h, int(seq_id), buf, n.value, ctypes.byref(n)))
        return list(buf[:n.value])

    def block_tables(self, seq_ids, width: int):
        """Padded [len(seq_ids), width] int32 tables and int32 lengths (numpy)."""
        import numpy as np

        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        tables = np.zeros((len(ids), max(width, 0)), np.int32)
        lens = np.zeros(len(ids), np.int32)
        _check(lib().pa_bm_block_tables(self._h, ids.ctypes.data, len(ids), tables.ctypes.data, int(width),
                                        lens.ctypes.data))
        return tables, lens

    def slot_mapping(self, seq_id: int, start: int, count: int):
        buf = (ctypes.c_int64 * max(count, 1))()
        _check(lib().pa_bm_slot_mapping(self._h, int(seq_id), int(start), int(count), buf))
        return list(buf[:count])

    def _info(self, seq_id):
        n, sw = _i64(), ctypes.c_int32()
        _check(lib().pa_bm_seq_info(self._h, int(seq_id), ctypes.byref(n), ctypes.byref(sw)))
        return n.value, bool(sw.value)

    def seq_len(self, seq_id: int) -> int:
        return self._info(seq_id)[0]

    def is_swapped(self, seq_id: int) -> bool:
        return self._info(seq_id)[1]

    def refcount(self, block: int) -> int:
        c = ctypes.c_int32()
        _check(lib().pa_bm_refcount(self._h, int(block), ctypes.byref(c)))
        return c.value

    def _stats(self):
        f, c, h, s = _i64(), _i64(), _i64(), _i64()
        _check(lib().pa_bm_stats(self._h, ctypes.byref(f), ctypes.byref(c), ctypes.byref(h), ctypes.byref(s)))
        return f.value, c.value, h.value, s.value

    def num_free(self) -> int:
        return self._stats()[0]

    def num_cached(self) -> int:
        return self._stats()[1]

    def num_host_free(self) -> int:
        return self._stats()[2]

    def num_seqs(self) -> int:
        return self._stats()[3]
