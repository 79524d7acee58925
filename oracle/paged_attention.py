"""fp64 CPU oracle: cache write and paged causal attention (test infrastructure).

Readings taken where the pages leave a step open (each is also pinned by a
CPU test):
  * Context includes this step's rows: new K/V are appended first, then the
    kernel reads history through the block table (quant67 §3.3, per-decode
    step order).  Row j of a request with n rows and context L sits at
    position L - n + j and sees keys 0 .. L - n + j (bottom-right causal).
  * GQA: query head h reads KV head h // G with G = Hq / Hkv (contiguous
    groups).
  * Pool layout: separate K and V pools ``[num_blocks, Hkv, block_size, D]``;
    one block id covers every KV head (the per-block byte count in quant67
    §8.3 includes num_kv_heads) and each head's block is a contiguous tile.
  * Slot encoding: slot = physical_block * block_size + offset (quant67 §3.3
    worked example: token 18 of table [17, 42] -> block 42, offset 2).
  * Negative slot = row already present, nothing written.  Duplicate slots
    are a precondition violation and raise.
  * scale is the fp32 value the caller passes, widened exactly to fp64.
"""

from __future__ import annotations

import math

import numpy as np


class OracleError(ValueError):
    """A precondition of the operation does not hold."""


# ---------------------------------------------------------------------------
# encodings


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of stored elements (fp32 values or bf16 bit patterns)."""
    if dtype == "bf16":
        return (np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "fp8":
        return fp8_e4m3_decode(x)
    raise OracleError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# 8-bit float cache encoding (OCP FP8 E4M3, the "FN" variant)
#
# The pages name FP8 KV caches as the next step for memory (quant67 §8.8 and
# §10.3) without fixing a format; the reading taken is the OCP 8-bit floating
# point E4M3 format: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
# bits; exponent 0 holds the subnormals m * 2^-9; there are no infinities;
# S.1111.111 is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448.
# Encoding rounds to nearest, ties to an even mantissa, and saturates
# magnitudes beyond 448 to 448.

FP8_MAX = 448.0


def fp8_e4m3_decode(codes) -> np.ndarray:
    """fp64 value of each E4M3 code (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def fp8_e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code of each fp32 value: ties to even, saturating at 448, NaN to 0x7F."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    out = np.empty(x.shape, np.uint8)
    flat_x, flat_o = x.reshape(-1), out.reshape(-1)
    for i, v in enumerate(flat_x.tolist()):
        if math.isnan(v):
            flat_o[i] = 0x7F
            continue
        sign = 0x80 if math.copysign(1.0, v) < 0 else 0
        a = abs(v)
        if a >= FP8_MAX:
            flat_o[i] = sign | 0x7E
            continue
        # the spacing of representable values around a: 2^-9 below 2^-6
        # (subnormals), else 2^(floor(log2 a) - 3)
        e = max(math.floor(math.log2(a)), -6) if a > 0 else -6
        quantum = 2.0 ** (e - 3)
        n = a / quantum                      # exact: a power-of-two scaling
        r = math.floor(n)
        frac = n - r
        if frac > 0.5 or (frac == 0.5 and r % 2 == 1):
            r += 1                           # round to nearest, ties to even
        val = r * quantum
        if val >= FP8_MAX:
            flat_o[i] = sign | 0x7E
        elif val < 2.0 ** -6:
            flat_o[i] = sign | int(round(val / 2.0 ** -9))
        else:
            ev = math.floor(math.log2(val))
            mant = int(round((val / 2.0 ** ev - 1.0) * 8))
            flat_o[i] = sign | ((ev + 7) << 3) | mant
    return out


def fp8_quantize_rows(x_bf16, scale) -> np.ndarray:
    """Cache codes of bf16 rows stored with a per-tensor scale: each value is
    divided by the fp32 scale in fp32 (rounded to nearest), then encoded."""
    xf = (np.asarray(x_bf16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    y = (xf / np.float32(scale)).astype(np.float32)
    return fp8_e4m3_encode(y)


# ---------------------------------------------------------------------------
# the three small rules the rest is built from


def physical_location(block_table_row: np.ndarray, t: int, block_size: int = 16):
    """(physical block, offset) of logical token t (quant67 §3.3 address rule)."""
    return int(block_table_row[t // block_size]), t % block_size


def kv_head_of(h: int, group: int) -> int:
    """KV head read by query head h when G = group query heads share one."""
    return h // group


def last_visible_key(seq_len: int, q_len: int, j: int) -> int:
    """Last key position row j may attend to (bottom-right causal alignment)."""
    return seq_len - q_len + j


def first_visible_key(seq_len: int, q_len: int, j: int, sliding_window: int = 0) -> int:
    """First key position row j may attend to: 0, or with a sliding window of
    W > 0 tokens the oldest of the last W positions up to its own (the pages
    list the sliding-window mask among the kernel variants, quant67 §10.8 FAQ,
    without defining it; the window is read as the row's own position and the
    W - 1 before it)."""
    if sliding_window <= 0:
        return 0
    return max(0, last_visible_key(seq_len, q_len, j) - sliding_window + 1)


# ---------------------------------------------------------------------------
# metadata


def validate_metadata(cu_seqlens, seq_lens, block_tables, num_blocks, block_size=16,
                      num_q_heads=None, num_kv_heads=None):
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    L = np.asarray(seq_lens, dtype=np.int64)
    bt = np.asarray(block_tables)
    B = L.shape[0]
    if cu.shape != (B + 1,):
        raise OracleError("cu_seqlens must have num_seqs + 1 entries")
    if cu[0] != 0 or (np.diff(cu) < 0).any():
        raise OracleError("cu_seqlens must start at 0 and be nondecreasing")
    n = np.diff(cu)
    if (n > L).any() or (L < 0).any():
        raise OracleError("need 0 <= q_len <= seq_len for every request")
    if bt.ndim != 2 or bt.shape[0] != B:
        raise OracleError("block_tables must be [num_seqs, max_blocks_per_seq]")
    for b in range(B):
        used = -(-int(L[b]) // block_size)
        if used > bt.shape[1]:
            raise OracleError(f"request {b}: {used} blocks exceed the table width")
        ids = bt[b, :used]
        if ((ids < 0) | (ids >= num_blocks)).any():
            raise OracleError(f"request {b}: block id out of range")
    if num_q_heads is not None and num_kv_heads is not None:
        if num_kv_heads <= 0 or num_q_heads % num_kv_heads:
            raise OracleError("num_q_heads must be a positive multiple of num_kv_heads")


# ---------------------------------------------------------------------------
# cache write (quant67 §3.3: the new token's K/V are appended to its block)


def oracle_cache_write(k_cache, v_cache, k_new, v_new, slot_mapping, block_size: int = 16):
    """Return copies of the pools with each new row stored at its slot.

    Row i goes to block ``slot // block_size``, offset ``slot % block_size``, for
    every KV head; rows with a negative slot are skipped.  The copy is of the
    stored encoding, so the result is exact.
    """
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    nb = k_out.shape[0]
    seen = set()
    for i, s in enumerate(slots.tolist()):
        if s < 0:
            continue
        if s >= nb * block_size:
            raise OracleError(f"row {i}: slot {s} outside the pool")
        if s in seen:
            raise OracleError(f"row {i}: slot {s} written twice")
        seen.add(s)
        blk, off = s // block_size, s % block_size
        k_out[blk, :, off, :] = k_new[i]
        v_out[blk, :, off, :] = v_new[i]
    return k_out, v_out


# ---------------------------------------------------------------------------
# attention


def gather_request_kv(cache, block_table_row, seq_len: int, dtype: str, block_size: int = 16):
    """Contiguous fp64 [seq_len, Hkv, D] copy of one request's cached tokens."""
    out = np.empty((seq_len, cache.shape[1], cache.shape[3]), np.float64)
    for t in range(0, seq_len, block_size):
        blk, _ = physical_location(block_table_row, t, block_size)
        m = min(block_size, seq_len - t)
        # cache[blk] is [Hkv, bs, D]; tokens t .. t+m-1 are its first m offsets
        out[t:t + m] = widen(cache[blk][:, :m, :], dtype).transpose(1, 0, 2)
    return out


def oracle_attention_varlen(q, k_cache, v_cache, cu_seqlens, seq_lens, block_tables,
                            scale, num_kv_heads: int, dtype: str, block_size: int = 16,
                            rows=None, validate: bool = True, kv_dtype: str | None = None,
                            k_scale: float = 1.0, v_scale: float = 1.0, sliding_window: int = 0):
    """Causal softmax attention of packed query rows over a paged KV cache.

    q: [total_q, Hq, D]; returns fp64 [total_q, Hq, D] (rows not computed stay
    NaN).  ``rows`` optionally limits the work to a subset of packed rows.
    For request b with rows cu[b] .. cu[b+1]-1 and context L_b, each query
    head h and row j:  s = scale * K[0..p] q,  o = softmax(s) V[0..p],  with
    p = L_b - n_b + j and K, V gathered through the block table.  The pools
    hold ``kv_dtype`` (default: ``dtype``); with 8-bit codes the cached values
    are the decoded codes times ``k_scale`` / ``v_scale`` (fp32, widened).
    With ``sliding_window`` W > 0 the keys are further limited to the last W
    positions up to p (``first_visible_key``).
    """
    q = np.asarray(q)
    total_q, Hq, D = q.shape
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    L_all = np.asarray(seq_lens, dtype=np.int64)
    bt = np.asarray(block_tables)
    if validate:
        validate_metadata(cu, L_all, bt, k_cache.shape[0], block_size, Hq, num_kv_heads)
    if cu[-1] != total_q:
        raise OracleError("cu_seqlens[-1] must equal the number of packed rows")
    G = Hq // num_kv_heads
    scale64 = float(np.float32(scale))
    kvd = dtype if kv_dtype is None else kv_dtype
    ks64, vs64 = float(np.float32(k_scale)), float(np.float32(v_scale))
    out = np.full((total_q, Hq, D), np.nan, np.float64)
    want = None if rows is None else set(int(r) for r in rows)

    for b in range(L_all.shape[0]):
        q0, q1 = int(cu[b]), int(cu[b + 1])
        n, L = q1 - q0, int(L_all[b])
        if n == 0:
            continue
        my_rows = [r for r in range(q0, q1) if want is None or r in want]
        if not my_rows:
            continue
        K = gather_request_kv(k_cache, bt[b], L, kvd, block_size) * ks64
        V = gather_request_kv(v_cache, bt[b], L, kvd, block_size) * vs64
        for r in my_rows:
            j = r - q0
            p = last_visible_key(L, n, j)
            lo = first_visible_key(L, n, j, sliding_window)
            qr = widen(q[r], dtype)  # [Hq, D]
            for h in range(Hq):
                kvh = kv_head_of(h, G)
                s = scale64 * (K[lo:p + 1, kvh, :] @ qr[h])
                w = np.exp(s - s.max())
                out[r, h] = (w @ V[lo:p + 1, kvh, :]) / w.sum()
    return out


# ---------------------------------------------------------------------------
# comparison against a device result


def compare_outputs(got: np.ndarray, want: np.ndarray, dtype: str):
    """(max |d|, mean |d|, ok) for a device output widened to fp64.

    Bounds: bf16 max 2e-2 and mean 2e-3; fp32 max 1e-5.  NaN anywhere fails.
    """
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    if got.shape != want.shape:
        raise OracleError("shape mismatch")
    if got.size == 0:
        return 0.0, 0.0, True
    d = np.abs(got - want)
    if not np.isfinite(d).all():
        return math.inf, math.inf, False
    mx, mean = float(d.max()), float(d.mean())
    if dtype == "bf16":
        return mx, mean, (mx <= 2e-2 and mean <= 2e-3)
    return mx, mean, mx <= 1e-5
