"""Seeded synthetic workloads: packed queries, a paged KV pool, block tables.

Every value is drawn from numpy's PCG64 through ``SeedSequence(seed,
spawn_key=(stream, chunk))``, so a case is a pure function of its seed and
its shape parameters, independent of the number of threads used to draw it.
Streams are drawn in one fixed order for every configuration:

    0 lengths, 1 pool permutation, 2 Q, 3 K pool, 4 V pool, 5 new K, 6 new V.

Values are N(0, 1) drawn in fp32; bf16 cases round them to bf16 with
round-to-nearest-even on the bit pattern and keep them as ``uint16``.

The pool layout is ``[num_blocks, num_kv_heads, block_size, head_dim]`` for K
and for V separately.  Token ``t`` of request ``b`` lives in physical block
``block_tables[b, t // block_size]`` at offset ``t % block_size``; this is the
scheduler-side bookkeeping that a serving engine does on the host, reproduced
here only to place the synthetic history and to emit ``slot_mapping``.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BLOCK_SIZE = 16
BF16_NAN_BITS = 0x7FC0
_CHUNK = 1 << 22

S_LENGTHS, S_POOL_PERM, S_Q, S_K_CACHE, S_V_CACHE, S_K_NEW, S_V_NEW = range(7)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _gen(seed: int, stream: int, chunk: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(int(seed), spawn_key=(int(stream), int(chunk)))
    return np.random.Generator(np.random.PCG64(ss))


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return the bits as uint16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    r = (b >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += b
    r >>= np.uint32(16)
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN_BITS
    return out


def _normal(shape, dtype: str, seed: int, stream: int, threads: int | None = None) -> np.ndarray:
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, np.uint16 if dtype == "bf16" else np.float32)
    nchunks = max(1, -(-n // _CHUNK))

    def work(i: int) -> None:
        lo = i * _CHUNK
        hi = min(n, lo + _CHUNK)
        x = _gen(seed, stream, i).standard_normal(hi - lo, dtype=np.float32)
        out[lo:hi] = bf16_bits_from_f32(x) if dtype == "bf16" else x

    if nchunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(threads or _threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out.reshape(shape)


@dataclass
class Case:
    """One batch of the paged-attention step, as numpy arrays on the host.

    ``q``, ``k_new``, ``v_new``, ``k_cache`` and ``v_cache`` hold float32 values
    for ``dtype == "f32"`` and bf16 bit patterns (uint16) for ``"bf16"``.
    ``k_cache``/``v_cache`` are the pool *before* this step's cache write.
    """

    name: str
    seed: int
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    scale: np.float32
    q_lens: np.ndarray          # int32 [B]   n_b, query rows of request b
    seq_lens: np.ndarray        # int32 [B]   L_b, context incl. this step's rows
    cu_seqlens: np.ndarray      # int32 [B+1]
    block_tables: np.ndarray    # int32 [B, max_blocks_per_seq]
    q: np.ndarray               # [total_q, Hq, D]
    k_cache: np.ndarray         # [NB, Hkv, bs, D]
    v_cache: np.ndarray
    k_new: np.ndarray           # [total_q, Hkv, D]
    v_new: np.ndarray
    slot_mapping: np.ndarray    # int64 [total_q]; -1 = row already present
    pad_block: int              # block id used for table entries past ceil(L/bs)
    poisoned: bool
    info: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_query_len(self) -> int:
        return int(self.q_lens.max()) if self.num_seqs else 0

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.num_seqs else 0


def build_case(
    name: str,
    seed: int,
    dtype: str,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    q_lens,
    seq_lens,
    *,
    max_blocks_per_seq: int | None = None,
    num_blocks: int | None = None,
    pool_factor: float = 1.25,
    share_groups=(),
    poison: bool = True,
    threads: int | None = None,
    info: dict | None = None,
    block_size: int = BLOCK_SIZE,
    rescale_tables: bool = False,
) -> Case:
    """Lay out a batch: block tables over a shuffled pool, history, new rows.

    ``share_groups`` is a sequence of ``(request_indices, num_blocks)``: the
    listed requests point their first ``num_blocks`` logical blocks at the same
    physical blocks (a shared prefix).  Rows whose token falls in a shared
    block are already present and get slot -1.
    With ``poison`` every slot that holds no history token, the slots the
    cache write will fill, and the padding block are set to NaN.
    """
    bs = int(block_size)
    if rescale_tables and bs != BLOCK_SIZE:
        # sizes given in 16-token blocks: keep the same token capacities
        def tok16(nb):
            return -(-int(nb) * BLOCK_SIZE // bs)
        max_blocks_per_seq = tok16(max_blocks_per_seq) if max_blocks_per_seq is not None else None
        num_blocks = tok16(num_blocks) if num_blocks is not None else None
        share_groups = [(m, int(nsh) * BLOCK_SIZE // bs) for m, nsh in share_groups]
    q_lens = np.asarray(q_lens, dtype=np.int64)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    B = int(seq_lens.shape[0])
    if q_lens.shape != seq_lens.shape:
        raise ValueError("q_lens and seq_lens differ in length")
    if (q_lens < 0).any() or (q_lens > seq_lens).any():
        raise ValueError("need 0 <= n_b <= L_b")
    if num_q_heads % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")

    nblk = -(-seq_lens // bs)
    shared_of = {}  # request index -> (group id, shared block count)
    for gi, (members, nsh) in enumerate(share_groups):
        for r in members:
            if nblk[r] < nsh:
                raise ValueError("request shorter than its shared prefix")
            shared_of[int(r)] = (gi, int(nsh))
    group_sizes = [int(nsh) for _, nsh in share_groups]
    need = int(sum(nblk[r] - shared_of.get(r, (0, 0))[1] for r in range(B)) + sum(group_sizes))
    if num_blocks is None:
        num_blocks = max(int(math.ceil(pool_factor * need)), need + 1)
    if num_blocks < need + 1:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {need} blocks plus a pad block")
    mbs = int(max_blocks_per_seq if max_blocks_per_seq is not None else max(1, int(nblk.max(initial=1))))
    if B and int(nblk.max()) > mbs:
        raise ValueError("max_blocks_per_seq too small")

    # 1: pool permutation -> physical ids handed out in order.
    perm = _gen(seed, S_POOL_PERM).permutation(num_blocks).astype(np.int32)
    ptr = 0
    group_ids = []
    for nsh in group_sizes:
        group_ids.append(perm[ptr:ptr + nsh].copy())
        ptr += nsh
    tables = np.empty((B, mbs), np.int32)
    for r in range(B):
        gi, nsh = shared_of.get(r, (None, 0))
        if nsh:
            tables[r, :nsh] = group_ids[gi]
        own = int(nblk[r]) - nsh
        tables[r, nsh:nsh + own] = perm[ptr:ptr + own]
        ptr += own
    pad_block = int(perm[ptr])
    for r in range(B):
        tables[r, int(nblk[r]):] = pad_block

    cu = np.zeros(B + 1, np.int64)
    np.cumsum(q_lens, out=cu[1:])
    total_q = int(cu[-1])

    # 2: queries.  3/4: pool contents.  5/6: new rows.
    q = _normal((total_q, num_q_heads, head_dim), dtype, seed, S_Q, threads)
    k_cache = _normal((num_blocks, num_kv_heads, bs, head_dim), dtype, seed, S_K_CACHE, threads)
    v_cache = _normal((num_blocks, num_kv_heads, bs, head_dim), dtype, seed, S_V_CACHE, threads)
    k_new = _normal((total_q, num_kv_heads, head_dim), dtype, seed, S_K_NEW, threads)
    v_new = _normal((total_q, num_kv_heads, head_dim), dtype, seed, S_V_NEW, threads)

    # slot_mapping: row j of request b carries the token at L_b - n_b + j.
    slots = np.empty(total_q, np.int64)
    present = np.zeros((num_blocks, bs), bool)
    for r in range(B):
        L, n = int(seq_lens[r]), int(q_lens[r])
        nsh = shared_of.get(r, (None, 0))[1]
        hist = np.arange(L - n)
        present[tables[r, hist // bs], hist % bs] = True
        pos = np.arange(L - n, L)
        lb = pos // bs
        s = tables[r, lb].astype(np.int64) * bs + pos % bs
        in_shared = lb < nsh
        s[in_shared] = -1
        if in_shared.any():
            pp = pos[in_shared]
            present[tables[r, pp // bs], pp % bs] = True
        slots[cu[r]:cu[r + 1]] = s
    if poison:
        nan = np.uint16(BF16_NAN_BITS) if dtype == "bf16" else np.float32(np.nan)
        bi, oi = np.nonzero(~present)
        k_cache[bi, :, oi, :] = nan
        v_cache[bi, :, oi, :] = nan
        k_cache[pad_block] = nan
        v_cache[pad_block] = nan

    return Case(
        name=name, seed=int(seed), dtype=dtype,
        num_q_heads=int(num_q_heads), num_kv_heads=int(num_kv_heads), head_dim=int(head_dim),
        block_size=bs, scale=np.float32(1.0 / math.sqrt(head_dim)),
        q_lens=q_lens.astype(np.int32), seq_lens=seq_lens.astype(np.int32),
        cu_seqlens=cu.astype(np.int32), block_tables=tables,
        q=q, k_cache=k_cache, v_cache=v_cache, k_new=k_new, v_new=v_new,
        slot_mapping=slots, pad_block=pad_block, poisoned=bool(poison),
        info=dict(info or {}),
    )


# ---------------------------------------------------------------------------
# The workload configurations.  Each draws its lengths from stream 0.


def _tiny_decode_f32(seed, **kw):
    g = _gen(seed, S_LENGTHS)
    L = g.integers(1, 100, size=4, endpoint=True)
    return build_case("tiny_decode_f32", seed, "f32", 8, 8, 64, np.ones(4, np.int64), L,
                      max_blocks_per_seq=7, num_blocks=64, **kw)


def _mha_decode_bf16(seed, **kw):
    g = _gen(seed, S_LENGTHS)
    L = g.integers(128, 2048, size=64, endpoint=True)
    return build_case("mha_decode_bf16", seed, "bf16", 32, 32, 128, np.ones(64, np.int64), L,
                      max_blocks_per_seq=128, **kw)


def _gqa_decode_bf16(seed, **kw):
    g = _gen(seed, S_LENGTHS)
    L = np.clip(np.rint(g.lognormal(math.log(1024.0), 1.0, size=256)), 16, 8192).astype(np.int64)
    return build_case("gqa_decode_bf16", seed, "bf16", 64, 8, 128, np.ones(256, np.int64), L,
                      max_blocks_per_seq=512, **kw)


def _gqa_decode_d256_bf16(seed, **kw):
    # the GQA decode layer's requests and lengths at head dim 256, 32 query / 8 KV heads
    g = _gen(seed, S_LENGTHS)
    L = np.clip(np.rint(g.lognormal(math.log(1024.0), 1.0, size=256)), 16, 8192).astype(np.int64)
    return build_case("gqa_decode_d256_bf16", seed, "bf16", 32, 8, 256, np.ones(256, np.int64), L,
                      max_blocks_per_seq=512, **kw)


def _gqa_decode_d256_g16_bf16(seed, **kw):
    # the GQA decode layer's requests and lengths at head dim 256 with 128 query / 8 KV heads:
    # 16 query heads per KV head, 8 work items per (KV head, partition)
    g = _gen(seed, S_LENGTHS)
    L = np.clip(np.rint(g.lognormal(math.log(1024.0), 1.0, size=256)), 16, 8192).astype(np.int64)
    return build_case("gqa_decode_d256_g16_bf16", seed, "bf16", 128, 8, 256, np.ones(256, np.int64), L,
                      max_blocks_per_seq=512, **kw)


def _mixed_prefill_bf16(seed, **kw):
    g = _gen(seed, S_LENGTHS)
    prior = g.integers(0, 4096, size=8, endpoint=True)
    dec = g.integers(256, 4096, size=248, endpoint=True)
    n = np.concatenate([np.full(8, 512), np.ones(248, np.int64)])
    L = np.concatenate([prior + 512, dec])
    return build_case("mixed_prefill_bf16", seed, "bf16", 32, 8, 128, n, L,
                      max_blocks_per_seq=288, **kw)


def _prefix_long_bf16(seed, **kw):
    g = _gen(seed, S_LENGTHS)
    priv = g.integers(0, 512, size=128, endpoint=True)
    L = np.concatenate([2048 + priv, np.full(4, 32768)])
    n = np.ones(132, np.int64)
    return build_case("prefix_long_bf16", seed, "bf16", 32, 8, 128, n, L,
                      max_blocks_per_seq=2048, share_groups=[(list(range(128)), 128)], **kw)


def _spec_verify_bf16(seed, **kw):
    # the GQA decode layer's requests, each verifying 1-7 draft tokens (2-8 query rows)
    g = _gen(seed, S_LENGTHS)
    L = np.clip(np.rint(g.lognormal(math.log(1024.0), 1.0, size=256)), 16, 8192).astype(np.int64)
    n = g.integers(2, 8, size=256, endpoint=True)
    return build_case("spec_verify_bf16", seed, "bf16", 64, 8, 128, n, L, max_blocks_per_seq=512, **kw)


_CONFIGS = {
    "tiny_decode_f32": _tiny_decode_f32,
    "mha_decode_bf16": _mha_decode_bf16,
    "gqa_decode_bf16": _gqa_decode_bf16,
    "gqa_decode_d256_bf16": _gqa_decode_d256_bf16,
    "gqa_decode_d256_g16_bf16": _gqa_decode_d256_g16_bf16,
    "mixed_prefill_bf16": _mixed_prefill_bf16,
    "prefix_long_bf16": _prefix_long_bf16,
    "spec_verify_bf16": _spec_verify_bf16,
}
CONFIG_NAMES = tuple(_CONFIGS)


def make_config(name: str, seed: int = 0, *, poison: bool = True, threads: int | None = None,
                block_size: int = BLOCK_SIZE) -> Case:
    """Build one of the named workloads for ``seed`` (``block_size`` tokens per block;
    table widths scale so every context still fits)."""
    if name not in _CONFIGS:
        raise KeyError(f"unknown config {name!r}; known: {CONFIG_NAMES}")
    if block_size == BLOCK_SIZE:
        return _CONFIGS[name](seed, poison=poison, threads=threads)
    return _CONFIGS[name](seed, poison=poison, threads=threads, block_size=block_size, rescale_tables=True)


# ---------------------------------------------------------------------------
# K/V rows that depend only on the token prefix (block-sharing workloads)


def prefix_kv_rows(tokens, start, count, num_kv_heads, head_dim, seed):
    """bf16 bits [count, 2, Hkv, D] of the K and V rows of positions start ..
    start+count-1 of a token sequence.

    Row i is drawn from a generator seeded by ``seed`` and the exact token
    prefix ``tokens[:i+1]``, the way a model's K/V at position i depend only
    on the tokens up to i.  Two sequences with equal prefixes therefore get
    bit-identical rows there, which is what makes sharing a cached block (or
    a forked one) valid.
    """
    import zlib

    out = np.empty((count, 2, num_kv_heads, head_dim), np.uint16)
    arr = np.asarray(tokens, dtype=np.int64)
    for j in range(count):
        i = start + j
        digest = zlib.crc32(arr[:i + 1].tobytes())
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), i, digest])))
        out[j] = bf16_bits_from_f32(g.standard_normal((2, num_kv_heads, head_dim), dtype=np.float32))
    return out
