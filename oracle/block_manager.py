"""Plain model of the KV block manager and of block copies (test infrastructure).

Test infrastructure only: the product library never imports this module.

What the pages fix, restated (quant67 "PagedAttention 与 Continuous
Batching"):
  * §3.3: a decode step appends the new token's K/V to the last block of the
    sequence if that block has room, else takes a physical block from the
    free pool; a request's blocks return to the pool when it finishes
    (lpnh.cn "大模型推理架构演进：从 PagedAttention 到 Prefill-Decode 分离的
    深度解析", §二 2.2, third step).
  * §3.5 / §3.8: parallel sampling shares the prompt's blocks among the
    samples (each share adds one to the block's reference count); a sample
    that must write into a block whose count is above one first copies it
    to a freshly allocated block, points its own table there and drops one
    reference from the old block (copy-on-write).  Worked example: three
    prompt blocks 0, 1, 2 shared by four samples have counts [4, 4, 4]; the
    first sample to decode copies block 2 into new block 7, its table
    becomes [0, 1, 7] and block 2's count falls to 3.
  * §3.9 / §6.1: preemption by swap moves a sequence's blocks to host
    memory and brings them back later.
  * §5.2: full blocks are keyed by a hash of the block's tokens together
    with the key of the previous block; a new request whose leading blocks
    hit the table points its block table at the existing blocks (one more
    reference each) and computes K/V only from the first block that misses;
    when the pool is full, blocks nobody references are evicted, least
    recently used first.

Readings taken where the pages leave a step open:
  * The free pool hands out blocks first in, first out, starting from block
    ids 0, 1, 2, ... in order (with other blocks in use this reproduces the
    §3.8 example's block 7).
  * A block whose count reaches zero goes back to the free pool unless it is
    a registered full block; registered blocks stay cached and join the
    eviction order instead.  Eviction happens only when the free pool is
    empty ("when the pool is full").  A sequence releases its blocks last
    to first, so its tail blocks are evicted before its prefix.
  * Copy-on-write happens only while the count is above one: the last
    sharer writes in place.
  * The key is the exact token content of the block and of every block
    before it, so two keys are equal only when the whole prefix is.
  * A prefix lookup never covers the block that holds the prompt's last
    token, so at least one prompt token is computed and no write lands in
    a shared block.  The lookup stops at the first miss.
  * A full block is registered when it becomes full (at allocation for full
    prompt blocks, on the append that fills it, on swap-in) and only if its
    key is not registered yet.
  * Swap-out copies every block of the sequence to host blocks and drops the
    sequence's device references.  Swap-in allocates fresh device blocks.
    Host blocks are never shared.
  * An operation that lacks free blocks fails with no change of state.
"""

from __future__ import annotations

from collections import OrderedDict, deque

import numpy as np

from .paged_attention import OracleError


class OutOfBlocks(OracleError):
    """Not enough free (or evictable) blocks; nothing was changed."""


class _Seq:
    def __init__(self, tokens, table):
        self.tokens = list(tokens)
        self.table = list(table)
        self.swapped = False


class OracleBlockManager:
    """Reference-counted block pool with copy-on-write, prefix keys and swap."""

    def __init__(self, num_blocks: int, block_size: int, num_host_blocks: int = 0, prefix_caching: bool = True):
        if num_blocks < 1 or block_size < 1 or num_host_blocks < 0:
            raise OracleError("bad pool sizes")
        self.block_size = block_size
        self.num_blocks = num_blocks
        self.prefix_caching = prefix_caching
        self.ref = [0] * num_blocks
        self.free_q = deque(range(num_blocks))
        self.evictable = OrderedDict()      # block -> None, least recently released first
        self.key_of = {}                    # block -> key (registered full blocks)
        self.block_of = {}                  # key -> block
        self.host_free = deque(range(num_host_blocks))
        self.num_host_blocks = num_host_blocks
        self.seqs = {}

    # -- keys --------------------------------------------------------------

    def _keys(self, tokens, nblocks):
        """Key of each of the first nblocks full blocks: (key of previous block, tokens)."""
        bs, keys, prev = self.block_size, [], None
        for i in range(nblocks):
            prev = (prev, tuple(tokens[i * bs:(i + 1) * bs]))
            keys.append(prev)
        return keys

    def _register(self, block, key):
        if self.prefix_caching and key not in self.block_of:
            self.block_of[key] = block
            self.key_of[block] = key

    # -- pool --------------------------------------------------------------

    def _available(self):
        return len(self.free_q) + len(self.evictable)

    def _alloc(self):
        if self.free_q:
            b = self.free_q.popleft()
        elif self.evictable:
            b, _ = self.evictable.popitem(last=False)
            del self.block_of[self.key_of.pop(b)]
        else:
            raise OutOfBlocks("no free block")
        self.ref[b] = 1
        return b

    def _release(self, b):
        self.ref[b] -= 1
        if self.ref[b] == 0:
            if b in self.key_of:
                self.evictable[b] = None
            else:
                self.free_q.append(b)

    def _take(self, b):
        """One more reference to a block found by a prefix lookup."""
        if self.ref[b] == 0:
            del self.evictable[b]
        self.ref[b] += 1

    def _seq(self, seq_id, swapped=False):
        s = self.seqs.get(seq_id)
        if s is None:
            raise OracleError(f"unknown sequence {seq_id}")
        if s.swapped != swapped:
            raise OracleError(f"sequence {seq_id} is {'' if s.swapped else 'not '}swapped out")
        return s

    # -- operations ----------------------------------------------------------

    def add_sequence(self, seq_id, tokens):
        """Blocks for a new prompt; returns how many leading tokens are already cached."""
        if seq_id in self.seqs:
            raise OracleError(f"sequence {seq_id} exists")
        if len(tokens) < 1:
            raise OracleError("empty prompt")
        bs = self.block_size
        nblocks = -(-len(tokens) // bs)
        nfull = len(tokens) // bs
        hits = []
        if self.prefix_caching:
            for key in self._keys(tokens, (len(tokens) - 1) // bs):
                b = self.block_of.get(key)
                if b is None:
                    break
                hits.append(b)
        need = nblocks - len(hits)
        if need > self._available() - sum(1 for b in hits if self.ref[b] == 0):
            raise OutOfBlocks(f"prompt needs {need} blocks")
        for b in hits:
            self._take(b)
        table = hits + [self._alloc() for _ in range(need)]
        keys = self._keys(tokens, nfull)
        for i in range(len(hits), nfull):
            self._register(table[i], keys[i])
        self.seqs[seq_id] = _Seq(tokens, table)
        return len(hits) * bs

    def fork(self, parent, child):
        """The child shares every block of the parent (one more reference each)."""
        p = self._seq(parent)
        if child in self.seqs:
            raise OracleError(f"sequence {child} exists")
        for b in p.table:
            self.ref[b] += 1
        self.seqs[child] = _Seq(p.tokens, p.table)

    def append_slot(self, seq_id, token):
        """Slot of the sequence's next token and the (src, dst) copy it needs, or -1s."""
        s = self._seq(seq_id)
        bs, n = self.block_size, len(s.tokens)
        src = dst = -1
        if n % bs == 0:
            if self._available() < 1:
                raise OutOfBlocks("no block for the next token")
            s.table.append(self._alloc())
        elif self.ref[s.table[-1]] > 1:
            if self._available() < 1:
                raise OutOfBlocks("no block for copy-on-write")
            src, dst = s.table[-1], self._alloc()
            self._release(src)
            s.table[-1] = dst
        s.tokens.append(token)
        if (n + 1) % bs == 0:
            self._register(s.table[-1], self._keys(s.tokens, (n + 1) // bs)[-1])
        return s.table[n // bs] * bs + n % bs, src, dst

    def free(self, seq_id):
        s = self.seqs.pop(seq_id, None)
        if s is None:
            raise OracleError(f"unknown sequence {seq_id}")
        if s.swapped:
            self.host_free.extend(reversed(s.table))
        else:
            for b in reversed(s.table):
                self._release(b)

    def swap_out(self, seq_id):
        """(device block, host block) pairs to copy; the sequence then lives in host blocks."""
        s = self._seq(seq_id)
        if len(self.host_free) < len(s.table):
            raise OutOfBlocks("not enough host blocks")
        host = [self.host_free.popleft() for _ in s.table]
        pairs = list(zip(s.table, host))
        for b in reversed(s.table):
            self._release(b)
        s.table, s.swapped = host, True
        return pairs

    def swap_in(self, seq_id):
        """(host block, device block) pairs to copy; the host blocks are freed."""
        s = self._seq(seq_id, swapped=True)
        if self._available() < len(s.table):
            raise OutOfBlocks("not enough device blocks")
        dev = [self._alloc() for _ in s.table]
        pairs = list(zip(s.table, dev))
        self.host_free.extend(reversed(s.table))
        nfull = len(s.tokens) // self.block_size
        for i, key in enumerate(self._keys(s.tokens, nfull)):
            self._register(dev[i], key)
        s.table, s.swapped = dev, False
        return pairs

    # -- queries -------------------------------------------------------------

    def table(self, seq_id):
        return list(self.seqs[seq_id].table)

    def seq_len(self, seq_id):
        return len(self.seqs[seq_id].tokens)

    def is_swapped(self, seq_id):
        return self.seqs[seq_id].swapped

    def refcount(self, block):
        return self.ref[block]

    def num_free(self):
        """Blocks an allocation may take: never used or released and evictable."""
        return self._available()

    def num_cached(self):
        return len(self.key_of)

    def num_host_free(self):
        return len(self.host_free)

    def slot_mapping(self, seq_id, start, count):
        s = self._seq(seq_id)
        bs = self.block_size
        return [s.table[i // bs] * bs + i % bs for i in range(start, start + count)]


# ---------------------------------------------------------------------------
# block copies (copy-on-write inside one pool, swap between two pools)


def _check_pairs(pairs, n_src, n_dst, same_pool):
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    src, dst = pairs[:, 0], pairs[:, 1]
    if ((src < 0) | (src >= n_src) | (dst < 0) | (dst >= n_dst)).any():
        raise OracleError("block index out of range")
    if len(set(dst.tolist())) != len(dst):
        raise OracleError("a destination block appears twice")
    if same_pool and set(dst.tolist()) & set(src.tolist()):
        raise OracleError("a destination block is also a source")
    return pairs


def oracle_copy_blocks(k_pool, v_pool, pairs):
    """Pools after copying block src to block dst for every (src, dst) pair (§3.8).

    The pools are arrays whose first axis is the block id; every element of
    the block (all KV heads, token slots and channels) is copied.
    """
    pairs = _check_pairs(pairs, len(k_pool), len(k_pool), True)
    k, v = np.array(k_pool, copy=True), np.array(v_pool, copy=True)
    for s, d in pairs.tolist():
        k[d] = k_pool[s]
        v[d] = v_pool[s]
    return k, v


def oracle_swap_blocks(dst_k, dst_v, src_k, src_v, pairs):
    """Destination pools after dst[d] = src[s] for every (s, d) pair (§3.9)."""
    pairs = _check_pairs(pairs, len(src_k), len(dst_k), False)
    k, v = np.array(dst_k, copy=True), np.array(dst_v, copy=True)
    for s, d in pairs.tolist():
        k[d] = src_k[s]
        v[d] = src_v[s]
    return k, v
