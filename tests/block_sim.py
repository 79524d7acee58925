"""Block-manager simulation used by the CPU tests (tests only).

A manager (the oracle's model or the native one, same method names) is
driven by a seeded random sequence of operations while a token-id pool
plays the part of the KV cache: every computed token's id is written at its
slot, copy-on-write and swap pairs are applied as block copies, and after
each step every live sequence must read back exactly its own tokens through
its block table.  This checks slots, sharing, copy-on-write, prefix hits and
swap by their effect on the data rather than by restating their rules.
"""

from __future__ import annotations

import numpy as np

import oracle
from oracle.block_manager import OutOfBlocks


class TokenPools:
    """Device and host pools of token ids, -1 where nothing was written."""

    def __init__(self, num_blocks, block_size, num_host_blocks):
        self.bs = block_size
        self.dev = np.full((num_blocks, block_size), -1, np.int64)
        self.host = np.full((max(num_host_blocks, 1), block_size), -1, np.int64)

    def write(self, slots, tokens):
        for s, t in zip(slots, tokens):
            self.dev[s // self.bs, s % self.bs] = t

    def copy(self, src, dst):
        self.dev, _ = oracle.oracle_copy_blocks(self.dev, self.dev, [(src, dst)])

    def swap_out(self, pairs):
        self.host, _ = oracle.oracle_swap_blocks(self.host, self.host, self.dev, self.dev, pairs)

    def swap_in(self, pairs):
        self.dev, _ = oracle.oracle_swap_blocks(self.dev, self.dev, self.host, self.host, pairs)

    def read(self, table, n, host=False):
        pool = self.host if host else self.dev
        return [int(pool[table[i // self.bs], i % self.bs]) for i in range(n)]


def check_state(mgr, seqs, pools, num_blocks):
    """Content and counting invariants of a manager after any operation."""
    refs = [0] * num_blocks
    for sid, toks in seqs.items():
        table = mgr.table(sid)
        assert len(table) == -(-len(toks) // pools.bs), sid
        swapped = mgr.is_swapped(sid)
        assert pools.read(table, len(toks), host=swapped) == toks, f"sequence {sid} reads other tokens"
        if not swapped:
            for b in table:
                refs[b] += 1
    for b in range(num_blocks):
        assert mgr.refcount(b) == refs[b], f"block {b}: count {mgr.refcount(b)}, tables hold {refs[b]}"
    assert mgr.num_free() == sum(1 for r in refs if r == 0)


def run_random(mgr, seed, num_blocks, block_size, num_host_blocks, steps, vocab=3, log=None,
               oob_errors=(OutOfBlocks,)):
    """Drive a manager with seeded random operations; returns the op log.

    A small vocabulary makes prompts share prefixes often, so prefix hits,
    shared blocks and copy-on-write all happen.  ``log`` (a list) records
    (op, args, result) so two managers can be compared step by step.
    """
    rng = np.random.default_rng(seed)
    pools = TokenPools(num_blocks, block_size, num_host_blocks)
    seqs = {}
    next_id = 0
    for _ in range(steps):
        live = [s for s in seqs if not mgr.is_swapped(s)]
        out = [s for s in seqs if mgr.is_swapped(s)]
        op = rng.choice(["add", "add", "fork", "append", "append", "append", "free", "swap_out", "swap_in"])
        try:
            if op == "add":
                n = int(rng.integers(1, 4 * block_size))
                base = int(rng.integers(0, 3))
                toks = [(base * 7 + i) % 11 if i < n // 2 else int(rng.integers(0, vocab)) for i in range(n)]
                cached = mgr.add_sequence(next_id, toks)
                assert cached % block_size == 0 and cached < n
                assert pools.read(mgr.table(next_id), cached) == toks[:cached], "prefix hit holds other tokens"
                pools.write(mgr.slot_mapping(next_id, cached, n - cached), toks[cached:])
                seqs[next_id] = toks
                res = (cached, mgr.table(next_id))
                next_id += 1
            elif op == "fork" and live:
                p = int(rng.choice(live))
                mgr.fork(p, next_id)
                seqs[next_id] = list(seqs[p])
                res = mgr.table(next_id)
                next_id += 1
            elif op == "append" and live:
                s = int(rng.choice(live))
                t = int(rng.integers(0, vocab))
                slot, src, dst = mgr.append_slot(s, t)
                if src >= 0:
                    pools.copy(src, dst)
                pools.write([slot], [t])
                seqs[s].append(t)
                res = (slot, src, dst)
            elif op == "free" and seqs:
                s = int(rng.choice(list(seqs)))
                mgr.free(s)
                del seqs[s]
                res = None
            elif op == "swap_out" and live and num_host_blocks:
                s = int(rng.choice(live))
                pairs = mgr.swap_out(s)
                pools.swap_out(pairs)
                res = pairs
            elif op == "swap_in" and out:
                s = int(rng.choice(out))
                pairs = mgr.swap_in(s)
                pools.swap_in(pairs)
                res = pairs
            else:
                continue
        except oob_errors:
            res = "out of blocks"
        if log is not None:
            log.append((str(op), res, mgr.num_free(), mgr.num_cached()))
        check_state(mgr, seqs, pools, num_blocks)
    return log
