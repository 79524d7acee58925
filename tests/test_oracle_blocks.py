"""Pins of the oracle's block manager and block copies.

Pinned by the copy-on-write worked example of quant67 §3.8, the prefix-key
behaviour of §5.2 (hits share blocks and add a reference, the walk stops at
the first miss, unreferenced cached blocks are evicted least recently used
first), and by seeded random operation sequences checked on their effect
on the data: a token-id pool stands in for the KV cache and every live
sequence must read back its own tokens through its block table.
"""

import numpy as np
import pytest

import oracle
from oracle.block_manager import OracleBlockManager, OutOfBlocks
from tests.block_sim import run_random

pytestmark = pytest.mark.cpu

BS = 16


def test_cow_worked_example():
    """Three prompt blocks shared by four samples: counts [4, 4, 4]; the first
    sample to decode copies block 2 into block 7 and gets table [0, 1, 7]."""
    m = OracleBlockManager(16, BS)
    m.add_sequence(0, list(range(40)))          # blocks 0, 1, 2 (block 2 holds 8 tokens)
    m.add_sequence(9, [100 + t for t in range(64)])   # an unrelated request holds blocks 3..6
    assert m.table(0) == [0, 1, 2] and m.table(9) == [3, 4, 5, 6]
    for child in (1, 2, 3):
        m.fork(0, child)
    assert [m.refcount(b) for b in (0, 1, 2)] == [4, 4, 4]
    slot, src, dst = m.append_slot(0, 999)
    assert (src, dst) == (2, 7) and slot == 7 * BS + 8
    assert m.table(0) == [0, 1, 7]
    assert [m.refcount(b) for b in (0, 1, 2, 7)] == [4, 4, 3, 1]
    # the other samples fork in turn; the last sharer writes in place
    assert m.append_slot(1, 5)[1:] == (2, 8)
    assert m.append_slot(2, 5)[1:] == (2, 9)
    slot3, s3, d3 = m.append_slot(3, 5)
    assert (s3, d3) == (-1, -1) and slot3 == 2 * BS + 8
    assert [m.refcount(b) for b in (0, 1, 2)] == [4, 4, 1]
    assert [m.table(s) for s in range(4)] == [[0, 1, 7], [0, 1, 8], [0, 1, 9], [0, 1, 2]]


def test_cow_needs_partial_block():
    """A fork whose last block is full needs no copy: the next token opens a new block."""
    m = OracleBlockManager(8, BS)
    m.add_sequence(0, list(range(32)))
    m.fork(0, 1)
    assert m.append_slot(1, 3) == (2 * BS, -1, -1)
    assert m.append_slot(0, 4) == (3 * BS, -1, -1)
    assert m.table(0) == [0, 1, 3] and m.table(1) == [0, 1, 2]


def test_prefix_hits_share_blocks_and_stop_at_first_miss():
    m = OracleBlockManager(32, BS)
    a = list(range(50))
    assert m.add_sequence(0, a) == 0
    assert m.table(0) == [0, 1, 2, 3] and m.num_cached() == 3
    b = a[:40] + [77] * 20                   # same first 2.5 blocks, then different
    assert m.add_sequence(1, b) == 32
    assert m.table(1)[:2] == [0, 1] and m.table(1)[2] == 4
    assert [m.refcount(x) for x in (0, 1, 2)] == [2, 2, 1]
    c = a[:16] + [5] * 16 + a[32:48]         # block 1 differs, block 2 equals a's block 2
    assert m.add_sequence(2, c + [1]) == 16  # the walk stops at block 1: block 2 is not reused
    assert m.table(2)[0] == 0 and 2 not in m.table(2)


def test_prefix_lookup_leaves_the_last_token_uncached():
    """A prompt equal to three cached full blocks reuses only two of them."""
    m = OracleBlockManager(16, BS)
    a = list(range(48))
    m.add_sequence(0, a)
    assert m.add_sequence(1, list(a)) == 32
    t = m.table(1)
    assert t[:2] == [0, 1] and t[2] not in (0, 1, 2)
    assert m.refcount(2) == 1 and m.num_cached() == 3   # the duplicate key is not registered twice


def test_lru_eviction_of_unreferenced_cached_blocks():
    m = OracleBlockManager(8, BS)
    m.add_sequence(0, list(range(33)))       # blocks 0, 1 full, block 2 partial
    m.add_sequence(1, [50 + t for t in range(33)])   # blocks 3, 4 full, block 5 partial
    m.free(0)                                # released 2 (to the free pool), then 1, 0 (cached)
    m.free(1)                                # then 5 (free pool), 4, 3 (cached)
    assert m.num_free() == 8 and m.num_cached() == 4
    m.add_sequence(2, [200 + t for t in range(65)])   # 5 blocks: free 6, 7, 2, 5, then evicts 1
    assert m.table(2) == [6, 7, 2, 5, 1]
    assert m.num_cached() == 3 + 4           # 0, 3, 4 still cached; 4 new full blocks of seq 2
    assert m.add_sequence(3, list(range(33))) == 16   # block 0 still hits, block 1 was evicted
    assert m.table(3)[0] == 0


def test_hit_on_evictable_block_takes_it_back():
    m = OracleBlockManager(4, BS)
    m.add_sequence(0, list(range(20)))
    m.free(0)
    assert m.num_free() == 4
    assert m.add_sequence(1, list(range(17))) == 16
    assert m.table(1)[0] == 0 and m.refcount(0) == 1 and m.num_free() == 2


def test_out_of_blocks_changes_nothing():
    m = OracleBlockManager(4, BS, num_host_blocks=1)
    m.add_sequence(0, list(range(40)))
    before = (m.table(0), m.num_free(), m.num_cached(), [m.refcount(b) for b in range(4)])
    with pytest.raises(OutOfBlocks):
        m.add_sequence(1, [9] * 40)
    with pytest.raises(OutOfBlocks):
        m.swap_out(0)                        # 3 blocks, 1 host block
    assert (m.table(0), m.num_free(), m.num_cached(), [m.refcount(b) for b in range(4)]) == before
    assert 1 not in m.seqs


def test_swap_round_trip():
    m = OracleBlockManager(8, BS, num_host_blocks=4)
    m.add_sequence(0, list(range(20)))
    m.fork(0, 1)
    pairs = m.swap_out(1)
    assert pairs == [(0, 0), (1, 1)] and m.is_swapped(1)
    assert [m.refcount(b) for b in (0, 1)] == [1, 1]
    with pytest.raises(oracle.OracleError):
        m.append_slot(1, 3)
    back = m.swap_in(1)
    assert [h for h, _ in back] == [0, 1] and m.num_host_free() == 4
    assert m.table(1) == [d for _, d in back] and not m.is_swapped(1)


def test_copy_and_swap_preconditions():
    pool = np.zeros((4, 2, 3), np.uint16)
    with pytest.raises(oracle.OracleError):
        oracle.oracle_copy_blocks(pool, pool, [(0, 1), (2, 1)])
    with pytest.raises(oracle.OracleError):
        oracle.oracle_copy_blocks(pool, pool, [(0, 1), (1, 2)])
    with pytest.raises(oracle.OracleError):
        oracle.oracle_copy_blocks(pool, pool, [(0, 4)])
    with pytest.raises(oracle.OracleError):
        oracle.oracle_swap_blocks(pool[:2], pool[:2], pool, pool, [(3, 2)])


def test_copy_moves_whole_blocks_only():
    rng = np.random.default_rng(0)
    k = rng.integers(0, 1 << 16, (6, 2, 4, 8)).astype(np.uint16)
    v = rng.integers(0, 1 << 16, (6, 2, 4, 8)).astype(np.uint16)
    k2, v2 = oracle.oracle_copy_blocks(k, v, [(1, 4), (0, 5)])
    for b, src in enumerate([0, 1, 2, 3, 1, 0]):
        assert np.array_equal(k2[b], k[src]) and np.array_equal(v2[b], v[src])


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("prefix", [True, False])
def test_random_operations_keep_every_sequence_intact(seed, prefix):
    m = OracleBlockManager(24, 4, num_host_blocks=10, prefix_caching=prefix)
    log = run_random(m, seed, 24, 4, 10, 400, log=[])
    ops = [e[0] for e in log]
    assert ops.count("append") > 50 and "swap_in" in ops
    if prefix:
        assert any(e[0] == "add" and e[1] != "out of blocks" and e[1][0] > 0 for e in log), "no prefix hit"
    assert any(e[0] == "append" and e[1] != "out of blocks" and e[1][1] >= 0 for e in log), "no copy-on-write"
