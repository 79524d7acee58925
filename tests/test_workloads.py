"""Statistics and structure of the seeded synthetic workloads (CPU only)."""

import numpy as np
import pytest

from workloads import bf16_bits_from_f32, build_case, make_config

pytestmark = pytest.mark.cpu


def _check_structure(c):
    bs = c.block_size
    assert c.cu_seqlens[0] == 0 and (np.diff(c.cu_seqlens) == c.q_lens).all()
    assert (c.q_lens <= c.seq_lens).all()
    used = []
    for b in range(c.num_seqs):
        nb = -(-int(c.seq_lens[b]) // bs)
        assert nb <= c.max_blocks_per_seq
        ids = c.block_tables[b, :nb]
        assert ((ids >= 0) & (ids < c.num_blocks)).all()
        assert (c.block_tables[b, nb:] == c.pad_block).all()
        used.append(ids)
    assert c.pad_block not in set(np.concatenate(used).tolist())
    s = c.slot_mapping[c.slot_mapping >= 0]
    assert len(np.unique(s)) == len(s)
    assert (s < c.num_blocks * bs).all()


def test_tiny_config_shape_and_determinism():
    a = make_config("tiny_decode_f32", 3)
    b = make_config("tiny_decode_f32", 3)
    c = make_config("tiny_decode_f32", 4)
    assert a.dtype == "f32" and a.num_blocks == 64 and a.max_blocks_per_seq == 7
    assert a.q.shape == (4, 8, 64) and a.k_cache.shape == (64, 8, 16, 64)
    assert ((a.seq_lens >= 1) & (a.seq_lens <= 100)).all()
    assert np.float32(a.scale) == np.float32(0.125)
    _check_structure(a)
    for f in ("q", "k_cache", "v_cache", "k_new", "slot_mapping", "block_tables"):
        assert np.array_equal(getattr(a, f), getattr(b, f), equal_nan=True)
    assert not np.array_equal(a.q, c.q)


def test_slot_of_each_new_row_is_its_position():
    c = make_config("tiny_decode_f32", 0)
    for b in range(c.num_seqs):
        pos = int(c.seq_lens[b]) - 1
        want = int(c.block_tables[b, pos // 16]) * 16 + pos % 16
        assert c.slot_mapping[c.cu_seqlens[b]] == want


def test_poison_marks_exactly_the_unowned_slots():
    c = build_case("t", 5, "f32", 2, 1, 8, [1, 3, 0], [5, 20, 17])
    present = np.zeros((c.num_blocks, 16), bool)
    for b in range(c.num_seqs):
        for t in range(int(c.seq_lens[b] - c.q_lens[b])):
            present[c.block_tables[b, t // 16], t % 16] = True
    nan = np.isnan(c.k_cache).all(axis=(1, 3))
    assert np.array_equal(nan, ~present)
    assert np.isfinite(c.k_cache[present.nonzero()[0], :, present.nonzero()[1]]).all()


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5, np.nan], np.float32)
    got = bf16_bits_from_f32(x).tolist()
    assert got[:5] == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020]
    assert got[5] == 0x7FC0


def test_shared_prefix_tables_and_negative_slots():
    c = build_case("p", 1, "bf16", 4, 2, 16, [1, 1, 1], [32, 40, 32], share_groups=[([0, 1, 2], 2)])
    assert (c.block_tables[0, :2] == c.block_tables[1, :2]).all()
    assert (c.block_tables[0, :2] == c.block_tables[2, :2]).all()
    # requests 0 and 2 end inside the shared prefix: their row is already present
    assert c.slot_mapping[0] == -1 and c.slot_mapping[2] == -1 and c.slot_mapping[1] >= 0
    _check_structure(c)


@pytest.mark.parametrize("name,lo,hi,B", [("mha_decode_bf16", 128, 2048, 64), ("gqa_decode_bf16", 16, 8192, 256),
                                          ("gqa_decode_d256_bf16", 16, 8192, 256),
                                          ("gqa_decode_d256_g16_bf16", 16, 8192, 256)])
def test_decode_config_lengths_and_pool(name, lo, hi, B):
    c = make_config(name, 0, poison=False)
    assert c.num_seqs == B and (c.q_lens == 1).all()
    assert c.seq_lens.min() >= lo and c.seq_lens.max() <= hi
    need = int(np.sum(-(-c.seq_lens // 16)))
    assert c.num_blocks == int(np.ceil(1.25 * need))
    _check_structure(c)
    if name.startswith("gqa_decode"):
        med = float(np.median(c.seq_lens))
        assert 700 < med < 1500     # log-normal, median 1024


def test_prefix_long_config():
    c = make_config("prefix_long_bf16", 0, poison=False)
    assert c.num_seqs == 132
    assert (c.seq_lens[128:] == 32768).all()
    priv = c.seq_lens[:128] - 2048
    assert priv.min() >= 0 and priv.max() <= 512
    first = c.block_tables[0, :128]
    assert all((c.block_tables[b, :128] == first).all() for b in range(128))
    _check_structure(c)
