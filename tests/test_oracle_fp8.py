"""Pins of the oracle's 8-bit float (OCP FP8 E4M3) cache encoding.

The decoder is pinned by closed forms of the format (bias 7, subnormals
m * 2^-9, largest finite 448, S.1111.111 = NaN) and by monotonicity; the
encoder by brute force against the decoder (nearest finite code, ties to the
even code, saturation at 448) and by round trips.
"""

import math

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.cpu

FINITE = [c for c in range(256) if (c & 0x7F) != 0x7F]


def test_decode_closed_forms():
    d = oracle.fp8_e4m3_decode
    assert d([0x38])[0] == 1.0
    assert d([0x30])[0] == 0.5
    assert d([0x40])[0] == 2.0
    assert d([0x7E])[0] == 448.0
    assert d([0xFE])[0] == -448.0
    assert d([0x01])[0] == 2.0 ** -9
    assert d([0x07])[0] == 7 * 2.0 ** -9
    assert d([0x08])[0] == 2.0 ** -6
    assert d([0x44])[0] == 3.0
    assert d([0xC4])[0] == -3.0
    assert d([0x00])[0] == 0.0 and math.copysign(1.0, d([0x80])[0]) < 0
    assert np.isnan(d([0x7F, 0xFF])).all()


def test_decode_monotonic_and_symmetric():
    v = oracle.fp8_e4m3_decode(np.arange(0x7F))
    assert (np.diff(v) > 0).all()
    assert np.array_equal(oracle.fp8_e4m3_decode(np.arange(0x80, 0xFF)), -v)


def _brute_encode(x):
    codes = np.array(FINITE)
    vals = oracle.fp8_e4m3_decode(codes)
    if math.isnan(x):
        return 0x7F
    if abs(x) >= 448.0:
        return 0x7E | (0x80 if x < 0 else 0)
    d = np.abs(vals - x)
    best = d.min()
    cand = codes[d == best]
    if len(cand) > 1:   # a tie: the code with the even mantissa, same sign as x
        cand = [c for c in cand if c % 2 == 0 and ((c & 0x80) != 0) == (math.copysign(1, x) < 0)] or list(cand)
    c = int(cand[0])
    if vals[FINITE.index(c)] == 0.0:   # zero keeps the sign of x
        c = 0x80 if math.copysign(1, x) < 0 else 0x00
    return c


def test_encode_matches_brute_force():
    rng = np.random.default_rng(3)
    mags = np.exp2(rng.uniform(-12, 9.5, 3000))
    xs = (mags * rng.choice([-1.0, 1.0], mags.size)).astype(np.float32)
    # exact midpoints between neighbouring codes (ties) and the boundary cases
    v = oracle.fp8_e4m3_decode(np.arange(0x7F))
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    xs = np.concatenate([xs, mids, -mids, np.array([0.0, -0.0, 448.0, 449.0, 464.0, 1e30, -1e30, 2.0 ** -10], np.float32)])
    got = oracle.fp8_e4m3_encode(xs)
    for x, g in zip(xs.tolist(), got.tolist()):
        assert g == _brute_encode(x), (x, g, _brute_encode(x))


def test_encode_round_trips_and_nan():
    codes = np.array(FINITE, np.uint8)
    assert np.array_equal(oracle.fp8_e4m3_encode(oracle.fp8_e4m3_decode(codes).astype(np.float32)), codes)
    assert oracle.fp8_e4m3_encode(np.array([np.nan], np.float32))[0] == 0x7F


def test_quantize_divides_by_the_scale_in_fp32():
    one, three = 0x3F80, 0x4040          # bf16 bit patterns of 1.0 and 3.0
    q = oracle.fp8_quantize_rows(np.array([one, three, 0xBF80], np.uint16), 0.5)
    assert q.tolist() == [0x40, 0x4C, 0xC0]   # 2.0, 6.0, -2.0
    # 1/3 is not exact in fp32: the quotient is rounded once, then encoded
    q3 = oracle.fp8_quantize_rows(np.array([one], np.uint16), 3.0)[0]
    assert q3 == oracle.fp8_e4m3_encode(np.array([np.float32(1.0) / np.float32(3.0)], np.float32))[0]


def test_widen_fp8_is_the_decoder():
    codes = np.arange(256, dtype=np.uint8)
    a, b = oracle.widen(codes, "fp8"), oracle.fp8_e4m3_decode(codes)
    assert np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)])


def test_attention_over_codes_equals_attention_over_decoded_values():
    """With 8-bit pools the oracle attends over decode(code) * scale: the same
    result as bf16-free fp64 pools holding those values (f32 pools that hold
    them exactly, since every E4M3 value times a power-of-two scale is an
    fp32 number)."""
    from workloads import build_case
    c = build_case("fp8pin", 4, "bf16", 8, 2, 64, [1, 3], [40, 70], poison=False)
    rng = np.random.default_rng(5)
    kc = rng.integers(0, 256, c.k_cache.shape).astype(np.uint8)
    vc = rng.integers(0, 256, c.v_cache.shape).astype(np.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x38
    vc[(vc & 0x7F) == 0x7F] = 0x38
    ks, vs = 0.25, 2.0
    got = oracle.oracle_attention_varlen(c.q, kc, vc, c.cu_seqlens, c.seq_lens, c.block_tables, c.scale,
                                         c.num_kv_heads, "bf16", kv_dtype="fp8", k_scale=ks, v_scale=vs)
    kf = (oracle.fp8_e4m3_decode(kc) * ks).astype(np.float32)
    vf = (oracle.fp8_e4m3_decode(vc) * vs).astype(np.float32)
    qf = oracle.widen(c.q, "bf16").astype(np.float32)
    want = oracle.oracle_attention_varlen(qf, kf, vf, c.cu_seqlens, c.seq_lens, c.block_tables, c.scale,
                                          c.num_kv_heads, "f32")
    assert np.array_equal(got, want)
