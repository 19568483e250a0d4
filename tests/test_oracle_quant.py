"""Pins of the oracle's quantisers and packers: sign rules, hand-packed bytes, extremes, error bounds."""

import numpy as np
import pytest

from oracle import quant, spec
from oracle.fwht import fwht_f32


# ------------------------------------------------------------------ sign extension (exhaustive)
def test_nibble_sign_rule_is_twos_complement():
    for v in range(16):
        expect = v - 16 if v >= 8 else v
        assert (v ^ 0x8) - 0x8 == expect
        assert quant.unpack_nibbles(np.array([v], dtype=np.uint8), signed=True)[0] == expect
    for code in range(-8, 8):
        b = quant.pack_nibbles(np.array([code, 0]))
        assert quant.unpack_nibbles(b, signed=True)[0] == code


def test_six_bit_sign_rule_is_twos_complement():
    for v in range(64):
        expect = v - 64 if v >= 32 else v
        assert (v ^ 0x20) - 0x20 == expect
    for code in range(-32, 32):
        blk = np.zeros(32, dtype=np.int64)
        blk[5] = code
        assert quant.unpack_q6(quant.pack_q6(blk))[5] == code


# ------------------------------------------------------------------ packing by hand
def test_q4_byte_holds_even_value_low_odd_value_high():
    # codes 1 and -2 (-2 = 0b1110) -> 0xE1; -8 and 7 -> 0x78
    b = quant.pack_nibbles(np.array([1, -2, -8, 7]))
    assert list(b) == [0xE1, 0x78]
    asym = quant.pack_nibbles(np.array([15, 0, 3, 12]))
    assert list(asym) == [0x0F, 0xC3]
    assert list(quant.unpack_nibbles(asym, signed=False)) == [15, 0, 3, 12]


def test_q6_planes_by_hand():
    codes = np.zeros(32, dtype=np.int64)
    codes[0] = 31        # 0b011111: low nibble 0xF, top bits 01
    codes[1] = -32       # 0b100000: low 0x0, top 10
    codes[6] = -1        # 0b111111: low 0xF, top 11
    codes[31] = 17       # 0b010001: low 0x1, top 01
    blk = quant.pack_q6(codes)
    assert blk.shape == (24,)
    assert blk[0] == 0x0F                # values 0 (low) and 1 (high nibble)
    assert blk[3] == 0x0F                # value 6 low nibble, value 7 = 0
    assert blk[15] == 0x10               # value 30 = 0 low, value 31 high nibble 1
    # high plane: value 4k+i -> byte 16+k, bits 2i..2i+1
    assert blk[16] == (0b01 << 0) | (0b10 << 2)   # values 0, 1
    assert blk[17] == (0b11 << 4)                 # value 6 = 4*1 + 2
    assert blk[23] == (0b01 << 6)                 # value 31 = 4*7 + 3
    np.testing.assert_array_equal(quant.unpack_q6(blk), codes)


@pytest.mark.parametrize("D", [32, 128, 256])
def test_pack_roundtrip_every_code(D, rng):
    c4 = rng.integers(-8, 8, size=(7, D))
    np.testing.assert_array_equal(quant.unpack_nibbles(quant.pack_nibbles(c4), signed=True), c4)
    u4 = rng.integers(0, 16, size=(7, D))
    np.testing.assert_array_equal(quant.unpack_nibbles(quant.pack_nibbles(u4), signed=False), u4)
    c6 = rng.integers(-32, 32, size=(7, D))
    p6 = quant.pack_q6(c6)
    assert p6.shape == (7, D // 32 * 24)
    np.testing.assert_array_equal(quant.unpack_q6(p6), c6)


# ------------------------------------------------------------------ quantiser extremes
def test_q4_0_extremes_map_to_minus8_and_7():
    x = np.zeros(32, dtype=np.float32)
    x[3], x[9] = -2.5, 2.5
    codes, d = quant.quantize_symmetric_blocks(x, spec.Q4_0)
    assert d[0] == 2.5 / 8
    assert codes[3] == -8 and codes[9] == 7


def test_q6_0_extremes_map_to_minus32_and_31():
    x = np.linspace(-4.0, 4.0, 32).astype(np.float32)
    codes, d = quant.quantize_symmetric_blocks(x, spec.Q6_0)
    assert d[0] == 4.0 / 32
    assert codes[0] == -32 and codes[-1] == 31


def test_had_int4_extremes_and_scale():
    x = np.random.default_rng(3).standard_normal(128).astype(np.float32)
    r, codes, s = quant.quantize_had_int4(x)
    np.testing.assert_array_equal(r, fwht_f32(x))
    amax = np.abs(r).max()
    assert s == float(np.float32(amax / 8.0))
    i = np.argmax(np.abs(r))
    assert codes[i] == (7 if r[i] > 0 else -8)
    assert codes.min() >= -8 and codes.max() <= 7


def test_int8_query_extremes():
    x = np.array([0.5, -3.0, 3.0, 0.0] + [0.1] * 28, dtype=np.float32)
    q8, sq = quant.quantize_q_int8(x)
    assert sq == float(np.float32(3.0 / 127.0))
    assert q8[1] == -127 and q8[2] == 127 and q8[3] == 0
    z, sz = quant.quantize_q_int8(np.zeros(16, dtype=np.float32))
    assert sz == 0 and not z.any()


def test_zero_blocks_give_zero_scale_and_codes():
    x = np.zeros((2, 64), dtype=np.float32)
    for layout in (spec.Q4_0, spec.Q6_0, spec.Q8_0):
        codes, d = quant.quantize_symmetric_blocks(x, layout)
        assert not codes.any() and not d.any()
    codes, s, z = quant.quantize_asym_g32(x)
    assert not codes.any() and not s.any() and not z.any()
    r, codes, s = quant.quantize_had_int4(np.zeros(128, dtype=np.float32))
    assert not codes.any() and s == 0


def test_constant_asym_group_is_exact_offset():
    x = np.full(32, 1.25, dtype=np.float32)
    codes, s, z = quant.quantize_asym_g32(x)
    assert s[0] == 0 and z[0] == 1.25 and not codes.any()
    np.testing.assert_array_equal(quant.dequantize(spec.ASYM_G32, codes, s, z), x)


def test_fp16_scale_saturates():
    x = np.zeros(32, dtype=np.float32)
    x[0] = 1e6
    x[1] = 100.0
    codes, d = quant.quantize_symmetric_blocks(x, spec.Q4_0)
    assert d[0] == 65504.0
    assert codes[0] == 7 and codes[1] == 0
    codes, s, z = quant.quantize_asym_g32(-x)
    assert z[0] == -65504.0


def test_asym_min_max_affine_map_by_hand():
    # min -1, max 2: s = 3/15 = 0.2 (f16 0.19995117), z = -1
    x = np.linspace(-1.0, 2.0, 32).astype(np.float32)
    codes, s, z = quant.quantize_asym_g32(x)
    assert s[0] == float(np.float16(np.float32(0.2)))
    assert z[0] == -1.0
    assert codes[0] == 0 and codes[-1] == 15
    assert np.all(np.diff(codes) >= 0)


# ------------------------------------------------------------------ error bounds
@pytest.mark.parametrize("layout", [spec.Q4_0, spec.Q6_0, spec.Q8_0])
def test_symmetric_error_bound(layout, rng):
    x = (rng.standard_normal((200, 128)) * rng.uniform(0.01, 50, size=(200, 1))).astype(np.float32)
    codes, d = quant.quantize_symmetric_blocks(x, layout)
    xh = quant.dequantize(layout, codes, d)
    M = spec.max_magnitude(layout)
    dd = np.repeat(d, 32, axis=-1)
    err = np.abs(x - xh)
    xr = x / dd
    inner = xr <= M - 0.5                        # not clipped at the positive end
    slack = 1e-6 * np.abs(x)                     # the f16 scale and f32 division roundings
    assert np.all(err[inner] <= dd[inner] / 2 + slack[inner])
    # clipped at the positive end: amax/d can exceed M by the fp16 rounding of d (2^-11 relative)
    assert np.all(err <= dd * (1 + M * 2.0**-11) + slack)
    # fp16 scale is the nearest f16 of amax / M
    amax = np.abs(x.reshape(200, -1, 32)).max(axis=-1)
    np.testing.assert_array_equal(d, np.float16(np.float32(amax) / np.float32(M)).astype(np.float64))


def test_asym_error_bound(rng):
    x = (rng.standard_t(3, size=(300, 128)) * 0.7 + rng.normal(size=(300, 1))).astype(np.float32)
    codes, s, z = quant.quantize_asym_g32(x)
    xh = quant.dequantize(spec.ASYM_G32, codes, s, z)
    xb = x.reshape(300, 4, 32).astype(np.float64)
    mn, mx = xb.min(-1), xb.max(-1)
    # s*n + z hits every value to half a step, plus the fp16 roundings of s and z
    slack = np.abs(z - mn) + 15 * np.abs(s - (mx - mn) / 15) + 1e-6 * (np.abs(mx) + np.abs(mn))
    bound = s / 2 + slack
    err = np.abs(xb - xh.reshape(300, 4, 32))
    assert np.all(err <= bound[..., None])
    assert codes.min() >= 0 and codes.max() <= 15


def test_had_roundtrip_error_bound(rng):
    x = rng.standard_normal((100, 128)).astype(np.float32)
    x[:, [3, 77]] *= 10.0                          # planted outlier channels
    r, codes, s = quant.quantize_had_int4(x)
    rh = codes * s[:, None]
    assert np.all(np.abs(r - rh) <= s[:, None] * (1 + 1e-6))


# ------------------------------------------------------------------ stored bytes
@pytest.mark.parametrize("layout,D", [(spec.HAD_INT4, 128), (spec.Q4_0, 128), (spec.Q6_0, 256),
                                      (spec.ASYM_G32, 128), (spec.Q4_0, 64), (spec.Q8_0, 128), (spec.Q8_0, 256)])
def test_encode_decode_bytes_roundtrip(layout, D, rng):
    x = rng.standard_normal((9, D)).astype(np.float32)
    e = quant.encode_rows(layout, x)
    assert e["payload"].shape == (9, spec.payload_bytes(layout, D))
    assert e["record"].shape == (9, spec.scale_bytes(layout, D))
    np.testing.assert_array_equal(quant.decode_codes(layout, e["payload"]), e["codes"])
    s, z = quant.decode_record(layout, e["record"], D)
    np.testing.assert_array_equal(s, e["scales"])
    if layout == spec.ASYM_G32:
        np.testing.assert_array_equal(z, e["zeros"])


def test_record_byte_order_by_hand():
    x = np.zeros(32, dtype=np.float32)
    x[0] = 8.0                                      # amax 8 -> d = 1.0 = 0x3C00
    e = quant.encode_rows(spec.Q4_0, x)
    assert list(e["record"]) == [0x00, 0x3C]
    y = np.zeros(32, dtype=np.float32)
    y[0], y[1] = -2.0, 13.0                          # s = 1.0 (0x3C00), z = -2.0 (0xC000)
    e = quant.encode_rows(spec.ASYM_G32, y)
    assert list(e["record"]) == [0x00, 0x3C, 0x00, 0xC0]
    assert e["codes"][0] == 0 and e["codes"][1] == 15 and e["codes"][2] == 2


def test_asym_codes_use_the_stored_fp16_zero():
    """Codes are computed against z = f16(min), not the f32 minimum.

    min = 1 + 2^-12 rounds to z = 1.0 in fp16; max - min = 15 so s = 1.0.  The value
    1.5 + 2^-12 is exactly half a step above the f32 minimum (ties to even -> 0) but
    more than half a step above z (-> 1).
    """
    e = 2.0 ** -12
    x = np.full(32, 1.0 + e, dtype=np.float32)
    x[1] = 1.5 + e
    x[2] = 16.0 + e
    codes, s, z = quant.quantize_asym_g32(x)
    assert z[0] == 1.0 and s[0] == 1.0
    assert codes[0] == 0 and codes[1] == 1 and codes[2] == 15


def test_q8_0_byte_codes_exhaustive():
    """Every code -128..127 packs into its two's-complement byte and back."""
    codes = np.arange(-128, 128, dtype=np.int64).reshape(8, 32)
    b = quant.pack_bytes(codes)
    assert b.dtype == np.uint8
    np.testing.assert_array_equal(b.astype(np.int64), codes & 0xFF)
    np.testing.assert_array_equal(quant.unpack_bytes(b), codes)


def test_q8_0_range_ends():
    """amax maps to 127 on the positive side (128 is out of range) and -128 on the negative side."""
    x = np.zeros(32, dtype=np.float32)
    x[0], x[1], x[2] = 2.0, -2.0, 1.0
    codes, d = quant.quantize_symmetric_blocks(x, spec.Q8_0)
    assert d[0] == float(np.float16(2.0 / 128.0))
    assert codes[0] == 127 and codes[1] == -128 and codes[2] == 64


# ------------------------------------------------------------------ exact ties (round half to even)
# Quotients that land exactly on k + 1/2 decide the rounding mode: half to even gives the even
# neighbour (0.5 -> 0, 1.5 -> 2, 2.5 -> 2, -2.5 -> -2), unlike half away from zero, half up or
# truncation.  Each block below has a scale of exactly 1, so the quotient is the value itself.
def _tie_block(amax, ties):
    x = np.zeros(32)
    x[0] = amax
    x[1:1 + len(ties)] = ties
    return x


def test_q4_0_ties_round_half_to_even():
    x = _tie_block(8.0, [0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, -3.5, 6.5, -7.5, 0.75])
    codes, d = quant.quantize_symmetric_blocks(x[None, :], spec.Q4_0)
    assert d[0, 0] == 1.0
    assert list(codes[0, :12]) == [7, 0, 2, 2, 4, 0, -2, -2, -4, 6, -8, 1]


def test_q6_0_ties_round_half_to_even():
    x = _tie_block(32.0, [0.5, 2.5, 30.5, -31.5, -0.5, 5.5, -4.5])
    codes, d = quant.quantize_symmetric_blocks(x[None, :], spec.Q6_0)
    assert d[0, 0] == 1.0
    assert list(codes[0, :8]) == [31, 0, 2, 30, -32, 0, 6, -4]


def test_q8_0_ties_round_half_to_even():
    x = _tie_block(128.0, [126.5, -127.5, 0.5, 1.5, -2.5, 125.5])
    codes, d = quant.quantize_symmetric_blocks(x[None, :], spec.Q8_0)
    assert d[0, 0] == 1.0
    assert list(codes[0, :7]) == [127, 126, -128, 0, 2, -2, 126]


def test_asym_ties_round_half_to_even():
    # min 0, max 15: s = 1, z = 0
    x = np.zeros(32)
    x[0], x[1:6] = 15.0, [0.5, 1.5, 2.5, 14.5, 13.5]
    codes, s, z = quant.quantize_asym_g32(x[None, :])
    assert (s[0, 0], z[0, 0]) == (1.0, 0.0)
    assert list(codes[0, :6]) == [15, 0, 2, 2, 14, 14]
    # min -8, max 7: s = 1, z = -8, so x - z = x + 8 carries the tie
    y = np.full(32, -8.0)
    y[0], y[1:4] = 7.0, [-5.5, -7.5, 6.5]
    codes, s, z = quant.quantize_asym_g32(y[None, :])
    assert (s[0, 0], z[0, 0]) == (1.0, -8.0)
    assert list(codes[0, :5]) == [15, 2, 0, 14, 0]


def test_int8_query_ties_round_half_to_even():
    x = np.zeros(128)
    x[0], x[1:7] = 127.0, [2.5, -0.5, 126.5, -126.5, 1.5, 0.5]
    q8, sq = quant.quantize_q_int8(x)
    assert sq == 1.0
    assert list(q8[:7]) == [127, 2, 0, 126, -126, 2, 0]


def test_had_int4_tie_in_the_rotated_basis():
    """x = 16 h0 + h1 - h2 + 1.5 h3 (rows of the +-1 Sylvester matrix): every butterfly sum is exact,
    so the rotated row is c * [2048, 128, -128, 192, 0, ...] with c = f32(1/sqrt(128)), where 2048 c
    and 128 c are exact and 192 c is one f32 rounding.  The scale is 2048 c / 8 = 256 c exactly;
    the quotients are 8 (clamped to 7), exactly +0.5 and -0.5 (half to even: 0 and 0; half away
    from zero would give 1 and -1) and about 0.75 (1; truncation would give 0)."""
    import scipy.linalg
    H = scipy.linalg.hadamard(128).astype(np.float64)
    x = 16 * H[0] + H[1] - H[2] + 1.5 * H[3]
    rot, codes, s = quant.quantize_had_int4(x[None, :])
    from oracle.fwht import norm_const_f32
    c = norm_const_f32(128)
    assert s[0] == 256 * c
    assert list(codes[0, :5]) == [7, 0, 0, 1, 0]
    assert not codes[0, 4:].any()
