"""Pins of the oracle's Hadamard transforms against scipy's Hadamard matrix and closed forms."""

import numpy as np
import pytest
import scipy.linalg

from oracle import fwht

POW2 = [1, 2, 4, 8, 16, 32, 64, 128, 256]


@pytest.mark.parametrize("D", POW2)
def test_matrix_equals_scipy_sylvester(D):
    np.testing.assert_array_equal(fwht.hadamard_matrix(D), scipy.linalg.hadamard(D))


@pytest.mark.parametrize("D", [2, 8, 64, 128, 256])
def test_f64_transform_equals_dense_orthonormal_hadamard(D, rng):
    x = rng.standard_normal((5, D))
    ref = x @ (scipy.linalg.hadamard(D).astype(np.float64) / np.sqrt(D)).T
    np.testing.assert_allclose(fwht.hadamard_f64(x), ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("D", [4, 128, 256])
def test_f64_transform_is_involution_and_isometry(D, rng):
    x = rng.standard_normal((3, D))
    y = fwht.hadamard_f64(x)
    np.testing.assert_allclose(fwht.hadamard_f64(y), x, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)


@pytest.mark.parametrize("D", [4, 128, 256])
def test_unit_vector_maps_to_constant(D):
    e0 = np.zeros(D)
    e0[0] = 1.0
    np.testing.assert_allclose(fwht.hadamard_f64(e0), np.full(D, 1.0 / np.sqrt(D)), atol=1e-15)


def test_rotation_invariance_of_scores(rng):
    """(QH)(KH)^T = QK^T: a shared orthonormal rotation leaves the scores unchanged."""
    q = rng.standard_normal((4, 128))
    k = rng.standard_normal((50, 128))
    np.testing.assert_allclose(fwht.hadamard_f64(q) @ fwht.hadamard_f64(k).T, q @ k.T, atol=1e-11)


def test_norm_constants():
    assert np.float32(fwht.norm_const_f32(128)).view(np.uint32) == 0x3DB504F3
    assert fwht.norm_const_f32(256) == 1.0 / 16.0
    assert fwht.norm_const_f32(64) == 1.0 / 8.0


def test_f32_butterfly_d2_by_hand():
    c = np.float32(1.0) / np.float32(np.sqrt(2.0))          # nearest f32 of 1/sqrt(2)
    assert np.float32(fwht.norm_const_f32(2)) == np.float32(0.70710677)
    y = fwht.fwht_f32(np.array([1.0, 2.0], dtype=np.float32))
    assert y[0] == float(np.float32(np.float32(3.0) * c))
    assert y[1] == float(np.float32(np.float32(-1.0) * c))


def test_f32_butterfly_d4_natural_order_by_hand():
    # stage h=1: [1+2, 1-2, 3+4, 3-4] = [3, -1, 7, -1]; stage h=2: [10, -2, -4, 0]; times 1/2
    y = fwht.fwht_f32(np.array([1.0, 2.0, 3.0, 4.0], dtype=np.float32))
    np.testing.assert_array_equal(y, [5.0, -1.0, -2.0, 0.0])


@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_f32_butterfly_is_close_to_definition(D, rng):
    x = rng.standard_normal((20, D)).astype(np.float32)
    y32 = fwht.fwht_f32(x)
    y64 = fwht.hadamard_f64(x.astype(np.float64))
    # every value is an f32
    np.testing.assert_array_equal(y32, y32.astype(np.float32).astype(np.float64))
    # f32 rounding only: log2(D) stages plus the scale, each at most half an ulp
    bound = (np.log2(D) + 2) * 2.0**-24 * np.sqrt(D) * np.abs(x).max(axis=-1, keepdims=True)
    assert np.all(np.abs(y32 - y64) <= bound)


def test_f32_butterfly_exact_on_small_integers():
    """Integer inputs whose partial sums stay exact in f32 give the exact transform for D=256."""
    x = np.arange(256, dtype=np.float32) % 7 - 3
    y = fwht.fwht_f32(x)
    ref = scipy.linalg.hadamard(256).astype(np.float64) @ x.astype(np.float64) / 16.0
    np.testing.assert_array_equal(y, ref)


def test_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        fwht.fwht_f32(np.zeros(96, dtype=np.float32))
    with pytest.raises(ValueError):
        fwht.hadamard_matrix(12)


# ------------------------------------------------------------------ rounding order, worked by hand
# A D = 8 row of one-decimal values, none of which is exact in binary, written out stage by stage as
# f32 bit patterns (each entry worked with one f32 add or subtract of the previous stage's pair,
# strides 1, 2, 4 in that order, then one f32 multiply by f32(1/sqrt(8)) = 0x3eb504f3).  Running the
# strides in descending order, or scaling before the butterflies, gives different bits here, so this
# pins the stage order and the scaling point the encoding reads from [tract-RFC] What's done (CPU).
_X8 = [0x40966666, 0x40A33333, 0x40F00000, 0x41180000, 0x3ECCCCCD, 0x3FC00000, 0x41033333, 0x41166666]
_STAGES8 = {
    1: [0x411CCCCC, 0xBECCCCD0, 0x41880000, 0xC0000000, 0x3FF33333, 0xBF8CCCCD, 0x418CCCCC, 0xBF999998],
    2: [0x41D66666, 0xC019999A, 0xC0E66668, 0x3FCCCCCC, 0x419BFFFF, 0xC0133332, 0xC17B3332, 0x3DCCCCB0],
    4: [0x42393332, 0xC0966666, 0xC1B73333, 0x3FD99997, 0x40E9999C, 0xBDCCCD00, 0x4107FFFE, 0x3FC00001],
}
_OUT8 = [0x4182F4C7, 0xBFD4B29D, 0xC1018ABE, 0x3F19DDCD, 0x40252E1F, 0xBD10D0E7, 0x4040553F, 0x3F07C3B7]


def _bits_to_f32(bits):
    return np.array(bits, dtype=np.uint32).view(np.float32)


def test_stage_table_is_consistent():
    """Each stage of the worked table is the f32 butterfly of the one before (the table's own check)."""
    prev = _bits_to_f32(_X8)
    for h in (1, 2, 4):
        cur = _bits_to_f32(_STAGES8[h])
        for i in range(8):
            if i & h == 0:
                assert cur[i] == np.float32(prev[i] + prev[i + h])
                assert cur[i + h] == np.float32(prev[i] - prev[i + h])
        prev = cur
    c = np.array([0x3EB504F3], dtype=np.uint32).view(np.float32)[0]
    np.testing.assert_array_equal((prev * c).astype(np.float32), _bits_to_f32(_OUT8))


def test_f32_butterfly_stage_order_and_scale_point():
    y = fwht.fwht_f32(_bits_to_f32(_X8))
    np.testing.assert_array_equal(np.asarray(y, dtype=np.float32).view(np.uint32), np.array(_OUT8, dtype=np.uint32))


def test_stage_order_and_scale_point_are_visible_in_the_worked_row():
    """The alternatives differ from the worked row, so a swapped order or scaling point fails above."""
    def variant(order, scale_first):
        y = _bits_to_f32(_X8).copy()
        c = np.float32(fwht.norm_const_f32(8))
        if scale_first:
            y = (y * c).astype(np.float32)
        for h in order:
            z = y.copy()
            for i in range(8):
                if i & h == 0:
                    z[i] = np.float32(y[i] + y[i + h])
                    z[i + h] = np.float32(y[i] - y[i + h])
            y = z
        return y if scale_first else (y * c).astype(np.float32)

    out = _bits_to_f32(_OUT8)
    assert not np.array_equal(variant((4, 2, 1), False), out)
    assert not np.array_equal(variant((1, 2, 4), True), out)
