"""Orthonormal Walsh-Hadamard transform.

Test infrastructure only (see the package docstring).

[tract-RFC] What's done (CPU) and Why this quant scheme: K and V rows are
rotated by a fixed orthonormal Hadamard matrix H (the fast transform, O(D log D)
butterflies) before per-token quantisation; Q is rotated by the same H so that
(QH)(KH)^T = QK^T, and the attention output is rotated back with H at the end
(Architecture > Data flow (decode), last step).

Two forms live here:

* ``hadamard_matrix`` / ``hadamard_f64`` -- the plain definition,
  H = H_D / sqrt(D) with Sylvester's H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]],
  computed in float64.
* ``fwht_f32`` -- the encoding step whose f32 result decides the stored codes.
  The pages leave the butterfly order and the normalisation point open; the
  reading taken is: stages with half-width h = 1, 2, 4, ..., D/2 in that order,
  each butterfly (a, b) -> (a + b, a - b) rounded to f32, natural (Sylvester)
  ordering, then every element multiplied by c_D = f32(1/sqrt(D)) and rounded
  to f32.
"""

import numpy as np


def _f32(x):
    """Round float64 values to the nearest float32 (ties to even), kept in f64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def _check_pow2(D):
    if D < 1 or D & (D - 1):
        raise ValueError("Hadamard transform needs a power-of-two length")


def hadamard_matrix(D):
    """Sylvester Hadamard matrix H_D (entries +-1), float64, built by doubling."""
    _check_pow2(D)
    H = np.ones((1, 1), dtype=np.float64)
    while H.shape[0] < D:
        H = np.block([[H, H], [H, -H]])
    return H


def hadamard_f64(x):
    """Plain definition: y = (H_D / sqrt(D)) x along the last axis, in float64."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    H = hadamard_matrix(D) / np.sqrt(D)
    return x @ H.T  # H is symmetric; the transpose only states the product


def norm_const_f32(D):
    """c_D = 1/sqrt(D) rounded to f32 (D=128 -> 0x3db504f3, D=256 -> 1/16)."""
    _check_pow2(D)
    return float(_f32(1.0 / np.sqrt(float(D))))


def fwht_f32(x):
    """Butterfly transform with f32 rounding at every step (the encoding step).

    ``x`` holds f32 values (any float dtype); the result is float64 holding
    f32 values.  Stage h pairs element i (bit h of i clear) with i + h: the
    lower slot gets f32(x_i + x_{i+h}), the upper slot f32(x_i - x_{i+h}).
    """
    y = _f32(np.array(x, dtype=np.float64, copy=True))
    D = y.shape[-1]
    _check_pow2(D)
    h = 1
    while h < D:
        y = y.reshape(y.shape[:-1] + (D // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = _f32(a + b)
        y[..., 1, :] = _f32(a - b)
        y = y.reshape(y.shape[:-3] + (D,))
        h *= 2
    return _f32(y * norm_const_f32(D))
