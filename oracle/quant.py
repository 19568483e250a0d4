"""Quantisers, packers and unpackers of the five cache encodings (float64 + explicit rounding).

Test infrastructure only (see the package docstring).

Rounding points.  The pages give the encodings but not every rounding step,
so the reading taken is: every value the cache stores or that decides a code
is the IEEE f32 (or f16, for the fp16 scale fields) rounding of the exact
result of one operation on the previous such values, with ties to even, and
code = clamp(round-half-even(f32(x / scale))).  Emulating one f32 operation as
"compute in float64, then round to f32" is exact for + - * / because float64
carries more than 2*24+2 significand bits, so the double rounding is
innocuous.

Inputs are assumed finite.
"""

import numpy as np

from . import spec
from .fwht import fwht_f32

F16_MAX = 65504.0


def f32(x):
    """Nearest f32 of float64 values (ties to even), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def f16(x):
    """Nearest f16 of values that are already f32 (ties to even), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float16).astype(np.float64)


def f16_sat(x):
    """f16 rounding of an f32 value clamped to the finite f16 range first.

    The fp16 scale/zero fields saturate at +-65504 instead of overflowing to
    infinity (a reading: the pages say nothing about overflow).  Clamping
    before rounding equals rounding and then replacing +-inf with +-65504.
    """
    return f16(np.clip(np.asarray(x, dtype=np.float64), -F16_MAX, F16_MAX))


def f16_bits(x):
    """Raw little-endian bit pattern (uint16) of values that are exactly f16."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def f32_bits(x):
    """Raw bit pattern (uint32) of values that are exactly f32."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32)


def _quantize_codes(x, scale, lo, hi):
    """code = clamp(rint(f32(x / scale)), lo, hi); all-zero codes where scale == 0."""
    scale = np.asarray(scale, dtype=np.float64)
    safe = np.where(scale == 0.0, 1.0, scale)
    n = np.rint(f32(x / safe))
    n = np.clip(n, lo, hi)
    return np.where(scale == 0.0, 0.0, n).astype(np.int64)


def _blocks(x):
    x = f32(x)
    D = x.shape[-1]
    if D % spec.BLOCK:
        raise ValueError("row length must be a multiple of 32")
    return x.reshape(x.shape[:-1] + (D // spec.BLOCK, spec.BLOCK))


# --------------------------------------------------------------------- symmetric block layouts
def quantize_symmetric_blocks(x, layout):
    """q4_0 / q6_0 / q8_0 encoding of rows ``x`` [..., D].

    [FreeToken-268] Summary and Storage layouts: per 32 values along head_dim,
    d = amax / max_magnitude stored as fp16 (8 for q4_0, so codes span
    [-8, 7]; 32 for q6_0, 128 for q8_0); the code is the value divided by the
    stored scale, rounded.

    Returns (codes int64 [..., D], d float64 [..., D/32] holding the fp16 values).
    """
    M = spec.max_magnitude(layout)
    lo, hi = spec.code_range(layout)
    xb = _blocks(x)
    amax = np.max(np.abs(xb), axis=-1)
    d = f16_sat(f32(amax / M))
    codes = _quantize_codes(xb, d[..., None], lo, hi)
    return codes.reshape(np.shape(x)), d


def quantize_asym_g32(x):
    """Per-group asymmetric int4 of rows ``x`` [..., D], g = 32.

    [Open-TQ-Metal] Background: each group of 32 consecutive elements gets its
    own scale and zero point; two 4-bit values per byte.  The formula itself is
    missing from the page; the reading taken is the min-max affine map
    s = (max - min) / 15, z = min (a float offset, fp16), code in [0, 15],
    x_hat = s * code + z, with s = f16(f32(f32(max - min) / 15)) and
    code = clamp(rint(f32(f32(x - z) / s)), 0, 15).

    Returns (codes int64 [..., D], s [..., D/32], z [..., D/32]) with s, z the fp16 values.
    """
    xb = _blocks(x)
    mn = np.min(xb, axis=-1)
    mx = np.max(xb, axis=-1)
    s = f16_sat(f32(f32(mx - mn) / 15.0))
    z = f16_sat(mn)
    codes = _quantize_codes(f32(xb - z[..., None]), s[..., None], 0, 15)
    return codes.reshape(np.shape(x)), s, z


def quantize_had_int4(x):
    """Per-token symmetric int4 in the Hadamard basis for rows ``x`` [..., D].

    [tract-RFC] What's done (CPU) and Architecture > Data flow (decode): rotate
    with the fixed Hadamard, then symmetric zero-point-free int4 with one f32
    scale per token.  The range follows the 4-bit symmetric rule, so
    s = f32(amax / 8) and codes in [-8, 7].

    Returns (rotated f32 row [..., D], codes int64 [..., D], s float64 [...]).
    """
    r = fwht_f32(f32(x))
    amax = np.max(np.abs(r), axis=-1)
    s = f32(amax / 8.0)
    codes = _quantize_codes(r, s[..., None], -8, 7)
    return r, codes, s


def quantize_q_int8(x):
    """Per-vector symmetric int8 of a query vector (already rotated for the Hadamard layout).

    [tract-RFC] Architecture > Data flow (decode): the score is int8(Q_rot)
    times int4(K_rot) accumulated in i32, with the scales applied outside.  The
    reading taken: sq = f32(amax / 127), q8 = clamp(rint(f32(x / sq)), -127, 127).

    Returns (q8 int64 [..., D], sq float64 [...]).
    """
    x = f32(x)
    amax = np.max(np.abs(x), axis=-1)
    sq = f32(amax / 127.0)
    q8 = _quantize_codes(x, sq[..., None], -127, 127)
    return q8, sq


# --------------------------------------------------------------------- packing
def pack_nibbles(codes):
    """Two codes per byte: byte j = (c[2j] & 0xF) | (c[2j+1] & 0xF) << 4.

    [FreeToken-268] Storage layouts (q4_0): val[2j] in the low nibble, val[2j+1]
    in the high nibble.  Negative codes are stored as 4-bit two's complement.
    """
    c = np.asarray(codes, dtype=np.int64) & 0xF
    lo = c[..., 0::2]
    hi = c[..., 1::2]
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed, signed):
    """Inverse of ``pack_nibbles``; signed nibbles use (v ^ 0x8) - 0x8."""
    b = np.asarray(packed, dtype=np.int64)
    lo = b & 0xF
    hi = (b >> 4) & 0xF
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    if signed:
        out = (out ^ 0x8) - 0x8
    return out


def pack_q6(codes):
    """q6_0 blocks: [16-byte low-nibble plane | 8-byte high plane] per 32 codes.

    [FreeToken-268] Storage layouts (q6_0): the low plane uses the q4_0 nibble
    order on the low 4 bits; the high plane holds the top two bits, four values
    per byte at bit positions 0, 2, 4, 6.  Reading: value 4k+i of the block goes
    to byte k, bits 2i..2i+1.
    """
    c = np.asarray(codes, dtype=np.int64) & 0x3F
    D = c.shape[-1]
    cb = c.reshape(c.shape[:-1] + (D // 32, 32))
    low = pack_nibbles(cb & 0xF)                                  # [..., nb, 16]
    top = (cb >> 4) & 0x3
    top4 = top.reshape(top.shape[:-1] + (8, 4))
    high = np.zeros(top4.shape[:-1], dtype=np.int64)
    for i in range(4):
        high |= top4[..., i] << (2 * i)
    blk = np.concatenate([low, high.astype(np.uint8)], axis=-1)   # [..., nb, 24]
    return blk.reshape(c.shape[:-1] + (D // 32 * 24,))


def unpack_q6(packed):
    """Inverse of ``pack_q6`` with the sign rule (v ^ 0x20) - 0x20."""
    b = np.asarray(packed, dtype=np.int64)
    nb = b.shape[-1] // 24
    blk = b.reshape(b.shape[:-1] + (nb, 24))
    low = unpack_nibbles(blk[..., :16], signed=False)             # [..., nb, 32]
    high = blk[..., 16:]
    top = np.empty(low.shape, dtype=np.int64)
    for i in range(4):
        top[..., i::4] = (high >> (2 * i)) & 0x3
    v = low | (top << 4)
    v = (v ^ 0x20) - 0x20
    return v.reshape(b.shape[:-1] + (nb * 32,))


def pack_bytes(codes):
    """q8_0 payload: code j of a row in byte j, as its two's-complement byte."""
    return (np.asarray(codes, dtype=np.int64) & 0xFF).astype(np.uint8)


def unpack_bytes(packed):
    """Inverse of pack_bytes: signed codes from bytes (v ^ 0x80) - 0x80."""
    v = np.asarray(packed, dtype=np.int64)
    return (v ^ 0x80) - 0x80


# --------------------------------------------------------------------- whole rows
def encode_rows(layout, x):
    """Encode rows ``x`` [..., D] into the stored cache bytes of ``layout``.

    Returns a dict with
      payload   uint8 [..., payload_bytes]
      record    uint8 [..., scale_bytes]   (little-endian; ASYM is (scale, zero) per group)
      codes     int64 [..., D]
      scales    float64 [..., n_groups]    (ASYM: the fp16 scales)
      zeros     float64 [..., n_groups]    (ASYM only, else None)
      rotated   float64 [..., D]           (HAD only: the f32 rotated row, else None)
    """
    x = f32(x)
    D = x.shape[-1]
    spec.check_head_dim(layout, D)
    zeros = None
    rotated = None
    if layout == spec.HAD_INT4:
        rotated, codes, s = quantize_had_int4(x)
        scales = s[..., None]
        payload = pack_nibbles(codes)
        record = np.ascontiguousarray(f32_bits(s)[..., None]).view(np.uint8)
    elif layout in (spec.Q4_0, spec.Q6_0, spec.Q8_0):
        codes, scales = quantize_symmetric_blocks(x, layout)
        if layout == spec.Q4_0:
            payload = pack_nibbles(codes)
        elif layout == spec.Q6_0:
            payload = pack_q6(codes)
        else:
            payload = pack_bytes(codes)
        record = np.ascontiguousarray(f16_bits(scales)).view(np.uint8)
    else:
        codes, scales, zeros = quantize_asym_g32(x)
        payload = pack_nibbles(codes)
        sz = np.stack([f16_bits(scales), f16_bits(zeros)], axis=-1)   # [..., ng, 2]
        record = np.ascontiguousarray(sz.reshape(sz.shape[:-2] + (-1,))).view(np.uint8)
    record = record.reshape(x.shape[:-1] + (spec.scale_bytes(layout, D),))
    return dict(payload=payload, record=record, codes=codes, scales=scales,
                zeros=zeros, rotated=rotated)


def decode_codes(layout, payload):
    """Codes of stored payload bytes [..., P] (sign rules of the layout)."""
    if layout == spec.Q6_0:
        return unpack_q6(payload)
    if layout == spec.Q8_0:
        return unpack_bytes(payload)
    return unpack_nibbles(payload, signed=(layout != spec.ASYM_G32))


def decode_record(layout, record, D):
    """(scales [..., ng], zeros [..., ng] or None) from stored record bytes."""
    rec = np.ascontiguousarray(np.asarray(record, dtype=np.uint8))
    if layout == spec.HAD_INT4:
        return rec.view(np.float32).astype(np.float64), None
    h = rec.view(np.float16).astype(np.float64)
    if layout == spec.ASYM_G32:
        return h[..., 0::2], h[..., 1::2]
    return h, None


def dequantize(layout, codes, scales, zeros=None):
    """x_hat per element, float64: d*n (block layouts, Hadamard basis for HAD), s*n + z (ASYM)."""
    codes = np.asarray(codes, dtype=np.float64)
    D = codes.shape[-1]
    g = D if layout == spec.HAD_INT4 else spec.BLOCK
    s = np.repeat(np.asarray(scales, dtype=np.float64), g, axis=-1)
    out = codes * s
    if layout == spec.ASYM_G32:
        out = out + np.repeat(np.asarray(zeros, dtype=np.float64), g, axis=-1)
    return out
