"""Layout constants of the five cache encodings.

Test infrastructure only (see the package docstring).

Each encoding stores, per token and per kv head and separately for K and V,
a payload of packed codes and a small record of scale values.

HAD_INT4   [tract-RFC] Architecture > Data flow (decode), "State = ..." paragraph:
           per-token int4 in the Hadamard basis, ceil(D/2) bytes of nibbles
           plus one f32 scale per token.
Q4_0       [FreeToken-268] Storage layouts: 32 values along head_dim share one
           fp16 scale, 16 payload bytes, two nibbles per byte.
Q6_0       [FreeToken-268] Storage layouts: 32 values, 16-byte low-nibble plane
           plus 8-byte plane of the top two bits, one fp16 scale.
ASYM_G32   [Open-TQ-Metal] Background, per-group asymmetric int4: groups of 32
           consecutive elements, per-group scale and zero point, two values
           per byte.  The scale and zero are stored as fp16 each.
Q8_0       [FreeToken-268] Summary and the memory table: the 8-bit block
           scheme at 1.0625 bytes per element, i.e. 32 one-byte codes plus one
           fp16 scale per 32 values along head_dim.
"""

HAD_INT4 = 0
Q4_0 = 1
Q6_0 = 2
ASYM_G32 = 3
Q8_0 = 4

LAYOUTS = (HAD_INT4, Q4_0, Q6_0, ASYM_G32, Q8_0)
NAMES = {HAD_INT4: "had_int4", Q4_0: "q4_0", Q6_0: "q6_0", ASYM_G32: "asym_int4_g32", Q8_0: "q8_0"}

BLOCK = 32  # elements per block / group for the block layouts


def check_head_dim(layout, D):
    """Raise ValueError when the layout cannot encode rows of length D."""
    if D <= 0 or D % BLOCK:
        raise ValueError("head_dim must be a positive multiple of 32")
    if layout == HAD_INT4 and D & (D - 1):
        raise ValueError("the Hadamard layout needs a power-of-two head_dim")
    if layout not in LAYOUTS:
        raise ValueError("unknown layout")


def n_groups(layout, D):
    """Number of scale groups per row (one for the per-token layout)."""
    check_head_dim(layout, D)
    return 1 if layout == HAD_INT4 else D // BLOCK


def payload_bytes(layout, D):
    """Packed code bytes per token per head per tensor."""
    check_head_dim(layout, D)
    if layout == Q6_0:
        return (D // BLOCK) * 24
    if layout == Q8_0:
        return D
    return D // 2


def scale_bytes(layout, D):
    """Scale-record bytes per token per head per tensor."""
    check_head_dim(layout, D)
    if layout == HAD_INT4:
        return 4                    # one f32
    if layout == ASYM_G32:
        return (D // BLOCK) * 4     # fp16 scale + fp16 zero per group
    return (D // BLOCK) * 2         # one fp16 scale per block


def bytes_per_element(layout, D):
    """Average stored bytes per cached element (payload plus scales)."""
    return (payload_bytes(layout, D) + scale_bytes(layout, D)) / D


def code_range(layout):
    """Inclusive (lo, hi) range of the integer codes of a layout."""
    if layout == Q6_0:
        return (-32, 31)
    if layout == Q8_0:
        return (-128, 127)
    if layout == ASYM_G32:
        return (0, 15)
    return (-8, 7)


def max_magnitude(layout):
    """Divisor M of the symmetric absmax scale d = amax / M.

    [FreeToken-268] Storage layouts: the 4-bit layout uses 8 (not 7), so the
    symmetric range is [-8, 7].  The 6-bit layout takes 2^(bits-1) = 32 by the
    same rule, the 8-bit layout 128 (range [-128, 127]); the Hadamard int4
    layout is symmetric int4 and takes 8.
    """
    if layout == Q6_0:
        return 32
    if layout == Q8_0:
        return 128
    if layout in (Q4_0, HAD_INT4):
        return 8
    raise ValueError("asymmetric layout has no max magnitude")
