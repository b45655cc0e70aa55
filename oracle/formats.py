"""Number formats used by the quantized linear, from their definitions.

Test infrastructure (see the package docstring): imported only by tests,
the smoke check and the bench's CPU baseline.

The abstract of 6Bit-Diffusion names NVFP4 and INT8 as the two activation
formats.  NVFP4 stores each element as OCP E2M1 (FP4) and each group of 16
elements carries one OCP E4M3 scale; an FP32 scale covers the tensor.  The
pages print neither the rounding mode nor the E4M3 variant; the reading
taken here is round-to-nearest with ties to the even code, saturating, and
the OCP "E4M3FN" variant (bias 7, largest finite 448, no infinities).

Every encoder below is written as "pick the nearest representable value,
ties to the even code": the two neighbours of the input in a sorted table
of the format's values are found and the input is compared with their
midpoint, exactly, in float64.
"""
import numpy as np

# E2M1 magnitudes, indexed by the 3 low bits of a code (bit 3 is the sign).
E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def _e4m3_value(code):
    """Value of a non-negative OCP E4M3FN code 0x00..0x7E (bias 7)."""
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0:                      # subnormal: m/8 * 2^(1-7)
        return m / 8.0 * 2.0 ** -6
    return (1.0 + m / 8.0) * 2.0 ** (e - 7)


# The 127 finite non-negative E4M3FN values in code order (strictly rising).
E4M3_VAL = np.array([_e4m3_value(c) for c in range(0x7F)], dtype=np.float64)
E4M3_MAX = E4M3_VAL[-1]          # 448.0, code 0x7E


def _nearest_even(table, a):
    """Index of the entry of the rising ``table`` nearest to each a >= 0.

    Ties go to the even index; inputs above the last entry saturate to it.
    All comparisons are exact: table entries and midpoints of neighbours are
    short dyadic numbers and ``a`` is float32-valued.
    """
    a = np.asarray(a, dtype=np.float64)
    last = len(table) - 1
    hi = np.minimum(np.searchsorted(table, a, side="left"), last)
    lo = np.maximum(hi - 1, 0)
    mid = (table[lo] + table[hi]) * 0.5
    pick = np.where(a < mid, lo, np.where(a > mid, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(table[hi] == a, hi, pick)     # exactly representable
    pick = np.where(a > table[last], last, pick)  # saturate
    return pick.astype(np.uint8)


def e2m1_decode(codes):
    """FP4 E2M1 code (0..15) -> value; bit 3 is the sign."""
    c = np.asarray(codes).astype(np.uint8)
    mag = E2M1_MAG[c & 7]
    return np.where((c & 8) != 0, -mag, mag)


def e2m1_encode(v):
    """float32 value -> E2M1 code, nearest with ties to the even code.

    Magnitudes at or above 6 saturate to 6.  The sign bit is the sign bit of
    the input, so a negative input that rounds to zero gives code 0x8.
    NaN and infinities are outside the contract.
    """
    v = np.asarray(v, dtype=np.float32)
    mag = _nearest_even(E2M1_MAG, np.abs(v).astype(np.float64))
    return (mag | (np.signbit(v).astype(np.uint8) << 3)).astype(np.uint8)


def e4m3_decode(codes):
    """OCP E4M3FN code -> value (0x7F and 0xFF are NaN)."""
    c = np.asarray(codes).astype(np.uint16)
    mag = np.where((c & 0x7F) == 0x7F, np.nan, E4M3_VAL[np.minimum(c & 0x7F, 0x7E)])
    return np.where((c & 0x80) != 0, -mag, mag)


def e4m3_encode_nonneg(a):
    """float32 value a >= 0 -> E4M3FN code, nearest with ties to the even
    code, saturating at 448 (code 0x7E).  Used for the group scales only."""
    a = np.asarray(a, dtype=np.float32)
    if np.any(a < 0) or np.any(~np.isfinite(a)):
        raise ValueError("E4M3 scale encoder takes finite non-negative values")
    return _nearest_even(E4M3_VAL, a.astype(np.float64))


# ---------------------------------------------------------------- bfloat16 --

def bf16_to_f64(bits):
    """bfloat16 bit patterns (uint16) -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def bf16_to_f32(bits):
    """bfloat16 bit patterns (uint16) -> float32 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def f64_to_bf16_rne(x):
    """float64 -> bfloat16 bits, round to nearest, ties to even.

    bfloat16 keeps 8 significant bits and the float32 exponent range; its
    smallest subnormal step is 2^-133.  The value is divided by its
    quantum, rounded half-to-even to an integer and scaled back, so there
    is one rounding of the exact input.  Results beyond the largest finite
    bfloat16 become infinity, as round-to-nearest prescribes.
    """
    x = np.asarray(x, dtype=np.float64)
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    _, e = np.frexp(xf)                       # |x| = m * 2^e, 0.5 <= m < 1
    q_exp = np.maximum(e - 8, -133)           # quantum of the 8-bit significand
    r = np.ldexp(np.rint(np.ldexp(xf, -q_exp)), q_exp)
    bf16_max = (2.0 - 2.0 ** -7) * 2.0 ** 127
    # one rounding above the largest finite value: RNE gives infinity from
    # the midpoint between max and 2^128 upward
    over = np.abs(xf) >= (bf16_max + 2.0 ** 119)
    r = np.where(over, np.copysign(np.inf, xf), np.where(np.abs(r) > bf16_max,
                                                          np.copysign(bf16_max, xf), r))
    out = np.asarray(np.where(finite, r, x), dtype=np.float64)
    bits = (out.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return bits


def f32_to_bf16_rne(x):
    """float32 -> bfloat16 bits, round to nearest, ties to even."""
    return f64_to_bf16_rne(np.asarray(x, dtype=np.float32).astype(np.float64))
