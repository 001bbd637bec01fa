"""Number formats for the oracle: bfloat16, OCP E4M3FN and E2M1 (FP4).

Test infrastructure only (see ``oracle/__init__.py``).

Every rounding here is "nearest representable value, ties to the value whose
last mantissa bit is 0", found by comparing distances to the enumerated
candidates.  Distances are taken in float64; for the inputs these functions
accept the candidates that can tie lie within a few binades of the input, so
those distances are exact and the tie test is exact.
"""

import numpy as np

# E2M1 (FP4) magnitudes indexed by the code's three low bits (exponent,
# mantissa).  Bit 3 of a code is the sign.  The rcap.io TRACE post rounds
# onto this grid; its listing clips to [-6, 6], the grid's end points.
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)

E4M3FN_MAX = 448.0


def _e4m3fn_field_value(byte: int) -> float:
    """Value of one OCP E4M3FN byte from its fields (bias 7, no infinities,
    S.1111.111 is NaN, exponent 0 encodes subnormals m * 2**-9)."""
    sign = -1.0 if byte & 0x80 else 1.0
    exp = (byte >> 3) & 0xF
    man = byte & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * man * 2.0 ** -9
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


E4M3FN_VALUES = np.array([_e4m3fn_field_value(b) for b in range(256)], dtype=np.float64)
# Non-negative finite codes 0x00..0x7E, increasing with the byte value.
_E4M3FN_POS = E4M3FN_VALUES[:0x7F]


def bf16_to_f32(bits) -> np.ndarray:
    """bfloat16 bit patterns -> float32 values (bf16 is the upper half of
    a binary32 pattern, so this is exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_rne(values) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even.

    The two candidates are the bf16 value obtained by dropping the low 16
    bits (toward zero) and the next bf16 value away from zero.  Above the
    largest finite bf16 the upper candidate is infinity, which takes part
    in the comparison with its IEEE overflow weight 2**128.  NaN maps to
    the quiet NaN 0x7FC0 with the input's sign.
    """
    v = np.ascontiguousarray(values, dtype=np.float32)
    bits = v.view(np.uint32)
    lo_bits = bits & np.uint32(0xFFFF0000)
    hi_bits = lo_bits + np.uint32(0x10000)
    x = v.astype(np.float64)
    with np.errstate(invalid="ignore"):
        lo_val = lo_bits.view(np.float32).astype(np.float64)
        hi_val = hi_bits.view(np.float32).astype(np.float64)
        hi_inf = np.isinf(hi_val) & ~np.isinf(v)
        hi_val = np.where(hi_inf, np.copysign(2.0 ** 128, x), hi_val)
        d_lo = np.abs(x - lo_val)
        d_hi = np.abs(hi_val - x)
    hi_even = ((hi_bits >> np.uint32(16)) & np.uint32(1)) == 0
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & hi_even)
    out = np.where(take_hi, hi_bits, lo_bits) >> np.uint32(16)
    out = out.astype(np.uint16)
    nan = np.isnan(v)
    if nan.any():
        out[nan] = (np.uint16(0x7FC0) | (bits[nan] >> np.uint32(16)).astype(np.uint16) & np.uint16(0x8000))
    return out


def e4m3fn_decode(byte_codes) -> np.ndarray:
    """E4M3FN bytes -> float64 values (exact; NaN for 0x7F and 0xFF)."""
    return E4M3FN_VALUES[np.asarray(byte_codes, dtype=np.uint8)]


def e4m3fn_encode_rne_sat(values) -> np.ndarray:
    """Non-negative float32 -> E4M3FN byte, nearest value with ties to the
    even byte, saturating: every value >= 448 (the largest finite E4M3FN
    value) encodes as 0x7E.  NaN encodes as 0x00 (a zero scale).

    Only non-negative inputs occur on this path (a block amax divided by
    positive constants); a negative input is an error.
    """
    v = np.asarray(values, dtype=np.float32).astype(np.float64)
    nan = np.isnan(v)
    if np.any(v[~nan] < 0):
        raise ValueError("e4m3fn_encode_rne_sat takes non-negative values")
    vv = np.where(nan, 0.0, np.minimum(v, E4M3FN_MAX))
    hi = np.searchsorted(_E4M3FN_POS, vv, side="left")  # first candidate >= v
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = np.abs(vv - _E4M3FN_POS[lo])
    d_hi = np.abs(_E4M3FN_POS[hi] - vv)
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    return np.where(take_hi, hi, lo).astype(np.uint8)


def e2m1_rne_index(a) -> np.ndarray:
    """Magnitude index (0..7) of the E2M1 value nearest to ``a`` (a float32
    array with values in [0, 6]); ties go to the even index, i.e. to the
    codeword whose mantissa bit is 0.

    The two candidates are the smallest grid value >= a and the one below
    it (the grid is sorted); their distances to a are exact in float64, so
    the nearer one wins and an exact tie goes to the even index."""
    v = np.asarray(a, dtype=np.float32).reshape(-1).astype(np.float64)
    hi = np.minimum(np.searchsorted(E2M1_MAGNITUDES, v, side="left"), 7)
    lo = np.maximum(hi - 1, 0)
    d_lo = np.abs(v - E2M1_MAGNITUDES[lo])
    d_hi = np.abs(E2M1_MAGNITUDES[hi] - v)
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    return np.where(take_hi, hi, lo).astype(np.uint8)


def e2m1_bracket(a):
    """Indices (lo, hi) of the two E2M1 magnitudes enclosing ``a`` in [0, 6]:
    lo = largest grid value <= a, hi = smallest grid value >= a.  They are
    equal exactly when ``a`` is itself a grid value.  On the sorted grid, the
    number of grid values <= a, minus one, is lo, and the number of grid
    values < a is hi."""
    v = np.asarray(a, dtype=np.float32).reshape(-1).astype(np.float64)
    lo = np.searchsorted(E2M1_MAGNITUDES, v, side="right") - 1
    hi = np.searchsorted(E2M1_MAGNITUDES, v, side="left")
    return lo.astype(np.uint8), hi.astype(np.uint8)
