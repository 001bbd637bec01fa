"""Oracle for the FP8 activation grid of the W4A8 setting (MXFP8, E4M3).

Test infrastructure only (see ``oracle/__init__.py``).

The rcap.io post "TRACE: Rollout-Guided Quantization-Aware Training for
FP4" reports (Ablations bullet) that the method carries over to MXFP4 W4A4
and W4A8 settings.  In W4A8 the activations -- the tensors the method rounds
on both sides -- are 8-bit.  The pages give no format; the reading taken
here is the OCP Microscaling Formats (MX) v1.0 concrete format MXFP8 with
E4M3 elements, the activation format that goes with MXFP4 weights:

* blocks of 32 consecutive elements along the last dimension, one E8M0
  scale byte each: byte b stands for 2^(b - 127); 0xFF (NaN) makes a
  zero-scale block, as on the MXFP4 path;
* the shared exponent is floor(log2(amax)) - 8, 8 being the exponent of
  E4M3's largest normal (448 = 1.75 * 2^8), clamped to [-127, 127], with
  the MXFP4 oracle's readings for NaN, zero and infinite maxima
  (``oracle.mx.mx_block_scales``; an infinite maximum gives byte 247);
* elements are OCP E4M3FN bytes, sign << 7 | magnitude code; the 127
  non-negative finite magnitudes (codes 0x00..0x7E: zero, the subnormals
  m * 2^-9 and the normals up to 448) increase with the code;
* the rule carries over with this grid in place of E2M1's:
  ``z = clip(fl32(x / s), -448, 448)``; the cached bit is the parity of the
  magnitude code (its last mantissa bit; adjacent codewords differ in it,
  also across +-0); the bracket, the guided, RNE and full-information
  choices, the clip mask ``|x / s| <= 448``, NaN inputs (z = +0, mask 0) and
  ``y = bf16(fl32(s * q*))`` are as on the E2M1 path;
* full information compares the rollout's signed codeword with the two
  bracket endpoints; a NaN byte (0x7F / 0xFF, which no capture writes)
  counts as +-480, the value the next code would have, beyond every
  codeword on its side.

Layouts: scales u8[n/32]; bits and mask u8[n/8] (bit k of byte j =
element 8j + k); codes u8[n], one E4M3FN byte per element.
"""

import numpy as np

from .formats import E4M3FN_VALUES, f32_to_bf16_rne
from .mx import mx_block_scales, mx_quotients
from .trace import pack_bits, unpack_bits

E4M3_EMAX = 8                        # 448 = 1.75 * 2^8
E4M3_MAX = np.float32(448.0)
# Non-negative finite E4M3FN magnitudes, indexed by the magnitude code 0x00..0x7E.
E4M3_MAGNITUDES = np.asarray(E4M3FN_VALUES[:0x7F], dtype=np.float64)
NAN_CODE_VALUE = 480.0               # reading: a NaN rollout byte sits beyond 448

_F32 = np.float32


def mx8_block_scales(x_bits) -> np.ndarray:
    """E8M0 byte per 32-element block for E4M3 elements."""
    return mx_block_scales(x_bits, elem_emax=E4M3_EMAX)


def e4m3_bracket(a):
    """Magnitude codes (lo, hi) of the two E4M3 magnitudes enclosing ``a``
    (float32 values in [0, 448]): lo = largest magnitude <= a, hi = smallest
    magnitude >= a; equal exactly when ``a`` is itself a magnitude."""
    v = np.asarray(a, dtype=np.float32).astype(np.float64).reshape(-1)
    lo = np.searchsorted(E4M3_MAGNITUDES, v, side="right") - 1
    hi = np.searchsorted(E4M3_MAGNITUDES, v, side="left")
    return lo.astype(np.int64), hi.astype(np.int64)


def e4m3_rne_code(a) -> np.ndarray:
    """Magnitude code of the E4M3 magnitude nearest to ``a`` (float32 in
    [0, 448]), ties to the even code (mantissa bit 0).  The distances are
    exact in float64: both ends are multiples of 2^-32 below 2^9 whenever
    lo > 0, and the distance is ``a`` itself when lo == 0."""
    v = np.asarray(a, dtype=np.float32).astype(np.float64).reshape(-1)
    lo, hi = e4m3_bracket(v)
    d_lo = v - E4M3_MAGNITUDES[lo]
    d_hi = E4M3_MAGNITUDES[hi] - v
    take_hi = (lo != hi) & ((d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0)))
    return np.where(take_hi, hi, lo).astype(np.int64)


def _sign_and_clipped(x, zr, valid):
    """Sign bit of z and |z| clipped to [0, 448]; NaN -> +0; a zero-scale
    block gives a zero with the input's sign."""
    nan = np.isnan(x)
    z = np.where(valid, zr, np.copysign(_F32(0), x))
    z = np.where(nan, _F32(0), z)
    sign = np.signbit(z)
    a = np.minimum(np.abs(z), E4M3_MAX).astype(np.float32)
    return sign, a


def _codes(sign, mag_code) -> np.ndarray:
    return ((sign.astype(np.uint8) << 7) | mag_code.astype(np.uint8)).astype(np.uint8)


def mx8_capture(x_bits, with_codes: bool = False) -> dict:
    """MXFP8 capture of a rollout site tensor: the E8M0 ``scales``
    (u8[n/32]), the parity ``bits`` of the round-to-nearest-even E4M3 codes
    (u8[n/8]) and, on request, the ``codes`` themselves (u8[n])."""
    scales = mx8_block_scales(x_bits)
    x, zr, _, valid = mx_quotients(x_bits, scales)
    sign, a = _sign_and_clipped(x, zr, valid)
    idx = np.where(valid & ~np.isnan(x), e4m3_rne_code(a), 0)
    out = {"scales": scales, "bits": pack_bits((idx & 1).astype(np.uint8))}
    if with_codes:
        out["codes"] = _codes(sign, idx)
    return out


def _finish(x, zr, s, valid, sign, m_code):
    """Clip mask, q* = copysign(magnitude, z), y = bf16(fl32(s * q*)) and
    the E4M3 codes of q*."""
    nan = np.isnan(x)
    ok = valid & ~nan
    with np.errstate(invalid="ignore"):
        mask = ok & (np.abs(zr) <= E4M3_MAX)
    m_code = np.where(ok, m_code, 0)
    m_val = E4M3_MAGNITUDES[m_code].astype(np.float32)
    q = np.where(sign, -m_val, m_val).astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        prod = np.where(ok, s * q, q).astype(np.float32)
    return {"y": f32_to_bf16_rne(prod), "mask": pack_bits(mask), "codes": _codes(sign, m_code)}


def mx8_guided_fwd(x_bits, scale_bytes, bits) -> dict:
    """Rollout-guided forward on the E4M3 grid: the bracket endpoint whose
    magnitude-code parity is the cached bit; |z| itself on a codeword."""
    x, zr, s, valid = mx_quotients(x_bits, scale_bytes)
    c = unpack_bits(bits, x.size).astype(np.int64)
    sign, a = _sign_and_clipped(x, zr, valid)
    lo, hi = e4m3_bracket(a)
    m = np.where((lo == hi) | ((lo & 1) == c), lo, hi)
    return _finish(x, zr, s, valid, sign, m)


def mx8_rne_fwd(x_bits, scale_bytes) -> dict:
    """Round-to-nearest-even forward on the E4M3 grid (the baseline)."""
    x, zr, s, valid = mx_quotients(x_bits, scale_bytes)
    sign, a = _sign_and_clipped(x, zr, valid)
    return _finish(x, zr, s, valid, sign, e4m3_rne_code(a))


def e4m3_signed_values(codes) -> np.ndarray:
    """Signed value of each E4M3FN byte, NaN bytes read as +-480."""
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    mag = np.where((c & 0x7F) == 0x7F, NAN_CODE_VALUE, E4M3FN_VALUES[c & 0x7F])
    return np.where(c & 0x80, -mag, mag)


def mx8_full_info_fwd(x_bits, scale_bytes, roll_codes) -> dict:
    """Full-information forward: the bracket endpoint nearest to the
    rollout's signed codeword (u8[n] E4M3FN bytes)."""
    x, zr, s, valid = mx_quotients(x_bits, scale_bytes)
    q_roll = e4m3_signed_values(roll_codes)
    if q_roll.size != x.size:
        raise ValueError("one rollout code byte per element is required")
    sign, a = _sign_and_clipped(x, zr, valid)
    lo, hi = e4m3_bracket(a)
    sgn = np.where(sign, -1.0, 1.0)
    d_lo = np.abs(sgn * E4M3_MAGNITUDES[lo] - q_roll)
    d_hi = np.abs(sgn * E4M3_MAGNITUDES[hi] - q_roll)
    m = np.where((lo == hi) | (d_lo < d_hi), lo, hi)
    return _finish(x, zr, s, valid, sign, m)


def mx8_mismatch_counts(x_train_bits, scale_bytes, roll_codes, bits) -> dict:
    """On the E4M3 grid: sites whose training RNE value differs from the
    rollout value, those among them that straddle (the rollout value is an
    endpoint of the training bracket) and those the guided rule recovers.
    Values are compared, so +0 and -0 agree."""
    x, zr, s, valid = mx_quotients(x_train_bits, scale_bytes)
    ok = valid & ~np.isnan(x)
    sign, a = _sign_and_clipped(x, zr, valid)
    lo, hi = e4m3_bracket(a)
    sgn = np.where(sign, -1.0, 1.0)
    q_roll = e4m3_signed_values(roll_codes)
    q_rne = sgn * E4M3_MAGNITUDES[e4m3_rne_code(a)]
    q_guided = e4m3_signed_values(mx8_guided_fwd(x_train_bits, scale_bytes, bits)["codes"])
    mism = ok & (q_rne != q_roll)
    straddle = mism & ((sgn * E4M3_MAGNITUDES[lo] == q_roll) | (sgn * E4M3_MAGNITUDES[hi] == q_roll))
    return {"n": int(x.size), "mismatched": int(mism.sum()), "straddle": int(straddle.sum()),
            "recovered": int((straddle & (q_guided == q_roll)).sum())}
