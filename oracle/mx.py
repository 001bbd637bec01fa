"""Oracle for the MXFP4 variant of the rollout-guided path.

Test infrastructure only (see ``oracle/__init__.py``).

The rcap.io post "TRACE: Rollout-Guided Quantization-Aware Training for
FP4" reports (Ablations bullet) that the method carries over to MXFP4 W4A4
and W4A8 settings, without giving MXFP4's parameters.  They are taken from
the OCP Microscaling Formats (MX) Specification v1.0 (section on the
MXFP4 concrete format and the conversion from a vector of scalars):

* a block is 32 consecutive elements along the last dimension;
* the shared scale is E8M0: byte b stands for 2^(b - 127), b = 0xFF is NaN;
* the shared exponent is floor(log2(amax)) - 2, where amax is the block's
  largest magnitude and 2 is the exponent of E2M1's largest normal
  (6 = 1.5 * 2^2), clamped to the E8M0 range [-127, 127];
* elements are E2M1 codes of ``x / X`` rounded to nearest (ties to even)
  and clamped to the largest normal 6.

Readings of points the specification leaves open:

* amax ignores NaN; an all-zero (or all-NaN) block gets the smallest scale,
  byte 0 (its elements are zeros anyway);
* an infinite element counts as exponent 128 (the position of the
  infinity's exponent field), so its block gets byte 128 - 2 + 127 = 253;
* there is no tensor-level scale;
* everything downstream of the block scale -- ``z = fl32(x / s)``, the
  clip mask, the E2M1 rounding, the guided, RNE and full-information rules,
  zero-scale blocks (byte 0xFF), NaN inputs, ``y = bf16(fl32(s * q*))`` --
  is exactly the NVFP4 path's (``oracle.trace``), with s = 2^(b - 127).
"""

import numpy as np

from .formats import bf16_to_f32
from .trace import capture_record, full_info_rule, guided_rule, rne_rule, unpack_bits, unpack_nibbles

MX_BLOCK = 32
E2M1_EMAX = 2          # 6 = 1.5 * 2^2
E8M0_BIAS = 127
INF_EXPONENT = 128     # reading: floor(log2(inf)) taken as the exponent field's position


def e8m0_decode(scale_bytes) -> np.ndarray:
    """E8M0 byte -> float32 2^(b - 127); 0xFF -> NaN.  2^-127 is a float32
    subnormal and exact."""
    b = np.asarray(scale_bytes, dtype=np.int64)
    v = np.ldexp(np.float64(1.0), b - E8M0_BIAS)
    return np.where(b == 0xFF, np.nan, v).astype(np.float32)


def floor_log2(a) -> np.ndarray:
    """floor(log2(a)) for positive finite float32 values, exactly: frexp
    gives a = m * 2^e with m in [0.5, 1), so floor(log2(a)) = e - 1."""
    _, e = np.frexp(np.asarray(a, dtype=np.float64))
    return (e - 1).astype(np.int64)


def _block_view(x_bits) -> np.ndarray:
    x = np.asarray(x_bits, dtype=np.uint16).reshape(-1)
    if x.size % MX_BLOCK:
        raise ValueError("tensor length must be a multiple of 32")
    return x.reshape(-1, MX_BLOCK)


def mx_block_scales(x_bits, elem_emax: int = E2M1_EMAX) -> np.ndarray:
    """One E8M0 byte per 32-element block: 127 + clamp(floor(log2(amax)) -
    elem_emax, -127, 127), elem_emax being the exponent of the element
    format's largest normal (2 for E2M1; ``oracle.mx8`` passes 8 for E4M3);
    amax ignores NaN; amax = 0 gives byte 0; an infinite amax counts as
    exponent 128."""
    f = bf16_to_f32(_block_view(x_bits))
    a = np.abs(f)
    a = np.where(np.isnan(a), np.float32(0), a)
    amax = a.max(axis=-1)
    pos = (amax > 0) & np.isfinite(amax)
    e = np.where(np.isinf(amax), INF_EXPONENT, 0)
    e = np.where(pos, floor_log2(np.where(pos, amax, 1)), e)
    shared = np.clip(e - elem_emax, -E8M0_BIAS, E8M0_BIAS)
    shared = np.where(amax == 0, -E8M0_BIAS, shared)
    return (shared + E8M0_BIAS).astype(np.uint8)


def mx_quotients(x_bits, scale_bytes):
    """Per element: x (float32), zr = fl32(x / s), s and the valid-scale
    flag, for 32-element blocks with E8M0 scale bytes."""
    xb = _block_view(x_bits)
    x = bf16_to_f32(xb)
    s = e8m0_decode(np.asarray(scale_bytes, dtype=np.uint8))
    if s.shape[0] != xb.shape[0]:
        raise ValueError("one scale byte per 32-element block is required")
    valid = np.isfinite(s) & (s > 0)
    s_safe = np.where(valid, s, np.float32(1))[:, None]
    with np.errstate(over="ignore", under="ignore", invalid="ignore", divide="ignore"):
        zr = x / s_safe
    return x.reshape(-1), zr.reshape(-1), np.repeat(s, MX_BLOCK), np.repeat(valid, MX_BLOCK)


def mx_capture(x_bits, with_codes: bool = False) -> dict:
    """MXFP4 capture: ``scales`` (E8M0, u8[n/32]), ``bits`` (u8[n/8]) and
    optional ``codes`` (u8[n/2]), element rounding as in ``trace.capture``."""
    scales = mx_block_scales(x_bits)
    x, zr, _, valid = mx_quotients(x_bits, scales)
    return {"scales": scales, **capture_record(x, zr, valid, with_codes)}


def mx_guided_fwd(x_bits, scale_bytes, bits) -> dict:
    """Rollout-guided fake-quant forward on MXFP4 scales."""
    x, zr, s, valid = mx_quotients(x_bits, scale_bytes)
    return guided_rule(x, zr, s, valid, unpack_bits(bits, x.size))


def mx_rne_fwd(x_bits, scale_bytes) -> dict:
    """Round-to-nearest-even fake-quant forward on MXFP4 scales."""
    x, zr, s, valid = mx_quotients(x_bits, scale_bytes)
    return rne_rule(x, zr, s, valid)


def mx_full_info_fwd(x_bits, scale_bytes, roll_codes) -> dict:
    """Full-information guided forward on MXFP4 scales."""
    x, zr, s, valid = mx_quotients(x_bits, scale_bytes)
    return full_info_rule(x, zr, s, valid, unpack_nibbles(roll_codes, x.size))
