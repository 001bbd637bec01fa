"""Exact rational helpers for the oracle pins (tests only).

They round a ``fractions.Fraction`` to IEEE binary32 / bfloat16 by the
textbook definition, independently of NumPy's float32 arithmetic and of the
oracle's candidate-distance rounding.
"""
import struct
from fractions import Fraction


def f32_of_bits(u):
    return struct.unpack("<f", struct.pack("<I", u & 0xFFFFFFFF))[0]


def bits_of_f32(f):
    return struct.unpack("<I", struct.pack("<f", f))[0]


def frac_of_f32(f):
    return Fraction(f)


def _floor_log2(fr):
    # floor(log2(fr)) for fr > 0
    n, d = fr.numerator, fr.denominator
    e = n.bit_length() - d.bit_length()
    if Fraction(2) ** e > fr:
        e -= 1
    return e


def round_to_binary(fr, mant_bits, emin, emax):
    """Round a Fraction to nearest (ties to even) in a binary format with
    ``mant_bits`` stored mantissa bits, normal exponents emin..emax and
    subnormals; returns a Fraction or +-inf (as float)."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = max(_floor_log2(a), emin)
    q = Fraction(2) ** (e - mant_bits)
    m = a / q
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = fl * q
    if val >= Fraction(2) ** (emax + 1):
        return sign * float("inf")
    return sign * val


def round_f32(fr):
    v = round_to_binary(Fraction(fr), 23, -126, 127)
    return float(v) if not isinstance(v, float) else v


def round_bf16(fr):
    v = round_to_binary(Fraction(fr), 7, -126, 127)
    return float(v) if not isinstance(v, float) else v
