"""Pins for the oracle's binary32 arithmetic: NumPy float32 division and
multiplication against exact rational arithmetic rounded to binary32 by the
textbook definition (CPU only)."""
from fractions import Fraction

import numpy as np

from oracle import formats as F
from tests.exact import round_f32


def _pairs(rng, n):
    # bf16 numerators of every exponent, fp32 denominators shaped like block
    # scales (E4M3 value times a tensor scale), plus ranges that produce
    # subnormal and overflowing quotients
    xb = rng.integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16)
    x = F.bf16_to_f32(xb)
    dec = F.E4M3FN_VALUES[rng.integers(1, 0x7F, size=n)].astype(np.float32)
    ts = (2.0 ** rng.uniform(-140, 120, size=n)).astype(np.float32)
    with np.errstate(all="ignore"):
        s = (dec * ts).astype(np.float32)
    ok = np.isfinite(x) & np.isfinite(s) & (s > 0)
    return x[ok], s[ok]


def test_float32_division_is_correctly_rounded():
    rng = np.random.default_rng(10)
    x, s = _pairs(rng, 40000)
    with np.errstate(all="ignore"):
        q = x / s
    for xi, si, qi in zip(x, s, q):
        want = round_f32(Fraction(float(xi)) / Fraction(float(si)))
        assert float(qi) == want or (np.isinf(want) and np.isinf(qi) and np.sign(want) == np.sign(qi)), (xi, si, qi, want)


def test_float32_division_subnormal_and_tiny_quotients():
    # quotients straddling the subnormal range and the 2**-150 rounding edge
    xs = F.bf16_to_f32(np.arange(1, 0x0100, dtype=np.uint16))  # bf16 subnormals
    ss = np.array([1.0, 3.0, 1e3, 65504.0, 3 * 2.0 ** 15, 2.0 ** 17, 1.7e4], np.float32)
    for s in ss:
        with np.errstate(all="ignore"):
            q = xs / np.float32(s)
        for xi, qi in zip(xs, q):
            want = round_f32(Fraction(float(xi)) / Fraction(float(s)))
            assert float(qi) == want, (xi, s, qi, want)


def test_float32_multiplication_is_correctly_rounded():
    rng = np.random.default_rng(11)
    x, s = _pairs(rng, 20000)
    g = F.E2M1_MAGNITUDES[rng.integers(0, 8, size=x.size)].astype(np.float32)
    with np.errstate(all="ignore"):
        p = s * g
        t = x * s
    for si, gi, pi, xi, ti in zip(s, g, p, x, t):
        assert float(pi) == round_f32(Fraction(float(si)) * Fraction(float(gi)))
        want = round_f32(Fraction(float(xi)) * Fraction(float(si)))
        assert float(ti) == want or (np.isinf(want) and np.isinf(ti))
