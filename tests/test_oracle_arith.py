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


def test_sharded_tensor_scale_is_the_max_of_local_scales():
    """Division by 2688 rounds monotonically, so max_i fl32(amax_i / 2688) =
    fl32(max_i amax_i / 2688): an all-reduce(max) of per-shard tensor scales
    gives the whole tensor's scale exactly (NaN, infinity and all-zero shards
    included)."""
    import oracle
    rng = np.random.default_rng(2688)
    for trial in range(200):
        n = 16 * int(rng.integers(1, 400))
        v = rng.standard_t(3, n) * 10.0 ** rng.uniform(-40, 38)
        if trial % 7 == 0:
            v[rng.integers(0, n)] = np.nan
        if trial % 11 == 0:
            v[rng.integers(0, n)] = np.inf
        if trial % 13 == 0:
            v[: n // 2] = 0.0
        with np.errstate(over="ignore"):  # values past the fp32 range become infinities, which the rule covers
            x = F.f32_to_bf16_rne(v.astype(np.float32))
        cuts = np.sort(rng.choice(np.arange(0, n + 1, 16), size=int(rng.integers(1, 6)), replace=True))
        shards = np.split(x, cuts)
        local = [np.float32(oracle.tensor_scale(s)) for s in shards]
        whole = np.float32(oracle.tensor_scale(x))
        assert np.float32(max(local)).view(np.uint32) == whole.view(np.uint32), trial
