"""Pin of the oracle's agreement statistics (``oracle.mismatch_stats``),
CPU only: every count recomputed element by element from the exact rational
twin of ``tests/test_oracle_twin.py`` (RNE and guided codes, the bracket of
|x_train / s|) and the definitions -- signed grid steps between rollout and
RNE codes, straddle = mismatch with the rollout codeword at an end of the
bracket, crossed = one-step mismatch that is no straddle, recovered =
mismatch where guided returns the rollout codeword, violation = guided value
farther from the rollout value than the RNE value -- on crafted tensors with
NaN, infinities, zero-scale and NaN scale bytes, random rollout codes
(both zeros included) and cached bits that do and do not match them."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import formats as F
from tests.exact import round_f32
from tests.test_oracle_twin import GRID, _tiny_tensor, twin_bracket, twin_element, twin_scale


def _si(code):
    return -(code & 7) if code & 8 else code & 7


def _val(code):
    v = GRID[code & 7]
    return -v if code & 8 else v


def _twin_counts(xt32, scales, ts, roll, cbits):
    hist = [0] * 15
    straddle = crossed = recovered = violations = 0
    for i, xv in enumerate(xt32):
        s = twin_scale(scales[i // 16], ts)
        r = int(roll[i])
        n_code, _, _ = twin_element(xv, s, "rne")
        g_code, _, _ = twin_element(xv, s, "guided", c=int(cbits[i]))
        steps = abs(_si(r) - _si(n_code))
        hist[steps] += 1
        if steps:
            # bracket endpoints as signed indices, with the sign of z (the code's sign bit)
            valid = np.isfinite(s) and s > 0
            if xv != xv or not valid:
                ends = {0}
            else:
                zr = xv if np.isinf(xv) else round_f32(Fraction(float(xv)) / Fraction(float(s)))
                lo, hi = twin_bracket(np.float32(min(abs(zr), 6.0)))
                sg = -1 if (n_code & 8) else 1
                ends = {sg * lo, sg * hi}
            st = _si(r) in ends
            straddle += st
            crossed += steps == 1 and not st
            recovered += _si(g_code) == _si(r)
        violations += abs(_val(g_code) - _val(r)) > abs(_val(n_code) - _val(r))
    return hist, straddle, crossed, recovered, violations


def _check(xt, scales, ts, roll, cbits):
    n = xt.size
    st = oracle.mismatch_stats(xt, scales, ts, oracle.pack_nibbles(roll), oracle.pack_bits(cbits.astype(np.uint8)))
    hist, straddle, crossed, recovered, violations = _twin_counts(F.bf16_to_f32(xt), scales, ts, roll, cbits)
    assert st["hist"] == hist
    assert (st["straddle"], st["crossed"], st["recovered"], st["violations"]) == \
        (straddle, crossed, recovered, violations)
    assert st["n"] == n and st["mismatched"] == n - hist[0]
    return st


@pytest.mark.parametrize("seed,consistent", [(0, True), (1, False)])
def test_mismatch_stats_specials(seed, consistent):
    """Crafted blocks (NaN, infinities, zeros, subnormals, huge values), NaN
    and zero scale bytes, rollout codes of every kind on 30% of the sites."""
    rng = np.random.default_rng(300 + seed)
    xr = np.concatenate([_tiny_tensor(rng) for _ in range(4)])
    xr32 = F.bf16_to_f32(xr)
    with np.errstate(over="ignore"):
        xt32 = np.where(np.isfinite(xr32), xr32 * (1 + 0.2 * rng.standard_normal(xr32.size)), xr32)
        xt = F.f32_to_bf16_rne(xt32.astype(np.float32))
    ts = oracle.tensor_scale(xr)
    cap = oracle.capture(xr, ts, with_codes=True)
    scales = cap["scales"].copy()
    scales[[1, 5]] = [0x7F, 0x00]
    n = xt.size
    roll = oracle.unpack_nibbles(cap["codes"], n).copy()
    flip = rng.random(n) < 0.3
    roll[flip] = rng.integers(0, 16, flip.sum())            # rollout codes of every kind, -0 included
    cbits = (roll & 1) if consistent else rng.integers(0, 2, n)
    st = _check(xt, scales, ts, roll, cbits)
    assert sum(st["hist"][1:]) > 50


@pytest.mark.parametrize("seed", [0, 1])
def test_mismatch_stats_near_rollout(seed):
    """Unit scale (byte 0x38, ts = 1, so z = x): z_train uniform over
    [-6.5, 6.5], the rollout's value within N(0, 0.3) of it and its code by
    RNE, so straddles, crossed moves and multi-step mismatches all occur;
    cached bits from the rollout codes (every straddle is recovered)."""
    rng = np.random.default_rng(400 + seed)
    n = 4096
    zt = rng.uniform(-6.5, 6.5, n)
    zr = zt + 0.3 * rng.standard_normal(n)
    xt, xr = (F.f32_to_bf16_rne(v.astype(np.float32)) for v in (zt, zr))
    scales = np.full(n // 16, 0x38, np.uint8)
    roll = oracle.unpack_nibbles(oracle.rne_fwd(xr, scales, np.float32(1))["codes"], n)
    st = _check(xt, scales, np.float32(1), roll, roll & 1)
    assert st["straddle"] > 200 and st["crossed"] > 20 and st["hist"][2] > 20
    assert st["recovered"] == st["straddle"]   # the guided rule recovers exactly the straddles
