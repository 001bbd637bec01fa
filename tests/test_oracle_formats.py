"""Pins for the oracle's number formats (CPU only).

Each test checks an oracle routine against something other than itself:
PyTorch's CPU casts, exact rational rounding, or an exhaustive sweep.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from tests.exact import round_bf16

ALL_BF16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def test_bf16_to_f32_matches_torch_all_patterns():
    ours = F.bf16_to_f32(ALL_BF16)
    ref = torch.from_numpy(ALL_BF16.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _torch_bf16_bits(v):
    return torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_f32_to_bf16_rne_matches_torch_random_and_ties():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    # exact ties: low half 0x8000, with odd and even kept LSBs
    ties = (rng.integers(0, 1 << 16, size=20000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    near = np.concatenate([ties - 1, ties + 1])
    top = np.arange(0x7F7F0000, 0x7F800000, 7, dtype=np.uint32)  # overflow region
    allb = np.concatenate([bits, ties, near, top, top | 0x80000000])
    v = allb.view(np.float32)
    v = v[~np.isnan(v)]
    assert np.array_equal(F.f32_to_bf16_rne(v), _torch_bf16_bits(v))


def test_f32_to_bf16_rne_exact_rational_sample():
    rng = np.random.default_rng(2)
    v = rng.integers(0, 1 << 32, size=3000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    v = v[np.isfinite(v)]
    ours = F.f32_to_bf16_rne(v)
    for x, b in zip(v, ours):
        want = round_bf16(Fraction(float(x)))
        got = float(F.bf16_to_f32(np.array([b]))[0])
        assert got == want or (np.isinf(want) and np.isinf(got) and np.sign(want) == np.sign(got)), (x, b)


def test_e4m3fn_table_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    ours = F.E4M3FN_VALUES
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def _torch_e4m3(v):
    return torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3fn_encode_matches_torch_below_max():
    # every non-negative bf16 magnitude below 448, random fp32, and every
    # midpoint between consecutive E4M3 values with its fp32 neighbours
    mags = F.bf16_to_f32(np.arange(0, 0x7F80, dtype=np.uint16))
    mags = mags[mags < 448]
    rng = np.random.default_rng(3)
    rnd = (rng.random(500_000) * 448).astype(np.float32)
    tiny = (rng.random(100_000) * 2.0 ** -5).astype(np.float32)
    vals = F.E4M3FN_VALUES[:0x7F]
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    nb = np.concatenate([np.nextafter(mids, np.float32(0)), mids, np.nextafter(mids, np.float32(1000))])
    v = np.concatenate([mags, rnd, tiny, nb]).astype(np.float32)
    v = v[v < 448]
    assert np.array_equal(F.e4m3fn_encode_rne_sat(v), _torch_e4m3(v))


def test_e4m3fn_encode_saturates_and_ties_even():
    v = np.array([448, 449, 464, 479, 1e30, np.inf], dtype=np.float32)
    assert np.all(F.e4m3fn_encode_rne_sat(v) == 0x7E)
    assert F.e4m3fn_encode_rne_sat(np.array([np.nan], np.float32))[0] == 0
    # 2**-10 lies halfway between 0 and the smallest subnormal -> even (0)
    assert F.e4m3fn_encode_rne_sat(np.array([2.0 ** -10], np.float32))[0] == 0x00
    # 3 * 2**-10 lies halfway between 0x01 and 0x02 -> 0x02
    assert F.e4m3fn_encode_rne_sat(np.array([3 * 2.0 ** -10], np.float32))[0] == 0x02
    # 1.0625 halfway between 1.0 (0x38) and 1.125 (0x39) -> 0x38
    assert F.e4m3fn_encode_rne_sat(np.array([1.0625], np.float32))[0] == 0x38
    with pytest.raises(ValueError):
        F.e4m3fn_encode_rne_sat(np.array([-1.0], np.float32))


def _e2m1_exact(a):
    """Nearest E2M1 magnitude index by exact rational distances, ties to the
    even index (mantissa bit 0)."""
    fa = Fraction(float(a))
    grid = [Fraction(g) for g in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
    d = [abs(fa - g) for g in grid]
    best = min(d)
    idx = [i for i, di in enumerate(d) if di == best]
    if len(idx) == 2:
        return idx[0] if idx[0] % 2 == 0 else idx[1]
    return idx[0]


def test_e2m1_rne_exhaustive_all_bf16():
    """All 65536 bf16 patterns as z: min(|z|, 6) rounded by the oracle equals
    exact nearest-with-ties-to-even."""
    z = F.bf16_to_f32(ALL_BF16)
    z = z[~np.isnan(z)]
    a = np.minimum(np.abs(z), np.float32(6))
    ours = F.e2m1_rne_index(a)
    want = np.array([_e2m1_exact(x) for x in a], dtype=np.uint8)
    assert np.array_equal(ours, want)
    # the listed tie-break cases
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    assert F.e2m1_rne_index(ties).tolist() == [0, 2, 2, 4, 4, 6, 6]


def test_e2m1_bracket_exhaustive_all_bf16():
    z = F.bf16_to_f32(ALL_BF16)
    z = z[~np.isnan(z)]
    a = np.minimum(np.abs(z), np.float32(6))
    lo, hi = F.e2m1_bracket(a)
    g = F.E2M1_MAGNITUDES
    assert np.all(g[lo] <= a) and np.all(g[hi] >= a)
    assert np.all(hi.astype(int) - lo.astype(int) <= 1)
    on_grid = np.isin(a.astype(np.float64), g)
    assert np.array_equal(lo == hi, on_grid)
    # nothing of the grid lies strictly inside a non-degenerate bracket
    assert np.all((hi == lo) | (hi == lo + 1))


def test_small_decoders_against_torch_and_definitions():
    """The oracle's byte decoders that the pins above reach only through the
    functions using them: E4M3FN decode of arbitrary arrays (torch's cast),
    the signed grid index of E2M1 codes (-7..7, both zeros 0) and the signed
    E4M3 values with NaN bytes read as +-480."""
    import torch
    import oracle
    b = np.arange(256, dtype=np.uint32).astype(np.uint8).reshape(16, 16)
    want = torch.from_numpy(b.copy()).view(torch.float8_e4m3fn).double().numpy()
    got = oracle.e4m3fn_decode(b)
    assert got.shape == b.shape
    assert np.array_equal(np.isnan(got), np.isnan(want)) and np.array_equal(got[~np.isnan(got)], want[~np.isnan(want)])
    codes = np.arange(16, dtype=np.uint8)
    assert oracle.signed_index(codes).tolist() == [0, 1, 2, 3, 4, 5, 6, 7, 0, -1, -2, -3, -4, -5, -6, -7]
    v = oracle.e4m3_signed_values(np.arange(256, dtype=np.uint32).astype(np.uint8))
    dec = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    finite = ~np.isnan(dec)
    assert np.array_equal(v[finite], dec[finite])
    assert v[0x7F] == 480.0 and v[0xFF] == -480.0 and v[0x80] == 0.0
