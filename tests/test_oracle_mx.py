"""Pins of the MXFP4 oracle (``oracle.mx``), CPU only.

* E8M0 decode against torch's ``float8_e8m0fnu`` for all 256 bytes;
* floor(log2) against the bf16 bit fields (exponent field, or the leading
  mantissa bit of a subnormal) for every positive finite bf16 value;
* block scale bytes against closed forms from the OCP MX definition
  (amax 6 -> scale 1, 7 -> 1 and saturates, 8 -> 2, ...) and against an
  exact-rational twin on random blocks;
* capture and the three forwards element by element against the exact twin
  of ``tests/test_oracle_twin.py`` with s = 2^(b - 127);
* the quotient by a power-of-two scale equals an exact ldexp wherever it
  does not underflow.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F
from tests.test_oracle_twin import _bf16, twin_element


def test_e8m0_decode_matches_torch():
    b = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(b).view(torch.float8_e8m0fnu).float().numpy()
    got = oracle.e8m0_decode(b)
    assert np.isnan(got[255]) and np.isnan(want[255])
    assert np.array_equal(got[:255].view(np.uint32), want[:255].view(np.uint32))


def _floor_log2_from_bits(bits):
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e:
        return int(e) - 127
    return int(m).bit_length() - 1 - 133  # value = m * 2^-133


def test_floor_log2_every_positive_bf16():
    bits = np.arange(1, 0x7F80, dtype=np.uint16)   # +subnormals and +normals
    vals = F.bf16_to_f32(bits)
    got = oracle.floor_log2(vals)
    want = np.array([_floor_log2_from_bits(int(b)) for b in bits])
    assert np.array_equal(got, want)


def _block(values):
    v = np.zeros(32, np.float32)
    v[: len(values)] = values
    return _bf16(v)


@pytest.mark.parametrize("amax,byte", [
    (6.0, 127),            # 6 = 1.5 * 2^2: scale 1, the plain E2M1 grid
    (7.0, 127),            # still scale 1; 7 saturates to 6
    (8.0, 128),            # scale 2
    (0.75, 124),           # floor(log2 0.75) = -1 -> scale 2^-3
    (1.0, 125),
    (0.0, 0),              # all-zero block: smallest scale
    (2.0 ** -130, 0),      # clamps at the bottom of E8M0
    (2.0 ** 127, 252),     # 127 - 2 + 127
    (3.0e38, 252),
    (float("inf"), 253),   # reading: infinity counts as exponent 128
])
def test_block_scale_closed_forms(amax, byte):
    xb = _block([amax, -amax / 3, amax / 7])
    assert oracle.mx_block_scales(xb)[0] == byte


def test_block_scale_ignores_nan_and_sign():
    assert oracle.mx_block_scales(_block([np.nan, -8.0, 1.0]))[0] == 128
    assert oracle.mx_block_scales(_block([np.nan]))[0] == 0


def _twin_mx_byte(vals):
    a = max([abs(Fraction(float(v))) for v in vals if v == v], default=Fraction(0))
    if a == 0:
        return 0
    e = 0
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    while Fraction(2) ** e > a:
        e -= 1
    return min(max(e - 2, -127), 127) + 127


def test_block_scale_against_exact_twin():
    rng = np.random.default_rng(3)
    blocks = [rng.standard_normal(32) * 10.0 ** rng.uniform(-40, 38) for _ in range(300)]
    x = _bf16(np.concatenate(blocks).astype(np.float32))
    got = oracle.mx_block_scales(x)
    f = F.bf16_to_f32(x).reshape(-1, 32)
    want = [_twin_mx_byte([v for v in row if np.isfinite(v)]) for row in f]
    assert np.array_equal(got, np.array(want, dtype=np.uint8))


def _mx_tensor(rng):
    blocks = [
        rng.standard_normal(32),
        rng.standard_normal(32) * 50,
        rng.standard_t(4, 32),
        np.zeros(32),
        np.r_[np.zeros(31), -0.0],
        rng.standard_normal(32) * 2.0 ** -128,          # subnormal block maximum, scale clamps
        rng.uniform(-6, 6, 32),                          # scale 1: the grid itself
        np.r_[rng.standard_normal(30), np.nan, 3.0],
        np.r_[rng.standard_normal(31), np.inf],
        np.r_[rng.standard_normal(31) * 1e30, 3e38],
        np.r_[np.full(31, 0.25), 6.0],                   # ties at scale 1
        np.r_[np.arange(-15, 16) * 0.5, 7.5],
    ]
    return _bf16(np.concatenate(blocks).astype(np.float32))


@pytest.mark.parametrize("seed", [0, 1])
def test_mx_path_matches_exact_twin(seed):
    rng = np.random.default_rng(seed)
    xr = _mx_tensor(rng)
    n = xr.size
    xt = _bf16(F.bf16_to_f32(xr) * (1 + 0.05 * rng.standard_normal(n)).astype(np.float32))
    cap = oracle.mx_capture(xr, with_codes=True)
    roll = oracle.unpack_nibbles(cap["codes"], n)
    bits = oracle.unpack_bits(cap["bits"], n)
    # a rollout code drawn at random for half the elements exercises full information off the captured codes
    rand_codes = np.where(rng.random(n) < 0.5, rng.integers(0, 16, n), roll).astype(np.uint8)
    packed_rand = oracle.pack_nibbles(rand_codes)
    gd = oracle.mx_guided_fwd(xt, cap["scales"], cap["bits"])
    rn = oracle.mx_rne_fwd(xt, cap["scales"])
    fi = oracle.mx_full_info_fwd(xt, cap["scales"], packed_rand)
    fr, ft = F.bf16_to_f32(xr), F.bf16_to_f32(xt)
    outs = {k: (oracle.unpack_nibbles(v["codes"], n), oracle.unpack_bits(v["mask"], n), v["y"])
            for k, v in (("guided", gd), ("rne", rn), ("full", fi))}
    for blk in range(n // 32):
        byte = _twin_mx_byte([v for v in fr[blk * 32:(blk + 1) * 32] if not np.isinf(v)] +
                             ([2.0 ** 128] if np.isinf(fr[blk * 32:(blk + 1) * 32]).any() else []))
        assert cap["scales"][blk] == byte, blk
        s = float(Fraction(2) ** (byte - 127))
        for i in range(blk * 32, (blk + 1) * 32):
            code, _, _ = twin_element(fr[i], s, "rne")
            assert roll[i] == code and bits[i] == (code & 1), i
            for rule, kw in (("guided", {"c": int(bits[i])}), ("rne", {}), ("full", {"roll_code": int(rand_codes[i])})):
                c2, m2, y2 = twin_element(ft[i], s, rule, **kw)
                qc, mk, y = outs[rule]
                assert qc[i] == c2 and mk[i] == m2 and y[i] == _bf16([y2])[0], (rule, i)


def test_quotient_is_exact_ldexp_without_underflow():
    """Dividing by 2^(b-127) is exact unless the quotient is subnormal."""
    bits = np.arange(0, 0x7F80, 97, dtype=np.uint16)
    x = F.bf16_to_f32(bits)
    for b in (0, 60, 100, 127, 150, 200, 254):
        xb = np.repeat(bits, 1)
        pad = (-xb.size) % 32
        xb = np.r_[xb, np.zeros(pad, np.uint16)]
        sb = np.full(xb.size // 32, b, np.uint8)
        out = oracle.mx_rne_fwd(xb, sb)
        # rebuild the quotient's E2M1 code independently from ldexp
        z = np.ldexp(np.r_[x, np.zeros(pad, np.float32)].astype(np.float64), 127 - b)
        ok = (z == 0) | (np.abs(z) >= 2.0 ** -126)
        a = np.minimum(np.abs(z), 6.0)
        idx = oracle.e2m1_rne_index(a.astype(np.float32))
        got = oracle.unpack_nibbles(out["codes"], xb.size) & 7
        assert np.array_equal(got[ok], idx[ok]), b
