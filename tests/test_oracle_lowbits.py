"""Pins of the b-bit cached-low-bits oracle (``capture_lowbits`` /
``lowbits_fwd``), CPU only, by brute force over every bf16 z with |z| <= 7
under a unit scale against every signed rollout codeword:

* b = 1 reproduces the guided rule and b = 4 the full-information rule
  (both pinned on their own in ``test_oracle_rule.py``);
* a rollout codeword within the window of 2^b signed indices centred on z's
  bracket is reconstructed exactly, so the result equals full information
  there (the recoverable window that b buys);
* the local guarantee (never farther from the rollout value than
  round-to-nearest) holds wherever the rollout codeword is in the window;
* capture's plane 0 is the b = 1 parity plane, and b = 4 planes determine
  the full code.
"""
import numpy as np
import pytest

import oracle
from oracle import formats as F
from tests.test_oracle_rule import SIGNED_GRID, _all_bf16_up_to, _signed_idx, _signed_val


def _planes_for(r_signed, n, b):
    res = np.mod(r_signed, 1 << b)
    return np.concatenate([oracle.pack_bits(np.full(n, (res >> k) & 1, np.uint8)) for k in range(b)])


@pytest.fixture(scope="module")
def sweep():
    x = _all_bf16_up_to(7.0)
    n = x.size
    scales = np.full(n // 16, 0x38, np.uint8)
    z = np.clip(F.bf16_to_f32(x).astype(np.float64), -6, 6)
    L = np.searchsorted(SIGNED_GRID, z, side="right") - 8
    H = np.searchsorted(SIGNED_GRID, z, side="left") - 7
    rne = _signed_idx(oracle.unpack_nibbles(oracle.rne_fwd(x, scales, 1.0)["codes"], n))
    out = {"x": x, "n": n, "scales": scales, "L": L, "H": H, "rne": rne, "res": {}}
    for r in range(-7, 8):
        code = (8 | -r) if r < 0 else r
        bits = oracle.pack_bits(np.full(n, abs(r) & 1, np.uint8))
        codes = oracle.pack_nibbles(np.full(n, code, np.uint8))
        g = oracle.unpack_nibbles(oracle.guided_fwd(x, scales, 1.0, bits)["codes"], n)
        f = oracle.unpack_nibbles(oracle.full_info_fwd(x, scales, 1.0, codes)["codes"], n)
        lb = {b: oracle.unpack_nibbles(oracle.lowbits_fwd(x, scales, 1.0, _planes_for(r, n, b), b)["codes"], n)
              for b in (1, 2, 3, 4)}
        out["res"][r] = (g, f, lb)
    return out


def test_b1_is_guided_and_b4_is_full_information(sweep):
    for r, (g, f, lb) in sweep["res"].items():
        assert np.array_equal(lb[1], g), r
        assert np.array_equal(lb[4], f), r


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_rollout_inside_the_window_is_recovered(sweep, b):
    """|r - (L + 1/2)| < 2^(b-1) for a strict bracket (L, L + 1): the result is
    the full-information result (the rollout codeword itself when it is an
    endpoint, else the endpoint on its side)."""
    L, H = sweep["L"], sweep["H"]
    half = 1 << (b - 1)
    strict = H == L + 1
    for r, (_, f, lb) in sweep["res"].items():
        inside = strict & (np.abs(2 * r - (2 * L + 1)) < 2 * half)
        assert np.array_equal(lb[b][inside], f[inside]), (b, r)
        onz = ~strict  # z is a codeword: always z itself
        assert np.array_equal(_signed_idx(lb[b][onz]), L[onz]), (b, r)


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_local_guarantee_inside_the_window(sweep, b):
    L, H, rne = sweep["L"], sweep["H"], sweep["rne"]
    half = 1 << (b - 1)
    for r, (_, _, lb) in sweep["res"].items():
        inside = np.abs(2 * r - (L + H)) < 2 * half
        got = np.abs(_signed_val(_signed_idx(lb[b])) - _signed_val(r))
        ref = np.abs(_signed_val(rne) - _signed_val(r))
        assert np.all(got[inside] <= ref[inside]), (b, r)


def test_recovered_set_grows_with_b(sweep):
    """More cached bits never recover fewer rollout codewords."""
    for r, (_, _, lb) in sweep["res"].items():
        prev = None
        for b in (1, 2, 3, 4):
            hit = _signed_idx(lb[b]) == r
            if prev is not None:
                assert np.all(hit[prev]), (b, r)
            prev = hit


def test_capture_planes():
    rng = np.random.default_rng(8)
    x = F.f32_to_bf16_rne(rng.standard_t(4, 64 * 48).astype(np.float32))
    ts = oracle.tensor_scale(x)
    cap = oracle.capture(x, ts, with_codes=True)
    n = x.size
    for b in (1, 2, 3, 4):
        lb = oracle.capture_lowbits(x, ts, b)
        assert lb["planes"].size == b * n // 8
        assert np.array_equal(lb["planes"][: n // 8], cap["bits"])
        assert np.array_equal(lb["scales"], cap["scales"])
    planes = oracle.capture_lowbits(x, ts, 4)["planes"].reshape(4, -1)
    res = sum(oracle.unpack_bits(planes[k], n).astype(np.int64) << k for k in range(4))
    si = np.where(res >= 8, res - 16, res)                 # two's complement back to -7..7
    codes = oracle.unpack_nibbles(cap["codes"], n)
    assert np.array_equal(si, _signed_idx(codes))


def test_residue_without_an_index_takes_the_endpoint_nearer_zero():
    """b = 4, residue 8: no signed index -7..7 has it (no capture writes it);
    the reading takes the bracket endpoint nearer zero for either sign."""
    z = np.array([0.3, -0.3, 2.4, -2.4, 5.0, -5.0, 1.0, -1.0] * 2, np.float32)
    x = F.f32_to_bf16_rne(z)
    scales = np.full(1, 0x38, np.uint8)
    planes = np.concatenate([oracle.pack_bits(np.full(16, (8 >> k) & 1, np.uint8)) for k in range(4)])
    out = oracle.lowbits_fwd(x, scales, 1.0, planes, 4)
    got = np.abs(_signed_val(_signed_idx(oracle.unpack_nibbles(out["codes"], 16))))
    want = np.array([0.0, 0.0, 2.0, 2.0, 4.0, 4.0, 1.0, 1.0] * 2)
    assert np.array_equal(got, want)
