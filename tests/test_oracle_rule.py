"""Pins for the rounding rule itself (CPU only): invariants that the
rcap.io TRACE post states or implies, checked by brute force, plus the
post's worked example and its compression figure."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import formats as F

HERE = os.path.dirname(os.path.abspath(__file__))
SIGNED_GRID = np.array([-6, -4, -3, -2, -1.5, -1, -0.5, 0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)


def _bf16(v):
    return F.f32_to_bf16_rne(np.asarray(v, np.float32))


def _signed_idx(codes):
    c = codes.astype(np.int16)
    return np.where(c & 8, -(c & 7), c & 7)


def _signed_val(si):
    return SIGNED_GRID[si + 7]


def _all_bf16_up_to(limit):
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = F.bf16_to_f32(b)
    keep = np.isfinite(v) & (np.abs(v) <= limit)
    b = b[keep]
    pad = (-b.size) % 16
    return np.concatenate([b, np.zeros(pad, np.uint16)])


@pytest.fixture(scope="module")
def sweep():
    """Every bf16 z with |z| <= 7 under a unit scale (byte 0x38 = 1.0,
    tensor scale 1), against every signed rollout codeword."""
    x = _all_bf16_up_to(7.0)
    n = x.size
    scales = np.full(n // 16, 0x38, np.uint8)
    z = F.bf16_to_f32(x).astype(np.float64)
    zc = np.clip(z, -6, 6)
    L = np.searchsorted(SIGNED_GRID, zc, side="right") - 8   # largest <= z
    H = np.searchsorted(SIGNED_GRID, zc, side="left") - 7    # smallest >= z
    rne = _signed_idx(oracle.unpack_nibbles(oracle.rne_fwd(x, scales, 1.0)["codes"], n))
    out = {"x": x, "n": n, "scales": scales, "L": L, "H": H, "rne": rne, "per_r": {}}
    for r in range(-7, 8):
        code = (8 | -r) if r < 0 else r
        bits = oracle.pack_bits(np.full(n, abs(r) & 1, np.uint8))
        codes = oracle.pack_nibbles(np.full(n, code, np.uint8))
        g = _signed_idx(oracle.unpack_nibbles(oracle.guided_fwd(x, scales, 1.0, bits)["codes"], n))
        f = _signed_idx(oracle.unpack_nibbles(oracle.full_info_fwd(x, scales, 1.0, codes)["codes"], n))
        out["per_r"][r] = (g, f)
    return out


def test_bracket_contains_rne_and_is_adjacent(sweep):
    L, H, rne = sweep["L"], sweep["H"], sweep["rne"]
    assert np.all((H - L >= 0) & (H - L <= 1))
    assert np.all((rne == L) | (rne == H))


def test_straddle_sites_recover_rollout_code(sweep):
    """A one-codeword mismatch whose rollout codeword is an endpoint of the
    training value's bracket is recovered exactly."""
    L, H = sweep["L"], sweep["H"]
    for r, (g, f) in sweep["per_r"].items():
        inb = (r == L) | (r == H)
        assert np.all(g[inb] == r), r
        assert np.all(f[inb] == r), r


def test_guided_picks_bracket_endpoint_with_cached_parity(sweep):
    L, H = sweep["L"], sweep["H"]
    for r, (g, _) in sweep["per_r"].items():
        assert np.all((g == L) | (g == H))
        nondeg = L != H
        assert np.all((np.abs(g[nondeg]) & 1) == (abs(r) & 1))
        assert np.all(g[~nondeg] == L[~nondeg])


def test_local_guarantee_holds_exactly_off_the_characterized_set(sweep):
    """|q* - q_roll| <= |q_RNE - q_roll| fails only when the rollout codeword
    lies outside the bracket, beyond q_RNE on q_RNE's side, an odd number of
    steps away; full-information guidance never fails it."""
    L, H, rne = sweep["L"], sweep["H"], sweep["rne"]
    v_rne = _signed_val(rne)
    for r, (g, f) in sweep["per_r"].items():
        vr = SIGNED_GRID[r + 7]
        viol = np.abs(_signed_val(g) - vr) > np.abs(v_rne - vr)
        outside = (r != L) & (r != H) & (L != H)
        odd = ((abs(r) - np.abs(rne)) & 1) == 1
        beyond = ((rne == H) & (r > H)) | ((rne == L) & (r < L))
        in_v = outside & odd & beyond
        assert np.array_equal(viol, in_v), r
        assert not np.any(np.abs(_signed_val(f) - vr) > np.abs(v_rne - vr)), r
        # two-codeword (even-step) mismatches fall back to RNE
        even = outside & ~odd
        assert np.all(g[even] == rne[even]), r


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_identical_inputs_give_identical_codes(seed):
    """x_train == x_roll: guided == RNE == rollout code at every site."""
    rng = np.random.default_rng(seed)
    parts = [rng.standard_normal(4096), rng.standard_t(4, 4096) * 30,
             rng.laplace(size=4096), rng.uniform(-1e-3, 1e-3, 4096)]
    x = np.concatenate(parts)
    x[rng.choice(x.size, 16, replace=False)] *= 200
    xb = _bf16(x)
    ts = oracle.tensor_scale(xb)
    cap = oracle.capture(xb, ts, with_codes=True)
    g = oracle.guided_fwd(xb, cap["scales"], ts, cap["bits"])
    r = oracle.rne_fwd(xb, cap["scales"], ts)
    assert np.array_equal(g["codes"], cap["codes"])
    assert np.array_equal(r["codes"], cap["codes"])
    assert np.array_equal(g["y"], r["y"])


def test_worked_example_from_the_post():
    with open(os.path.join(HERE, "golden", "worked_example.json")) as fh:
        ex = json.load(fh)
    e = ex["expect"]
    xr = np.zeros(32, np.float32)
    xt = np.zeros(32, np.float32)
    xr[0:2] = ex["block"]["x_roll"]
    xt[0:2] = ex["block"]["x_train"]
    xr[16] = xt[16] = ex["tensor_amax"]
    xr_b, xt_b = _bf16(xr), _bf16(xt)
    ts = oracle.tensor_scale(xr_b)
    assert float(ts) == e["tensor_scale"]
    cap = oracle.capture(xr_b, ts, with_codes=True)
    assert cap["scales"][0] == e["scale_byte"]
    s, valid = oracle.decode_scales(cap["scales"][:1], ts)
    assert valid[0] and float(s[0]) == e["decoded_scale"]
    rc = oracle.unpack_nibbles(cap["codes"], 32)
    assert oracle.unpack_bits(cap["bits"], 32)[1] == e["rollout_bit"]
    roll_val = float(s[0]) * oracle.E2M1_MAGNITUDES[rc[1] & 7]
    rne = F.bf16_to_f32(oracle.rne_fwd(xt_b, cap["scales"], ts)["y"])
    gd = F.bf16_to_f32(oracle.guided_fwd(xt_b, cap["scales"], ts, cap["bits"])["y"])
    assert roll_val == e["rollout_value"]
    assert rne[1] == e["rne_train_value"] and gd[1] == e["guided_train_value"]
    assert roll_val - rne[1] == e["fp4_gap_rne"] and roll_val - gd[1] == e["fp4_gap_guided"]
    assert abs(float(F.bf16_to_f32(xr_b)[1] - F.bf16_to_f32(xt_b)[1]) - 0.48) < 0.05


def test_compression_matches_the_posts_six_fold_figure():
    """One bit plus scale metadata for the deeper half of the layers against
    full FP4 codes everywhere: about 6x (bandwidth paragraph; 20 of 40 layers
    in the ablation bullet)."""
    acc = oracle.compact_cache_bytes(262144 * 2048, captured_layers=20, total_layers=40)
    assert acc["bits_per_elem_compact"] == 1.5 and acc["bits_per_elem_full"] == 4.5
    assert acc["compact_bytes"] == 2_013_265_920
    assert acc["full_nvfp4_bytes"] == 12_079_595_520
    assert acc["ratio_per_layer"] == 3.0 and acc["ratio"] == 6.0
