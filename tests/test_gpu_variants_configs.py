"""The MXFP4, MXFP8 and b-cached-low-bits variants at full workload sizes: the KV
cache workload (2 x 131072 x 512) and the ragged large-hidden workload
(65573 x 7168, half of the training values placed near codeword midpoints),
every output on sampled rows (first, last, ragged tail, random) against the
oracle, bit for bit."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import to_np_u8, to_np_u16
from tests.workload_place import oracle_block_scales, place_kv, place_near_midpoints

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _rows(rows, k, seed):
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(rows, size=min(k, rows), replace=False).tolist())
    pick.update([0, rows - 1, rows - 2])
    return np.array(sorted(pick))


def _take(t, idx, per_row, u16=False):
    v = (t.view(torch.int16) if u16 else t).reshape(-1, per_row)[torch.from_numpy(idx).to(t.device)]
    return to_np_u16(v) if u16 else to_np_u8(v)


def _check(ctx, got, want):
    for k, w in want.items():
        g = got[k]
        if not np.array_equal(g.reshape(-1), np.asarray(w).reshape(-1)):
            bad = np.flatnonzero(g.reshape(-1) != np.asarray(w).reshape(-1))
            raise AssertionError(f"{ctx}: {k} differs at {bad.size} positions, first {bad[:6].tolist()}")


def _mx_site(name, x_roll, x_train, k_rows, seed):
    import fp4_rollout_guided_amd as tr
    rows, cols = x_roll.shape
    _say(f"case {name}: MXFP4 {rows}x{cols}")
    sc, bt, cd = tr.mx_capture(x_roll, want_codes=True)
    yg, mg, qg = tr.mx_guided_fakequant_fwd(x_train, sc, bt, want_codes=True)
    yf, mf, qf = tr.mx_full_info_fakequant_fwd(x_train, sc, cd, want_codes=True)
    torch.cuda.synchronize()
    idx = _rows(rows, k_rows, seed)
    xr, xt = _take(x_roll, idx, cols, True), _take(x_train, idx, cols, True)
    cap = oracle.mx_capture(xr, with_codes=True)
    gd = oracle.mx_guided_fwd(xt, cap["scales"], cap["bits"])
    fi = oracle.mx_full_info_fwd(xt, cap["scales"], cap["codes"])
    got = {"scales": _take(sc, idx, cols // 32), "bits": _take(bt, idx, cols // 8), "codes": _take(cd, idx, cols // 2),
           "y_g": _take(yg, idx, cols, True), "m_g": _take(mg, idx, cols // 8), "q_g": _take(qg, idx, cols // 2),
           "y_f": _take(yf, idx, cols, True), "m_f": _take(mf, idx, cols // 8), "q_f": _take(qf, idx, cols // 2)}
    want = {"scales": cap["scales"], "bits": cap["bits"], "codes": cap["codes"], "y_g": gd["y"], "m_g": gd["mask"],
            "q_g": gd["codes"], "y_f": fi["y"], "m_f": fi["mask"], "q_f": fi["codes"]}
    _check(name, got, want)


def _mx8_site(name, x_roll, x_train, k_rows, seed):
    import fp4_rollout_guided_amd as tr
    rows, cols = x_roll.shape
    _say(f"case {name}: MXFP8 {rows}x{cols}")
    sc, bt, cd = tr.mx8_capture(x_roll, want_codes=True)
    yg, mg, qg = tr.mx8_guided_fakequant_fwd(x_train, sc, bt, want_codes=True)
    yf, mf, qf = tr.mx8_full_info_fakequant_fwd(x_train, sc, cd, want_codes=True)
    torch.cuda.synchronize()
    idx = _rows(rows, k_rows, seed)
    xr, xt = _take(x_roll, idx, cols, True), _take(x_train, idx, cols, True)
    cap = oracle.mx8_capture(xr, with_codes=True)
    gd = oracle.mx8_guided_fwd(xt, cap["scales"], cap["bits"])
    fi = oracle.mx8_full_info_fwd(xt, cap["scales"], cap["codes"])
    got = {"scales": _take(sc, idx, cols // 32), "bits": _take(bt, idx, cols // 8), "codes": _take(cd, idx, cols),
           "y_g": _take(yg, idx, cols, True), "m_g": _take(mg, idx, cols // 8), "q_g": _take(qg, idx, cols),
           "y_f": _take(yf, idx, cols, True), "m_f": _take(mf, idx, cols // 8), "q_f": _take(qf, idx, cols)}
    want = {"scales": cap["scales"], "bits": cap["bits"], "codes": cap["codes"], "y_g": gd["y"], "m_g": gd["mask"],
            "q_g": gd["codes"], "y_f": fi["y"], "m_f": fi["mask"], "q_f": fi["codes"]}
    _check(name, got, want)


def _lowbits_site(name, x_roll, x_train, nbits, k_rows, seed):
    import fp4_rollout_guided_amd as tr
    rows, cols = x_roll.shape
    _say(f"case {name}: b = {nbits} low bits {rows}x{cols}")
    ts = tr.tensor_scale(x_roll)
    sc, pl, _ = tr.capture_lowbits(x_roll, ts, nbits)
    y, m, q = tr.lowbits_fakequant_fwd(x_train, sc, ts, nbits, pl, want_codes=True)
    torch.cuda.synchronize()
    tsf = np.float32(ts.cpu().numpy()[0])
    idx = _rows(rows, k_rows, seed)
    xr, xt = _take(x_roll, idx, cols, True), _take(x_train, idx, cols, True)
    cap = oracle.capture_lowbits(xr, tsf, nbits)
    out = oracle.lowbits_fwd(xt, cap["scales"], tsf, cap["planes"], nbits)
    n = rows * cols
    planes = pl.reshape(nbits, n // 8)
    got = {"scales": _take(sc, idx, cols // 16),
           "planes": np.concatenate([_take(planes[k], idx, cols // 8) for k in range(nbits)]),
           "y": _take(y, idx, cols, True), "mask": _take(m, idx, cols // 8), "codes": _take(q, idx, cols // 2)}
    want = {"scales": cap["scales"], "planes": cap["planes"], "y": out["y"], "mask": out["mask"],
            "codes": out["codes"]}
    _check(name, got, want)


@pytest.fixture(scope="module")
def workload4(device):
    x_roll = workloads.cfg4_rollout(device)
    _, s_block = oracle_block_scales(x_roll)
    return x_roll, place_near_midpoints(x_roll, s_block)


def test_mx_workload4(device, workload4):
    _mx_site("workload 4", *workload4, k_rows=96, seed=41)


def test_mx8_workload4(device, workload4):
    _mx8_site("workload 4", *workload4, k_rows=96, seed=47)


@pytest.mark.parametrize("nbits", [2, 3])
def test_lowbits_workload4(device, workload4, nbits):
    _lowbits_site("workload 4", *workload4, nbits=nbits, k_rows=96, seed=42 + nbits)


@pytest.mark.parametrize("which", ["k", "v"])
def test_variants_workload2(device, which):
    x_roll = workloads.cfg2_rollout(device, which)
    _, s_block = oracle_block_scales(x_roll)
    x_train = place_kv(x_roll, which, s_block)
    shape2d = (x_roll.shape[0], x_roll.shape[1] * x_roll.shape[2])
    _mx_site(f"workload 2 {which}", x_roll.reshape(shape2d), x_train.reshape(shape2d), k_rows=256, seed=21)
    _mx8_site(f"workload 2 {which}", x_roll.reshape(shape2d), x_train.reshape(shape2d), k_rows=256, seed=23)
    _lowbits_site(f"workload 2 {which}", x_roll.reshape(shape2d), x_train.reshape(shape2d), nbits=2, k_rows=256,
                  seed=22)
