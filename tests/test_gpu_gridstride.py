"""The grid-stride paths of every kernel (and the batch entry points'
small-grid splits), and the non-temporal instantiations.  Production grids
cover a tensor in one pass up to 2^34 elements, so these loops only run for
larger tensors; the small-grid build of the same sources (grids capped at 3
workgroups) runs them for several iterations on test-sized tensors.  That
build also streams every tensor with the non-temporal hint, which
production applies past 256 MiB only, so the comparison pins those
instantiations on a ragged tensor with NaN and infinite blocks as well.
Every entry point's outputs must equal the production build's bit for bit
(which the other GPU tests tie to the oracle); capture is also checked
against the oracle directly."""
import contextlib
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F
from tests.gpu_util import from_np_u16, to_np_u8, to_np_u16

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@contextlib.contextmanager
def _small_grid():
    import fp4_rollout_guided_amd as tr
    saved = tr.lib
    tr.lib = tr.load_library(tr.SMALLGRID_LIB_PATH)
    try:
        yield
    finally:
        tr.lib = saved


def _host(v):
    if v is None:
        return None
    if v.dtype in (torch.bfloat16, torch.int16):
        return to_np_u16(v)
    if v.dtype == torch.float32:
        return v.cpu().numpy().view(np.uint32)
    if v.dtype == torch.int64:
        return v.cpu().numpy()
    return to_np_u8(v)


def _everything(tr, xr, xt, g, offsets, perm):
    """Run every entry point once; return host copies keyed by name."""
    out = {}
    ts = tr.tensor_scale(xr)
    sc, bt, cd = tr.capture(xr, ts, want_codes=True)
    out.update(ts=ts, scales=sc, bits=bt, codes=cd)
    for name, fn in (("g", lambda: tr.guided_fakequant_fwd(xt, sc, ts, bt, want_codes=True)),
                     ("r", lambda: tr.rne_fakequant_fwd(xt, sc, ts, want_codes=True)),
                     ("f", lambda: tr.full_info_fakequant_fwd(xt, sc, ts, cd, want_codes=True))):
        y, m, q = fn()
        out.update({f"y_{name}": y, f"m_{name}": m, f"q_{name}": q})
    out["gin"] = tr.ste_bwd(g, out["m_g"])
    gb, gs, gc = tr.gather_records(bt, sc, cd, xr.shape[1], perm)
    out.update(gather_bits=gb, gather_scales=gs, gather_codes=gc)
    gts = tr.grouped_tensor_scale(xr, offsets)
    gsc, gbt, gcd = tr.grouped_capture(xr, offsets, gts, want_codes=True)
    out.update(gts=gts, gsc=gsc, gbt=gbt, gcd=gcd)
    for name, fn in (("gg", lambda: tr.grouped_guided_fakequant_fwd(xt, offsets, gsc, gts, gbt, want_codes=True)),
                     ("gr", lambda: tr.grouped_rne_fakequant_fwd(xt, offsets, gsc, gts, want_codes=True)),
                     ("gf", lambda: tr.grouped_full_info_fakequant_fwd(xt, offsets, gsc, gts, gcd, want_codes=True))):
        y, m, q = fn()
        out.update({f"y_{name}": y, f"m_{name}": m, f"q_{name}": q})
    # forwards on records read back in place: x_train gets one row per entry
    # of perm (a waves-inside-rows width), and the same record read as rows
    # of 64 elements (waves spanning rows; the record is in flat order)
    rows, cols = xr.shape
    xg = torch.cat([xt, xt[:perm.numel() - rows]])
    n64 = xr.numel() // 64
    perm64 = torch.cat([torch.randperm(n64, generator=torch.Generator(device=xr.device).manual_seed(5),
                                       device=xr.device),
                        torch.tensor([-1, n64], dtype=torch.int64, device=xr.device)])
    x64 = torch.cat([xt.reshape(n64, 64), xt.reshape(n64, 64)[:2]])
    for name, fn in (("xg", lambda: tr.gathered_guided_fakequant_fwd(xg, perm, sc, ts, bt, want_codes=True)),
                     ("xf", lambda: tr.gathered_full_info_fakequant_fwd(xg, perm, sc, ts, cd, want_codes=True)),
                     ("xgg", lambda: tr.gathered_guided_fakequant_fwd(xg, perm, gsc, gts, gbt, offsets=offsets,
                                                                      want_codes=True)),
                     ("x64", lambda: tr.gathered_guided_fakequant_fwd(x64, perm64, sc, ts, bt, want_codes=True)),
                     ("x64f", lambda: tr.gathered_full_info_fakequant_fwd(x64, perm64, sc, ts, cd, want_codes=True)),
                     ("xr", lambda: tr.gathered_rne_fakequant_fwd(xg, perm, gsc, gts, offsets=offsets, want_codes=True)),
                     ("x64r", lambda: tr.gathered_rne_fakequant_fwd(x64, perm64, sc, ts, want_codes=True))):
        y, m, q = fn()
        out.update({f"y_{name}": y, f"m_{name}": m, f"q_{name}": q})
    msc, mbt, mcd = tr.mx_capture(xr, want_codes=True)
    out.update(msc=msc, mbt=mbt, mcd=mcd)
    for name, fn in (("mg", lambda: tr.mx_guided_fakequant_fwd(xt, msc, mbt, want_codes=True)),
                     ("mr", lambda: tr.mx_rne_fakequant_fwd(xt, msc, want_codes=True)),
                     ("mf", lambda: tr.mx_full_info_fakequant_fwd(xt, msc, mcd, want_codes=True))):
        y, m, q = fn()
        out.update({f"y_{name}": y, f"m_{name}": m, f"q_{name}": q})
    esc, ebt, ecd = tr.mx8_capture(xr, want_codes=True)
    out.update(esc=esc, ebt=ebt, ecd=ecd)
    for name, fn in (("eg", lambda: tr.mx8_guided_fakequant_fwd(xt, esc, ebt, want_codes=True)),
                     ("er", lambda: tr.mx8_rne_fakequant_fwd(xt, esc, want_codes=True)),
                     ("ef", lambda: tr.mx8_full_info_fakequant_fwd(xt, esc, ecd, want_codes=True))):
        y, m, q = fn()
        out.update({f"y_{name}": y, f"m_{name}": m, f"q_{name}": q})
    lsc, lpl, _ = tr.capture_lowbits(xr, ts, 3)
    y, m, q = tr.lowbits_fakequant_fwd(xt, lsc, ts, 3, lpl, want_codes=True)
    out.update(lsc=lsc, lpl=lpl, y_l=y, m_l=m, q_l=q)
    out["stats"] = tr.mismatch_stats(xt, sc, ts, bt, cd)
    # a batch of three sites (rows of the same tensor): in the small-grid build
    # the tensor scale pass splits three workgroups among them and the capture
    # falls back to one grid-stride launch per site
    sites = [xr[0:100], xr[100:], xr[5:6]]
    for i, (t, (bsc, bbt, bcd)) in enumerate(zip(tr.tensor_scale_batch(sites),
                                                 tr.capture_batch(sites, tr.tensor_scale_batch(sites),
                                                                  want_codes=True))):
        out.update({f"batch_ts{i}": t, f"batch_sc{i}": bsc, f"batch_bt{i}": bbt, f"batch_cd{i}": bcd})
    torch.cuda.synchronize()
    return {k: _host(v) for k, v in out.items()}


def test_grid_stride_paths_match_the_production_build(device):
    import fp4_rollout_guided_amd as tr
    _say("case grid-stride paths (small-grid build)")
    rows, cols = 257, 4096
    rng = np.random.default_rng(17)
    v = rng.standard_t(4, (rows, cols)) * 10.0 ** rng.uniform(-2, 2, (rows, 1))
    v[3, 5] = np.nan
    v[100, 7:9] = np.inf
    xr = F.f32_to_bf16_rne(v.reshape(-1).astype(np.float32))
    xt = F.f32_to_bf16_rne((F.bf16_to_f32(xr) * (1 + 0.2 * rng.standard_normal(xr.size))).astype(np.float32))
    g = F.f32_to_bf16_rne(rng.standard_normal(xr.size).astype(np.float32))
    shape = (rows, cols)
    xrd, xtd, gd = (from_np_u16(a, device, shape) for a in (xr, xt, g))
    offsets = torch.tensor(np.r_[0, np.sort(rng.integers(0, rows, 30)), rows], dtype=torch.int64, device=device)
    perm = torch.from_numpy(np.r_[rng.permutation(rows), [-1, rows]].astype(np.int64)).to(device)
    ref = _everything(tr, xrd, xtd, gd, offsets, perm)
    with _small_grid():
        assert tr.lib.trace_tensor_scale_workspace_bytes(rows * cols) == 12  # three amax partials
        got = _everything(tr, xrd, xtd, gd, offsets, perm)
    for k in ref:
        if ref[k] is None:
            continue
        assert np.array_equal(got[k], ref[k]), k
    cap = oracle.capture(xr, np.float32(ref["ts"].view(np.float32)[0]), with_codes=True)
    assert np.array_equal(got["scales"], cap["scales"]) and np.array_equal(got["bits"], cap["bits"])
    assert np.array_equal(got["codes"], cap["codes"])
