"""The boundary of the non-temporal streams: a tensor of exactly 256 MiB (the
size of MI355X's last-level cache) runs the plain instantiations, one more
row the hinted ones (loads of x and stores of every output with the
non-temporal hint, record stores in the capture).  On both sides, every
element of every output against the oracle, bit for bit:

* the whole path (tensor scale, capture with codes, the guided, RNE and
  full-information forwards, the STE backward);
* the per-expert path (128 seeded row groups: tensor scales, capture, the
  three forwards);
* the forwards on records read back in a shuffled row order with two
  out-of-range indices, with one tensor scale and with per-expert scales."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.full_compare import (Shared, compare_every_element, compare_gathered_every_element,
                                compare_grouped_every_element, tensor_scale_of)
from tests.gpu_util import to_np_u16

pytestmark = pytest.mark.gpu
COLS = 2048
LLC_BYTES = 256 << 20


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _inputs(device, rows):
    g = workloads.generator(device, "stream threshold", rows, "x")
    x = workloads.normal((rows, COLS), g, device)
    workloads.scale_channels(x, workloads.outlier_channels(COLS, 2, g, device), 100.0)
    x_roll = workloads.bf16(x)
    del x
    x_train = workloads.relative_noise(x_roll, 0.02, workloads.generator(device, "stream threshold", rows, "noise"))
    grad = workloads.grad_for((rows, COLS), device, "stream threshold", rows)
    return x_roll, x_train, grad


@pytest.mark.parametrize("rows", [LLC_BYTES // (2 * COLS), LLC_BYTES // (2 * COLS) + 1], ids=["at", "past"])
def test_both_sides_of_the_stream_threshold(device, rows):
    import fp4_rollout_guided_amd as tr
    nbytes = rows * COLS * 2
    _say(f"case stream threshold: {rows}x{COLS} bf16, {nbytes} bytes "
         f"({'hinted' if nbytes > LLC_BYTES else 'plain'} instantiations)")
    x_roll, x_train, grad = _inputs(device, rows)

    # the whole path
    ts = tr.tensor_scale(x_roll)
    sc, bt, cd = tr.capture(x_roll, ts, want_codes=True)
    got = {"scales": sc, "bits": bt, "codes": cd}
    got["y_g"], got["mask_g"], got["q_g"] = tr.guided_fakequant_fwd(x_train, sc, ts, bt, want_codes=True)
    got["y_r"], got["mask_r"], got["q_r"] = tr.rne_fakequant_fwd(x_train, sc, ts, want_codes=True)
    got["y_f"], got["mask_f"], got["q_f"] = tr.full_info_fakequant_fwd(x_train, sc, ts, cd, want_codes=True)
    got["gin"] = tr.ste_bwd(grad, got["mask_g"])
    torch.cuda.synchronize()
    with Shared({"xr": x_roll, "xt": x_train, "g": grad}) as sh:
        ts_o = tensor_scale_of(sh)
        assert ts.cpu().numpy().view(np.uint32)[0] == np.float32(ts_o).view(np.uint32)
        compare_every_element(f"{rows} rows, whole path", sh, got, ts_o)
    del got

    # the per-expert path
    rng = np.random.default_rng(rows)
    off = np.r_[0, np.sort(rng.integers(0, rows + 1, 127)), rows].astype(np.int64)
    offsets = torch.from_numpy(off).to(device)
    gts = tr.grouped_tensor_scale(x_roll, offsets)
    gsc, gbt, gcd = tr.grouped_capture(x_roll, offsets, gts, want_codes=True)
    got = {"scales": gsc, "bits": gbt, "codes": gcd}
    got["y_g"], got["mask_g"], got["q_g"] = tr.grouped_guided_fakequant_fwd(x_train, offsets, gsc, gts, gbt,
                                                                           want_codes=True)
    got["y_r"], got["mask_r"], got["q_r"] = tr.grouped_rne_fakequant_fwd(x_train, offsets, gsc, gts, want_codes=True)
    got["y_f"], got["mask_f"], got["q_f"] = tr.grouped_full_info_fakequant_fwd(x_train, offsets, gsc, gts, gcd,
                                                                              want_codes=True)
    torch.cuda.synchronize()
    xr_h, xt_h = to_np_u16(x_roll), to_np_u16(x_train)
    gts_o = oracle.grouped_tensor_scale(xr_h, rows, COLS, off)
    assert np.array_equal(gts.cpu().numpy().view(np.uint32), gts_o.view(np.uint32))
    compare_grouped_every_element(f"{rows} rows, per-expert path", xr_h, xt_h, rows, COLS, off, gts_o, got)
    del got

    # the forwards on records read back in a shuffled row order
    perm = workloads.trainer_order(rows, device).clone()
    perm[5], perm[rows // 2] = -1, rows  # rows the rollout never produced: zero-scale blocks
    for label, rec, scales_ts, offs, ts_ref in (("one tensor scale", (sc, bt, cd), ts, None, ts_o),
                                                ("per-expert scales", (gsc, gbt, gcd), gts, offsets, gts_o)):
        r_sc, r_bt, r_cd = rec
        got = {}
        got["y_g"], got["mask_g"], got["q_g"] = tr.gathered_guided_fakequant_fwd(
            x_train, perm, r_sc, scales_ts, r_bt, offsets=offs, want_codes=True)
        got["y_f"], got["mask_f"], got["q_f"] = tr.gathered_full_info_fakequant_fwd(
            x_train, perm, r_sc, scales_ts, r_cd, offsets=offs, want_codes=True)
        got["y_r"], got["mask_r"], got["q_r"] = tr.gathered_rne_fakequant_fwd(
            x_train, perm, r_sc, scales_ts, offsets=offs, want_codes=True)
        torch.cuda.synchronize()
        n = compare_gathered_every_element(f"{rows} rows, read back, {label}", xr_h, rows, xt_h,
                                           perm.cpu().numpy(), COLS, None if offs is None else off, ts_ref, got)
        _say(f"  {rows} rows, read back with {label}: {n} elements equal to the oracle")
        del got
