"""Pins of ``oracle.gathered_fwd``, the training side's forward on records
read back in its own row order (the trainer reads the rollout's records
back), against independent paths through already pinned functions:

* a per-row loop: each destination row through ``guided_fwd`` /
  ``full_info_fwd`` / ``rne_fwd`` with that row's record bytes taken by hand from the
  source row and its group's scalar tensor scale;
* the identity order: equal to the ungrouped and per-expert forwards;
* rows whose index is out of range: the zero-scale rule written out
  (y = a zero with the input's sign, NaN -> +0, mask 0)."""
import numpy as np
import pytest

import oracle
from oracle import formats as F


def _rollout(rng, rows, cols, off=None):
    v = rng.standard_t(4, (rows, cols))
    if off is not None:
        for g, (a, b) in enumerate(zip(off, off[1:])):
            v[a:b] *= 10.0 ** (g - 2)
    xr = F.f32_to_bf16_rne(v.astype(np.float32).reshape(-1))
    return xr


def _train(rng, xr):
    return F.f32_to_bf16_rne((F.bf16_to_f32(xr) * (1 + 0.05 * rng.standard_normal(xr.size))).astype(np.float32))


def _record(xr, rows, cols, off):
    if off is None:
        ts = np.array([oracle.tensor_scale(xr)], dtype=np.float32)
        cap = oracle.capture(xr, ts[0], with_codes=True)
    else:
        ts = oracle.grouped_tensor_scale(xr, rows, cols, off)
        cap = oracle.grouped_capture(xr, rows, cols, off, ts, with_codes=True)
    return cap, ts


@pytest.mark.parametrize("grouped", [False, True])
@pytest.mark.parametrize("mode", ["guided", "full", "rne"])
def test_gathered_against_a_per_row_loop(grouped, mode):
    rng = np.random.default_rng(11 + grouped + 2 * ["guided", "full", "rne"].index(mode))
    src_rows, cols, dst_rows = 40, 96, 57
    off = np.array([0, 7, 7, 20, 33, 40], dtype=np.int64) if grouped else None
    xr = _rollout(rng, src_rows, cols, off)
    cap, ts = _record(xr, src_rows, cols, off)
    idx = rng.integers(0, src_rows, dst_rows).astype(np.int64)
    idx[[3, 9, 20]] = [-1, src_rows, 1 << 40]
    xt = _train(rng, F.f32_to_bf16_rne(rng.standard_t(4, dst_rows * cols).astype(np.float32)))
    xt[9 * cols + 5] = 0x7FC0          # a NaN in an out-of-range row
    got = oracle.gathered_fwd(mode, xt, cols, cap, src_rows, idx, ts, off)
    sb, bb, cb = cols // 16, cols // 8, cols // 2
    for r in range(dst_rows):
        s = int(idx[r])
        x = xt[r * cols:(r + 1) * cols]
        if 0 <= s < src_rows:
            g = 0 if off is None else int(np.flatnonzero((off[:-1] <= s) & (s < off[1:]))[0])
            t = ts[g]
            scales, bits, codes = cap["scales"][s * sb:(s + 1) * sb], cap["bits"][s * bb:(s + 1) * bb], \
                cap["codes"][s * cb:(s + 1) * cb]
        else:
            t = ts[0]
            scales, bits, codes = (np.zeros(k, np.uint8) for k in (sb, bb, cb))
        want = (oracle.guided_fwd(x, scales, t, bits) if mode == "guided" else
                oracle.full_info_fwd(x, scales, t, codes) if mode == "full" else oracle.rne_fwd(x, scales, t))
        assert np.array_equal(got["y"][r * cols:(r + 1) * cols], want["y"]), r
        assert np.array_equal(got["mask"][r * bb:(r + 1) * bb], want["mask"]), r
        assert np.array_equal(got["codes"][r * cb:(r + 1) * cb], want["codes"]), r


def test_gathered_identity_order_equals_the_forwards():
    rng = np.random.default_rng(12)
    rows, cols = 48, 64
    off = np.array([0, 5, 30, 30, 48], dtype=np.int64)
    idx = np.arange(rows, dtype=np.int64)
    xr = _rollout(rng, rows, cols, off)
    xt = _train(rng, xr)
    cap, ts = _record(xr, rows, cols, None)
    for k in ("y", "mask", "codes"):
        assert np.array_equal(oracle.gathered_fwd("guided", xt, cols, cap, rows, idx, ts)[k],
                              oracle.guided_fwd(xt, cap["scales"], ts[0], cap["bits"])[k])
        assert np.array_equal(oracle.gathered_fwd("full", xt, cols, cap, rows, idx, ts)[k],
                              oracle.full_info_fwd(xt, cap["scales"], ts[0], cap["codes"])[k])
        assert np.array_equal(oracle.gathered_fwd("rne", xt, cols, cap, rows, idx, ts)[k],
                              oracle.rne_fwd(xt, cap["scales"], ts[0])[k])
    capg, tsg = _record(xr, rows, cols, off)
    for k in ("y", "mask", "codes"):
        assert np.array_equal(oracle.gathered_fwd("guided", xt, cols, capg, rows, idx, tsg, off)[k],
                              oracle.grouped_guided_fwd(xt, rows, cols, off, capg["scales"], tsg, capg["bits"])[k])
        assert np.array_equal(oracle.gathered_fwd("full", xt, cols, capg, rows, idx, tsg, off)[k],
                              oracle.grouped_full_info_fwd(xt, rows, cols, off, capg["scales"], tsg, capg["codes"])[k])
        assert np.array_equal(oracle.gathered_fwd("rne", xt, cols, capg, rows, idx, tsg, off)[k],
                              oracle.grouped_rne_fwd(xt, rows, cols, off, capg["scales"], tsg)[k])


def test_gathered_out_of_range_rows_are_zero_scale():
    rng = np.random.default_rng(13)
    src_rows, cols = 8, 32
    xr = _rollout(rng, src_rows, cols)
    cap, ts = _record(xr, src_rows, cols, None)
    vals = np.array([1.5, -2.0, 0.0, -0.0, np.nan, np.inf, -np.inf, 3e38] * 4, dtype=np.float32)
    xt = F.f32_to_bf16_rne(np.tile(vals, 2))
    out = oracle.gathered_fwd("guided", xt, cols, cap, src_rows, np.array([-5, src_rows], np.int64), ts)
    sign = (xt >> 15).astype(np.uint16)
    nan = np.isnan(F.bf16_to_f32(xt))
    assert np.array_equal(out["y"], np.where(nan, 0, sign << 15).astype(np.uint16))
    assert not out["mask"].any()
    codes = oracle.unpack_nibbles(out["codes"], xt.size)
    assert np.array_equal(codes, np.where(nan, 0, sign << 3).astype(np.uint8))


def test_gathered_rejects_a_bad_mode_and_bad_offsets():
    rng = np.random.default_rng(14)
    xr = _rollout(rng, 4, 16)
    cap, ts = _record(xr, 4, 16, None)
    with pytest.raises(ValueError):
        oracle.gathered_fwd("nearest", xr, 16, cap, 4, np.arange(4), ts)
    with pytest.raises(ValueError):
        oracle.gathered_fwd("guided", xr, 16, cap, 4, np.arange(4), ts, np.array([0, 3, 2, 4]))
