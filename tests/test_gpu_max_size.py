"""A site tensor past 2^32 elements: (2^21 + 37) x 2048 = 4,295,043,072
elements, 8 GiB per bf16 tensor, so element indices pass 2^32 and byte
offsets 2^33 in every kernel.  Every element of every NVFP4 output is
checked against the whole-tensor properties of ``tests/full_props.py``; the
tensor scale against torch's amax of the whole tensor; sampled rows --
around the 2^31-byte and 2^32-element boundaries, the ragged end and random
rows -- against the oracle, for the NVFP4 path, per-expert scales (64 row
groups), the forward on records read back in a shuffled row order (source
rows around the same boundaries, and out of range) and the MXFP4 and MXFP8
variants.  Inputs are generated on the
device: N(0, 1) with 2 outlier channels x100 and x_train = x_roll plus 2%
relative noise, as in the deeper-half sweep."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.full_props import check_nvfp4_outputs
from tests.gpu_util import assert_same, oracle_path, to_np_u8, to_np_u16

pytestmark = pytest.mark.gpu

ROWS, COLS = (1 << 21) + 37, 2048
CHUNK_ROWS = 1 << 18


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def big(device):
    free, _ = torch.cuda.mem_get_info(device)
    if free < (100 << 30):
        pytest.skip("needs 100 GiB of free device memory")
    _say(f"case max size: generating {ROWS}x{COLS} ({ROWS * COLS} elements)")
    x_roll = torch.empty(ROWS, COLS, dtype=torch.bfloat16, device=device)
    x_train = torch.empty_like(x_roll)
    grad = torch.empty_like(x_roll)
    gx = workloads.generator(device, "max", "x")
    chans = workloads.outlier_channels(COLS, 2, gx, device)
    for r0 in range(0, ROWS, CHUNK_ROWS):
        r1 = min(ROWS, r0 + CHUNK_ROWS)
        x = workloads.normal((r1 - r0, COLS), gx, device)
        workloads.scale_channels(x, chans, 100.0)
        x_roll[r0:r1] = workloads.bf16(x)
        del x
        x_train[r0:r1] = workloads.relative_noise(x_roll[r0:r1], 0.02, workloads.generator(device, "max", "n", r0))
        grad[r0:r1] = workloads.bf16(workloads.normal((r1 - r0, COLS), workloads.generator(device, "max", "g", r0),
                                                      device))
    torch.cuda.synchronize()
    rng = np.random.default_rng(2024)
    b31 = (1 << 31) // (2 * COLS)        # first row past 2^31 bytes of bf16
    b32 = (1 << 32) // COLS              # first row past 2^32 elements
    rows = {0, 1, b31 - 1, b31, b32 - 1, b32, b32 + 1, ROWS - 2, ROWS - 1}
    rows.update(rng.choice(ROWS, 24, replace=False).tolist())
    idx = np.array(sorted(rows))
    yield {"x_roll": x_roll, "x_train": x_train, "grad": grad, "idx": idx}
    del x_roll, x_train, grad
    torch.cuda.empty_cache()


def _rows_of(t, idx, per_row, u16=False):
    v = t.reshape(-1, per_row)[torch.from_numpy(idx).to(t.device)]
    return to_np_u16(v.view(torch.int16)) if u16 else to_np_u8(v)


def test_max_size_nvfp4_path(device, big):
    import fp4_rollout_guided_amd as tr
    x_roll, x_train, grad, idx = big["x_roll"], big["x_train"], big["grad"], big["idx"]
    _say("case max size: NVFP4 path")
    ts = tr.tensor_scale(x_roll)
    amax = np.float32(x_roll.abs().max().float().item())
    assert ts.cpu().numpy().view(np.uint32)[0] == (amax / np.float32(2688)).view(np.uint32)
    scales, bits, codes = tr.capture(x_roll, ts, want_codes=True)
    out = {"scales": scales, "bits": bits, "codes": codes}
    for k, fn in (("g", lambda: tr.guided_fakequant_fwd(x_train, scales, ts, bits, want_codes=True)),
                  ("r", lambda: tr.rne_fakequant_fwd(x_train, scales, ts, want_codes=True)),
                  ("f", lambda: tr.full_info_fakequant_fwd(x_train, scales, ts, codes, want_codes=True))):
        out[f"y_{k}"], out[f"mask_{k}"], out[f"q_{k}"] = fn()
    out["gin"] = tr.ste_bwd(grad, out["mask_g"])
    torch.cuda.synchronize()
    check_nvfp4_outputs("max size", x_roll, x_train, grad, ts, out)
    want = oracle_path(_rows_of(x_roll, idx, COLS, True), _rows_of(x_train, idx, COLS, True),
                       _rows_of(grad, idx, COLS, True), ts=ts.item())
    per = {"scales": COLS // 16, "bits": COLS // 8, "codes": COLS // 2, "mask_g": COLS // 8, "q_g": COLS // 2,
           "mask_r": COLS // 8, "q_r": COLS // 2, "mask_f": COLS // 8, "q_f": COLS // 2}
    got = {k: _rows_of(out[k], idx, n) for k, n in per.items()}
    for k in ("y_g", "y_r", "y_f", "gin"):
        got[k] = _rows_of(out[k], idx, COLS, True)
    assert_same(got, want, keys=list(per) + ["y_g", "y_r", "y_f", "gin"], ctx="max size")


def test_max_size_grouped(device, big):
    import fp4_rollout_guided_amd as tr
    x_roll, x_train, idx = big["x_roll"], big["x_train"], big["idx"]
    _say("case max size: 64 row groups")
    rng = np.random.default_rng(77)
    off_np = np.r_[0, np.sort(rng.choice(np.arange(1, ROWS), 63, replace=False)), ROWS].astype(np.int64)
    offsets = torch.from_numpy(off_np).to(device)
    gts = tr.grouped_tensor_scale(x_roll, offsets)
    scales, bits, _ = tr.grouped_capture(x_roll, offsets, gts)
    y, mask, q = tr.grouped_guided_fakequant_fwd(x_train, offsets, scales, gts, bits, want_codes=True)
    torch.cuda.synchronize()
    gts_np = gts.cpu().numpy()
    for g in range(64):
        amax = np.float32(x_roll[off_np[g]:off_np[g + 1]].abs().max().float().item())
        assert gts_np[g].view(np.uint32) == (amax / np.float32(2688)).view(np.uint32), g
    group_of = np.searchsorted(off_np, idx, side="right") - 1
    xr, xt = _rows_of(x_roll, idx, COLS, True), _rows_of(x_train, idx, COLS, True)
    for j, r in enumerate(idx):
        ts = gts_np[group_of[j]]
        row = slice(j * COLS, (j + 1) * COLS)
        cap = oracle.capture(xr[row], ts)
        gd = oracle.guided_fwd(xt[row], cap["scales"], ts, cap["bits"])
        got = {"scales": _rows_of(scales, idx[j:j + 1], COLS // 16), "bits": _rows_of(bits, idx[j:j + 1], COLS // 8),
               "y": _rows_of(y, idx[j:j + 1], COLS, True), "mask": _rows_of(mask, idx[j:j + 1], COLS // 8),
               "codes": _rows_of(q, idx[j:j + 1], COLS // 2)}
        assert_same(got, {"scales": cap["scales"], "bits": cap["bits"], "y": gd["y"], "mask": gd["mask"],
                          "codes": gd["codes"]}, ctx=f"max size grouped row {r}")


def test_max_size_gathered(device, big):
    """The guided forward on records read back in place: destination row r
    reads source row perm[r] (a seeded permutation), with the sampled
    destination rows pointed at source rows around the 2^31-byte and
    2^32-element boundaries, the ragged end and two out-of-range indices."""
    import fp4_rollout_guided_amd as tr
    x_roll, x_train, idx = big["x_roll"], big["x_train"], big["idx"]
    _say("case max size: forward on records read back in a shuffled row order")
    ts = tr.tensor_scale(x_roll)
    scales, bits, _ = tr.capture(x_roll, ts)
    b31, b32 = (1 << 31) // (2 * COLS), (1 << 32) // COLS
    perm = workloads.trainer_order(ROWS, device).clone()
    for r, src in zip(idx[::2], (b31 - 1, b31, b32 - 1, b32, b32 + 1, ROWS - 1, -1, ROWS)):
        perm[int(r)] = src
    y, mask, q = tr.gathered_guided_fakequant_fwd(x_train, perm, scales, ts, bits, want_codes=True)
    torch.cuda.synchronize()
    src = perm.cpu().numpy()[idx]
    live = sorted({int(v) for v in src if 0 <= v < ROWS})
    pos = {v: i for i, v in enumerate(live)}
    ts_v = np.float32(ts.item())
    rec = oracle.capture(_rows_of(x_roll, np.array(live), COLS, True), ts_v)   # the record of the rows read
    row_index = np.array([pos.get(int(v), -1) for v in src], dtype=np.int64)
    want = oracle.gathered_fwd("guided", _rows_of(x_train, idx, COLS, True), COLS, rec, len(live), row_index, ts_v)
    got = {"y": _rows_of(y, idx, COLS, True), "mask": _rows_of(mask, idx, COLS // 8), "codes": _rows_of(q, idx, COLS // 2)}
    assert_same(got, {"y": want["y"], "mask": want["mask"], "codes": want["codes"]}, ctx="max size read back")


def test_max_size_mx_variants(device, big):
    import fp4_rollout_guided_amd as tr
    x_roll, x_train, idx = big["x_roll"], big["x_train"], big["idx"]
    xr, xt = _rows_of(x_roll, idx, COLS, True), _rows_of(x_train, idx, COLS, True)
    _say("case max size: MXFP4")
    sc, bt, _ = tr.mx_capture(x_roll)
    y, m, q = tr.mx_guided_fakequant_fwd(x_train, sc, bt, want_codes=True)
    torch.cuda.synchronize()
    cap = oracle.mx_capture(xr)
    gd = oracle.mx_guided_fwd(xt, cap["scales"], cap["bits"])
    got = {"scales": _rows_of(sc, idx, COLS // 32), "bits": _rows_of(bt, idx, COLS // 8),
           "y": _rows_of(y, idx, COLS, True), "mask": _rows_of(m, idx, COLS // 8), "codes": _rows_of(q, idx, COLS // 2)}
    assert_same(got, {"scales": cap["scales"], "bits": cap["bits"], "y": gd["y"], "mask": gd["mask"],
                      "codes": gd["codes"]}, ctx="max size MXFP4")
    del sc, bt, y, m, q
    _say("case max size: MXFP8")
    sc, bt, _ = tr.mx8_capture(x_roll)
    y, m, q = tr.mx8_guided_fakequant_fwd(x_train, sc, bt, want_codes=True)
    torch.cuda.synchronize()
    cap = oracle.mx8_capture(xr)
    gd = oracle.mx8_guided_fwd(xt, cap["scales"], cap["bits"])
    got = {"scales": _rows_of(sc, idx, COLS // 32), "bits": _rows_of(bt, idx, COLS // 8),
           "y": _rows_of(y, idx, COLS, True), "mask": _rows_of(m, idx, COLS // 8), "codes": _rows_of(q, idx, COLS)}
    assert_same(got, {"scales": cap["scales"], "bits": cap["bits"], "y": gd["y"], "mask": gd["mask"],
                      "codes": gd["codes"]}, ctx="max size MXFP8")
