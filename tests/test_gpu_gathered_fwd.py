"""GPU parity of the training-side forwards on records read back in place
(trace_gathered_{guided,full_info,rne}_fakequant_fwd)
against ``oracle.gathered_fwd``: permuted, repeated and out-of-range row
indices, one tensor scale or per-expert groups of source rows (balanced,
unbalanced, empty, fewer than three), row widths whose waves each lie inside
one row and widths whose waves span rows, in place and without codes; then
every element of the routed-expert site of the MoE layer read back in a
seeded trainer order, and the fused call against the record gather followed
by the forward."""
import json
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import formats as F
from tests.full_compare import compare_gathered_every_element
from tests.gpu_util import assert_same, from_np_u16, to_np_u8, to_np_u16

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _offsets(kind, rows, rng):
    if kind is None:
        return None
    if kind == "balanced":
        g = 16
        return np.r_[0, np.sort(rng.integers(0, rows + 1, g - 1)), rows].astype(np.int64)
    if kind == "unbalanced":       # one large group among many small ones: the window misses, binary search
        cuts = np.r_[np.arange(1, 40), rows - 3, rows - 2]
        return np.r_[0, cuts, rows].astype(np.int64)
    if kind == "two":
        return np.array([0, rows // 3, rows], dtype=np.int64)
    if kind == "empty":            # empty first, middle and last groups
        return np.array([0, 0, rows // 4, rows // 4, rows // 4, rows // 2, rows, rows], dtype=np.int64)
    if kind == "one":
        return np.array([0, rows], dtype=np.int64)
    raise ValueError(kind)


def _index(rng, src_rows, dst_rows):
    idx = rng.integers(0, max(src_rows, 1), dst_rows).astype(np.int64)
    k = min(dst_rows, src_rows)
    idx[:k] = rng.permutation(src_rows)[:k]
    if dst_rows >= 6:
        idx[1] = -1
        idx[2] = src_rows
        idx[3] = np.iinfo(np.int64).max
        idx[4] = np.iinfo(np.int64).min
    if src_rows == 0:
        idx[:] = rng.integers(-3, 3, dst_rows)
    return idx


def _inputs(rng, src_rows, dst_rows, cols, idx):
    v = rng.standard_t(4, (max(src_rows, 1), cols)) * 10.0 ** rng.uniform(-3, 3, (max(src_rows, 1), 1))
    xr = F.f32_to_bf16_rne(v[:src_rows].reshape(-1).astype(np.float32))
    base = np.where((idx >= 0) & (idx < src_rows), np.clip(idx, 0, max(src_rows - 1, 0)), 0)
    t = v[base] * (1 + 0.03 * rng.standard_normal((dst_rows, cols)))
    t = t.reshape(-1)
    if t.size >= 64:               # special values in the trainer's input
        t[:8] = [np.nan, -np.nan, np.inf, -np.inf, 0.0, -0.0, 1e-40, -3e38]
        t[-3:] = [np.inf, np.nan, -0.0]
    xt = F.f32_to_bf16_rne(t.astype(np.float32))
    return xr, xt


@pytest.mark.parametrize("src_rows,dst_rows,cols,groups", [
    (1, 1, 16, None), (9, 40, 48, None), (300, 257, 4112, None), (64, 64, 7168, None), (0, 5, 32, None),
    (1000, 3, 2048, None), (200, 300, 768, "balanced"), (512, 512, 2048, "balanced"),
    (333, 400, 512, "unbalanced"), (50, 60, 96, "two"), (40, 50, 2048, "empty"), (1, 3, 16, "one"),
    (0, 7, 512, "one"),
])
def test_gathered_fwd_bit_exact(device, src_rows, dst_rows, cols, groups):
    _say("case gathered fwd", src_rows, dst_rows, cols, groups)
    import fp4_rollout_guided_amd as tr
    rng = np.random.default_rng(src_rows * 131 + dst_rows * 7 + cols + len(str(groups)))
    idx = _index(rng, src_rows, dst_rows)
    xr, xt = _inputs(rng, src_rows, dst_rows, cols, idx)
    off = _offsets(groups, src_rows, rng)
    if off is None:
        ts = np.float32(oracle.tensor_scale(xr))
        rec = oracle.capture(xr, ts, with_codes=True)
    else:
        ts = oracle.grouped_tensor_scale(xr, src_rows, cols, off)
        rec = oracle.grouped_capture(xr, src_rows, cols, off, ts, with_codes=True)
    rec = {k: v.copy() for k, v in rec.items()}
    if rec["scales"].size >= 8:    # zero-scale and large-scale blocks in the record
        rec["scales"][0] = 0x7F
        rec["scales"][1] = 0xFF
        rec["scales"][2] = 0x00
        rec["scales"][-1] = 0x7E
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    x_train = from_np_u16(xt, device, (dst_rows, cols))
    row_index = dev(idx)
    ts_d = dev(np.atleast_1d(np.asarray(ts, dtype=np.float32)))
    off_d = dev(off) if off is not None else None
    sc, bt, cd = dev(rec["scales"]), dev(rec["bits"]), dev(rec["codes"])
    got = {}
    y, m, q = tr.gathered_guided_fakequant_fwd(x_train, row_index, sc, ts_d, bt, offsets=off_d, want_codes=True)
    got.update(y_g=y, mask_g=m, q_g=q)
    y, m, q = tr.gathered_full_info_fakequant_fwd(x_train, row_index, sc, ts_d, cd, offsets=off_d, want_codes=True)
    got.update(y_f=y, mask_f=m, q_f=q)
    y, m, q = tr.gathered_rne_fakequant_fwd(x_train, row_index, sc, ts_d, offsets=off_d, want_codes=True)
    got.update(y_r=y, mask_r=m, q_r=q)
    # without codes, and in place (y is x_train)
    y_nc, m_nc, _ = tr.gathered_guided_fakequant_fwd(x_train, row_index, sc, ts_d, bt, offsets=off_d)
    inplace = x_train.clone()
    y_ip, m_ip, _ = tr.gathered_full_info_fakequant_fwd(inplace, row_index, sc, ts_d, cd, offsets=off_d, y=inplace)
    torch.cuda.synchronize()
    want = {}
    for mode, tag in (("guided", "g"), ("full", "f"), ("rne", "r")):
        r = oracle.gathered_fwd(mode, xt, cols, rec, src_rows, idx, ts, off)
        want.update({f"y_{tag}": r["y"], f"mask_{tag}": r["mask"], f"q_{tag}": r["codes"]})
    host = {k: (to_np_u16(v) if k.startswith("y") else to_np_u8(v)) for k, v in got.items()}
    assert_same(host, want, ctx=f"gathered {src_rows}->{dst_rows}x{cols} {groups}")
    assert np.array_equal(to_np_u16(y_nc), want["y_g"]) and np.array_equal(to_np_u8(m_nc), want["mask_g"])
    assert y_ip.data_ptr() == inplace.data_ptr()
    assert np.array_equal(to_np_u16(inplace), want["y_f"]) and np.array_equal(to_np_u8(m_ip), want["mask_f"])


def test_gathered_fwd_wide_index_rows_use_their_own_group(device):
    """Rows of one wave but of different destination rows (narrow rows)
    whose source rows fall in different groups: each lane keeps its row's
    group scale."""
    _say("case gathered fwd, narrow rows over many groups")
    import fp4_rollout_guided_amd as tr
    rng = np.random.default_rng(99)
    src_rows, dst_rows, cols = 4096, 5000, 32
    idx = rng.integers(0, src_rows, dst_rows).astype(np.int64)
    xr, xt = _inputs(rng, src_rows, dst_rows, cols, idx)
    off = np.r_[0, np.sort(rng.integers(0, src_rows, 200)), src_rows].astype(np.int64)
    ts = oracle.grouped_tensor_scale(xr, src_rows, cols, off)
    assert len(np.unique(ts)) > 100
    rec = oracle.grouped_capture(xr, src_rows, cols, off, ts, with_codes=True)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    y, m, q = tr.gathered_guided_fakequant_fwd(from_np_u16(xt, device, (dst_rows, cols)), dev(idx),
                                               dev(rec["scales"]), dev(ts), dev(rec["bits"]), offsets=dev(off),
                                               want_codes=True)
    torch.cuda.synchronize()
    want = oracle.gathered_fwd("guided", xt, cols, rec, src_rows, idx, ts, off)
    assert_same({"y": to_np_u16(y), "mask": to_np_u8(m), "codes": to_np_u8(q)}, want, ctx="narrow rows")


def test_moe_expert_site_read_back_in_trainer_order(device):
    """The routed-expert site of the MoE layer workload (131072 x 2048, 128
    experts, per-expert tensor scales) captured in routing order and read
    back by the trainer in a seeded random row order: every element of the
    fused forwards against the oracle; with one tensor scale, the fused
    call equals the record gather followed by the forward."""
    import fp4_rollout_guided_amd as tr
    with open(os.path.join(HERE, "golden", "moe_layer_sigma.json")) as fh:
        sigma = json.load(fh)["sigma"]
    _say("case MoE layer expert site read back in trainer order")
    d = workloads.moe_layer(device, sigma, sites=["expert_in"])["expert_in"]
    _, experts = workloads.moe_routing(device)
    offsets = workloads.moe_expert_offsets(experts)
    x_roll, x_train_src = d["x_roll"], d["x_train"]
    rows, cols = x_roll.shape
    perm = workloads.trainer_order(rows, device)
    x_train = x_train_src[perm]
    gts = tr.grouped_tensor_scale(x_roll, offsets)
    sc, bt, cd = tr.grouped_capture(x_roll, offsets, gts, want_codes=True)
    got = {}
    y, m, q = tr.gathered_guided_fakequant_fwd(x_train, perm, sc, gts, bt, offsets=offsets, want_codes=True)
    got.update(y_g=y, mask_g=m, q_g=q)
    y, m, q = tr.gathered_full_info_fakequant_fwd(x_train, perm, sc, gts, cd, offsets=offsets, want_codes=True)
    got.update(y_f=y, mask_f=m, q_f=q)
    y, m, q = tr.gathered_rne_fakequant_fwd(x_train, perm, sc, gts, offsets=offsets, want_codes=True)
    got.update(y_r=y, mask_r=m, q_r=q)
    # one tensor scale: fused == gather + forward (both paths on the GPU)
    ts1 = tr.tensor_scale(x_roll)
    sc1, bt1, cd1 = tr.capture(x_roll, ts1, want_codes=True)
    yf, mf, qf = tr.gathered_guided_fakequant_fwd(x_train, perm, sc1, ts1, bt1, want_codes=True)
    b2, s2, c2 = tr.gather_records(bt1, sc1, cd1, cols, perm)
    y2, m2, q2 = tr.guided_fakequant_fwd(x_train, s2, ts1, b2, want_codes=True)
    yff, mff, qff = tr.gathered_full_info_fakequant_fwd(x_train, perm, sc1, ts1, cd1, want_codes=True)
    y3, m3, q3 = tr.full_info_fakequant_fwd(x_train, s2, ts1, c2, want_codes=True)
    torch.cuda.synchronize()
    for a, b, name in ((yf, y2, "y"), (mf, m2, "mask"), (qf, q2, "codes"), (yff, y3, "y full"),
                       (mff, m3, "mask full"), (qff, q3, "codes full")):
        assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                           b.view(torch.uint8) if b.dtype != torch.uint8 else b), name
    off = offsets.cpu().numpy()
    xr_h = to_np_u16(x_roll)
    ts = oracle.grouped_tensor_scale(xr_h, rows, cols, off)
    assert np.array_equal(gts.cpu().numpy().view(np.uint32), ts.view(np.uint32))
    host = {k: (to_np_u16(v) if k.startswith("y") else to_np_u8(v)) for k, v in got.items()}
    n = compare_gathered_every_element("expert site, trainer order", xr_h, rows, to_np_u16(x_train),
                                       perm.cpu().numpy(), cols, off, ts, host)
    _say(f"  expert site read back: {n} elements of the three forwards equal to the oracle")


# Row widths around the kernel's row modes (half blocks per row = cols / 8):
# 512 (64, one row per segment, every segment a new row), 528 (66: segments
# span two rows), 768 (96), 1008 (126), 1024 (128), 1536 (192), 2560 (320),
# 496 (62: per lane), with row counts that leave a partial last segment.
@pytest.mark.parametrize("cols", [496, 512, 528, 768, 1008, 1024, 1536, 2560])
@pytest.mark.parametrize("grouped", [False, True])
def test_gathered_fwd_row_mode_edges(device, cols, grouped):
    _say("case gathered fwd row-mode edges", cols, grouped)
    import fp4_rollout_guided_amd as tr
    rng = np.random.default_rng(cols * 2 + grouped)
    for src_rows, dst_rows in ((37, 53), (130, 7), (3, 129)):
        idx = _index(rng, src_rows, dst_rows)
        xr, xt = _inputs(rng, src_rows, dst_rows, cols, idx)
        off = np.r_[0, np.sort(rng.integers(0, src_rows + 1, 5)), src_rows].astype(np.int64) if grouped else None
        if off is None:
            ts = np.float32(oracle.tensor_scale(xr))
            rec = oracle.capture(xr, ts, with_codes=True)
        else:
            ts = oracle.grouped_tensor_scale(xr, src_rows, cols, off)
            rec = oracle.grouped_capture(xr, src_rows, cols, off, ts, with_codes=True)
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
        x_train = from_np_u16(xt, device, (dst_rows, cols))
        args = (dev(idx), dev(rec["scales"]), dev(np.atleast_1d(np.asarray(ts, dtype=np.float32))))
        kw = {"offsets": dev(off)} if grouped else {}
        y, m, q = tr.gathered_guided_fakequant_fwd(x_train, *args, dev(rec["bits"]), want_codes=True, **kw)
        yf, mf, qf = tr.gathered_full_info_fakequant_fwd(x_train, *args, dev(rec["codes"]), want_codes=True, **kw)
        yr, mr, qr = tr.gathered_rne_fakequant_fwd(x_train, *args, want_codes=True, **kw)
        torch.cuda.synchronize()
        g = oracle.gathered_fwd("guided", xt, cols, rec, src_rows, idx, ts, off)
        f = oracle.gathered_fwd("full", xt, cols, rec, src_rows, idx, ts, off)
        r = oracle.gathered_fwd("rne", xt, cols, rec, src_rows, idx, ts, off)
        ctx = f"cols {cols} grouped {grouped} {src_rows}->{dst_rows}"
        assert_same({"y": to_np_u16(y), "mask": to_np_u8(m), "codes": to_np_u8(q)}, g, ctx=ctx + " guided")
        assert_same({"y": to_np_u16(yf), "mask": to_np_u8(mf), "codes": to_np_u8(qf)}, f, ctx=ctx + " full")
        assert_same({"y": to_np_u16(yr), "mask": to_np_u8(mr), "codes": to_np_u8(qr)}, r, ctx=ctx + " rne")
