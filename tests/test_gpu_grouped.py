"""GPU parity of the per-expert (row-group) entry points: grouped tensor
scale, capture and the three forwards through the C ABI against the
oracle's grouped functions, bit for bit.  Groups are laid out so that group
starts fall inside waves (3 blocks per row), groups are empty or one row
long, every row is its own group, and group magnitudes differ by orders of
magnitude (a wrong group's tensor scale changes the scale bytes)."""
import json
import os
import sys
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import formats as F
from tests.full_compare import compare_grouped_every_element
from tests.full_props import check_nvfp4_outputs
from tests.gpu_util import from_np_u16, to_np_u8, to_np_u16

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _partition(rng, rows, groups, empties=0):
    cuts = np.sort(rng.integers(0, rows + 1, groups - 1))
    off = np.r_[0, cuts, rows].astype(np.int64)
    for _ in range(empties):  # force some empty groups
        g = rng.integers(1, groups)
        off[g] = off[g - 1]
    return np.maximum.accumulate(off)


CASES = [
    ("tiny", 7, 32, lambda rng: np.array([0, 2, 2, 5, 7])),
    ("one", 1, 16, lambda rng: np.array([0, 1])),
    ("mid-wave", 300, 48, lambda rng: _partition(rng, 300, 40, empties=5)),
    ("row-each", 64, 16, lambda rng: np.arange(65)),
    ("leading-empty", 129, 4112, lambda rng: np.array([0, 0, 0, 64, 64, 129, 129])),
    ("single", 1024, 2048, lambda rng: np.array([0, 1024])),
    ("many", 2000, 96, lambda rng: _partition(rng, 2000, 128, empties=10)),
    # equal groups: the lookup's first guess lands in the group or next to it
    ("balanced-3", 300, 32, lambda rng: np.array([0, 100, 200, 300])),
    ("balanced-16", 1024, 64, lambda rng: np.arange(0, 1025, 64)),
    ("near-balanced", 4096, 32, lambda rng: np.r_[0, np.arange(1, 64) * 64 + rng.integers(-25, 25, 63), 4096]),
    ("balanced-empties", 960, 48, lambda rng: np.array([0, 0, 240, 240, 480, 720, 720, 960, 960])),
    # more groups than blocks: the fixed-point ratio clamps, the binary search finds the group
    ("more-groups-than-blocks", 3, 16, lambda rng: np.array([0, 0, 0, 1, 1, 1, 2, 2, 3, 3, 3])),
]


def _grouped_values(rng, rows, cols, off):
    v = rng.standard_t(4, (rows, cols))
    mags = 10.0 ** rng.uniform(-3, 3, len(off) - 1)
    for g, (a, b) in enumerate(zip(off, off[1:])):
        v[a:b] *= mags[g]
    return F.f32_to_bf16_rne(v.astype(np.float32).reshape(-1))


def _gpu_grouped(x_roll, x_train, offsets):
    import fp4_rollout_guided_amd as tr
    ts = tr.grouped_tensor_scale(x_roll, offsets)
    sc, bt, cd = tr.grouped_capture(x_roll, offsets, ts, want_codes=True)
    yg, mg, qg = tr.grouped_guided_fakequant_fwd(x_train, offsets, sc, ts, bt, want_codes=True)
    yr, mr, qr = tr.grouped_rne_fakequant_fwd(x_train, offsets, sc, ts, want_codes=True)
    yf, mf, qf = tr.grouped_full_info_fakequant_fwd(x_train, offsets, sc, ts, cd, want_codes=True)
    torch.cuda.synchronize()
    return {"ts": ts, "scales": sc, "bits": bt, "codes": cd, "y_g": yg, "mask_g": mg, "q_g": qg,
            "y_r": yr, "mask_r": mr, "q_r": qr, "y_f": yf, "mask_f": mf, "q_f": qf}


def _oracle_grouped(xr, xt, rows, cols, off, ts):
    cap = oracle.grouped_capture(xr, rows, cols, off, ts, with_codes=True)
    gd = oracle.grouped_guided_fwd(xt, rows, cols, off, cap["scales"], ts, cap["bits"])
    rn = oracle.grouped_rne_fwd(xt, rows, cols, off, cap["scales"], ts)
    fi = oracle.grouped_full_info_fwd(xt, rows, cols, off, cap["scales"], ts, cap["codes"])
    return {"scales": cap["scales"], "bits": cap["bits"], "codes": cap["codes"],
            "y_g": gd["y"], "mask_g": gd["mask"], "q_g": gd["codes"],
            "y_r": rn["y"], "mask_r": rn["mask"], "q_r": rn["codes"],
            "y_f": fi["y"], "mask_f": fi["mask"], "q_f": fi["codes"]}


def _host(got):
    out = {}
    for k, v in got.items():
        if k == "ts":
            continue
        out[k] = to_np_u16(v) if k.startswith("y_") else to_np_u8(v)
    return out


def _compare(got, want, ctx):
    for k in want:
        if not np.array_equal(got[k], want[k]):
            bad = np.flatnonzero(got[k] != want[k])
            raise AssertionError(f"{ctx}: {k} differs at {bad.size} positions, first {bad[:6].tolist()}")


@pytest.mark.parametrize("name,rows,cols,make", CASES, ids=[c[0] for c in CASES])
def test_grouped_bit_exact(device, name, rows, cols, make):
    _say("case grouped", name, rows, cols)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    off = np.asarray(make(rng), dtype=np.int64)
    xr = _grouped_values(rng, rows, cols, off)
    xt = F.f32_to_bf16_rne(F.bf16_to_f32(xr) * (1 + 0.03 * rng.standard_normal(xr.size)).astype(np.float32))
    offsets = torch.from_numpy(off).to(device)
    got = _gpu_grouped(from_np_u16(xr, device, (rows, cols)), from_np_u16(xt, device, (rows, cols)), offsets)
    ts = oracle.grouped_tensor_scale(xr, rows, cols, off)
    assert np.array_equal(got["ts"].cpu().numpy().view(np.uint32), ts.view(np.uint32)), name
    _compare(_host(got), _oracle_grouped(xr, xt, rows, cols, off, ts), name)


@pytest.mark.parametrize("peak_row", [2048, 4998, 0])
def test_grouped_tensor_scale_long_groups(device, peak_row):
    """Groups longer than one pass of the group fold (2048 row maxima per
    workgroup pass): group 0 holds 4999 rows, with its largest magnitude at
    the start of the second pass, in the last (partial) pass, or in the
    first row.  Every group's tensor scale against the oracle, bit for bit."""
    _say("case grouped long groups, peak row", peak_row)
    import fp4_rollout_guided_amd as tr
    rows, cols = 6000, 16
    off = np.array([0, 4999, 5000, 6000], dtype=np.int64)
    rng = np.random.default_rng(peak_row + 11)
    v = rng.standard_normal((rows, cols)).astype(np.float32)
    v[peak_row, 5] = -700.0     # group 0's maximum
    v[4999, 3] = 3.0e-3         # group 1: one small row
    v[5000:] *= 1.0e4           # group 2 orders of magnitude larger
    xr = F.f32_to_bf16_rne(v.reshape(-1))
    ts = tr.grouped_tensor_scale(from_np_u16(xr, device, (rows, cols)), torch.from_numpy(off).to(device))
    torch.cuda.synchronize()
    want = oracle.grouped_tensor_scale(xr, rows, cols, off)
    assert np.array_equal(ts.cpu().numpy().view(np.uint32), want.view(np.uint32))
    assert want[0] == np.float32(700.0) / np.float32(2688.0)


def test_single_group_equals_ungrouped(device):
    """With one group the grouped entry points reproduce the ungrouped ones."""
    _say("case grouped single == ungrouped")
    import fp4_rollout_guided_amd as tr
    d = workloads.single_site(device)
    xr, xt = d["x_roll"], d["x_train"]
    offsets = torch.tensor([0, xr.shape[0]], dtype=torch.int64, device=device)
    got = _host(_gpu_grouped(xr, xt, offsets))
    ts = tr.tensor_scale(xr)
    sc, bt, cd = tr.capture(xr, ts, want_codes=True)
    yg, mg, qg = tr.guided_fakequant_fwd(xt, sc, ts, bt, want_codes=True)
    torch.cuda.synchronize()
    ref = {"scales": to_np_u8(sc), "bits": to_np_u8(bt), "codes": to_np_u8(cd), "y_g": to_np_u16(yg),
           "mask_g": to_np_u8(mg), "q_g": to_np_u8(qg)}
    _compare(got, ref, "single group")


def test_moe_expert_site_per_expert_scales(device):
    """The packed routed-expert site of the MoE layer workload (131072 x 2048,
    rows grouped by 128 experts) with per-expert tensor scales: every scale
    against the oracle, and sampled rows of every output."""
    with open(os.path.join(HERE, "golden", "moe_layer_sigma.json")) as fh:
        sigma = json.load(fh)["sigma"]
    _say("case MoE layer expert site, per-expert scales")
    d = workloads.moe_layer(device, sigma, sites=["expert_in"])["expert_in"]
    _, experts = workloads.moe_routing(device)
    offsets = workloads.moe_expert_offsets(experts)
    x_roll, x_train = d["x_roll"], d["x_train"]
    rows, cols = x_roll.shape
    got = _gpu_grouped(x_roll, x_train, offsets)
    off = offsets.cpu().numpy()
    xr_all = to_np_u16(x_roll)
    ts = oracle.grouped_tensor_scale(xr_all, rows, cols, off)
    del xr_all
    assert np.array_equal(got["ts"].cpu().numpy().view(np.uint32), ts.view(np.uint32))
    assert len(np.unique(ts)) > 1
    # sampled rows: a few per expert, including each group's first and last row
    rng = np.random.default_rng(5)
    pick = []
    for a, b in zip(off, off[1:]):
        if b > a:
            pick += [a, b - 1] + rng.integers(a, b, 2).tolist()
    idx = np.unique(np.array(pick, dtype=np.int64))
    group = np.searchsorted(off, idx, side="right") - 1
    sub_off = np.r_[0, np.cumsum(np.bincount(group, minlength=len(off) - 1))].astype(np.int64)
    it = torch.from_numpy(idx).to(device)

    def rows_of(t, per_row, u16=False):
        v = t.view(torch.int16) if u16 else t
        v = v.reshape(-1, per_row)[it]
        return to_np_u16(v) if u16 else to_np_u8(v)

    xr = rows_of(x_roll, cols, True)
    xt = rows_of(x_train, cols, True)
    want = _oracle_grouped(xr, xt, idx.size, cols, sub_off, ts)
    per = {"scales": cols // 16, "bits": cols // 8, "codes": cols // 2, "mask_g": cols // 8, "q_g": cols // 2,
           "mask_r": cols // 8, "q_r": cols // 2, "mask_f": cols // 8, "q_f": cols // 2}
    sampled = {k: rows_of(got[k], n) for k, n in per.items()}
    for k in ("y_g", "y_r", "y_f"):
        sampled[k] = rows_of(got[k], cols, True)
    _compare(sampled, want, "expert site")
    _say(f"  expert site: {idx.size} sampled rows over {int((np.diff(off) > 0).sum())} experts, "
         f"ts range {ts.min():.3e}..{ts.max():.3e}")
    # every element of every output against the whole-tensor properties, with
    # each row's own group scale
    import fp4_rollout_guided_amd as tr
    grad = workloads.grad_for(x_roll.shape, device, 1, "expert_in")
    got["gin"] = tr.ste_bwd(grad, got["mask_g"])
    row_ts = got["ts"].repeat_interleave(torch.from_numpy(np.diff(off)).to(device))
    torch.cuda.synchronize()
    check_nvfp4_outputs("expert site", x_roll, x_train, grad, row_ts, got)
    # every element of every output against the oracle, with the oracle's
    # per-expert tensor scales
    host = {k: (to_np_u16(v) if k in ("y_g", "y_r", "y_f") else to_np_u8(v))
            for k, v in got.items() if k not in ("ts", "gin")}
    compare_grouped_every_element("expert site", to_np_u16(x_roll), to_np_u16(x_train), rows, cols, off, ts, host)
