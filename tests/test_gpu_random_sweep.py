"""Seeded random sweep over the entry points, every output element against
the oracle, bit for bit.

Each case draws from its own seed:
- a family:
  - the whole path, with the tensor scale computed or held by the caller;
  - per-expert groups;
  - forwards on records read back in a shuffled row order;
  - the record gather;
  - b low bits;
  - MXFP4 and MXFP8;
  - batches of sites;
  - the agreement statistics;
  - the allocation-free tensor scale;
- a ragged shape of up to a few hundred thousand elements;
- a value recipe: per-row magnitudes spread over up to 60 decades, heavy
  tails, outlier channels, zero rows, and IEEE specials sprinkled into either
  side;
- a build: production, or the small-grid build, whose grids cap at three
  workgroups and whose non-temporal threshold is zero.

The hand-picked cases of the other files pin known edges; this sweep looks
for the combinations nobody listed."""
import contextlib
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F
from tests.gpu_util import assert_same, from_np_u16, gpu_path, oracle_path, to_np_u8, to_np_u16

pytestmark = pytest.mark.gpu
CASES = 110
FAMILIES = ["path", "path_ts", "grouped", "gathered", "gather", "lowbits", "mx", "mx8", "batch", "stats",
            "noalloc"]
SPECIALS = np.array([np.nan, -np.nan, np.inf, -np.inf, 0.0, -0.0, 1e-40, -1e-42, 3.3e38, -3.3e38, 1.2e-38,
                     6.0, -6.0, 2688.0], dtype=np.float32)


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@contextlib.contextmanager
def _build(tr, build):
    saved = tr.lib
    if build == "small-grid":
        tr.lib = tr.load_library(tr.SMALLGRID_LIB_PATH)
    try:
        yield
    finally:
        tr.lib = saved


def _shape(rng, unit, max_elems=300_000):
    while True:
        rows = int(np.exp(rng.uniform(0, np.log(700))))
        cols = unit * int(np.exp(rng.uniform(0, np.log(320 * 16 // unit))))
        if rows * cols <= max_elems:
            return rows, cols


def _f32(rng, rows, cols):
    kind = rng.integers(0, 4)
    if kind == 0:
        v = rng.standard_normal((rows, cols))
    elif kind == 1:
        v = rng.standard_t(2, (rows, cols))
    elif kind == 2:
        v = rng.standard_normal((rows, cols))
        ch = rng.choice(cols, max(1, cols // 128), replace=False)
        v[:, ch] *= rng.uniform(10, 1e4, ch.size)
    else:
        v = rng.uniform(-1, 1, (rows, cols)) ** 5
    spread = 30 if rng.random() < 0.3 else 3
    v = v * 10.0 ** rng.uniform(-spread, spread, (rows, 1))
    if rows > 2 and rng.random() < 0.5:
        v[rng.integers(rows)] = 0.0
    return v.astype(np.float32)


def _sprinkle(rng, flat, p=0.5):
    if flat.size and rng.random() < p:
        k = int(rng.integers(1, 12))
        flat[rng.integers(0, flat.size, k)] = rng.choice(SPECIALS, k)
    return flat


def _pair(rng, rows, cols):
    """(x_roll, x_train, grad) as bf16 bit arrays."""
    v = _f32(rng, rows, cols)
    xr = F.f32_to_bf16_rne(_sprinkle(rng, v.reshape(-1).copy()))
    if rng.random() < 0.1:
        t = _f32(rng, rows, cols).reshape(-1)
    else:
        eps = rng.choice([0.0, 1e-3, 0.03, 0.5])
        with np.errstate(over="ignore", invalid="ignore"):
            t = (F.bf16_to_f32(xr).astype(np.float64) * (1 + eps * rng.standard_normal(xr.size))).astype(np.float32)
    xt = F.f32_to_bf16_rne(_sprinkle(rng, t))
    g = F.f32_to_bf16_rne(rng.standard_normal(xr.size).astype(np.float32))
    return xr, xt, g


def _partition(rng, rows):
    groups = int(rng.integers(1, min(rows, 40) + 2))
    off = np.r_[0, np.sort(rng.integers(0, rows + 1, groups - 1)), rows].astype(np.int64)
    return off


def _host(got):
    return {k: (to_np_u16(v) if k.startswith(("y", "gin")) else to_np_u8(v)) for k, v in got.items()}


def _fwd_dict(r, tag):
    return {f"y_{tag}": r["y"], f"mask_{tag}": r["mask"], f"q_{tag}": r["codes"]}


def _run_path(tr, rng, device, ctx, caller_ts):
    rows, cols = _shape(rng, 16)
    xr, xt, g = _pair(rng, rows, cols)
    ts = None
    if caller_ts:
        ts = np.float32(rng.choice([2.0 ** -20, 2.0 ** -60, 1e30, 3e-39, rng.uniform(1e-3, 10)]))
    _say(f"{ctx}: path {rows}x{cols}, ts {'computed' if ts is None else ts}")
    dev = lambda a: from_np_u16(a, device, (rows, cols))
    ts_d = None if ts is None else torch.tensor([ts], dtype=torch.float32, device=device)
    got = gpu_path(dev(xr), dev(xt), dev(g), ts=ts_d)
    assert_same(got, oracle_path(xr, xt, g, ts=ts), ctx=ctx)


def _run_grouped(tr, rng, device, ctx):
    rows, cols = _shape(rng, 16)
    xr, xt, _ = _pair(rng, rows, cols)
    off = _partition(rng, rows)
    _say(f"{ctx}: grouped {rows}x{cols}, {len(off) - 1} groups")
    offsets = torch.from_numpy(off).to(device)
    x_roll, x_train = from_np_u16(xr, device, (rows, cols)), from_np_u16(xt, device, (rows, cols))
    ts = tr.grouped_tensor_scale(x_roll, offsets)
    sc, bt, cd = tr.grouped_capture(x_roll, offsets, ts, want_codes=True)
    got = {"scales": sc, "bits": bt, "codes": cd}
    got["y_g"], got["mask_g"], got["q_g"] = tr.grouped_guided_fakequant_fwd(x_train, offsets, sc, ts, bt,
                                                                           want_codes=True)
    got["y_r"], got["mask_r"], got["q_r"] = tr.grouped_rne_fakequant_fwd(x_train, offsets, sc, ts, want_codes=True)
    got["y_f"], got["mask_f"], got["q_f"] = tr.grouped_full_info_fakequant_fwd(x_train, offsets, sc, ts, cd,
                                                                              want_codes=True)
    torch.cuda.synchronize()
    ts_o = oracle.grouped_tensor_scale(xr, rows, cols, off)
    assert np.array_equal(ts.cpu().numpy().view(np.uint32), ts_o.view(np.uint32)), ctx
    cap = oracle.grouped_capture(xr, rows, cols, off, ts_o, with_codes=True)
    want = {"scales": cap["scales"], "bits": cap["bits"], "codes": cap["codes"]}
    want.update(_fwd_dict(oracle.grouped_guided_fwd(xt, rows, cols, off, cap["scales"], ts_o, cap["bits"]), "g"))
    want.update(_fwd_dict(oracle.grouped_rne_fwd(xt, rows, cols, off, cap["scales"], ts_o), "r"))
    want.update(_fwd_dict(oracle.grouped_full_info_fwd(xt, rows, cols, off, cap["scales"], ts_o, cap["codes"]), "f"))
    assert_same(_host(got), want, ctx=ctx)


def _index(rng, src_rows, dst_rows):
    idx = rng.integers(0, max(src_rows, 1), dst_rows).astype(np.int64)
    if dst_rows and rng.random() < 0.5:
        k = int(rng.integers(1, min(dst_rows, 4) + 1))
        idx[rng.integers(0, dst_rows, k)] = rng.choice([-1, -7, src_rows, src_rows + 3], k)
    return idx


def _run_gathered(tr, rng, device, ctx):
    src_rows, cols = _shape(rng, 16)
    dst_rows = int(rng.integers(1, max(2, 300_000 // cols)))
    dst_rows = min(dst_rows, 700)
    grouped = rng.random() < 0.5
    xr = F.f32_to_bf16_rne(_sprinkle(rng, _f32(rng, src_rows, cols).reshape(-1)))
    idx = _index(rng, src_rows, dst_rows)
    base = np.clip(idx, 0, src_rows - 1)
    with np.errstate(over="ignore", invalid="ignore"):
        t = (F.bf16_to_f32(xr).reshape(src_rows, cols)[base].astype(np.float64)
             * (1 + 0.03 * rng.standard_normal((dst_rows, cols)))).astype(np.float32).reshape(-1)
    xt = F.f32_to_bf16_rne(_sprinkle(rng, t))
    off = _partition(rng, src_rows) if grouped else None
    _say(f"{ctx}: gathered {src_rows}->{dst_rows}x{cols}, {'per-expert' if grouped else 'one'} scale")
    if off is None:
        ts = np.float32(oracle.tensor_scale(xr))
        rec = oracle.capture(xr, ts, with_codes=True)
    else:
        ts = oracle.grouped_tensor_scale(xr, src_rows, cols, off)
        rec = oracle.grouped_capture(xr, src_rows, cols, off, ts, with_codes=True)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    x_train = from_np_u16(xt, device, (dst_rows, cols))
    row_index, off_d = dev(idx), (dev(off) if off is not None else None)
    ts_d = dev(np.atleast_1d(np.asarray(ts, dtype=np.float32)))
    sc, bt, cd = dev(rec["scales"]), dev(rec["bits"]), dev(rec["codes"])
    got = {}
    got["y_g"], got["mask_g"], got["q_g"] = tr.gathered_guided_fakequant_fwd(x_train, row_index, sc, ts_d, bt,
                                                                             offsets=off_d, want_codes=True)
    got["y_f"], got["mask_f"], got["q_f"] = tr.gathered_full_info_fakequant_fwd(x_train, row_index, sc, ts_d, cd,
                                                                                offsets=off_d, want_codes=True)
    got["y_r"], got["mask_r"], got["q_r"] = tr.gathered_rne_fakequant_fwd(x_train, row_index, sc, ts_d,
                                                                          offsets=off_d, want_codes=True)
    torch.cuda.synchronize()
    want = {}
    for mode, tag in (("guided", "g"), ("full", "f"), ("rne", "r")):
        want.update(_fwd_dict(oracle.gathered_fwd(mode, xt, cols, rec, src_rows, idx, ts, off), tag))
    assert_same(_host(got), want, ctx=ctx)


def _run_gather(tr, rng, device, ctx):
    src_rows, cols = _shape(rng, 16)
    dst_rows = min(700, int(rng.integers(1, max(2, 300_000 // cols))))
    n = src_rows * cols
    rec = {"bits": rng.integers(0, 256, n // 8, dtype=np.uint8),
           "scales": rng.integers(0, 256, n // 16, dtype=np.uint8),
           "codes": rng.integers(0, 256, n // 2, dtype=np.uint8) if rng.random() < 0.5 else None}
    idx = _index(rng, src_rows, dst_rows)
    _say(f"{ctx}: record gather {src_rows}->{dst_rows}x{cols}, codes {rec['codes'] is not None}")
    dev = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device)
    bits, scales, codes = tr.gather_records(dev(rec["bits"]), dev(rec["scales"]), dev(rec["codes"]), cols, dev(idx))
    torch.cuda.synchronize()
    want = oracle.gather_records(rec, idx, src_rows, cols)
    got = {"bits": to_np_u8(bits), "scales": to_np_u8(scales)}
    if rec["codes"] is not None:
        got["codes"] = to_np_u8(codes)
    assert_same(got, want, ctx=ctx)


def _run_lowbits(tr, rng, device, ctx):
    rows, cols = _shape(rng, 16)
    xr, xt, _ = _pair(rng, rows, cols)
    nb = int(rng.integers(1, 5))
    _say(f"{ctx}: low bits b={nb} {rows}x{cols}")
    x_roll, x_train = from_np_u16(xr, device, (rows, cols)), from_np_u16(xt, device, (rows, cols))
    ts = tr.tensor_scale(x_roll)
    sc, planes, cd = tr.capture_lowbits(x_roll, ts, nb, want_codes=True)
    y, m, q = tr.lowbits_fakequant_fwd(x_train, sc, ts, nb, planes, want_codes=True)
    torch.cuda.synchronize()
    ts_o = np.float32(oracle.tensor_scale(xr))
    cap = oracle.capture_lowbits(xr, ts_o, nb)
    full = oracle.capture(xr, ts_o, with_codes=True)
    want = {"scales": cap["scales"], "planes": cap["planes"], "codes": full["codes"]}
    want.update(_fwd_dict(oracle.lowbits_fwd(xt, cap["scales"], ts_o, cap["planes"], nb), "l"))
    got = {"scales": to_np_u8(sc), "planes": to_np_u8(planes), "codes": to_np_u8(cd),
           "y_l": to_np_u16(y), "mask_l": to_np_u8(m), "q_l": to_np_u8(q)}
    assert_same(got, want, ctx=ctx)


def _run_mx(tr, rng, device, ctx, eight):
    rows, cols = _shape(rng, 32)
    xr, xt, g = _pair(rng, rows, cols)
    _say(f"{ctx}: {'mx8' if eight else 'mx'} {rows}x{cols}")
    dev = lambda a: from_np_u16(a, device, (rows, cols))
    x_roll, x_train, grad = dev(xr), dev(xt), dev(g)
    pre = "mx8_" if eight else "mx_"
    sc, bt, cd = getattr(tr, pre + "capture")(x_roll, want_codes=True)
    got = {"scales": sc, "bits": bt, "codes": cd}
    got["y_g"], got["mask_g"], got["q_g"] = getattr(tr, pre + "guided_fakequant_fwd")(x_train, sc, bt, want_codes=True)
    got["y_r"], got["mask_r"], got["q_r"] = getattr(tr, pre + "rne_fakequant_fwd")(x_train, sc, want_codes=True)
    got["y_f"], got["mask_f"], got["q_f"] = getattr(tr, pre + "full_info_fakequant_fwd")(x_train, sc, cd,
                                                                                        want_codes=True)
    got["gin"] = tr.ste_bwd(grad, got["mask_g"])
    torch.cuda.synchronize()
    o = {"capture": oracle.mx8_capture if eight else oracle.mx_capture,
         "guided": oracle.mx8_guided_fwd if eight else oracle.mx_guided_fwd,
         "rne": oracle.mx8_rne_fwd if eight else oracle.mx_rne_fwd,
         "full": oracle.mx8_full_info_fwd if eight else oracle.mx_full_info_fwd}
    cap = o["capture"](xr, with_codes=True)
    want = {"scales": cap["scales"], "bits": cap["bits"], "codes": cap["codes"]}
    gd = o["guided"](xt, cap["scales"], cap["bits"])
    want.update(_fwd_dict(gd, "g"))
    want.update(_fwd_dict(o["rne"](xt, cap["scales"]), "r"))
    want.update(_fwd_dict(o["full"](xt, cap["scales"], cap["codes"]), "f"))
    want["gin"] = oracle.ste_bwd(g, gd["mask"], xt.size)
    assert_same(_host(got), want, ctx=ctx)


def _run_batch(tr, rng, device, ctx):
    k = int(rng.integers(1, 9))
    shapes = [_shape(rng, 16, 300_000 // k) for _ in range(k)]
    _say(f"{ctx}: batch of {k} sites {shapes}")
    xs = [F.f32_to_bf16_rne(_sprinkle(rng, _f32(rng, r, c).reshape(-1), 0.3)) for r, c in shapes]
    dev = [from_np_u16(x, device, s) for x, s in zip(xs, shapes)]
    ts = tr.tensor_scale_batch(dev)
    rec = tr.capture_batch(dev, ts, want_codes=True)
    torch.cuda.synchronize()
    for i, (x, (sc, bt, cd)) in enumerate(zip(xs, rec)):
        ts_o = np.float32(oracle.tensor_scale(x))
        assert ts[i].cpu().numpy().view(np.uint32)[0] == ts_o.view(np.uint32), (ctx, i)
        cap = oracle.capture(x, ts_o, with_codes=True)
        assert_same({"scales": to_np_u8(sc), "bits": to_np_u8(bt), "codes": to_np_u8(cd)},
                    {"scales": cap["scales"], "bits": cap["bits"], "codes": cap["codes"]}, ctx=f"{ctx} site {i}")


def _run_stats(tr, rng, device, ctx):
    rows, cols = _shape(rng, 16)
    xr, xt, _ = _pair(rng, rows, cols)
    n = xr.size
    ts = np.float32(oracle.tensor_scale(xr))
    cap = oracle.capture(xr, ts, with_codes=True)
    roll = oracle.unpack_nibbles(cap["codes"], n).copy()
    flip = rng.random(n) < rng.choice([0.0, 0.02, 0.5])
    roll[flip] = rng.integers(0, 16, int(flip.sum()))
    cbits = (roll & 1) if rng.random() < 0.7 else rng.integers(0, 2, n)
    codes, bits = oracle.pack_nibbles(roll), oracle.pack_bits(cbits.astype(np.uint8))
    _say(f"{ctx}: agreement statistics {rows}x{cols}, {int(flip.sum())} rollout codes replaced")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    got = tr.mismatch_stats(from_np_u16(xt, device, (rows, cols)), dev(cap["scales"]),
                            dev(np.array([ts], np.float32)), dev(bits), dev(codes))
    torch.cuda.synchronize()
    st = oracle.mismatch_stats(xt, cap["scales"], ts, codes, bits)
    want = st["hist"] + [st["straddle"], st["crossed"], st["recovered"], st["violations"], st["n"]]
    assert got.cpu().numpy().tolist() == want, ctx


def _run_noalloc(tr, rng, device, ctx):
    sizes = [_shape(rng, 16) for _ in range(2)]
    sizes.sort(key=lambda rc: -rc[0] * rc[1])      # the second call smaller, as the entry point's callers reuse it
    _say(f"{ctx}: allocation-free tensor scale on {sizes}")
    for rows, cols in sizes:
        x = F.f32_to_bf16_rne(_sprinkle(rng, _f32(rng, rows, cols).reshape(-1)))
        got = tr.tensor_scale_noalloc(from_np_u16(x, device, (rows, cols)))
        torch.cuda.synchronize()
        want = np.float32(oracle.tensor_scale(x))
        assert got.cpu().numpy().view(np.uint32)[0] == want.view(np.uint32), (ctx, rows, cols)


@pytest.mark.parametrize("seed", range(CASES), ids=[f"seed{s}" for s in range(CASES)])
def test_random_sweep(device, seed):
    import fp4_rollout_guided_amd as tr
    rng = np.random.default_rng(0x7ACE0000 + seed)
    family = FAMILIES[seed % len(FAMILIES)]
    build = "small-grid" if rng.random() < 0.4 else "production"
    ctx = f"random sweep seed {seed} ({family}, {build} build)"
    with _build(tr, build):
        if family in ("path", "path_ts"):
            _run_path(tr, rng, device, ctx, caller_ts=family == "path_ts")
        elif family == "grouped":
            _run_grouped(tr, rng, device, ctx)
        elif family == "gathered":
            _run_gathered(tr, rng, device, ctx)
        elif family == "gather":
            _run_gather(tr, rng, device, ctx)
        elif family == "lowbits":
            _run_lowbits(tr, rng, device, ctx)
        elif family in ("mx", "mx8"):
            _run_mx(tr, rng, device, ctx, eight=family == "mx8")
        elif family == "batch":
            _run_batch(tr, rng, device, ctx)
        elif family == "stats":
            _run_stats(tr, rng, device, ctx)
        else:
            _run_noalloc(tr, rng, device, ctx)
