"""GPU parity where the capture's quotient x / s leaves binary32.

A caller may hand the capture any tensor scale (an engine that keeps its
own).  Under a small one, a block with a huge element saturates its scale
byte at 0x7E, s = 448 * ts, and |x| / s can exceed the largest float: the
oracle's quotient is then +-inf, its magnitude clips to 6 and the code is
+-7 with the element's sign.  These blocks, and blocks just below and above
that threshold, go through every capture entry point (per site, batch,
per-expert groups, b low bits) and the forwards that read their record,
against the oracle bit for bit."""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F
from tests.gpu_util import assert_same, from_np_u16, gpu_path, oracle_path, to_np_u8, to_np_u16

pytestmark = pytest.mark.gpu

# tensor scales: inside the fast range with saturation reachable (2^-20,
# 2^-60, 2^-100), at its top where only the largest bf16 values overflow
# (2^-9), past it (2^-8: 448 ts > 1, no overflow possible), and one
# unrelated value
TENSOR_SCALES = [2.0 ** -20, 2.0 ** -60, 2.0 ** -100, 2.0 ** -9, 2.0 ** -8, 1e-30]


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _bf16_np(v):
    return F.f32_to_bf16_rne(np.asarray(v, np.float64).astype(np.float32))


def overflow_blocks(ts, rng):
    """Blocks around the overflow of x / (448 ts): elements near
    2^128 * 448 * ts, exact powers of two at and around 2^117, the largest
    bf16 values, mixed signs, small values and zeros beside them."""
    edge = 2.0 ** 128 * 448.0 * float(np.float32(ts))          # |x| / s = 2^128 here
    bf16_max = float(F.bf16_to_f32(np.array([0x7F7F], np.uint16))[0])
    pool = [edge * f for f in (0.25, 0.5, 0.999, 1.0, 1.001, 1.5, 2.0, 4.0)]
    pool += [2.0 ** e for e in (100, 116, 117, 118, 126, 127)] + [bf16_max, 3e38, 1.0, 0.5, 2.0 ** -100]
    pool = np.array([p for p in pool if p <= bf16_max])
    blocks = [
        [2.0 ** 117, -2.0 ** 117, 2.0 ** 116, -2.0 ** 100, 1.0, -1.0, 0.0, -0.0,
         2.0 ** -100, bf16_max, -bf16_max, 2.0 ** 127, -2.0 ** 126, 5.0, -6.0, 2.0 ** 64],
        [-2.0 ** 117] * 16,                                      # every element negative
        [2.0 ** 117] * 16,
        [bf16_max] + [-(2.0 ** k) for k in range(100, 115)],
        [-bf16_max] + [0.0] * 7 + [-0.0] * 8,
    ]
    for _ in range(123):                                        # random mixes from the pool
        b = rng.choice(pool, 16) * np.where(rng.random(16) < 0.5, -1.0, 1.0)
        b[rng.random(16) < 0.2] = 0.0
        blocks.append(b.tolist())
    return _bf16_np(np.array(blocks, np.float64).reshape(-1))


def _train_values(xr, rng):
    xt = F.bf16_to_f32(xr).astype(np.float64)
    xt = np.where(rng.random(xt.size) < 0.5, xt, xt * (1 + 0.3 * rng.standard_normal(xt.size)))
    return _bf16_np(np.clip(xt, -3.3e38, 3.3e38))


@pytest.mark.parametrize("ts", TENSOR_SCALES)
def test_capture_and_forwards_past_binary32(device, ts):
    _say("case overflow, per site, ts", ts)
    rng = np.random.default_rng(117)
    xr = overflow_blocks(ts, rng)
    xt = _train_values(xr, rng)
    g = _bf16_np(rng.standard_normal(xr.size))
    shape = (xr.size // 64, 64)
    tsf = np.float32(ts)
    got = gpu_path(from_np_u16(xr, device, shape), from_np_u16(xt, device, shape), from_np_u16(g, device, shape),
                   ts=torch.tensor([tsf], dtype=torch.float32, device=device))
    want = oracle_path(xr, xt, g, ts=tsf)
    assert_same(got, want, ctx=f"overflow ts={ts}")
    # the class this covers: saturated scale bytes with overflowing quotients
    s = F.e4m3fn_decode(want["scales"]).astype(np.float32) * tsf
    with np.errstate(over="ignore", invalid="ignore"):
        q = np.abs(F.bf16_to_f32(xr).reshape(-1, 16) / s[:, None])
    hits = int(np.isinf(q).sum())
    _say(f"  ts={ts}: {hits} quotients overflow binary32")
    if ts <= 2.0 ** -20:
        assert hits > 100


def test_batch_capture_past_binary32(device):
    import fp4_rollout_guided_amd as tr
    _say("case overflow, batch")
    rng = np.random.default_rng(118)
    host = [overflow_blocks(ts, rng) for ts in TENSOR_SCALES]
    dev = [from_np_u16(x, device, (x.size // 32, 32)) for x in host]
    tss = [torch.tensor([np.float32(ts)], dtype=torch.float32, device=device) for ts in TENSOR_SCALES]
    rec = tr.capture_batch(dev, tss, want_codes=True)
    torch.cuda.synchronize()
    for i, (x, ts) in enumerate(zip(host, TENSOR_SCALES)):
        cap = oracle.capture(x, np.float32(ts), with_codes=True)
        for k, got in zip(("scales", "bits", "codes"), rec[i]):
            assert np.array_equal(to_np_u8(got), cap[k]), (ts, k)


def test_grouped_capture_past_binary32(device):
    import fp4_rollout_guided_amd as tr
    _say("case overflow, per-expert groups")
    rng = np.random.default_rng(119)
    parts = [overflow_blocks(ts, rng) for ts in TENSOR_SCALES]
    cols = 64
    rows_per = [p.size // cols for p in parts]
    off = np.concatenate([[0], np.cumsum(rows_per)]).astype(np.int64)
    xr = np.concatenate(parts)
    xt = _train_values(xr, rng)
    rows = int(off[-1])
    ts = np.array(TENSOR_SCALES, dtype=np.float32)
    offsets = torch.from_numpy(off).to(device)
    tsd = torch.from_numpy(ts).to(device)
    xrd, xtd = from_np_u16(xr, device, (rows, cols)), from_np_u16(xt, device, (rows, cols))
    sc, bt, cd = tr.grouped_capture(xrd, offsets, tsd, want_codes=True)
    yg, mg, qg = tr.grouped_guided_fakequant_fwd(xtd, offsets, sc, tsd, bt, want_codes=True)
    yf, mf, qf = tr.grouped_full_info_fakequant_fwd(xtd, offsets, sc, tsd, cd, want_codes=True)
    torch.cuda.synchronize()
    cap = oracle.grouped_capture(xr, rows, cols, off, ts, with_codes=True)
    gd = oracle.grouped_guided_fwd(xt, rows, cols, off, cap["scales"], ts, cap["bits"])
    fi = oracle.grouped_full_info_fwd(xt, rows, cols, off, cap["scales"], ts, cap["codes"])
    assert_same({"scales": to_np_u8(sc), "bits": to_np_u8(bt), "codes": to_np_u8(cd)}, cap, ctx="grouped capture")
    assert_same({"y": to_np_u16(yg), "mask": to_np_u8(mg), "codes": to_np_u8(qg)}, gd, ctx="grouped guided")
    assert_same({"y": to_np_u16(yf), "mask": to_np_u8(mf), "codes": to_np_u8(qf)}, fi, ctx="grouped full info")


@pytest.mark.parametrize("nbits", [1, 2, 3, 4])
def test_lowbits_capture_past_binary32(device, nbits):
    import fp4_rollout_guided_amd as tr
    _say("case overflow, low bits", nbits)
    rng = np.random.default_rng(120 + nbits)
    for ts in (2.0 ** -20, 2.0 ** -100):
        xr = overflow_blocks(ts, rng)
        xt = _train_values(xr, rng)
        shape = (xr.size // 64, 64)
        tsf = np.float32(ts)
        tsd = torch.tensor([tsf], dtype=torch.float32, device=device)
        xrd, xtd = from_np_u16(xr, device, shape), from_np_u16(xt, device, shape)
        sc, pl, cd = tr.capture_lowbits(xrd, tsd, nbits, want_codes=True)
        y, m, q = tr.lowbits_fakequant_fwd(xtd, sc, tsd, nbits, pl, want_codes=True)
        torch.cuda.synchronize()
        cap = oracle.capture_lowbits(xr, tsf, nbits)
        want = oracle.lowbits_fwd(xt, cap["scales"], tsf, cap["planes"], nbits)
        assert_same({"scales": to_np_u8(sc), "planes": to_np_u8(pl)}, cap, ctx=f"lowbits capture b={nbits} ts={ts}")
        assert_same({"codes": to_np_u8(cd)}, {"codes": oracle.capture(xr, tsf, with_codes=True)["codes"]},
                    ctx=f"lowbits codes b={nbits} ts={ts}")
        assert_same({"y": to_np_u16(y), "mask": to_np_u8(m), "codes": to_np_u8(q)}, want,
                    ctx=f"lowbits fwd b={nbits} ts={ts}")
