"""GPU parity of the MXFP4 variant: capture and the guided / RNE /
full-information forwards (and the STE backward on their mask) through the
C ABI against ``oracle.mx``, bit for bit.  Covers ragged shapes over several
tiles, every bf16 pattern under every E8M0 scale byte, block maxima over
every finite bf16 magnitude, tiny elements beside large ones, specials,
in-place use, and every element of a layer of the deeper-half sweep."""
import contextlib
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import formats as F
from tests.gpu_util import from_np_u16, to_np_u8, to_np_u16

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _bf16_np(v):
    return F.f32_to_bf16_rne(np.asarray(v, np.float32))


def _gpu_mx(xr, xt, g, roll=None):
    import fp4_rollout_guided_amd as tr
    sc, bt, cd = tr.mx_capture(xr, want_codes=True)
    yg, mg, qg = tr.mx_guided_fakequant_fwd(xt, sc, bt, want_codes=True)
    yr, mr, qr = tr.mx_rne_fakequant_fwd(xt, sc, want_codes=True)
    yf, mf, qf = tr.mx_full_info_fakequant_fwd(xt, sc, cd if roll is None else roll, want_codes=True)
    gin = tr.ste_bwd(g, mg)
    torch.cuda.synchronize()
    return {"scales": to_np_u8(sc), "bits": to_np_u8(bt), "codes": to_np_u8(cd),
            "y_g": to_np_u16(yg), "mask_g": to_np_u8(mg), "q_g": to_np_u8(qg),
            "y_r": to_np_u16(yr), "mask_r": to_np_u8(mr), "q_r": to_np_u8(qr),
            "y_f": to_np_u16(yf), "mask_f": to_np_u8(mf), "q_f": to_np_u8(qf), "gin": to_np_u16(gin)}


def _oracle_mx(xr, xt, g, roll=None):
    cap = oracle.mx_capture(xr, with_codes=True)
    gd = oracle.mx_guided_fwd(xt, cap["scales"], cap["bits"])
    rn = oracle.mx_rne_fwd(xt, cap["scales"])
    fi = oracle.mx_full_info_fwd(xt, cap["scales"], cap["codes"] if roll is None else roll)
    return {"scales": cap["scales"], "bits": cap["bits"], "codes": cap["codes"],
            "y_g": gd["y"], "mask_g": gd["mask"], "q_g": gd["codes"],
            "y_r": rn["y"], "mask_r": rn["mask"], "q_r": rn["codes"],
            "y_f": fi["y"], "mask_f": fi["mask"], "q_f": fi["codes"],
            "gin": oracle.ste_bwd(g, gd["mask"], xt.size)}


def _same(got, want, ctx):
    for k in want:
        a, b = np.asarray(got[k]).reshape(-1), np.asarray(want[k]).reshape(-1)
        assert a.shape == b.shape, (ctx, k)
        if not np.array_equal(a, b):
            bad = np.flatnonzero(a != b)
            raise AssertionError(f"{ctx}: {k} differs at {bad.size} of {b.size}; first {bad[:6].tolist()} "
                                 f"got {a[bad[:6]].tolist()} want {b[bad[:6]].tolist()}")


@pytest.mark.parametrize("shape", [(1, 32), (37, 64), (3, 4128), (129, 4096 + 32 * 5), (17, 7168), (1024, 2048)])
def test_mx_small_shapes_bit_exact(device, shape):
    _say("case mx small", shape)
    rows, cols = shape
    rng = np.random.default_rng(rows * 100003 + cols)
    v = rng.standard_t(4, (rows, cols))
    v[:, rng.choice(cols, max(1, cols // 256), replace=False)] *= 60
    xr = _bf16_np(v.reshape(-1))
    xt = _bf16_np(F.bf16_to_f32(xr) * (1 + 0.03 * rng.standard_normal(xr.size)))
    g = _bf16_np(rng.standard_normal(xr.size))
    got = _gpu_mx(*(from_np_u16(a, device, shape) for a in (xr, xt, g)))
    _same(got, _oracle_mx(xr, xt, g), f"mx {shape}")


def test_mx_fwd_exhaustive_bf16_by_scale_byte(device):
    """Every bf16 pattern as x_train under every E8M0 byte 0x00..0xFF (0xFF:
    zero-scale blocks), guided with random cached bits, RNE, and full
    information with random rollout codes."""
    import fp4_rollout_guided_amd as tr
    _say("case mx exhaustive fwd")
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = np.tile(pats, 256)
    scales = np.repeat(np.arange(256, dtype=np.uint32).astype(np.uint8), (1 << 16) // 32)
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 256, size=x.size // 8, dtype=np.uint8)
    roll = rng.integers(0, 256, size=x.size // 2, dtype=np.uint8)
    xd = from_np_u16(x, device, (x.size // 32, 32))
    sd, bd, rd = (torch.from_numpy(a).to(device) for a in (scales, bits, roll))
    yg, mg, qg = tr.mx_guided_fakequant_fwd(xd, sd, bd, want_codes=True)
    yr, mr, qr = tr.mx_rne_fakequant_fwd(xd, sd, want_codes=True)
    yf, mf, qf = tr.mx_full_info_fakequant_fwd(xd, sd, rd, want_codes=True)
    torch.cuda.synchronize()
    for name, (y, m, q), want in (("guided", (yg, mg, qg), oracle.mx_guided_fwd(x, scales, bits)),
                                  ("rne", (yr, mr, qr), oracle.mx_rne_fwd(x, scales)),
                                  ("full", (yf, mf, qf), oracle.mx_full_info_fwd(x, scales, roll))):
        _same({"y": to_np_u16(y), "mask": to_np_u8(m), "codes": to_np_u8(q)}, want, f"mx exhaustive {name}")


def test_mx_capture_exhaustive_block_amax(device):
    """Block maxima over every finite positive bf16 magnitude (plus +Inf),
    the other 31 elements random fractions of the maximum, NaN elements here
    and there: every E8M0 byte the capture can produce."""
    import fp4_rollout_guided_amd as tr
    _say("case mx capture amax sweep")
    rng = np.random.default_rng(42)
    mags = F.bf16_to_f32(np.arange(1, 0x7F81, dtype=np.uint16)).astype(np.float64)
    nb = mags.size
    frac = rng.uniform(-1, 1, size=(nb, 31))
    blocks = np.concatenate([mags[:, None] * np.where(rng.random((nb, 1)) < 0.5, 1, -1), mags[:, None] * frac], axis=1)
    blocks = np.where(np.isfinite(blocks), blocks, np.where(np.isinf(blocks) & (np.arange(32) > 0), 0.0, blocks))
    xr = _bf16_np(blocks.reshape(-1))
    xr[rng.choice(xr.size, 64, replace=False)] = 0x7FC1
    sc, bt, cd = tr.mx_capture(from_np_u16(xr, device, (nb, 32)), want_codes=True)
    torch.cuda.synchronize()
    _same({"scales": to_np_u8(sc), "bits": to_np_u8(bt), "codes": to_np_u8(cd)},
          oracle.mx_capture(xr, with_codes=True), "mx capture sweep")


def test_mx_tiny_elements_and_specials(device):
    """Blocks with one large element setting the scale anywhere in E8M0's
    range and otherwise subnormals, tiny normals, signed zeros, NaN and Inf;
    x_train perturbed on 30% of the elements."""
    _say("case mx tiny + specials")
    rng = np.random.default_rng(77)
    big = np.repeat(2.0 ** np.arange(-133, 128, dtype=np.float64), 8) * rng.uniform(1, 2, 261 * 8)
    nb = big.size
    pool = np.concatenate([F.bf16_to_f32(np.arange(1, 0x80, dtype=np.uint16)).astype(np.float64),
                           2.0 ** rng.uniform(-126, -96, 400), np.array([0.0, -0.0, np.nan, np.inf, -np.inf]),
                           rng.standard_normal(200)])
    rest = rng.choice(pool, size=(nb, 31)) * np.where(rng.random((nb, 31)) < 0.5, -1, 1)
    tame = rng.random((nb, 31)) > 0.1           # keep NaN / Inf on about a tenth of the draws
    rest[tame] = np.where(np.isfinite(rest), rest, 0.0)[tame]
    blocks = np.concatenate([big[:, None] * np.where(rng.random((nb, 1)) < 0.5, -1, 1), rest], axis=1)
    xr = _bf16_np(blocks.reshape(-1))
    xt = xr.copy()
    flip = rng.random(xt.size) < 0.3
    xt[flip] = _bf16_np(F.bf16_to_f32(xt[flip]) * (1 + 0.3 * rng.standard_normal(flip.sum())))
    g = _bf16_np(rng.standard_normal(xr.size))
    shape = (nb, 32)
    got = _gpu_mx(*(from_np_u16(a, device, shape) for a in (xr, xt, g)))
    _same(got, _oracle_mx(xr, xt, g), "mx tiny/specials")


@pytest.mark.parametrize("build", ["production", "small-grid"])
def test_mx_in_place(device, build):
    """y written over x_train equals y in a separate buffer; also through the
    small-grid build, which streams every tensor with the non-temporal hint
    (production does past 256 MiB)."""
    import fp4_rollout_guided_amd as tr
    _say("case mx in place", build)
    with _build(tr, build):
        _test_mx_in_place(tr, device)


@contextlib.contextmanager
def _build(tr, build):
    saved = tr.lib
    if build == "small-grid":
        tr.lib = tr.load_library(tr.SMALLGRID_LIB_PATH)
    try:
        yield
    finally:
        tr.lib = saved


def _test_mx_in_place(tr, device):
    rng = np.random.default_rng(9)
    xr = _bf16_np(rng.standard_normal(64 * 2048))
    xt = _bf16_np(F.bf16_to_f32(xr) * (1 + 0.05 * rng.standard_normal(xr.size)))
    xrd = from_np_u16(xr, device, (64, 2048))
    sc, bt, _ = tr.mx_capture(xrd)
    ref, _, _ = tr.mx_guided_fakequant_fwd(from_np_u16(xt, device, (64, 2048)), sc, bt)
    inplace = from_np_u16(xt, device, (64, 2048))
    out, _, _ = tr.mx_guided_fakequant_fwd(inplace, sc, bt, y=inplace)
    torch.cuda.synchronize()
    assert out.data_ptr() == inplace.data_ptr()
    assert np.array_equal(to_np_u16(out), to_np_u16(ref))


def test_mx_deeper_half_layer(device):
    """One 262144x2048 layer of the deeper-half sweep on MXFP4 scales: the
    capture, guided, RNE and full-information outputs and the STE backward
    on the guided mask against the oracle, bit for bit, every element."""
    from tests.full_compare import compare_variant_every_element
    _say("case mx deeper-half layer 0, every element")
    d = workloads.deeper_half_layer(device, 0)
    got = _gpu_mx(d["x_roll"], d["x_train"], d["grad"])
    ren = {"mask_g": "m_g", "mask_r": "m_r", "mask_f": "m_f"}
    got = {ren.get(k, k): v for k, v in got.items()}
    rows, cols = d["x_roll"].shape
    xr, xt, g = (to_np_u16(d[k]) for k in ("x_roll", "x_train", "grad"))
    compare_variant_every_element("mx deeper-half layer 0", "mx", xr, xt, got, extra="with_rne", g=g)
