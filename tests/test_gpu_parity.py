"""GPU parity: the HIP path (through the C ABI) against the oracle, element by
element, bit-exact, at sizes the oracle finishes in seconds.  Covers several
workgroup tiles and ragged tails, crafted special values, and exhaustive
sweeps over bf16 inputs and scale bytes."""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F
from tests.gpu_util import assert_same, from_np_u16, gpu_path, oracle_path, to_np_u8, to_np_u16

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _bf16_np(v):
    return F.f32_to_bf16_rne(np.asarray(v, np.float32))


def _rand_tensor(rng, rows, cols, kind="normal"):
    if kind == "normal":
        v = rng.standard_normal((rows, cols))
    elif kind == "t":
        v = rng.standard_t(4, (rows, cols))
    else:
        v = rng.laplace(size=(rows, cols))
    ch = rng.choice(cols, size=max(1, cols // 256), replace=False)
    v[:, ch] *= 60
    return _bf16_np(v)


def _run_both(xr, xt, g, shape, device, ts=None):
    got = gpu_path(from_np_u16(xr, device, shape), from_np_u16(xt, device, shape), from_np_u16(g, device, shape),
                   ts=None if ts is None else torch.tensor([ts], dtype=torch.float32, device=device))
    want = oracle_path(xr, xt, g, ts=ts)
    return got, want


@pytest.mark.parametrize("shape", [(1, 16), (37, 48), (3, 4112), (129, 4096 + 16 * 5), (17, 7168), (1024, 2048)])
def test_small_shapes_bit_exact(device, shape):
    _say("case small", shape)
    rng = np.random.default_rng(hash(shape) % 2**32)
    rows, cols = shape
    xr = _rand_tensor(rng, rows, cols, ["normal", "t", "laplace"][rows % 3]).reshape(-1)
    xt = _bf16_np(F.bf16_to_f32(xr) * (1 + 0.03 * rng.standard_normal(xr.size)))
    g = _bf16_np(rng.standard_normal(xr.size))
    got, want = _run_both(xr, xt, g, shape, device)
    assert_same(got, want, ctx=f"shape {shape}")


def _special_tensor():
    """Blocks of crafted values under tensor scale 1 (the tensor holds 2688)."""
    blocks = []
    ties = [6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0, 0.0]
    blocks.append(ties)                                             # exact midpoints, s = 1
    blocks.append([6.0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -1, -1.5, -2, -3, -4, -6, -0.0])  # codewords
    blocks.append([0.0] * 15 + [-0.0])                              # zero block (scale byte 0)
    blocks.append([float("nan"), 1.0, -2.0, 3.0] + [0.5] * 12)      # NaN ignored by the amax
    blocks.append([2688.0] + [1.0] * 15)                            # the tensor amax
    sub = [2.0 ** -133 * (k + 1) * (-1) ** k for k in range(16)]    # bf16 subnormals only
    blocks.append(sub)
    blocks.append([1e-30 * (k - 7.5) for k in range(16)])
    blocks.append([2688.0] + [-2688.0] + [1.0] * 14)               # top of the E4M3 range
    blocks.append([2.0 ** -6 * 6 * 1.0001] + [2.0 ** -9] * 15)      # E4M3 subnormal/normal boundary
    blocks.append([6.0 * 2.0 ** -10] + [1e-5] * 15)                 # v = 2^-10: tie to scale byte 0
    blocks.append([6.0 * 3 * 2.0 ** -10] + [-1e-5] * 15)            # v = 3*2^-10: tie to byte 2
    return _bf16_np(np.array(blocks, np.float64).reshape(-1))


def test_special_values_bit_exact(device):
    _say("case special values")
    xr = _special_tensor()
    rng = np.random.default_rng(5)
    xt = xr.copy()
    xt32 = F.bf16_to_f32(xt)
    xt32 = np.where(np.isfinite(xt32), xt32 * (1 + 0.1 * rng.standard_normal(xt.size)), xt32)
    xt = _bf16_np(xt32)
    # training-side specials: +-Inf, NaN, huge values, and exact copies of rollout ties
    xt[[3, 20, 50, 70]] = _bf16_np([np.inf, -np.inf, np.nan, -3e38])
    xt[:16] = xr[:16]
    g = _bf16_np(rng.standard_normal(xr.size))
    g[[1, 2]] = _bf16_np([np.nan, np.inf])
    shape = (xr.size // 16, 16)
    got, want = _run_both(xr, xt, g, shape, device)
    assert_same(got, want, ctx="special")
    # also with an infinite tensor scale (all blocks zero-scale) and ts = 0
    for ts in (0.5, 1.0, 2.0 ** -20, np.inf, 0.0, -1.0, np.nan):
        got, want = _run_both(xr, xt, g, shape, device, ts=np.float32(ts))
        assert_same(got, want, ctx=f"special ts={ts}")
    # a +-2^117 block under ts = 2^-20: scale byte 0x7E, |x| / s past the largest float
    big = _bf16_np([2.0 ** 117, -2.0 ** 117, 2.0 ** 117, -1.0] + [-2.0 ** 117] * 4 + [3.0, -0.0] + [2.0 ** 116] * 6)
    xr2, xt2, g2 = np.concatenate([xr, big]), np.concatenate([xt, big]), np.concatenate([g, g[:16]])
    got, want = _run_both(xr2, xt2, g2, (xr2.size // 16, 16), device, ts=np.float32(2.0 ** -20))
    # s = 448 * 2^-20: every quotient clips to +-6 (code 7 with the sign), -0 stays -0 (0x8)
    assert want["codes"][-8:].tolist() == [0xF7, 0xF7, 0xFF, 0xFF, 0x87, 0x77, 0x77, 0x77]
    assert_same(got, want, ctx="special +-2^117 block, ts=2^-20")


def test_tensor_scale_cases(device):
    import fp4_rollout_guided_amd as tr
    rng = np.random.default_rng(9)
    cases = {
        "normal": _bf16_np(rng.standard_normal(4096 * 37)),
        "nan_ignored": _bf16_np(np.r_[rng.standard_normal(4096), np.nan, -7.0, np.zeros(14)]),
        "inf": _bf16_np(np.r_[rng.standard_normal(64), -np.inf, np.zeros(15)]),
        "zeros": np.zeros(4096, np.uint16),
        "all_nan": _bf16_np(np.full(32, np.nan)),
        "subnormal": _bf16_np(np.full(16, 2.0 ** -130)),
        "big": _bf16_np(np.r_[3.3e38, np.zeros(15)]),
        "many_groups": _bf16_np(rng.standard_normal(4096 * 2100 + 16)),
    }
    for name, x in cases.items():
        _say("case tensor_scale", name)
        got = tr.tensor_scale(from_np_u16(x, device)).cpu().numpy().view(np.uint32)[0]
        want = np.float32(oracle.tensor_scale(x)).view(np.uint32)
        assert got == want, (name, hex(got), hex(want))
    empty = torch.empty(0, dtype=torch.bfloat16, device=device)
    out = torch.full((1,), 7.0, device=device)
    tr.tensor_scale(empty, out=out)
    assert out.item() == 0.0


@pytest.mark.parametrize("ts", [1.0, 0.0123456, 3.0e-39, 1.0e30, 2.0 ** -100, 146.0, 2.0 ** -90])
def test_fwd_exhaustive_bf16_by_scale_byte(device, ts):
    """Every bf16 pattern as x_train under every scale byte (0x00..0xFF),
    for guided (random cached bits), RNE and full-information (random
    rollout codes) forward."""
    import fp4_rollout_guided_amd as tr
    _say("case exhaustive fwd ts", ts)
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = np.tile(pats, 256)
    scales = np.repeat(np.arange(256, dtype=np.uint32).astype(np.uint8), (1 << 16) // 16)
    rng = np.random.default_rng(int(ts * 1000) % 2**31)
    bits = rng.integers(0, 256, size=x.size // 8, dtype=np.uint8)
    tsf = np.float32(ts)
    xd = from_np_u16(x, device, (x.size // 16, 16))
    sd = torch.from_numpy(scales).to(device)
    bd = torch.from_numpy(bits).to(device)
    tsd = torch.tensor([tsf], dtype=torch.float32, device=device)
    yg, mg, qg = tr.guided_fakequant_fwd(xd, sd, tsd, bd, want_codes=True)
    yr, mr, qr = tr.rne_fakequant_fwd(xd, sd, tsd, want_codes=True)
    torch.cuda.synchronize()
    roll = rng.integers(0, 256, size=x.size // 2, dtype=np.uint8)   # every rollout code, both nibbles
    yf, mf, qf = tr.full_info_fakequant_fwd(xd, sd, tsd, torch.from_numpy(roll).to(device), want_codes=True)
    torch.cuda.synchronize()
    wg = oracle.guided_fwd(x, scales, tsf, bits)
    wr = oracle.rne_fwd(x, scales, tsf)
    wf = oracle.full_info_fwd(x, scales, tsf, roll)
    assert_same({"y": to_np_u16(yg), "mask": to_np_u8(mg), "codes": to_np_u8(qg)}, wg, ctx=f"guided ts={ts}")
    assert_same({"y": to_np_u16(yr), "mask": to_np_u8(mr), "codes": to_np_u8(qr)}, wr, ctx=f"rne ts={ts}")
    assert_same({"y": to_np_u16(yf), "mask": to_np_u8(mf), "codes": to_np_u8(qf)}, wf, ctx=f"full ts={ts}")


@pytest.mark.parametrize("ts", [1.0, 0.0123456, 7.5e-37, 1.0e30, 2.0 ** -20, 2.0 ** -60])
def test_capture_exhaustive_block_amax(device, ts):
    """Block maxima over every finite positive bf16 magnitude (plus Inf and
    NaN blocks), the other 15 elements random fractions of the maximum,
    under an explicit tensor scale: exercises every scale-byte path.  Under
    2^-20 and 2^-60 the largest maxima saturate the scale byte and their
    quotients pass the largest float (codes +-7)."""
    import fp4_rollout_guided_amd as tr
    _say("case capture amax sweep ts", ts)
    rng = np.random.default_rng(42)
    mags = F.bf16_to_f32(np.arange(1, 0x7F81, dtype=np.uint16)).astype(np.float64)  # incl. +Inf
    nb = mags.size
    frac = rng.uniform(-1, 1, size=(nb, 15))
    blocks = np.concatenate([mags[:, None] * np.where(rng.random((nb, 1)) < 0.5, 1, -1), mags[:, None] * frac], axis=1)
    blocks = np.where(np.isfinite(blocks), blocks, np.where(np.isinf(blocks) & (np.arange(16) > 0), 0.0, blocks))
    xr = _bf16_np(blocks.reshape(-1))
    xr[rng.choice(xr.size, 64, replace=False)] = 0x7FC1  # NaN elements here and there
    tsf = np.float32(ts)
    xd = from_np_u16(xr, device, (nb, 16))
    tsd = torch.tensor([tsf], dtype=torch.float32, device=device)
    scales, bits, codes = tr.capture(xd, tsd, want_codes=True)
    torch.cuda.synchronize()
    want = oracle.capture(xr, tsf, with_codes=True)
    assert_same({"scales": to_np_u8(scales), "bits": to_np_u8(bits), "codes": to_np_u8(codes)}, want,
                ctx=f"capture ts={ts}")


@pytest.mark.parametrize("ts", [1.0, 146.0, 2.0 ** -88, 0.0123456])
def test_tiny_elements_beside_large_ones(device, ts):
    """Blocks holding one large element (setting the block scale anywhere in
    the E4M3 range) and otherwise bf16 subnormals, tiny normals, signed zeros
    and small values: capture codes and guided / RNE outputs keep the sign
    and the zero-ness of every tiny quotient."""
    import fp4_rollout_guided_amd as tr
    _say("case tiny elements ts", ts)
    rng = np.random.default_rng(77)
    tsf = np.float32(ts)
    dec = F.E4M3FN_VALUES[1:0x7F]
    big = np.repeat(6.0 * dec * float(tsf), 64)
    nb = big.size
    tiny_pool = np.concatenate([
        F.bf16_to_f32(np.arange(1, 0x80, dtype=np.uint16)).astype(np.float64),      # subnormals
        2.0 ** rng.uniform(-126, -96, 400),                                           # tiny normals
        np.array([0.0, -0.0]),
        rng.standard_normal(200) * float(tsf)])
    rest = rng.choice(tiny_pool, size=(nb, 15)) * np.where(rng.random((nb, 15)) < 0.5, -1, 1)
    blocks = np.concatenate([big[:, None] * np.where(rng.random((nb, 1)) < 0.5, -1, 1), rest], axis=1)
    xr = _bf16_np(blocks.reshape(-1))
    xt = xr.copy()
    flip = rng.random(xt.size) < 0.3
    xt[flip] = _bf16_np(F.bf16_to_f32(xt[flip]) * (1 + 0.3 * rng.standard_normal(flip.sum())))
    g = _bf16_np(rng.standard_normal(xr.size))
    shape = (nb, 16)
    got = gpu_path(from_np_u16(xr, device, shape), from_np_u16(xt, device, shape), from_np_u16(g, device, shape),
                   ts=torch.tensor([tsf], dtype=torch.float32, device=device))
    want = oracle_path(xr, xt, g, ts=tsf)
    assert_same(got, want, ctx=f"tiny ts={ts}")


@pytest.mark.parametrize("build", ["production", "small-grid"])
def test_in_place_and_guard_bytes(device, build):
    """y written over x_train and grad_in over grad_out give the same bytes
    as separate buffers; bytes around every output stay untouched.  Also
    through the small-grid build, whose kernels loop over their grids and
    stream every tensor with the non-temporal hint (production does past
    256 MiB)."""
    import fp4_rollout_guided_amd as tr
    _say("case in-place + guards", build)
    saved = tr.lib
    if build == "small-grid":
        tr.lib = tr.load_library(tr.SMALLGRID_LIB_PATH)
    try:
        _in_place_and_guard_bytes(tr, device)
    finally:
        tr.lib = saved


def _in_place_and_guard_bytes(tr, device):
    rng = np.random.default_rng(3)
    rows, cols = 300, 2064
    n = rows * cols
    xr = _rand_tensor(rng, rows, cols).reshape(-1)
    xt = _bf16_np(F.bf16_to_f32(xr) * (1 + 0.03 * rng.standard_normal(n)))
    g = _bf16_np(rng.standard_normal(n))
    want = oracle_path(xr, xt, g)
    G = 256  # guard bytes on each side

    def guarded_u8(nbytes):
        buf = torch.full((nbytes + 2 * G,), 0xA5, dtype=torch.uint8, device=device)
        return buf, buf[G:G + nbytes]

    def guarded_bf16(count):
        buf = torch.full((count + G,), -23131, dtype=torch.int16, device=device)  # 0xA5A5
        return buf, buf[G // 2:G // 2 + count].view(torch.bfloat16)

    xr_d = from_np_u16(xr, device, (rows, cols))
    ts = tr.tensor_scale(xr_d)
    sc_buf, sc = guarded_u8(n // 16)
    bt_buf, bt = guarded_u8(n // 8)
    cd_buf, cd = guarded_u8(n // 2)
    tr.capture(xr_d, ts, scales=sc, bits=bt, codes=cd)
    xt_buf, xt_d = guarded_bf16(n)
    xt_d.copy_(from_np_u16(xt, device))
    mk_buf, mk = guarded_u8(n // 8)
    tr.guided_fakequant_fwd(xt_d.view(rows, cols), sc, ts, bt, y=xt_d.view(rows, cols), mask=mk)  # in place
    g_buf, g_d = guarded_bf16(n)
    g_d.copy_(from_np_u16(g, device))
    tr.ste_bwd(g_d, mk, grad_in=g_d)  # in place
    torch.cuda.synchronize()
    assert np.array_equal(to_np_u8(sc), want["scales"])
    assert np.array_equal(to_np_u8(bt), want["bits"])
    assert np.array_equal(to_np_u8(cd), want["codes"])
    assert np.array_equal(to_np_u16(xt_d), want["y_g"])
    assert np.array_equal(to_np_u8(mk), want["mask_g"])
    assert np.array_equal(to_np_u16(g_d), want["gin"])
    for name, buf, inner in (("scales", sc_buf, n // 16), ("bits", bt_buf, n // 8), ("codes", cd_buf, n // 2),
                             ("mask", mk_buf, n // 8)):
        h = to_np_u8(buf)
        assert np.all(h[:G] == 0xA5) and np.all(h[G + inner:] == 0xA5), name
    for name, buf in (("y", xt_buf), ("grad_in", g_buf)):
        h = buf.cpu().numpy().view(np.uint16)
        assert np.all(h[:G // 2] == 0xA5A5) and np.all(h[G // 2 + n:] == 0xA5A5), name


def test_autograd_wrapper(device):
    import fp4_rollout_guided_amd as tr
    rng = np.random.default_rng(11)
    rows, cols = 64, 256
    xr = _rand_tensor(rng, rows, cols).reshape(-1)
    xt = _bf16_np(F.bf16_to_f32(xr) * 1.05)
    g = _bf16_np(rng.standard_normal(xr.size))
    want = oracle_path(xr, xt, g)
    xr_d = from_np_u16(xr, device, (rows, cols))
    ts = tr.tensor_scale(xr_d)
    sc, bt, _ = tr.capture(xr_d, ts)
    x = from_np_u16(xt, device, (rows, cols)).requires_grad_(True)
    y = tr.GuidedFakeQuant.apply(x, sc, ts, bt)
    y.backward(from_np_u16(g, device, (rows, cols)))
    assert np.array_equal(to_np_u16(y.detach()), want["y_g"])
    assert np.array_equal(to_np_u16(x.grad), want["gin"])


@pytest.mark.parametrize("tiles", [2047, 2048, 2049, 4096 + 5, 6143])
def test_ste_bwd_tile_runs(device, tiles):
    """The STE backward hands tiles (256 vectors of 8 elements) to the XCDs in
    runs once its grid holds a whole group of 8 x 256 workgroups; a partial
    last group keeps dispatch order.  Grids just below, at and past whole
    groups, with a ragged last tile: every element against the oracle."""
    import fp4_rollout_guided_amd as tr
    nvec = 256 * tiles - 2                  # 8-element vectors; the last tile is ragged
    n = 8 * nvec                            # a multiple of 16 (nvec is even)
    _say("case ste tile runs", tiles, n)
    rng = np.random.default_rng(tiles)
    grad = rng.integers(0, 1 << 16, n, dtype=np.uint16)
    mask = rng.integers(0, 256, n // 8, dtype=np.uint8)
    gin = tr.ste_bwd(from_np_u16(grad, device, (1, n)), torch.from_numpy(mask).to(device))
    torch.cuda.synchronize()
    assert np.array_equal(to_np_u16(gin), oracle.ste_bwd(grad, mask, n)), tiles
