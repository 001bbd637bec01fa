"""GPU parity of the b-cached-low-bits path (b = 1..4): capture's bit-planes
and the forward from them through the C ABI against ``oracle.capture_lowbits``
/ ``oracle.lowbits_fwd``, bit for bit, on ragged shapes with training
values far enough from the rollout's to cross several codewords, and
exhaustively over every bf16 x_train under every scale byte with random
residues; b = 1 and b = 4 also against the guided and full-information
kernels."""
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


def _bf16_np(v):
    return F.f32_to_bf16_rne(np.asarray(v, np.float32))


def _same(got, want, ctx):
    for k in want:
        a, b = np.asarray(got[k]).reshape(-1), np.asarray(want[k]).reshape(-1)
        assert a.shape == b.shape, (ctx, k)
        if not np.array_equal(a, b):
            bad = np.flatnonzero(a != b)
            raise AssertionError(f"{ctx}: {k} differs at {bad.size} of {b.size}; first {bad[:6].tolist()} "
                                 f"got {a[bad[:6]].tolist()} want {b[bad[:6]].tolist()}")


@pytest.mark.parametrize("nbits", [1, 2, 3, 4])
@pytest.mark.parametrize("shape", [(1, 16), (37, 48), (129, 4176), (256, 2048)])
def test_lowbits_bit_exact(device, nbits, shape):
    import fp4_rollout_guided_amd as tr
    _say("case lowbits", nbits, shape)
    rows, cols = shape
    rng = np.random.default_rng(nbits * 7919 + rows * 31 + cols)
    v = rng.standard_t(4, (rows, cols))
    v[:, rng.choice(cols, max(1, cols // 256), replace=False)] *= 40
    xr = _bf16_np(v.reshape(-1))
    xt = _bf16_np(F.bf16_to_f32(xr) * (1 + 0.4 * rng.standard_normal(xr.size)))  # multi-codeword moves
    xrd, xtd = from_np_u16(xr, device, shape), from_np_u16(xt, device, shape)
    ts = tr.tensor_scale(xrd)
    sc, pl, cd = tr.capture_lowbits(xrd, ts, nbits, want_codes=True)
    y, m, q = tr.lowbits_fakequant_fwd(xtd, sc, ts, nbits, pl, want_codes=True)
    torch.cuda.synchronize()
    tsf = np.float32(ts.cpu().numpy()[0])
    cap = oracle.capture_lowbits(xr, tsf, nbits)
    want = oracle.lowbits_fwd(xt, cap["scales"], tsf, cap["planes"], nbits)
    _same({"scales": to_np_u8(sc), "planes": to_np_u8(pl)}, cap, f"lowbits capture b={nbits} {shape}")
    _same({"codes": to_np_u8(cd)}, {"codes": oracle.capture(xr, tsf, with_codes=True)["codes"]}, "codes")
    _same({"y": to_np_u16(y), "mask": to_np_u8(m), "codes": to_np_u8(q)}, want, f"lowbits fwd b={nbits} {shape}")
    if nbits in (1, 4):
        if nbits == 1:
            yr, mr, qr = tr.guided_fakequant_fwd(xtd, sc, ts, pl, want_codes=True)
        else:
            yr, mr, qr = tr.full_info_fakequant_fwd(xtd, sc, ts, cd, want_codes=True)
        torch.cuda.synchronize()
        assert np.array_equal(to_np_u16(y), to_np_u16(yr)) and np.array_equal(to_np_u8(q), to_np_u8(qr))


@pytest.mark.parametrize("nbits", [2, 3, 4])
def test_lowbits_fwd_exhaustive(device, nbits):
    """Every bf16 pattern as x_train under every scale byte (tensor scale 1)
    with random residues: every (sign, bracket, residue) decision."""
    import fp4_rollout_guided_amd as tr
    _say("case lowbits exhaustive", nbits)
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = np.tile(pats, 256)
    scales = np.repeat(np.arange(256, dtype=np.uint32).astype(np.uint8), (1 << 16) // 16)
    rng = np.random.default_rng(100 + nbits)
    planes = rng.integers(0, 256, size=nbits * (x.size // 8), dtype=np.uint8)
    xd = from_np_u16(x, device, (x.size // 16, 16))
    sd, pd = torch.from_numpy(scales).to(device), torch.from_numpy(planes).to(device)
    tsd = torch.ones(1, dtype=torch.float32, device=device)
    y, m, q = tr.lowbits_fakequant_fwd(xd, sd, tsd, nbits, pd, want_codes=True)
    torch.cuda.synchronize()
    want = oracle.lowbits_fwd(x, scales, np.float32(1.0), planes, nbits)
    _same({"y": to_np_u16(y), "mask": to_np_u8(m), "codes": to_np_u8(q)}, want, f"lowbits exhaustive b={nbits}")
