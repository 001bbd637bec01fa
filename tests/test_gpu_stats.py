"""GPU parity of the agreement statistics (``trace_mismatch_stats``) with
``oracle.mismatch_stats``: every count exact (histogram of signed steps,
straddle, crossed, recovered, violations, elements) on ragged shapes, on
crafted specials with NaN / zero scale bytes and rollout codes of every
kind, with cached bits that do and do not match the rollout codes, and on
every bf16 pattern under every scale byte; calls accumulate and an empty
tensor adds nothing."""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F
from tests.gpu_util import from_np_u16
from tests.test_oracle_twin import _tiny_tensor

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _want(st):
    return st["hist"] + [st["straddle"], st["crossed"], st["recovered"], st["violations"], st["n"]]


def _gpu(xt, shape, scales, ts, roll, cbits, device, stats=None):
    import fp4_rollout_guided_amd as tr
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    out = tr.mismatch_stats(from_np_u16(xt, device, shape), dev(scales), dev(np.array([ts], np.float32)),
                            dev(oracle.pack_bits(cbits.astype(np.uint8))), dev(oracle.pack_nibbles(roll)), stats)
    torch.cuda.synchronize()
    return out.cpu().numpy().tolist()


def _case(rng, rows, cols, noise, flip_frac, consistent):
    v = rng.standard_t(4, (rows, cols))
    v[:, rng.choice(cols, max(1, cols // 256), replace=False)] *= 60
    xr = F.f32_to_bf16_rne(v.reshape(-1).astype(np.float32))
    xt = F.f32_to_bf16_rne((F.bf16_to_f32(xr) * (1 + noise * rng.standard_normal(xr.size))).astype(np.float32))
    ts = oracle.tensor_scale(xr)
    cap = oracle.capture(xr, ts, with_codes=True)
    n = xr.size
    roll = oracle.unpack_nibbles(cap["codes"], n).copy()
    flip = rng.random(n) < flip_frac
    roll[flip] = rng.integers(0, 16, flip.sum())
    cbits = (roll & 1) if consistent else rng.integers(0, 2, n)
    return xt, cap["scales"], ts, roll, cbits


@pytest.mark.parametrize("shape,consistent", [((1, 16), True), ((37, 48), True), ((129, 4176), True),
                                              ((17, 7168), False), ((1024, 2048), True)])
def test_stats_small_shapes(device, shape, consistent):
    _say("case stats", shape, consistent)
    rng = np.random.default_rng(shape[0] * 31 + shape[1])
    xt, scales, ts, roll, cbits = _case(rng, *shape, noise=0.05, flip_frac=0.02, consistent=consistent)
    want = _want(oracle.mismatch_stats(xt, scales, ts, oracle.pack_nibbles(roll),
                                       oracle.pack_bits(cbits.astype(np.uint8))))
    assert _gpu(xt, shape, scales, ts, roll, cbits, device) == want


def _step_codes(rng, roll, frac):
    """Move a fraction of the codes one signed grid step up or down (either
    zero for index 0), so that rollout and training codes sit one step apart."""
    out = roll.copy()
    pick = np.flatnonzero(rng.random(roll.size) < frac)
    m = (roll[pick] & 7).astype(np.int16)
    si = np.where(roll[pick] & 8, -m, m) + rng.choice(np.array([-1, 1], np.int16), pick.size)
    si = np.clip(si, -7, 7)
    zero_sign = rng.integers(0, 2, pick.size).astype(np.uint8) << 3
    out[pick] = np.where(si < 0, 8 | (-si), np.where(si == 0, zero_sign, si)).astype(np.uint8)
    return out


@pytest.mark.parametrize("consistent", [True, False])
def test_stats_one_step_neighbours(device, consistent):
    """Rollout codes one step from the training side's on 5% of the sites (the
    nibble-parallel path: up, down, through zero), with cached bits from the
    rollout codes or random (guided moving toward or away from the rollout)."""
    _say("case stats one-step", consistent)
    rng = np.random.default_rng(11 + consistent)
    rows, cols = 96, 2048
    v = rng.standard_t(4, (rows, cols)) * 0.5
    xr = F.f32_to_bf16_rne(v.reshape(-1).astype(np.float32))
    ts = oracle.tensor_scale(xr)
    cap = oracle.capture(xr, ts, with_codes=True)
    roll = _step_codes(rng, oracle.unpack_nibbles(cap["codes"], xr.size), 0.05)
    cbits = (roll & 1) if consistent else rng.integers(0, 2, xr.size)
    st = oracle.mismatch_stats(xr, cap["scales"], ts, oracle.pack_nibbles(roll), oracle.pack_bits(cbits.astype(np.uint8)))
    assert st["hist"][1] > 1000 and (consistent or st["violations"] > 1000)
    assert _gpu(xr, (rows, cols), cap["scales"], ts, roll, cbits, device) == _want(st)


def test_stats_specials(device):
    """Crafted blocks (NaN, infinities, zeros, subnormals, huge values) with
    NaN and zero scale bytes and random rollout codes on 30% of the sites."""
    _say("case stats specials")
    rng = np.random.default_rng(5)
    xr = np.concatenate([_tiny_tensor(rng) for _ in range(16)])
    xr32 = F.bf16_to_f32(xr)
    with np.errstate(over="ignore"):
        xt = F.f32_to_bf16_rne(np.where(np.isfinite(xr32), xr32 * (1 + 0.2 * rng.standard_normal(xr.size)),
                                        xr32).astype(np.float32))
    ts = oracle.tensor_scale(xr)
    cap = oracle.capture(xr, ts, with_codes=True)
    scales = cap["scales"].copy()
    scales[rng.choice(scales.size, 12, replace=False)] = rng.choice([0x00, 0x7F, 0x80, 0xFF], 12)
    n = xt.size
    roll = oracle.unpack_nibbles(cap["codes"], n).copy()
    flip = rng.random(n) < 0.3
    roll[flip] = rng.integers(0, 16, flip.sum())
    for consistent in (True, False):
        cbits = (roll & 1) if consistent else rng.integers(0, 2, n)
        want = _want(oracle.mismatch_stats(xt, scales, ts, oracle.pack_nibbles(roll),
                                           oracle.pack_bits(cbits.astype(np.uint8))))
        assert _gpu(xt, (n // 64, 64), scales, ts, roll, cbits, device) == want, consistent


def test_stats_exhaustive_bf16_by_scale_byte(device):
    """Every bf16 pattern as x_train under every scale byte (ts = 1), random
    rollout codes and cached bits."""
    _say("case stats exhaustive")
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = np.tile(pats, 256)
    scales = np.repeat(np.arange(256, dtype=np.uint32).astype(np.uint8), (1 << 16) // 16)
    rng = np.random.default_rng(6)
    roll = rng.integers(0, 16, x.size).astype(np.uint8)
    cbits = rng.integers(0, 2, x.size)
    want = _want(oracle.mismatch_stats(x, scales, np.float32(1), oracle.pack_nibbles(roll),
                                       oracle.pack_bits(cbits.astype(np.uint8))))
    assert _gpu(x, (x.size // 4096, 4096), scales, 1.0, roll, cbits, device) == want


def test_stats_accumulate_and_empty(device):
    import fp4_rollout_guided_amd as tr
    _say("case stats accumulate")
    rng = np.random.default_rng(7)
    xt, scales, ts, roll, cbits = _case(rng, 64, 256, noise=0.05, flip_frac=0.05, consistent=True)
    once = _gpu(xt, (64, 256), scales, ts, roll, cbits, device)
    acc = torch.zeros(20, dtype=torch.int64, device=device)
    _gpu(xt, (64, 256), scales, ts, roll, cbits, device, stats=acc)
    twice = _gpu(xt, (64, 256), scales, ts, roll, cbits, device, stats=acc)
    assert twice == [2 * v for v in once]
    empty = torch.empty(0, 256, dtype=torch.bfloat16, device=device)
    e8 = torch.empty(0, dtype=torch.uint8, device=device)
    tr.mismatch_stats(empty, e8, torch.ones(1, device=device), e8, e8, stats=acc)
    torch.cuda.synchronize()
    assert acc.cpu().numpy().tolist() == twice
