"""Placement of training values relative to the rollout's FP4 grid, for the
KV-cache and large-hidden workloads (test infrastructure).

The per-block rollout scales come from the oracle; the random draws come
from ``workloads``; the arithmetic here (z = x/s, a target z, x_train =
bf16(s * z_target)) shapes inputs only.  Both the HIP path and the oracle
then consume the same x_train, and the achieved statistics are measured by
the oracle.
"""
import numpy as np
import torch

import oracle
import workloads

SIGNED_GRID = torch.tensor([-6, -4, -3, -2, -1.5, -1, -0.5, 0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=torch.float32)


def oracle_block_scales(x_roll_bf16):
    """Oracle tensor scale and per-block decoded scales (float32 numpy) of a
    device tensor."""
    xr = x_roll_bf16.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)
    ts = oracle.tensor_scale(xr)
    sb = oracle.block_scales(xr, ts)
    s, valid = oracle.decode_scales(sb, ts)
    return ts, np.where(valid, s, np.float32(np.nan)).astype(np.float32)


def _nearest_grid_index(z, chunk=1 << 24):
    grid = SIGNED_GRID.to(z.device)
    out = torch.empty(z.shape, dtype=torch.long, device=z.device)
    for i in range(0, z.numel(), chunk):
        seg = z[i:i + chunk]
        out[i:i + chunk] = (seg[:, None] - grid[None, :]).abs().argmin(dim=1)
    return out


def place_kv(x_roll, which, s_block):
    """~1% one-codeword straddles and ~0.01% two-codeword moves in z-space;
    all other sites keep x_train = x_roll."""
    dev = x_roll.device
    x = x_roll.float().reshape(-1)
    n = x.numel()
    d = workloads.kv_cache_perturbation_draws(dev, which, n)
    s = torch.from_numpy(s_block).to(dev).repeat_interleave(16)
    ok = torch.isfinite(s)
    z = torch.where(ok, x / torch.where(ok, s, torch.ones_like(s)), torch.zeros_like(x))
    k = _nearest_grid_index(z)
    grid = SIGNED_GRID.to(dev)
    step = torch.where(d["up"], 1, -1)
    k1 = k + step
    k1 = torch.where((k1 < 0) | (k1 > 14), k - step, k1)
    mid = 0.5 * (grid[k] + grid[k1])
    z1 = mid + d["u"] * (grid[k1] - mid)
    k2 = k + 2 * step
    k2 = torch.where((k2 < 0) | (k2 > 14), k - 2 * step, k2)
    gap = torch.minimum((grid[torch.clamp(k2 + 1, max=14)] - grid[k2]).abs().clamp(min=1e-9),
                       (grid[k2] - grid[torch.clamp(k2 - 1, min=0)]).abs().clamp(min=1e-9))
    z2 = grid[k2] + 0.2 * gap * d["w"]
    xt = x.clone()
    one = d["one"] & ok
    two = d["two"] & ok
    xt[one] = s[one] * z1[one]
    xt[two] = s[two] * z2[two]
    return xt.to(torch.bfloat16).reshape(x_roll.shape)


def place_near_midpoints(x_roll, s_block):
    """~50% of elements moved to within 1e-3 (in z) of the E2M1 midpoint
    nearest to their rollout value (then rounded to bf16); the rest keep
    x_train = x_roll."""
    dev = x_roll.device
    x = x_roll.float().reshape(-1)
    n = x.numel()
    d = workloads.large_hidden_draws(dev, n)
    s = torch.from_numpy(s_block).to(dev).repeat_interleave(16)
    ok = torch.isfinite(s)
    z = torch.where(ok, x / torch.where(ok, s, torch.ones_like(s)), torch.zeros_like(x))
    grid = SIGNED_GRID.to(dev)
    mids = 0.5 * (grid[1:] + grid[:-1])
    k = torch.bucketize(z.clamp(-6, 6), mids).clamp(max=13)   # nearest midpoint: candidates k-1, k
    km = torch.clamp(k - 1, min=0)
    take_lo = (z - mids[km]).abs() < (z - mids[k]).abs()
    m = torch.where(take_lo, mids[km], mids[k])
    xt = x.clone()
    sel = d["near"] & ok
    xt[sel] = s[sel] * (m[sel] + d["off"][sel])
    return xt.to(torch.bfloat16).reshape(x_roll.shape)
