"""Seeded synthetic inputs for the capture workloads.

Random draws only: this module holds no part of the quantizer's arithmetic
(no scales, no grid, no rounding rule).  Where a workload places training
values relative to the rollout's FP4 grid, this module supplies the raw
draws (which sites, which direction, where inside an interval) and the
caller combines them with scales it computed itself.

Every draw comes from a ``torch.Generator`` seeded from (workload, site,
layer, stream), on the device the caller names; the same call on the same
device type returns the same tensor.  Values are drawn in fp32, scaled, and
rounded to bf16 by PyTorch's round-to-nearest-even cast.

Workloads (sizes in elements, bf16):

0. one capture site 1024 x 2048, N(0,1) with 8 outlier channels x50;
   x_train = x_roll + N(0, (0.02 |x_roll|)^2); grad ~ N(0,1).
1. one MoE layer for 16384 tokens, hidden 2048: attention input 16384 x 2048,
   o_proj input 16384 x 4096, expert inputs 131072 x 2048 after seeded
   top-8-of-128 uniform routing (rows grouped by expert, then token), expert
   down_proj inputs 131072 x 768; Student-t(4) values.
2. KV cache for one layer at 131072 tokens: K and V each 131072 x 4 heads x
   128 head_dim, N(0,1), 2 outlier dims per head x20.
3. 20 captured layers (the deeper half of 40), each 262144 x 2048
   (64 trajectories x 4096 tokens), N(0,1) with 0.1% outlier channels x100.
4. 65573 x 7168 (65536 + 37 rows), Laplace(0,1), 16 outlier channels x200.
"""
import hashlib

import torch

SEED_BASE = 20261006

SHAPES = {
    0: {"x": (1024, 2048)},
    1: {"attn_in": (16384, 2048), "o_proj_in": (16384, 4096),
        "expert_in": (131072, 2048), "down_proj_in": (131072, 768)},
    2: {"k": (131072, 4, 128), "v": (131072, 4, 128)},
    3: {"x": (262144, 2048)},
    4: {"x": (65573, 7168)},
}
CFG3_LAYERS = 20
CFG3_TOTAL_LAYERS = 40
MOE_TOKENS, MOE_EXPERTS, MOE_TOPK = 16384, 128, 8


def generator(device, *key) -> torch.Generator:
    """Generator seeded from SEED_BASE and an integer/string key."""
    h = hashlib.sha256(repr((SEED_BASE,) + tuple(key)).encode()).digest()
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(int.from_bytes(h[:8], "little") & ((1 << 63) - 1))
    return g


def _dev(device):
    return torch.device(device)


def normal(shape, g, device):
    return torch.randn(shape, generator=g, device=_dev(device), dtype=torch.float32)


def uniform(shape, g, device):
    return torch.rand(shape, generator=g, device=_dev(device), dtype=torch.float32)


def exponential(shape, g, device):
    # -ln(1 - U), U in [0, 1): finite and >= 0
    return -torch.log1p(-uniform(shape, g, device))


def laplace(shape, g, device):
    return exponential(shape, g, device) - exponential(shape, g, device)


def student_t4(shape, g, device):
    # t_4 = N / sqrt(chi2_4 / 4), chi2_4 = 2 (E1 + E2)
    z = normal(shape, g, device)
    chi = exponential(shape, g, device) + exponential(shape, g, device)
    return z / torch.sqrt(torch.clamp(chi, min=1e-30) * 0.5)


def outlier_channels(cols, k, g, device):
    return torch.randperm(cols, generator=g, device=_dev(device))[:k]


def scale_channels(x, channels, factor):
    x[..., channels] *= factor
    return x


def bf16(x):
    return x.to(torch.bfloat16)


def relative_noise(x_bf16, sigma, g):
    """bf16(x + N(0, (sigma |x|)^2)) with x the fp32 value of x_bf16."""
    x = x_bf16.float()
    return bf16(x + sigma * x.abs() * normal(x.shape, g, x.device))


# ----------------------------------------------------------------------------
# single site (1024 x 2048)
# ----------------------------------------------------------------------------

def single_site(device):
    rows, cols = SHAPES[0]["x"]
    g = generator(device, 0, "x")
    x = normal((rows, cols), g, device)
    scale_channels(x, outlier_channels(cols, 8, g, device), 50.0)
    x_roll = bf16(x)
    x_train = relative_noise(x_roll, 0.02, generator(device, 0, "noise"))
    grad = bf16(normal((rows, cols), generator(device, 0, "grad"), device))
    return {"x_roll": x_roll, "x_train": x_train, "grad": grad}


# ----------------------------------------------------------------------------
# MoE layer; x_train is relative noise whose sigma the caller
# chooses (tuned so that ~3% of sites straddle an E2M1 midpoint)
# ----------------------------------------------------------------------------

def moe_routing(device):
    """Seeded top-8-of-128 routing of 16384 tokens from i.i.d. U(0,1) scores.
    Returns (token_of_row, expert_of_row) for the 131072 packed rows, grouped
    by expert and, inside an expert, by token."""
    g = generator(device, 1, "router")
    scores = uniform((MOE_TOKENS, MOE_EXPERTS), g, device)
    experts = torch.topk(scores, MOE_TOPK, dim=1).indices            # [T, 8]
    tokens = torch.arange(MOE_TOKENS, device=_dev(device)).repeat_interleave(MOE_TOPK)
    experts = experts.reshape(-1)
    order = torch.argsort(experts * MOE_TOKENS + tokens)
    return tokens[order], experts[order]


def moe_expert_offsets(expert_of_row):
    """Row offsets of the expert groups of packed rows sorted by expert:
    int64[experts + 1], group e = rows [off[e], off[e+1]) (empty experts give
    empty groups)."""
    counts = torch.bincount(expert_of_row, minlength=MOE_EXPERTS)
    return torch.cat([torch.zeros(1, dtype=torch.int64, device=counts.device), torch.cumsum(counts, 0)])


def trainer_order(rows, device):
    """The training side's row order for records read back from the
    rollout: a seeded random permutation of the rows (int64 on device)."""
    return torch.randperm(rows, generator=generator(device, "trainer order"), device=_dev(device))


def moe_layer(device, sigma, sites=None):
    """Dict site -> {x_roll, x_train, grad} for the MoE layer sites."""
    sites = sites or list(SHAPES[1])
    out = {}
    tok = None
    for site in sites:
        rows, cols = SHAPES[1][site]
        if site == "expert_in":
            if tok is None:
                tok, _ = moe_routing(device)
            h = bf16(student_t4((MOE_TOKENS, cols), generator(device, 1, "h"), device))
            h_train = relative_noise(h, sigma, generator(device, 1, "h", "noise"))
            x_roll, x_train = h[tok], h_train[tok]
        else:
            x_roll = bf16(student_t4((rows, cols), generator(device, 1, site), device))
            x_train = relative_noise(x_roll, sigma, generator(device, 1, site, "noise"))
        grad = bf16(normal((rows, cols), generator(device, 1, site, "grad"), device))
        out[site] = {"x_roll": x_roll.contiguous(), "x_train": x_train.contiguous(), "grad": grad}
    return out


# ----------------------------------------------------------------------------
# KV cache
# ----------------------------------------------------------------------------

def kv_cache_rollout(device, which):
    """K or V rollout tensor [131072, 4, 128]: N(0,1), per head 2 of 128
    dims scaled x20 (separate draws for K and V and for every head)."""
    tokens, heads, hd = SHAPES[2][which]
    g = generator(device, 2, which)
    x = normal((tokens, heads, hd), g, device)
    for h in range(heads):
        x[:, h, outlier_channels(hd, 2, g, device)] *= 20.0
    return bf16(x)


def kv_cache_perturbation_draws(device, which, n):
    """Raw draws for placing training values near the rollout grid:
    ``one`` / ``two`` = disjoint site masks of ~1% and ~0.01%, ``up`` = the
    direction (+1 / -1) of the neighbour to move toward, ``u`` in [0, 1) =
    where inside the target interval, ``w`` in [-1, 1) = jitter."""
    g = generator(device, 2, which, "place")
    r = uniform((n,), g, device)
    one = r < 0.01
    two = (r >= 0.01) & (r < 0.0101)
    up = uniform((n,), g, device) < 0.5
    u = uniform((n,), g, device)
    w = uniform((n,), g, device) * 2 - 1
    return {"one": one, "two": two, "up": up, "u": u, "w": w}


# ----------------------------------------------------------------------------
# deeper-half sweep, one layer per call
# ----------------------------------------------------------------------------

def deeper_half_layer(device, layer, with_grad=True):
    rows, cols = SHAPES[3]["x"]
    g = generator(device, 3, layer, "x")
    x = normal((rows, cols), g, device)
    k = round(0.001 * cols)   # 0.1% of 2048 channels -> 2
    scale_channels(x, outlier_channels(cols, k, g, device), 100.0)
    x_roll = bf16(x)
    del x
    x_train = relative_noise(x_roll, 0.02, generator(device, 3, layer, "noise"))
    out = {"x_roll": x_roll, "x_train": x_train}
    if with_grad:
        out["grad"] = bf16(normal((rows, cols), generator(device, 3, layer, "grad"), device))
    return out


# ----------------------------------------------------------------------------
# large hidden, ragged rows
# ----------------------------------------------------------------------------

def large_hidden_rollout(device):
    rows, cols = SHAPES[4]["x"]
    g = generator(device, 4, "x")
    x = laplace((rows, cols), g, device)
    scale_channels(x, outlier_channels(cols, 16, g, device), 200.0)
    return bf16(x)


def large_hidden_draws(device, n):
    """``near`` = the ~50% of elements placed near a codeword midpoint,
    ``off`` in [-1e-3, 1e-3) = their offset from it."""
    g = generator(device, 4, "place")
    near = uniform((n,), g, device) < 0.5
    off = (uniform((n,), g, device) * 2 - 1) * 1e-3
    return {"near": near, "off": off}


def grad_for(shape, device, *key):
    return bf16(normal(shape, generator(device, "grad", *key), device))
