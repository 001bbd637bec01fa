"""Tune the relative noise of the MoE-layer workload so that ~3% of sites
straddle an E2M1 midpoint, and store it in moe_layer_sigma.json.

    python tests/golden/make_moe_layer_sigma.py

A site straddles when its rollout codeword and the training value's RNE
codeword differ and the rollout codeword is an endpoint of the training
value's bracket (the post's rounding-boundary example).  The rate is
measured by the oracle on a CPU-generated sample of the attention-input site
(Student-t(4) values); x_train = bf16(x_roll + sigma |x_roll| N(0,1)).
Bisection on sigma; only the oracle and the seeded generators are used.
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402
import torch  # noqa: E402

import oracle  # noqa: E402
import workloads  # noqa: E402

TARGET = 0.03
ROWS = 256


def straddle_rate(x_roll_t, sigma):
    x_train_t = workloads.relative_noise(x_roll_t, sigma, workloads.generator("cpu", "tune", sigma))
    xr = x_roll_t.view(torch.int16).numpy().view(np.uint16).reshape(-1)
    xt = x_train_t.view(torch.int16).numpy().view(np.uint16).reshape(-1)
    ts = oracle.tensor_scale(xr)
    cap = oracle.capture(xr, ts, with_codes=True)
    st = oracle.mismatch_stats(xt, cap["scales"], ts, cap["codes"], cap["bits"])
    return st["straddle"] / st["n"], st


def main():
    rows, cols = workloads.SHAPES[1]["attn_in"]
    x = workloads.bf16(workloads.student_t4((rows, cols), workloads.generator("cpu", 1, "attn_in"), "cpu"))
    sample = x[:ROWS].contiguous()
    lo, hi = 0.0, 0.2
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        r, _ = straddle_rate(sample, mid)
        if r < TARGET:
            lo = mid
        else:
            hi = mid
    sigma = round(0.5 * (lo + hi), 6)
    rate, st = straddle_rate(sample, sigma)
    out = {
        "sigma": sigma,
        "target_straddle_rate": TARGET,
        "straddle_rate_on_tuning_sample": rate,
        "tuning_sample": f"first {ROWS} rows of the attention-input site (Student-t(4), 16384x2048), CPU generator",
        "mismatch_histogram_on_tuning_sample": st["hist"][:5],
        "written_by": "tests/golden/make_moe_layer_sigma.py (oracle + workloads only)",
    }
    with open(os.path.join(HERE, "moe_layer_sigma.json"), "w") as fh:
        json.dump(out, fh, indent=2)
    print(json.dumps(out, indent=2))


if __name__ == "__main__":
    main()
