#!/usr/bin/env python3
"""Throughput of the rollout-guided FP4 rounding path on one MI355X.

Workload: the deeper-half capture sweep -- 20 captured layers (of 40), each
one bf16 site of 262144 x 2048 (64 trajectories x 4096 tokens), Gaussian with
0.1% outlier channels x100, x_train = x_roll + N(0, (0.02|x_roll|)^2),
grad ~ N(0, 1).  All 20 layers' inputs are generated on the GPU and resident
in HBM (distinct 1 GiB buffers, far larger than the 256 MB last-level cache)
before timing starts.

One step = the rollout side over every layer (tensor scale, i.e. the amax
pass, then capture: scale bytes + parity bit-plane), then the training side
over every layer (guided fake-quant forward: y + clip mask, plain RNE
fake-quant forward: y + clip mask, STE backward), the order of an RL step's
rollout and training phases.  A HIP event
marker on the kernels' stream sits before the first kernel and after every
kernel, so each kernel is timed between the markers around it; the step's
wall time is taken between device synchronizations.  After the timed steps, a separate
pass times the rows beyond the hot path (capture with full 4-bit codes, the
full-information forward, MXFP4 capture and guided forward, and capture to
and forward from b = 3 cached low bits, on the same layers) and reports them
under ``next_rows``; another
times the per-expert (grouped) tensor scale, capture and guided forward and
the record gather, and the forwards on records read back in a shuffled row
order, on the packed routed-expert site of the MoE layer workload
(``moe_expert_site``); ``kernels_cold`` times one layer's tensor scale and
capture after a read-only pass; a last one runs the step's kernels on the sites of
the other workloads, cold and repeated (``other_workloads``).

Prints one JSON line (last line of stdout).  ``value`` is the algorithmic
bytes of the whole step divided by its wall time, in GB/s; per-kernel GB/s,
Gelem/s and the fraction of the 8 TB/s HBM peak are reported beside it, with
the CPU oracle timed on a bounded sample of the same workload and, under
``practical_ceiling``, the GB/s of a plain copy, the same copy with
non-temporal loads and stores, a read-only and a write-only stream on the
same GPU, and of plain copies of 12 to 192 MiB (``bench_ceiling.hip``).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GB/s and Gelem/s for capture + guided fakequant fwd/bwd; % of HBM peak"
HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, AMD specification
LAYERS, TOTAL_LAYERS = 20, 40
ROWS, COLS = 262144, 2048
# Algorithmic bytes per element each kernel must move (reads + writes).
BYTES_PER_ELEM = {
    "tensor_scale": 2.0,                       # read x
    "capture": 2.0 + 1 / 8 + 1 / 16,           # read x; write bits + scale bytes
    "guided_fwd": 2.0 + 1 / 8 + 1 / 16 + 2.0 + 1 / 8,  # read x, bits, scales; write y, mask
    "rne_fwd": 2.0 + 1 / 16 + 2.0 + 1 / 8,     # read x, scales; write y, mask
    "ste_bwd": 2.0 + 1 / 8 + 2.0,              # read grad, mask; write grad_in
}
KERNELS = list(BYTES_PER_ELEM)
# Rows beyond the hot path, timed in a separate pass after the step.
NEXT_BYTES_PER_ELEM = {
    "capture_codes": 2.0 + 1 / 8 + 1 / 16 + 1 / 2,        # capture that also writes the 4-bit codes
    "full_info_fwd": 2.0 + 1 / 16 + 1 / 2 + 2.0 + 1 / 8,  # read x, scales, codes; write y, mask
    "mismatch_stats": 2.0 + 1 / 16 + 1 / 8 + 1 / 2,       # agreement statistics: read x_train, scales, bits, codes
    "mx_capture": 2.0 + 1 / 8 + 1 / 32,                   # MXFP4: read x; write bits + E8M0 scale bytes
    "mx_guided_fwd": 2.0 + 1 / 8 + 1 / 32 + 2.0 + 1 / 8,  # MXFP4: read x, bits, scales; write y, mask
    "mx8_capture": 2.0 + 1 / 8 + 1 / 32,                  # MXFP8 (E4M3): read x; write bits + E8M0 scale bytes
    "mx8_guided_fwd": 2.0 + 1 / 8 + 1 / 32 + 2.0 + 1 / 8, # MXFP8: read x, bits, scales; write y, mask
    "capture_lowbits3": 2.0 + 3 / 8 + 1 / 16,             # b = 3 cached low bits: three bit-planes
    "lowbits3_fwd": 2.0 + 3 / 8 + 1 / 16 + 2.0 + 1 / 8,   # forward from three bit-planes
}
# Per-expert rows on the packed routed-expert site of the MoE layer workload
# (131072 x 2048, rows grouped by 128 experts), timed in their own pass.
MOE_BYTES_PER_ELEM = {
    "grouped_tensor_scale": 2.0,                                   # read x (+ one word per row)
    "grouped_capture": 2.0 + 1 / 8 + 1 / 16,
    "grouped_guided_fwd": 2.0 + 1 / 8 + 1 / 16 + 2.0 + 1 / 8,
    "gather_records": 2 * (1 / 8 + 1 / 16),                        # read + write bits and scale bytes
    "gather_records_runs": 2 * (1 / 8 + 1 / 16),                   # the same, rows moved in runs
}
# records read back in the trainer's (shuffled) row order, then the guided
# forward: the gather and the forward as two launches, against one fused
# launch that reads the record rows in place (one tensor scale, and
# per-expert scales, which only the fused call can apply in that order)
READBACK_BYTES_PER_ELEM = {
    "gather_then_guided_fwd": 2 * (1 / 8 + 1 / 16) + 2.0 + 1 / 8 + 1 / 16 + 2.0 + 1 / 8,
    "fused_guided_fwd": 2.0 + 1 / 8 + 1 / 16 + 2.0 + 1 / 8,
    "fused_guided_fwd_per_expert": 2.0 + 1 / 8 + 1 / 16 + 2.0 + 1 / 8,
}
GATHER_RUN = 256         # rows per run in the run-ordered gather
MOE_REPS, MOE_WARM_S = 8, 0.1  # timed reps of the routed-expert site rows, after this long of untimed ones
CPU_SHARE = 16           # host cores granted to a process driving one GPU
CPU_BUDGET_S = 12.0      # wall-clock budget of the CPU oracle leg
CHUNK_ROWS = 128


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------
# CPU oracle leg (runs in worker processes started before the GPU is touched)
# ----------------------------------------------------------------------------

def _oracle_chunk(args):
    import numpy as np
    import oracle
    xr, xt, g, ts = args
    t0 = time.perf_counter()
    oracle.tensor_scale(xr)                      # the amax pass over this chunk
    cap = oracle.capture(xr, ts)
    gd = oracle.guided_fwd(xt, cap["scales"], ts, cap["bits"])
    rn = oracle.rne_fwd(xt, cap["scales"], ts)
    gin = oracle.ste_bwd(g, gd["mask"], xt.size)
    dt = time.perf_counter() - t0
    return dt, {"scales": cap["scales"], "bits": cap["bits"], "y_g": gd["y"], "mask_g": gd["mask"],
                "y_r": rn["y"], "mask_r": rn["mask"], "gin": gin}


def make_pool():
    import multiprocessing as mp
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    cores = max(1, min(cores, CPU_SHARE))
    ctx = mp.get_context("forkserver")
    pool = ctx.Pool(cores)
    pool.map(_noop, range(cores))   # start every worker now, before any GPU call
    return pool, cores


def _noop(_):
    import numpy  # noqa: F401
    import oracle  # noqa: F401
    return 0


# ----------------------------------------------------------------------------
# GPU leg
# ----------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--layers", type=int, default=LAYERS, help=argparse.SUPPRESS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB bf16 device copy (reference kernel for HBM byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this library's path runs on a single MI355X and has no "
              "multi-GPU mode (every 16-element block is independent; a sharded tensor would need one "
              "all-reduce(max) of its tensor amax, which this library does not implement). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy()
        return
    pool, cores = (None, 0) if args.no_cpu_baseline else make_pool()

    import numpy as np
    import torch

    import fp4_rollout_guided_amd as tr
    import workloads

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    L = args.layers
    n = ROWS * COLS
    log(f"generating {L} layers of {ROWS}x{COLS} bf16 on {torch.cuda.get_device_name(dev)}")
    layers = []
    for l in range(L):
        d = workloads.deeper_half_layer(dev, l)
        d["scales"] = torch.empty(n // 16, dtype=torch.uint8, device=dev)
        d["bits"] = torch.empty(n // 8, dtype=torch.uint8, device=dev)
        d["ts"] = torch.empty(1, dtype=torch.float32, device=dev)
        layers.append(d)
    y_g = torch.empty(ROWS, COLS, dtype=torch.bfloat16, device=dev)
    y_r = torch.empty_like(y_g)
    gin = torch.empty_like(y_g)
    mask_g = torch.empty(n // 8, dtype=torch.uint8, device=dev)
    mask_r = torch.empty_like(mask_g)
    ws = torch.empty(tr.lib.trace_tensor_scale_workspace_bytes(n), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)

    # An RL step runs the rollout (which captures every layer's site) and then
    # the training pass (which reads every layer's record back), so a step
    # here is the rollout side over all layers, then the training side over
    # all layers.  STEP_ORDER names the kernel of each launch in that order.
    STEP_ORDER = ["tensor_scale", "capture"] * L + ["guided_fwd", "rne_fwd", "ste_bwd"] * L

    def step(markers=None):
        """One pass over all layers.  markers: None, or len(STEP_ORDER) + 1
        timing events, recorded before the first kernel and after every
        kernel (one shared marker between consecutive kernels: a kernel's
        duration is the time between the markers around it; two markers per
        kernel would add a second queue barrier per launch)."""
        it = iter(markers) if markers is not None else None

        def mark():
            if it is not None:
                next(it).record(stream)
        mark()
        for d in layers:  # rollout side
            tr.tensor_scale(d["x_roll"], out=d["ts"], workspace=ws)
            mark()
            tr.capture(d["x_roll"], d["ts"], scales=d["scales"], bits=d["bits"])
            mark()
        for d in layers:  # training side
            tr.guided_fakequant_fwd(d["x_train"], d["scales"], d["ts"], d["bits"], y=y_g, mask=mask_g)
            mark()
            tr.rne_fakequant_fwd(d["x_train"], d["scales"], d["ts"], y=y_r, mask=mask_r)
            mark()
            tr.ste_bwd(d["grad"], mask_g, grad_in=gin)
            mark()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    per_kernel_ms = {k: 0.0 for k in KERNELS}
    # every step records its own markers, so the steps run back to back with
    # no host synchronization between them; the markers are read after the
    # timed region
    markers = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STEP_ORDER) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(markers[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for m in markers:
        for i, k in enumerate(STEP_ORDER):
            per_kernel_ms[k] += m[i].elapsed_time(m[i + 1])
    ms_per_step = 1e3 * wall / args.steps
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step")

    launches = args.steps * L
    bytes_step = L * n * sum(BYTES_PER_ELEM.values())
    value = bytes_step / (ms_per_step * 1e-3) / 1e9
    kernels = {}
    for k in KERNELS:
        avg_ms = per_kernel_ms[k] / launches
        gbs = BYTES_PER_ELEM[k] * n / (avg_ms * 1e-3) / 1e9
        kernels[k] = {"avg_us": round(avg_ms * 1e3, 2), "GB_s": round(gbs, 1),
                      "Gelem_s": round(n / (avg_ms * 1e-3) / 1e9, 2),
                      "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                      "bytes_per_launch": int(BYTES_PER_ELEM[k] * n)}
    dominant = max(KERNELS, key=lambda k: per_kernel_ms[k])
    dk = kernels[dominant]

    # rows beyond the hot path: capture with full codes, the full-information
    # forward and the agreement statistics, the MXFP4 and MXFP8 variants,
    # b = 3 cached low bits
    codes = torch.empty(n // 2, dtype=torch.uint8, device=dev)
    mx_scales = torch.empty(n // 32, dtype=torch.uint8, device=dev)
    mx_bits = torch.empty(n // 8, dtype=torch.uint8, device=dev)
    planes3 = torch.empty(3 * (n // 8), dtype=torch.uint8, device=dev)
    stats_acc = torch.zeros(20, dtype=torch.int64, device=dev)
    next_ms = {k: 0.0 for k in NEXT_BYTES_PER_ELEM}
    next_steps = max(1, min(args.steps, 3))
    flush_next = torch.empty(1, dtype=torch.float32, device=dev)
    zero_flush = torch.zeros(1 << 29, dtype=torch.bfloat16, device=dev) if L == 1 else None
    for it in range(next_steps + 1):
        ev = {k: [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(L)] for k in NEXT_BYTES_PER_ELEM}
        for li, d in enumerate(layers):
            def timed(k, fn):
                # each kernel after a read-only 1 GiB pass: these rows are not
                # part of the step, and a kernel right after a writer would
                # carry that writer's cache write-back
                # (over another layer's tensor, so no input line is left cached)
                tr.tensor_scale(zero_flush if L == 1 else layers[(li + 1) % L]["x_roll"], out=flush_next)
                ev[k][li][0].record(stream)
                fn()
                ev[k][li][1].record(stream)
            timed("capture_codes", lambda: tr.capture(d["x_roll"], d["ts"], scales=d["scales"], bits=d["bits"],
                                                      codes=codes))
            timed("full_info_fwd", lambda: tr.full_info_fakequant_fwd(d["x_train"], d["scales"], d["ts"], codes, y=y_g,
                                                                      mask=mask_g))
            timed("mismatch_stats", lambda: tr.mismatch_stats(d["x_train"], d["scales"], d["ts"], d["bits"], codes,
                                                              stats=stats_acc))
            timed("mx_capture", lambda: tr.mx_capture(d["x_roll"], scales=mx_scales, bits=mx_bits))
            timed("mx_guided_fwd", lambda: tr.mx_guided_fakequant_fwd(d["x_train"], mx_scales, mx_bits, y=y_g,
                                                                      mask=mask_g))
            timed("mx8_capture", lambda: tr.mx8_capture(d["x_roll"], scales=mx_scales, bits=mx_bits))
            timed("mx8_guided_fwd", lambda: tr.mx8_guided_fakequant_fwd(d["x_train"], mx_scales, mx_bits, y=y_g,
                                                                        mask=mask_g))
            timed("capture_lowbits3", lambda: tr.capture_lowbits(d["x_roll"], d["ts"], 3, scales=d["scales"],
                                                                 planes=planes3))
            timed("lowbits3_fwd", lambda: tr.lowbits_fakequant_fwd(d["x_train"], d["scales"], d["ts"], 3, planes3,
                                                                   y=y_g, mask=mask_g))
        stream.synchronize()
        if it > 0:  # the first pass warms up
            for k in NEXT_BYTES_PER_ELEM:
                next_ms[k] += sum(ev[k][li][0].elapsed_time(ev[k][li][1]) for li in range(L))
    next_rows = {}
    for k, bpe in NEXT_BYTES_PER_ELEM.items():
        avg_ms = next_ms[k] / (next_steps * L)
        gbs = bpe * n / (avg_ms * 1e-3) / 1e9
        next_rows[k] = {"avg_us": round(avg_ms * 1e3, 2), "GB_s": round(gbs, 1),
                        "Gelem_s": round(n / (avg_ms * 1e-3) / 1e9, 2), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                        "bytes_per_launch": int(bpe * n)}

    cold = cold_rows(tr, torch, dev, stream, layers, next_steps)
    moe = moe_rows(tr, workloads, torch, dev, stream, layers, next_steps)
    other = workload_rows(tr, workloads, torch, dev, stream)

    cache = {
        "compact_bytes_20_layers": L * (n // 8 + n // 16),
        "full_nvfp4_bytes_40_layers": TOTAL_LAYERS * (n // 2 + n // 16),
    }
    cache["ratio"] = round(cache["full_nvfp4_bytes_40_layers"] / cache["compact_bytes_20_layers"], 4)
    # layer-selection policies (5 / 20 / 40 captured layers) and b cached low
    # bits: b bit-planes + one scale byte per 16 elements + a 4-byte tensor
    # scale per captured site, against full NVFP4 codes for all 40 layers
    full40 = TOTAL_LAYERS * (n // 2 + n // 16 + 4)
    cache["policies"] = [{"captured_layers": lc, "bits": b, "bytes": lc * (b * n // 8 + n // 16 + 4),
                          "ratio_vs_full_40": round(full40 / (lc * (b * n // 8 + n // 16 + 4)), 4)}
                         for lc in (5, 20, 40) for b in (1, 2, 3, 4)]

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"deeper-half capture sweep: {L} of {TOTAL_LAYERS} layers, one {ROWS}x{COLS} "
                               f"bf16 site per layer (64 trajectories x 4096 tokens), Gaussian with 0.1% outlier "
                               f"channels x100",
                   "layers": L, "rows": ROWS, "cols": COLS, "elements_per_step": L * n,
                   "step": "rollout side (tensor_scale + capture) over all layers, then training side "
                           "(guided_fwd + rne_fwd + ste_bwd) over all layers"},
        "gelem_per_s": round(L * n / (ms_per_step * 1e-3) / 1e9, 3),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "kernels": kernels,
        "kernels_cold": cold,
        "next_rows": next_rows,
        "moe_expert_site": moe,
        "other_workloads": other,
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": dk["GB_s"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": dk["frac_hbm_peak"], "traffic": read_traffic(dominant)},
        "cache": cache,
        "cpu_baseline": None,
    }

    result["practical_ceiling"] = practical_ceiling()

    if pool is not None:
        result["cpu_baseline"] = cpu_leg(pool, cores, layers[0], n, y_g, mask_g, y_r, mask_r, gin, np, torch, tr)
        pool.close()
        pool.join()
    print(json.dumps(result), flush=True)


def cold_rows(tr, torch, dev, stream, layers, reps):
    """The tensor scale and the capture of one deeper-half layer without the
    step's neighbours: each after a read-only 1 GiB pass over another
    layer's tensor (which evicts the 256 MB last-level cache and leaves no
    dirty lines), and the capture right after the tensor scale of the same
    tensor (as a rollout runs them).  In the step, the capture follows the
    tensor scale and reads first the lines that pass read last, so part of
    its input comes from the last-level cache; these rows give its figure
    from HBM alone."""
    d = layers[0]
    flush = layers[-1]["x_roll"] if len(layers) > 1 else torch.zeros(1 << 29, dtype=torch.bfloat16, device=dev)
    flush_ts = torch.empty(1, dtype=torch.float32, device=dev)
    n = d["x_roll"].numel()
    ws = torch.empty(tr.lib.trace_tensor_scale_workspace_bytes(n), dtype=torch.uint8, device=dev)
    names = ("tensor_scale_after_read", "capture_after_read", "capture_after_tensor_scale")
    t = {k: 0.0 for k in names}
    for it in range(reps + 1):
        ev = {k: [torch.cuda.Event(enable_timing=True) for _ in range(2)] for k in names}
        tr.tensor_scale(flush, out=flush_ts)
        ev["tensor_scale_after_read"][0].record(stream)
        tr.tensor_scale(d["x_roll"], out=d["ts"], workspace=ws)
        ev["tensor_scale_after_read"][1].record(stream)
        tr.tensor_scale(flush, out=flush_ts)
        ev["capture_after_read"][0].record(stream)
        tr.capture(d["x_roll"], d["ts"], scales=d["scales"], bits=d["bits"])
        ev["capture_after_read"][1].record(stream)
        tr.tensor_scale(flush, out=flush_ts)
        tr.tensor_scale(d["x_roll"], out=d["ts"], workspace=ws)
        ev["capture_after_tensor_scale"][0].record(stream)
        tr.capture(d["x_roll"], d["ts"], scales=d["scales"], bits=d["bits"])
        ev["capture_after_tensor_scale"][1].record(stream)
        stream.synchronize()
        if it > 0:
            for k in names:
                t[k] += ev[k][0].elapsed_time(ev[k][1])
    out = {"protocol": "layer 0 of the sweep; 'after_read': after a read-only 1 GiB pass over another layer "
                       "(no last-level-cache reuse, no dirty lines); 'capture_after_tensor_scale': right after the "
                       "tensor scale of the same tensor, itself after such a pass (the capture then reads part of "
                       "its input from the 256 MB last-level cache, as in the step)"}
    for k in names:
        bpe = BYTES_PER_ELEM["tensor_scale" if k.startswith("tensor") else "capture"]
        avg = t[k] / reps
        gbs = bpe * n / (avg * 1e-3) / 1e9
        out[k] = {"avg_us": round(avg * 1e3, 2), "GB_s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    return out


def rollout_side_rows(tr, torch, dev, stream, sites, flush, flush_ts, reps):
    """The rollout side of a multi-site workload (tensor scale and capture of
    every site): per-site calls against the batch entry points, each timed
    between two HIP events after a read-only 1 GiB pass."""
    xs = [d["x_roll"].reshape(d["x_roll"].shape[0], -1) for d in sites.values()]
    tss = [torch.empty(1, dtype=torch.float32, device=dev) for _ in xs]
    recs = [(torch.empty(x.numel() // 16, dtype=torch.uint8, device=dev),
             torch.empty(x.numel() // 8, dtype=torch.uint8, device=dev), None) for x in xs]
    ws1 = [torch.empty(tr.lib.trace_tensor_scale_workspace_bytes(x.numel()), dtype=torch.uint8, device=dev) for x in xs]
    wsb = torch.empty(max(4, tr.lib.trace_tensor_scale_batch_workspace_bytes(tr._sites(xs, tss), len(xs))),
                      dtype=torch.uint8, device=dev)

    def per_site():
        for x, t, w, (sc, bt, _) in zip(xs, tss, ws1, recs):
            tr.tensor_scale(x, out=t, workspace=w)
            tr.capture(x, t, scales=sc, bits=bt)

    def batched():
        tr.tensor_scale_batch(xs, outs=tss, workspace=wsb)
        tr.capture_batch(xs, tss, records=recs)

    per_site()
    batched()
    t = {"per_site": 0.0, "batched": 0.0}
    for _ in range(reps):
        for name, fn in (("per_site", per_site), ("batched", batched)):
            tr.tensor_scale(flush, out=flush_ts)        # read-only 1 GiB pass
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            stream.synchronize()
            t[name] += e0.elapsed_time(e1) / reps
    nbytes = sum((BYTES_PER_ELEM["tensor_scale"] + BYTES_PER_ELEM["capture"]) * x.numel() for x in xs)
    return {"sites": len(xs), "algorithmic_bytes": int(nbytes),
            "per_site_us": round(t["per_site"] * 1e3, 1), "batched_us": round(t["batched"] * 1e3, 1),
            "per_site_GB_s": round(nbytes / (t["per_site"] * 1e-3) / 1e9, 1),
            "batched_GB_s": round(nbytes / (t["batched"] * 1e-3) / 1e9, 1)}


def workload_rows(tr, workloads, torch, dev, stream, reps=3):
    """The step's five kernels on each site of the other workloads (the MoE
    layer's four sites, K and V of the KV cache, the ragged large-hidden
    site, and the small 1024x2048 case), timed per kernel with HIP events.
    Cold: every rep follows a 1 GiB read-only pass, which evicts the 256 MB
    last-level cache without leaving dirty lines; warm: the same step again
    at once (sites under 256 MB then read from the cache).  x_train follows
    the relative-noise rule of each workload where it is one (the MoE layer:
    its tuned sigma; elsewhere the small case's 2%): the kernels have no
    data-dependent path on finite inputs, so where values land does not
    change the time."""
    import json as _json
    with open(os.path.join(ROOT, "tests", "golden", "moe_layer_sigma.json")) as fh:
        sigma = _json.load(fh)["sigma"]
    flush = torch.zeros(1 << 29, dtype=torch.bfloat16, device=dev)   # 1 GiB
    flush_ts = torch.empty(1, dtype=torch.float32, device=dev)

    def noisy(x, *key):
        return workloads.relative_noise(x, 0.02, workloads.generator(dev, *key))

    sites = {"small 1024x2048": {"x": workloads.single_site(dev)}}
    sites["MoE layer"] = workloads.moe_layer(dev, sigma)
    kv = {}
    for which in ("k", "v"):
        xr = workloads.kv_cache_rollout(dev, which)
        kv[which] = {"x_roll": xr, "x_train": noisy(xr, 2, which, "bench"), "grad": workloads.grad_for(xr.shape, dev, 2, which)}
    sites["KV cache"] = kv
    xr = workloads.large_hidden_rollout(dev)
    sites["large hidden 65573x7168"] = {"x": {"x_roll": xr, "x_train": noisy(xr, 4, "bench"),
                                              "grad": workloads.grad_for(xr.shape, dev, 4)}}
    # sustained untimed work first (the step's kernels on the large-hidden
    # site): after the data generation the clocks settle over ~20-40 ms of it
    # (see moe_rows)
    wd = sites["large hidden 65573x7168"]["x"]
    w_ts = torch.empty(1, dtype=torch.float32, device=dev)
    w_sc, w_bt, _ = tr.capture(wd["x_roll"], tr.tensor_scale(wd["x_roll"], out=w_ts))
    w_y = torch.empty_like(wd["x_train"])
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < MOE_WARM_S:
        tr.tensor_scale(wd["x_roll"], out=w_ts)
        tr.capture(wd["x_roll"], w_ts, scales=w_sc, bits=w_bt)
        tr.guided_fakequant_fwd(wd["x_train"], w_sc, w_ts, w_bt, y=w_y)
        torch.cuda.synchronize()
    del w_sc, w_bt, w_y
    bpe_step = sum(BYTES_PER_ELEM.values())
    out = {"protocol": "cold: each of %d reps after a 1 GiB read-only pass (evicts the 256 MB last-level cache, "
                       "leaves no dirty lines); warm: the same step again at once (small sites' inputs partly "
                       "cache-resident, the first run's output lines still being written back); GB/s = algorithmic "
                       "bytes of the five kernels / the sum of their HIP-event times; x_train by relative noise" % reps}
    for wname, ws_ in sites.items():
        tot = {"bytes": 0.0, "cold_s": 0.0, "warm_s": 0.0}
        res = {}
        for sname, d in ws_.items():
            x_roll = d["x_roll"].reshape(d["x_roll"].shape[0], -1)
            x_train = d["x_train"].reshape(x_roll.shape)
            grad = d["grad"].reshape(x_roll.shape)
            n = x_roll.numel()
            ts = torch.empty(1, dtype=torch.float32, device=dev)
            ws = torch.empty(tr.lib.trace_tensor_scale_workspace_bytes(n), dtype=torch.uint8, device=dev)
            scales = torch.empty(n // 16, dtype=torch.uint8, device=dev)
            bits = torch.empty(n // 8, dtype=torch.uint8, device=dev)
            y = torch.empty_like(x_train)
            mask = torch.empty(n // 8, dtype=torch.uint8, device=dev)
            gin = torch.empty_like(grad)

            def run(evs):
                evs[0].record(stream)
                tr.tensor_scale(x_roll, out=ts, workspace=ws)
                evs[1].record(stream)
                tr.capture(x_roll, ts, scales=scales, bits=bits)
                evs[2].record(stream)
                tr.guided_fakequant_fwd(x_train, scales, ts, bits, y=y, mask=mask)
                evs[3].record(stream)
                tr.rne_fakequant_fwd(x_train, scales, ts, y=y, mask=mask)
                evs[4].record(stream)
                tr.ste_bwd(grad, mask, grad_in=gin)
                evs[5].record(stream)

            def events():
                return [torch.cuda.Event(enable_timing=True) for _ in range(6)]

            run(events())                                   # warm-up
            cold = [0.0] * 5
            warm = [0.0] * 5
            for _ in range(reps):
                tr.tensor_scale(flush, out=flush_ts)        # read-only 1 GiB pass
                ec, ew = events(), events()
                run(ec)
                run(ew)
                stream.synchronize()
                for k in range(5):
                    cold[k] += ec[k].elapsed_time(ec[k + 1]) / reps
                    warm[k] += ew[k].elapsed_time(ew[k + 1]) / reps
            nbytes = bpe_step * n
            cs, wsec = sum(cold) * 1e-3, sum(warm) * 1e-3
            res[sname] = {"elements": n, "cold_us": round(cs * 1e6, 1), "cold_GB_s": round(nbytes / cs / 1e9, 1),
                          "cold_frac_hbm_peak": round(nbytes / cs / 1e9 / HBM_PEAK_GBS, 4),
                          "warm_us": round(wsec * 1e6, 1), "warm_GB_s": round(nbytes / wsec / 1e9, 1),
                          "cold_kernel_us": {k: round(cold[i] * 1e3, 1) for i, k in enumerate(KERNELS)}}
            tot["bytes"] += nbytes
            tot["cold_s"] += cs
            tot["warm_s"] += wsec
        out[wname] = {"sites": res, "cold_GB_s": round(tot["bytes"] / tot["cold_s"] / 1e9, 1),
                      "warm_GB_s": round(tot["bytes"] / tot["warm_s"] / 1e9, 1)}
        log(f"workload {wname}: cold {out[wname]['cold_GB_s']} GB/s, warm {out[wname]['warm_GB_s']} GB/s")
        if len(ws_) > 1:
            out[wname]["rollout_side"] = rollout_side_rows(tr, torch, dev, stream, ws_, flush, flush_ts, reps)
            log(f"  rollout side of {wname}: {out[wname]['rollout_side']}")
    del sites, flush
    return out


def moe_rows(tr, workloads, torch, dev, stream, layers, reps):
    """Per-expert tensor scales on the packed routed-expert site (the
    sequence tensor scale, capture, guided forward: in sequence, and each rep
    after a read-only 1 GiB pass), the trainer-side gather of its records
    into a shuffled row order (single rows, and runs of GATHER_RUN
    consecutive rows), and the trainer's forward on its rows in that order
    (gather then forward, against the fused read-back forwards); every
    gather and read-back variant after a read-only 1 GiB pass, and the
    read-back variants also rep after rep.  Medians of MOE_REPS reps."""
    sigma = 0.02
    d = workloads.moe_layer(dev, sigma, sites=["expert_in"])["expert_in"]
    _, experts = workloads.moe_routing(dev)
    offsets = workloads.moe_expert_offsets(experts)
    x_roll, x_train = d["x_roll"], d["x_train"]
    rows, cols = x_roll.shape
    n = rows * cols
    perm = workloads.trainer_order(rows, dev)
    # the same rows as shuffled runs of RUN consecutive rows (a trainer that
    # moves whole token runs rather than single rows)
    run_order = torch.randperm(rows // GATHER_RUN, generator=workloads.generator(dev, "trainer runs"), device=dev)
    runs = (run_order[:, None] * GATHER_RUN + torch.arange(GATHER_RUN, device=dev)[None, :]).reshape(-1)
    flush_ts = torch.empty(1, dtype=torch.float32, device=dev)
    groups = offsets.numel() - 1
    ts = torch.empty(groups, dtype=torch.float32, device=dev)
    ws = torch.empty(max(4, tr.lib.trace_grouped_tensor_scale_workspace_bytes(rows)), dtype=torch.uint8, device=dev)
    scales = torch.empty(n // 16, dtype=torch.uint8, device=dev)
    bits = torch.empty(n // 8, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x_train)
    mask = torch.empty(n // 8, dtype=torch.uint8, device=dev)
    flush = layers[0]["x_roll"]

    def medians(run, names):
        """run(ev) enqueues one rep, recording ev[name] = (start, end) events;
        returns the median microseconds of each name over MOE_REPS reps.
        Untimed reps run first for MOE_WARM_S seconds: after the data
        generation the GPU's clocks settle over ~20-40 ms of sustained work,
        during which the capture and the forward measured up to 40% and 15%
        slower.  The timed reps are all enqueued before the host waits, so
        the GPU runs them back to back: with a wait after each rep, a start
        event fires on an idle GPU while the host is still issuing the
        launch, and that gap (~4 us on the per-expert forward) lands inside
        the interval."""
        t = {k: [] for k in names}
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < MOE_WARM_S:
            run({k: (torch.cuda.Event(), torch.cuda.Event()) for k in names})
            stream.synchronize()
        evs = []
        for _ in range(MOE_REPS):
            evs.append({k: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                        for k in names})
            run(evs[-1])
        stream.synchronize()
        for ev in evs:
            for k in names:
                t[k].append(ev[k][0].elapsed_time(ev[k][1]) * 1e3)
        return {k: statistics.median(v) for k, v in t.items()}

    def timed(ev, k, fn):
        ev[k][0].record(stream)
        fn()
        ev[k][1].record(stream)

    def seq_medians(calls):
        """calls: (name, fn) pairs run in order, rep after rep, with one
        marker event after each call (as the step times its kernels, rather
        than a start and an end event around each): the median microseconds
        of each name over MOE_REPS reps, after MOE_WARM_S seconds of untimed
        reps."""
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < MOE_WARM_S:
            for _, fn in calls:
                fn()
            stream.synchronize()
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(MOE_REPS * len(calls) + 1)]
        marks[0].record(stream)
        i = 0
        for _ in range(MOE_REPS):
            for _, fn in calls:
                fn()
                i += 1
                marks[i].record(stream)
        stream.synchronize()
        t = {k: [] for k, _ in calls}
        for j in range(MOE_REPS * len(calls)):
            t[calls[j % len(calls)][0]].append(marks[j].elapsed_time(marks[j + 1]) * 1e3)
        return {k: statistics.median(v) for k, v in t.items()}

    seq_names = ("grouped_tensor_scale", "grouped_capture", "grouped_guided_fwd")

    def rollout_side(ev):
        tr.tensor_scale(flush, out=flush_ts)  # read-only 1 GiB pass
        timed(ev, "grouped_tensor_scale", lambda: tr.grouped_tensor_scale(x_roll, offsets, out=ts, workspace=ws))
        timed(ev, "grouped_capture", lambda: tr.grouped_capture(x_roll, offsets, ts, scales=scales, bits=bits))

    def training_side(ev):
        tr.tensor_scale(flush, out=flush_ts)
        timed(ev, "grouped_guided_fwd",
              lambda: tr.grouped_guided_fakequant_fwd(x_train, offsets, scales, ts, bits, y=y, mask=mask))

    # in the step's phase order: the rollout side rep after rep, then the
    # training side rep after rep; and each rep after a read-only pass
    us = seq_medians((("grouped_tensor_scale", lambda: tr.grouped_tensor_scale(x_roll, offsets, out=ts, workspace=ws)),
                      ("grouped_capture", lambda: tr.grouped_capture(x_roll, offsets, ts, scales=scales, bits=bits))))
    us.update(seq_medians((("grouped_guided_fwd",
                            lambda: tr.grouped_guided_fakequant_fwd(x_train, offsets, scales, ts, bits, y=y,
                                                                    mask=mask)),)))
    us_cold = medians(rollout_side, seq_names[:2])
    us_cold.update(medians(training_side, seq_names[2:]))

    # the gathers are short (0.375 B per element): each is timed after a
    # read-only 1 GiB pass, outside the previous kernel's write-back
    def gathers(ev):
        for k, order in (("gather_records", perm), ("gather_records_runs", runs)):
            tr.tensor_scale(flush, out=flush_ts)
            timed(ev, k, lambda: tr.gather_records(bits, scales, None, cols, order))

    us.update(medians(gathers, ("gather_records", "gather_records_runs")))

    # the trainer's forward on its rows in its own order, each variant after
    # a read-only 1 GiB pass
    xt_perm = x_train[perm]
    ts1 = tr.tensor_scale(x_roll)
    sc1, bt1, _ = tr.capture(x_roll, ts1)

    def two_step():
        g_bits, g_scales, _ = tr.gather_records(bt1, sc1, None, cols, perm)
        tr.guided_fakequant_fwd(xt_perm, g_scales, ts1, g_bits, y=y, mask=mask)

    rb_calls = (("gather_then_guided_fwd", two_step),
                ("fused_guided_fwd",
                 lambda: tr.gathered_guided_fakequant_fwd(xt_perm, perm, sc1, ts1, bt1, y=y, mask=mask)),
                ("fused_guided_fwd_per_expert",
                 lambda: tr.gathered_guided_fakequant_fwd(xt_perm, perm, scales, ts, bits, offsets=offsets,
                                                          y=y, mask=mask)))

    def readback(ev):
        for k, fn in rb_calls:
            tr.tensor_scale(flush, out=flush_ts)
            timed(ev, k, fn)

    us_rb = medians(readback, tuple(READBACK_BYTES_PER_ELEM))
    # and each variant rep after rep, as a training step streams its
    # forwards: each rep then also pays the write-back the previous one left
    # in the last-level cache, which the read-only pass above takes off
    us_rb_seq = {}
    for k, fn in rb_calls:
        us_rb_seq.update(seq_medians(((k, fn),)))

    def row(k_us, bpe):
        gbs = bpe * n / (k_us * 1e-6) / 1e9
        return {"median_us": round(k_us, 2), "GB_s": round(gbs, 1), "Gelem_s": round(n / (k_us * 1e-6) / 1e9, 2),
                "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": int(bpe * n)}

    out = {"site": f"routed-expert input {rows}x{cols} bf16, rows grouped by {groups} experts "
                   f"(top-8 of 128 routing of 16384 tokens), Student-t(4)",
           "timing": f"median of {MOE_REPS} reps after {MOE_WARM_S} s of untimed ones, HIP events",
           "kernels": {k: row(us[k], bpe) for k, bpe in MOE_BYTES_PER_ELEM.items()}}
    out["protocol"] = ("kernels: as the step, the rollout side (grouped tensor scale, capture) rep after rep, "
                       "then the training side (guided forward) rep after rep")
    out["kernels_cold"] = {"protocol": "the same, each rep after a read-only 1 GiB pass (no last-level-cache "
                                       "reuse, no dirty lines)"}
    out["kernels_cold"].update({k: row(us_cold[k], MOE_BYTES_PER_ELEM[k]) for k in seq_names})
    out["readback_trainer_order"] = {k: row(us_rb[k], bpe) for k, bpe in READBACK_BYTES_PER_ELEM.items()}
    out["readback_trainer_order"]["protocol"] = "each rep after a read-only 1 GiB pass"
    out["readback_trainer_order_in_sequence"] = {k: row(us_rb_seq[k], bpe)
                                                 for k, bpe in READBACK_BYTES_PER_ELEM.items()}
    out["readback_trainer_order_in_sequence"]["protocol"] = "each variant rep after rep"
    del d, x_roll, x_train, y, xt_perm
    return out


def practical_ceiling():
    """Copy (plain and non-temporal), read and fill streams over 1 GiB
    (``bench_ceiling.hip``, built into _build/), back to back, after a
    read-only pass and after a 1 GiB write: the practical ceilings for the
    kernels' access mixes; and plain copies of 12 to 192 MiB
    (``copy_by_size``), the ceiling of the smaller sites' kernels.  Run as a
    child process after the timed work; None if it is not built."""
    import subprocess
    exe = os.path.join(ROOT, "_build", "bench_ceiling")
    if not os.path.exists(exe):
        log("practical ceiling: _build/bench_ceiling is not built (python fp4_rollout_guided_amd/build.py)")
        return None
    try:
        res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    except subprocess.TimeoutExpired:
        log("practical ceiling: probe timed out")
        return None
    if res.returncode != 0:
        log(f"practical ceiling: probe failed ({res.returncode}): {res.stderr.strip()[-300:]}")
        return None
    return json.loads(res.stdout.strip().splitlines()[-1])


def calibrate_copy():
    """A plain copy of ROWS x COLS bf16 (1 GiB read, 1 GiB written), three
    times: the counter reading of a kernel whose HBM bytes are known."""
    import torch
    dev = torch.device("cuda", 0)
    src = torch.randn(ROWS, COLS, device=dev).to(torch.bfloat16)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(3):
        dst.copy_(src)
    ev[1].record()
    torch.cuda.synchronize()
    us = ev[0].elapsed_time(ev[1]) * 1e3 / 3
    nbytes = src.numel() * 2
    log(f"copy {nbytes} B read + {nbytes} B written: {us:.1f} us per copy, {2 * nbytes / us / 1e3:.1f} GB/s")
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "avg_us": round(us, 2),
                      "GB_s": round(2 * nbytes / us / 1e3, 1)}), flush=True)


def read_traffic(kernel):
    """HBM traffic per launch from the committed counter summary, or None
    when there is none for this kernel or the kernel source changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_deeper_half.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    recorded = (kv.get("kernel_sources_sha256") or "-").split()[0]   # the digest, then the file list
    if recorded != kernel_sources_digest() or "traffic_bytes_per_launch" not in kv:
        return None
    return float(kv["traffic_bytes_per_launch"])


KERNEL_SOURCES = ("kernels.hip", "fp4_block.h", "device_math.h", "nvfp4_scale.h", "launch.h")


def kernel_sources_digest():
    """SHA-256 over the sources that make up the NVFP4 kernels' code; the
    committed counter summaries record it, so they are ignored once any of
    these files changes."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "fp4_rollout_guided_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def cpu_leg(pool, cores, d0, n, y_g, mask_g, y_r, mask_r, gin, np, torch, tr):
    """Oracle on rows of layer 0 (its outputs recomputed on the GPU for
    those rows are compared bit for bit), within CPU_BUDGET_S of wall time."""
    import oracle
    from tests.gpu_util import to_np_u16, to_np_u8
    # layer-0 outputs of the last step are still in y_g/... for the last layer only;
    # recompute layer 0 so that the GPU outputs of the sampled rows are at hand
    tr.tensor_scale(d0["x_roll"], out=d0["ts"])
    tr.capture(d0["x_roll"], d0["ts"], scales=d0["scales"], bits=d0["bits"])
    tr.guided_fakequant_fwd(d0["x_train"], d0["scales"], d0["ts"], d0["bits"], y=y_g, mask=mask_g)
    tr.rne_fakequant_fwd(d0["x_train"], d0["scales"], d0["ts"], y=y_r, mask=mask_r)
    tr.ste_bwd(d0["grad"], mask_g, grad_in=gin)
    torch.cuda.synchronize()
    ts_gpu = np.float32(d0["ts"].item())
    xr_all = to_np_u16(d0["x_roll"])
    ts_oracle = oracle.tensor_scale(xr_all)
    ts_match = bool(np.float32(ts_oracle).view(np.uint32) == ts_gpu.view(np.uint32))
    del xr_all

    per = CHUNK_ROWS * COLS
    done_rows, busy, exact = 0, 0.0, ts_match
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < CPU_BUDGET_S and done_rows + cores * CHUNK_ROWS <= ROWS:
        lo, hi = done_rows, done_rows + cores * CHUNK_ROWS
        sl = slice(lo * COLS, hi * COLS)
        xr = to_np_u16(d0["x_roll"].view(-1)[sl])
        xt = to_np_u16(d0["x_train"].view(-1)[sl])
        g = to_np_u16(d0["grad"].view(-1)[sl])
        tasks = [(xr[i * per:(i + 1) * per], xt[i * per:(i + 1) * per], g[i * per:(i + 1) * per], ts_oracle)
                 for i in range(cores)]
        res = pool.map(_oracle_chunk, tasks)
        busy += sum(r[0] for r in res)
        want = {k: np.concatenate([r[1][k] for r in res]) for k in res[0][1]}
        got = {
            "scales": to_np_u8(d0["scales"][lo * COLS // 16:hi * COLS // 16]),
            "bits": to_np_u8(d0["bits"][lo * COLS // 8:hi * COLS // 8]),
            "y_g": to_np_u16(y_g.view(-1)[sl]), "mask_g": to_np_u8(mask_g[lo * COLS // 8:hi * COLS // 8]),
            "y_r": to_np_u16(y_r.view(-1)[sl]), "mask_r": to_np_u8(mask_r[lo * COLS // 8:hi * COLS // 8]),
            "gin": to_np_u16(gin.view(-1)[sl]),
        }
        exact = exact and all(np.array_equal(got[k], want[k]) for k in want)
        done_rows = hi
    wall = time.perf_counter() - t0
    elems = done_rows * COLS
    eps = elems / wall
    bpe = sum(BYTES_PER_ELEM.values())
    log(f"cpu oracle: {elems} elements in {wall:.2f} s on {cores} processes; bit-exact={exact}")
    return {"value": round(eps * bpe / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "elem_per_s": round(eps, 1),
            "one_core_value": round(elems * bpe / busy / 1e9, 4) if busy > 0 else None,
            "one_core_elem_per_s": round(elems / busy, 1) if busy > 0 else None,
            "sample": f"rows 0..{done_rows} of layer 0 ({elems} elements) through the whole step, "
                      f"tensor scale of the full layer; {cores} worker processes, "
                      f"{busy:.1f} s of CPU time in {wall:.1f} s wall",
            "sample_bit_exact_vs_gpu": exact}


if __name__ == "__main__":
    main()
