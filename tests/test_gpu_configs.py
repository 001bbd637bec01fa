"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark uses (one call per site tensor): every element of every output of
every site against the oracle, bit for bit (``tests/full_compare.py``), on
every workload including all 20 layers of the deeper-half sweep (one case
per layer), and on sampled rows (the first row, random rows and the last
rows, which include the ragged tail of the large-hidden workload).  The
tensor scale of every site is checked over the whole tensor, and every
element of every output against the whole-tensor properties of
``tests/full_props.py``.  Where a workload is built around rollout /
training agreement, the oracle's mismatch statistics on the sample are
checked against what the rule guarantees (straddle sites are recovered,
two-codeword mismatches fall back to RNE) and printed."""
import json
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.full_compare import Shared, compare_every_element, tensor_scale_of
from tests.full_props import check_nvfp4_outputs
from tests.gpu_util import assert_same, oracle_path, to_np_u16, to_np_u8
from tests.workload_place import oracle_block_scales, place_kv, place_near_midpoints

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _gpu_full(x_roll, x_train, grad):
    import fp4_rollout_guided_amd as tr
    ts = tr.tensor_scale(x_roll)
    sc, bt, cd = tr.capture(x_roll, ts, want_codes=True)
    yg, mg, qg = tr.guided_fakequant_fwd(x_train, sc, ts, bt, want_codes=True)
    yr, mr, qr = tr.rne_fakequant_fwd(x_train, sc, ts, want_codes=True)
    yf, mf, qf = tr.full_info_fakequant_fwd(x_train, sc, ts, cd, want_codes=True)
    gin = tr.ste_bwd(grad, mg)
    torch.cuda.synchronize()
    return {"ts": ts, "scales": sc, "bits": bt, "codes": cd, "y_g": yg, "mask_g": mg, "q_g": qg,
            "y_r": yr, "mask_r": mr, "q_r": qr, "y_f": yf, "mask_f": mf, "q_f": qf, "gin": gin}


def _rows(rows, k, seed):
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(rows, size=min(k, rows), replace=False).tolist())
    pick.update([0, rows - 1, rows - 2, rows - 37 if rows > 37 else 0])
    return np.array(sorted(pick))


def _gather(t, idx, per_row, u16=False):
    v = t.reshape(-1, per_row)[torch.from_numpy(idx).to(t.device)]
    return to_np_u16(v) if u16 else to_np_u8(v)


def check_site(name, x_roll, x_train, grad, k_rows=128, seed=0):
    rows, cols = x_roll.shape[0], x_roll.numel() // x_roll.shape[0]
    _say(f"case {name}: {tuple(x_roll.shape)} ({x_roll.numel()} elements), every element, then {k_rows} sampled rows")
    with Shared({"xr": x_roll, "xt": x_train, "g": grad}) as sh:
        ts = tensor_scale_of(sh)          # the oracle's, over the whole tensor
        got = _gpu_full(x_roll, x_train, grad)
        check_nvfp4_outputs(name, x_roll, x_train, grad, got["ts"], got)
        assert got["ts"].cpu().numpy().view(np.uint32)[0] == np.float32(ts).view(np.uint32), name
        # every element of every output against the oracle
        compare_every_element(name, sh, {k: v for k, v in got.items() if k != "ts"}, ts)
    idx = _rows(rows, k_rows, seed)
    xr = _gather(x_roll.view(torch.int16), idx, cols, True)
    xt = _gather(x_train.view(torch.int16), idx, cols, True)
    g = _gather(grad.view(torch.int16), idx, cols, True)
    want = oracle_path(xr, xt, g, ts=ts)
    per = {"scales": cols // 16, "bits": cols // 8, "codes": cols // 2, "mask_g": cols // 8, "q_g": cols // 2,
           "mask_r": cols // 8, "q_r": cols // 2, "mask_f": cols // 8, "q_f": cols // 2}
    sampled = {k: _gather(got[k], idx, n) for k, n in per.items()}
    for k in ("y_g", "y_r", "y_f", "gin"):
        sampled[k] = _gather(got[k].view(torch.int16), idx, cols, True)
    assert_same(sampled, want, keys=list(per) + ["y_g", "y_r", "y_f", "gin"], ctx=name)
    st = oracle.mismatch_stats(xt, want["scales"], ts, want["codes"], want["bits"])
    _say(f"  {name}: sample {st['n']} sites, mismatched {st['mismatched']}, straddle {st['straddle']}, "
         f"crossed {st['crossed']}, recovered {st['recovered']}, violations {st['violations']}, "
         f"hist {st['hist'][:4]}")
    # agreement statistics on the GPU: the sampled rows against the oracle's
    # counts, then the whole tensor (every straddle recovered)
    import fp4_rollout_guided_amd as tr
    pick = torch.from_numpy(idx).to(x_train.device)
    rows_t = lambda t, per: t.reshape(-1, per)[pick].contiguous()
    g_sample = tr.mismatch_stats(rows_t(x_train.view(-1, cols), cols), rows_t(got["scales"], cols // 16), got["ts"],
                                 rows_t(got["bits"], cols // 8), rows_t(got["codes"], cols // 2))
    assert g_sample.cpu().numpy().tolist() == st["hist"] + [st["straddle"], st["crossed"], st["recovered"],
                                                            st["violations"], st["n"]], name
    full = tr.mismatch_stats(x_train.view(-1, cols), got["scales"], got["ts"], got["bits"], got["codes"])
    full = full.cpu().numpy().tolist()
    assert sum(full[:15]) == full[19] == rows * cols and full[17] == full[15], name
    _say(f"  {name}: whole tensor {full[19]} sites, mismatched {full[19] - full[0]}, straddle {full[15]}, "
         f"crossed {full[16]}, violations {full[18]}, hist {full[:4]}")
    st["full"] = full
    # full tensor: where x_train == x_roll, guided == RNE (identical inputs give identical codes)
    same = (x_train.view(torch.int16) == x_roll.view(torch.int16)).reshape(-1)
    if bool(same.any()):
        yg = got["y_g"].view(torch.int16).reshape(-1)
        yr = got["y_r"].view(torch.int16).reshape(-1)
        assert bool((yg[same] == yr[same]).all()), name
    return st


def test_single_site_every_element(device):
    """1024 x 2048: every element against the oracle."""
    d = workloads.single_site(device)
    _say("case single site, every element")
    from tests.gpu_util import gpu_path
    got = gpu_path(d["x_roll"], d["x_train"], d["grad"])
    want = oracle_path(to_np_u16(d["x_roll"]), to_np_u16(d["x_train"]), to_np_u16(d["grad"]))
    assert_same(got, want, ctx="single site")


def test_moe_layer(device):
    with open(os.path.join(HERE, "golden", "moe_layer_sigma.json")) as fh:
        sigma = json.load(fh)["sigma"]
    sites = workloads.moe_layer(device, sigma)
    total = {"n": 0, "straddle": 0, "full_n": 0, "full_straddle": 0}
    for i, (name, d) in enumerate(sites.items()):
        st = check_site(f"MoE layer {name}", d["x_roll"], d["x_train"], d["grad"], seed=10 + i)
        total["n"] += st["n"]
        total["straddle"] += st["straddle"]
        total["full_n"] += st["full"][19]
        total["full_straddle"] += st["full"][15]
        assert st["recovered"] >= st["straddle"]
    rate = total["straddle"] / total["n"]
    _say(f"  MoE layer straddle rate on the samples: {rate:.4f}")
    assert 0.02 < rate < 0.04
    full_rate = total["full_straddle"] / total["full_n"]
    _say(f"  MoE layer straddle rate over the whole layer: {full_rate:.4f}")
    assert 0.02 < full_rate < 0.04


@pytest.mark.parametrize("which", ["k", "v"])
def test_kv_cache(device, which):
    x_roll = workloads.kv_cache_rollout(device, which)
    _, s_block = oracle_block_scales(x_roll)
    x_train = place_kv(x_roll, which, s_block)
    grad = workloads.grad_for(x_roll.shape, device, 2, which)
    shape2d = (x_roll.shape[0], x_roll.shape[1] * x_roll.shape[2])
    st = check_site(f"KV cache {which}", x_roll.reshape(shape2d), x_train.reshape(shape2d), grad.reshape(shape2d),
                    k_rows=256, seed=20)
    assert st["recovered"] >= st["straddle"]
    # all mismatches on the sample are the placed one- and two-codeword moves
    assert st["hist"][1] > 0 and sum(st["hist"][4:]) == 0


@pytest.mark.parametrize("layer", range(20))
def test_deeper_half_layer(device, layer):
    """One layer of the deeper-half sweep per case (the latter 20 of 40
    layers): every element of every output against the oracle and against
    the whole-tensor properties, the oracle's agreement statistics on
    sampled rows and the GPU's over the whole layer."""
    d = workloads.deeper_half_layer(device, layer)
    st = check_site(f"deeper-half layer {layer}", d["x_roll"], d["x_train"], d["grad"], seed=30 + layer)
    assert st["recovered"] >= st["straddle"]
    del d


def test_large_hidden_ragged(device):
    x_roll = workloads.large_hidden_rollout(device)
    _, s_block = oracle_block_scales(x_roll)
    x_train = place_near_midpoints(x_roll, s_block)
    grad = workloads.grad_for(x_roll.shape, device, 4)
    st = check_site("large hidden", x_roll, x_train, grad, k_rows=96, seed=40)
    assert st["recovered"] >= st["straddle"]
