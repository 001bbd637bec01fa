"""GPU parity of the batch entry points (trace_tensor_scale_batch,
trace_capture_batch): several site tensors in one tensor-scale pass and one
capture launch.  Small mixed sites (empty, one block, ragged widths, tensor
scales orders of magnitude apart, NaN and infinity) against the oracle bit
for bit; the MoE layer's four sites and the KV cache's K and V against the
per-site entry points (which the other GPU tests tie to the oracle), with
every tensor scale against the oracle's."""
import json
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import formats as F
from tests.gpu_util import from_np_u16, to_np_u8, to_np_u16

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _ts_bits(t):
    return t.cpu().numpy().view(np.uint32)[0]


def _mixed_sites(rng, shapes, device):
    host, dev = [], []
    for i, (rows, cols) in enumerate(shapes):
        v = rng.standard_t(4, (rows, cols)) * 10.0 ** rng.uniform(-30, 30)
        if rows * cols > 64 and i % 2 == 0:
            v.reshape(-1)[rng.integers(0, rows * cols)] = np.nan
        if rows * cols > 64 and i % 3 == 0:
            v.reshape(-1)[rng.integers(0, rows * cols)] = -np.inf
        x = F.f32_to_bf16_rne(v.reshape(-1).astype(np.float32))
        host.append(x)
        dev.append(from_np_u16(x, device, (rows, cols)))
    return host, dev


SHAPES = [(1, 16), (37, 48), (0, 32), (3, 4112), (129, 4096 + 80), (17, 7168), (256, 16), (1000, 64)]


@pytest.mark.parametrize("count", [1, 3, 8])
def test_batch_mixed_sites_against_the_oracle(device, count):
    import fp4_rollout_guided_amd as tr
    _say("case batch of", count, "mixed sites")
    rng = np.random.default_rng(100 + count)
    shapes = SHAPES[:count] if count < 8 else SHAPES
    host, dev = _mixed_sites(rng, shapes, device)
    ts = tr.tensor_scale_batch(dev)
    rec = tr.capture_batch(dev, ts, want_codes=True)
    torch.cuda.synchronize()
    for i, x in enumerate(host):
        want_ts = np.float32(oracle.tensor_scale(x))
        assert _ts_bits(ts[i]) == want_ts.view(np.uint32), (i, shapes[i])
        if x.size == 0:
            continue
        cap = oracle.capture(x, want_ts, with_codes=True)
        sc, bt, cd = rec[i]
        for k, got in (("scales", sc), ("bits", bt), ("codes", cd)):
            assert np.array_equal(to_np_u8(got), cap[k]), (i, shapes[i], k)


def test_batch_capture_with_a_shared_tensor_scale(device):
    """Two sites captured with one tensor scale (an input shared by both),
    and one tensor given as two sites."""
    import fp4_rollout_guided_amd as tr
    _say("case batch capture, shared ts")
    rng = np.random.default_rng(7)
    host, dev = _mixed_sites(rng, [(64, 512), (64, 512)], device)
    ts = tr.tensor_scale(dev[0])
    rec = tr.capture_batch(dev, [ts, ts], want_codes=True)
    torch.cuda.synchronize()
    for i, x in enumerate(host):
        cap = oracle.capture(x, np.float32(oracle.tensor_scale(host[0])), with_codes=True)
        for k, got in zip(("scales", "bits", "codes"), rec[i]):
            assert np.array_equal(to_np_u8(got), cap[k]), (i, k)
    # one input tensor in two sites of a batch (inputs may be shared)
    ts2 = tr.tensor_scale_batch([dev[1], dev[1]])
    rec2 = tr.capture_batch([dev[1], dev[1]], ts2, want_codes=True)
    torch.cuda.synchronize()
    assert _ts_bits(ts2[0]) == _ts_bits(ts2[1]) == np.float32(oracle.tensor_scale(host[1])).view(np.uint32)
    for a, b in zip(rec2[0], rec2[1]):
        assert torch.equal(a, b)


def _against_per_site(name, xs):
    import fp4_rollout_guided_amd as tr
    ts_b = tr.tensor_scale_batch(xs)
    rec_b = tr.capture_batch(xs, ts_b, want_codes=True)
    for i, x in enumerate(xs):
        ts = tr.tensor_scale(x)
        sc, bt, cd = tr.capture(x, ts, want_codes=True)
        torch.cuda.synchronize()
        want_ts = np.float32(oracle.tensor_scale(to_np_u16(x)))
        assert _ts_bits(ts_b[i]) == _ts_bits(ts) == want_ts.view(np.uint32), (name, i)
        for k, a, b in zip(("scales", "bits", "codes"), rec_b[i], (sc, bt, cd)):
            assert torch.equal(a, b), (name, i, k)
    _say(f"  {name}: {len(xs)} sites, batch == per site")


def test_batch_moe_layer_sites(device):
    with open(os.path.join(HERE, "golden", "moe_layer_sigma.json")) as fh:
        sigma = json.load(fh)["sigma"]
    _say("case batch, MoE layer sites")
    sites = workloads.moe_layer(device, sigma)
    _against_per_site("MoE layer", [d["x_roll"] for d in sites.values()])


def test_batch_kv_cache(device):
    _say("case batch, KV cache K and V")
    xs = [workloads.kv_cache_rollout(device, w) for w in ("k", "v")]
    _against_per_site("KV cache", [x.reshape(x.shape[0], -1) for x in xs])
