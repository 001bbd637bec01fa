"""The library on several streams and under HIP graph capture.

* Two host threads, each with a stream of its own, run the whole path on
  different tensors at the same time, repeatedly; every output equals the
  same calls made one after another on one stream (the library keeps no
  state between calls, so concurrent calls on different streams cannot
  interfere).
* The path (tensor scale with a caller's workspace, capture, guided and RNE
  forwards, STE backward) captured into a HIP graph through torch's graph
  API: each of several replays, with eager work and synchronizations
  between them, equals the eager results bit for bit (the library issues
  only kernel launches, no memsets or allocations, so the captured graph
  holds kernel nodes only); on a small site and on one past 256 MiB, whose
  kernels are the non-temporal instantiations."""
import sys
import threading

import numpy as np
import pytest
import torch

from oracle import formats as F
from tests.gpu_util import to_np_u8, to_np_u16

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _site(seed, rows, cols, device):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((rows, cols)).astype(np.float32) * 10.0 ** rng.uniform(-2, 2)
    xr = F.f32_to_bf16_rne(v.reshape(-1))
    xt = F.f32_to_bf16_rne((v * (1 + 0.03 * rng.standard_normal(v.shape))).astype(np.float32).reshape(-1))
    g = F.f32_to_bf16_rne(rng.standard_normal(v.size).astype(np.float32))
    to = lambda a: torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16).reshape(rows, cols)
    return to(xr), to(xt), to(g)


def _path(tr, xr, xt, g, out):
    """The path into preallocated outputs (a dict of tensors) on the
    current stream."""
    tr.tensor_scale(xr, out=out["ts"], workspace=out["ws"])
    tr.capture(xr, out["ts"], scales=out["scales"], bits=out["bits"], codes=out["codes"])
    tr.guided_fakequant_fwd(xt, out["scales"], out["ts"], out["bits"], y=out["y_g"], mask=out["m_g"])
    tr.rne_fakequant_fwd(xt, out["scales"], out["ts"], y=out["y_r"], mask=out["m_r"])
    tr.ste_bwd(g, out["m_g"], grad_in=out["gin"])


def _outputs(tr, xr, device):
    n = xr.numel()
    return {"ts": torch.empty(1, dtype=torch.float32, device=device),
            "ws": torch.empty(tr.lib.trace_tensor_scale_workspace_bytes(n), dtype=torch.uint8, device=device),
            "scales": torch.empty(n // 16, dtype=torch.uint8, device=device),
            "bits": torch.empty(n // 8, dtype=torch.uint8, device=device),
            "codes": torch.empty(n // 2, dtype=torch.uint8, device=device),
            "y_g": torch.empty_like(xr), "m_g": torch.empty(n // 8, dtype=torch.uint8, device=device),
            "y_r": torch.empty_like(xr), "m_r": torch.empty(n // 8, dtype=torch.uint8, device=device),
            "gin": torch.empty_like(xr)}


def _host(out):
    return {k: (to_np_u16(v) if v.dtype == torch.bfloat16 else
                v.cpu().numpy().view(np.uint32) if v.dtype == torch.float32 else to_np_u8(v))
            for k, v in out.items() if k != "ws"}


def test_two_threads_on_their_own_streams(device):
    import fp4_rollout_guided_amd as tr
    _say("case two host threads, two streams")
    sites = [_site(s, 2048, 2064, device) for s in (1, 2)]
    ref = []
    for xr, xt, g in sites:  # one after another on the current stream
        out = _outputs(tr, xr, device)
        _path(tr, xr, xt, g, out)
        torch.cuda.synchronize()
        ref.append(_host(out))
    errors, results = [], [None, None]

    def worker(i):
        try:
            xr, xt, g = sites[i]
            stream = torch.cuda.Stream(device=device)
            outs = [_outputs(tr, xr, device) for _ in range(4)]
            with torch.cuda.stream(stream):
                for out in outs:
                    _path(tr, xr, xt, g, out)
            stream.synchronize()
            results[i] = [_host(o) for o in outs]
        except Exception as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    for i in range(2):
        for rep, got in enumerate(results[i]):
            for k in ref[i]:
                assert np.array_equal(got[k], ref[i][k]), (i, rep, k)


@pytest.mark.parametrize("rows,cols", [(1024, 4096), (65537, 2048)], ids=["small", "past-256MiB"])
def test_graph_replays_equal_eager(device, rows, cols):
    import fp4_rollout_guided_amd as tr
    _say("case HIP graph capture and replay", rows, cols)
    xr, xt, g = _site(3, rows, cols, device)
    eager = _outputs(tr, xr, device)
    _path(tr, xr, xt, g, eager)
    torch.cuda.synchronize()
    want = _host(eager)
    out = _outputs(tr, xr, device)
    side = torch.cuda.Stream(device=device)
    side.wait_stream(torch.cuda.current_stream(device))
    with torch.cuda.stream(side):  # warm-up on the side stream, as torch's graph API asks
        _path(tr, xr, xt, g, out)
    torch.cuda.current_stream(device).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _path(tr, xr, xt, g, out)
    for rep in range(4):
        for v in out.values():  # eager work between replays: overwrite every output
            v.fill_(0x5A if v.dtype == torch.uint8 else 3)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _host(out)
        for k in want:
            assert np.array_equal(got[k], want[k]), (rep, k)
    del graph
