"""trace_tensor_scale_noalloc (the tensor scale for callers that cannot
allocate: its partial maxima go to the library's per-GPU scratch array)
against trace_tensor_scale (caller-provided workspace) and the oracle, bit
for bit, on consecutive calls that share the scratch array: a large tensor,
then a smaller one (whose call reads only the words it wrote), then the
large one again on another stream of the same device, and an empty tensor."""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F
from tests.gpu_util import from_np_u16

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _bits(t):
    return int(t.cpu().numpy().view(np.uint32)[0])


def _tensor(rng, n, peak):
    v = rng.standard_normal(n).astype(np.float32)
    v[rng.integers(0, n)] = peak
    v[rng.integers(0, n, 3)] = np.nan
    return F.f32_to_bf16_rne(v)


def test_noalloc_tensor_scale_matches_the_workspace_entry_point(device):
    import fp4_rollout_guided_amd as tr
    rng = np.random.default_rng(2026)
    big = _tensor(rng, 4096 * 6000 + 48, -3.0e5)        # more tiles than the scratch array's 1536 words
    small = _tensor(rng, 4096 * 3 + 16, 77.0)           # four partial words
    tiny = _tensor(rng, 16, 0.5)                        # one partial word
    stream2 = torch.cuda.Stream(device)
    for i, (name, x, stream) in enumerate((("large", big, None), ("small", small, None), ("tiny", tiny, None),
                                           ("large again, second stream", big, stream2))):
        _say(f"case no-alloc call {i}: {name}, {x.size} elements")
        xd = from_np_u16(x, device)
        with torch.cuda.stream(stream if stream is not None else torch.cuda.current_stream(device)):
            got = tr.tensor_scale_noalloc(xd)
            ref = tr.tensor_scale(xd)
        torch.cuda.synchronize()
        want = np.float32(oracle.tensor_scale(x)).view(np.uint32)
        assert _bits(got) == _bits(ref) == int(want), (name, hex(_bits(got)), hex(_bits(ref)), hex(int(want)))
    empty = torch.empty(0, dtype=torch.bfloat16, device=device)
    out = torch.full((1,), 7.0, device=device)
    tr.tensor_scale_noalloc(empty, out=out)
    torch.cuda.synchronize()
    assert out.item() == 0.0
