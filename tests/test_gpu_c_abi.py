"""The library from plain C: `_build/trace_c_smoke` (tests/c/trace_c_smoke.c,
built by build() with the host C compiler against include/trace.h and
libtrace.so) allocates with hipMalloc, runs the tensor scale, capture,
guided and RNE forwards and the STE backward on the default stream, with no
PyTorch in the process, and its outputs equal the oracle's bit for bit."""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
from oracle import formats as F
from tests.gpu_util import assert_same, oracle_path

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "_build", "trace_c_smoke")


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def test_c_caller_matches_the_oracle(tmp_path):
    if not os.path.exists(BIN):
        pytest.fail(f"{BIN} is missing: run fp4_rollout_guided_amd/build.py first")
    rows, cols = 97, 2064   # ragged: neither a multiple of the 256-block tile nor of 64 rows
    _say("case C caller", rows, cols)
    rng = np.random.default_rng(2026)
    v = rng.standard_normal((rows, cols)).astype(np.float32)
    v[:, rng.choice(cols, 4, replace=False)] *= 50
    v[5, 7], v[6, 0:16] = np.nan, 0.0
    xr = F.f32_to_bf16_rne(v.reshape(-1))
    t = (v * (1 + 0.02 * rng.standard_normal(v.shape))).astype(np.float32)
    t[7, 3], t[8, 9] = np.inf, -1e30
    xt = F.f32_to_bf16_rne(t.reshape(-1))
    g = F.f32_to_bf16_rne(rng.standard_normal(v.size).astype(np.float32))
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as fh:
        fh.write(np.array([rows, cols], dtype=np.int64).tobytes())
        for a in (xr, xt, g):
            fh.write(a.astype(np.uint16).tobytes())
    p = subprocess.run([BIN, str(inp), str(out)], stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True,
                       timeout=120)
    _say(p.stdout.strip(), p.stderr.strip())
    assert p.returncode == 0, p.stderr
    n = rows * cols
    raw = np.fromfile(out, dtype=np.uint8)
    got, pos = {}, 0

    def take(name, nbytes, dtype=np.uint8):
        nonlocal pos
        got[name] = raw[pos:pos + nbytes].view(dtype).copy()
        pos += nbytes

    take("ts", 4, np.uint32)
    take("scales", n // 16)
    take("bits", n // 8)
    take("codes", n // 2)
    take("y_g", 2 * n, np.uint16)
    take("mask_g", n // 8)
    take("y_r", 2 * n, np.uint16)
    take("mask_r", n // 8)
    take("gin", 2 * n, np.uint16)
    assert pos == raw.size
    got["ts"] = got["ts"][0]
    want = oracle_path(xr, xt, g)
    assert_same(got, want, keys=["ts", "scales", "bits", "codes", "y_g", "mask_g", "y_r", "mask_r", "gin"],
                ctx="C caller")
    assert np.float32(oracle.tensor_scale(xr)).view(np.uint32) == got["ts"]
