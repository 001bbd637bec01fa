"""GPU parity of the trainer-side record gather: the HIP gather (through the
C ABI) against ``oracle.gather_records``, byte for byte, with permuted,
repeated and out-of-range row indices, with and without 4-bit codes; and the
gathered record driving the guided forward on rows in the trainer's order."""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F
from tests.gpu_util import from_np_u16, to_np_u8, to_np_u16

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _index(rng, src_rows, dst_rows):
    idx = rng.integers(0, max(src_rows, 1), dst_rows).astype(np.int64)
    if dst_rows >= 4:
        idx[0] = -1
        idx[1] = src_rows
        idx[2] = np.iinfo(np.int64).max
        idx[3] = np.iinfo(np.int64).min
    return idx


@pytest.mark.parametrize("src_rows,dst_rows,cols", [(1, 1, 16), (9, 40, 48), (300, 257, 4112), (64, 64, 7168),
                                                    (0, 5, 32), (1000, 3, 2048)])
@pytest.mark.parametrize("with_codes", [False, True])
def test_gather_records_bit_exact(device, src_rows, dst_rows, cols, with_codes):
    _say("case gather", src_rows, dst_rows, cols, with_codes)
    import fp4_rollout_guided_amd as tr
    rng = np.random.default_rng(src_rows * 7919 + dst_rows * 31 + cols + with_codes)
    n = src_rows * cols
    rec = {"bits": rng.integers(0, 256, n // 8, dtype=np.uint8),
           "scales": rng.integers(0, 256, n // 16, dtype=np.uint8),
           "codes": rng.integers(0, 256, n // 2, dtype=np.uint8) if with_codes else None}
    idx = _index(rng, src_rows, dst_rows)
    dev = lambda a: torch.from_numpy(a).to(device)
    got = tr.gather_records(dev(rec["bits"]), dev(rec["scales"]), dev(rec["codes"]) if with_codes else None, cols,
                            dev(idx))
    torch.cuda.synchronize()
    want = oracle.gather_records(rec, idx, src_rows, cols)
    for name, g in zip(("bits", "scales", "codes"), got):
        if name == "codes" and not with_codes:
            assert g is None
            continue
        np.testing.assert_array_equal(to_np_u8(g), want[name], err_msg=name)


def test_gathered_record_drives_guided_fwd(device):
    """Rollout rows captured in one order, trained in another: the guided
    forward over the gathered record equals the oracle's on the same rows."""
    _say("case gather+guided")
    import fp4_rollout_guided_amd as tr
    rng = np.random.default_rng(77)
    rows, cols = 96, 4096 + 48
    xr = F.f32_to_bf16_rne(rng.standard_normal(rows * cols).astype(np.float32))
    idx = rng.permutation(rows).astype(np.int64)[: rows - 10]
    xt_rows = F.bf16_to_f32(xr).reshape(rows, cols)[idx] * (1 + 0.02 * rng.standard_normal((idx.size, cols)))
    xt = F.f32_to_bf16_rne(xt_rows.astype(np.float32).reshape(-1))
    ts = oracle.tensor_scale(xr)
    cap = oracle.capture(xr, ts, with_codes=True)
    want_rec = oracle.gather_records(cap, idx, rows, cols)
    want = oracle.guided_fwd(xt, want_rec["scales"], ts, want_rec["bits"])
    want_fi = oracle.full_info_fwd(xt, want_rec["scales"], ts, want_rec["codes"])

    x_roll = from_np_u16(xr, device, (rows, cols))
    x_train = from_np_u16(xt, device, (idx.size, cols))
    ts_gpu = tr.tensor_scale(x_roll)
    scales, bits, codes = tr.capture(x_roll, ts_gpu, want_codes=True)
    b2, s2, c2 = tr.gather_records(bits, scales, codes, cols, torch.from_numpy(idx).to(device))
    y, mask, q = tr.guided_fakequant_fwd(x_train, s2, ts_gpu, b2, want_codes=True)
    yf, maskf, qf = tr.full_info_fakequant_fwd(x_train, s2, ts_gpu, c2, want_codes=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np_u16(y), want["y"])
    np.testing.assert_array_equal(to_np_u8(mask), want["mask"])
    np.testing.assert_array_equal(to_np_u8(q), want["codes"])
    np.testing.assert_array_equal(to_np_u16(yf), want_fi["y"])
    np.testing.assert_array_equal(to_np_u8(maskf), want_fi["mask"])
    np.testing.assert_array_equal(to_np_u8(qf), want_fi["codes"])
