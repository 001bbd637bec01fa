"""The MXFP4, MXFP8 and b-cached-low-bits variants at full workload sizes: the KV
cache workload (2 x 131072 x 512) and the ragged large-hidden workload
(65573 x 7168, half of the training values placed near codeword midpoints),
every element of every output against the oracle, bit for bit
(``tests/full_compare.py``)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.full_compare import compare_variant_every_element
from tests.gpu_util import to_np_u8, to_np_u16
from tests.workload_place import oracle_block_scales, place_kv, place_near_midpoints

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _mx_site(name, x_roll, x_train, kind):
    import fp4_rollout_guided_amd as tr
    rows, cols = x_roll.shape
    _say(f"case {name}: {'MXFP4' if kind == 'mx' else 'MXFP8'} {rows}x{cols}, every element")
    cap, gfwd, ffwd = ((tr.mx_capture, tr.mx_guided_fakequant_fwd, tr.mx_full_info_fakequant_fwd) if kind == "mx" else
                       (tr.mx8_capture, tr.mx8_guided_fakequant_fwd, tr.mx8_full_info_fakequant_fwd))
    sc, bt, cd = cap(x_roll, want_codes=True)
    yg, mg, qg = gfwd(x_train, sc, bt, want_codes=True)
    yf, mf, qf = ffwd(x_train, sc, cd, want_codes=True)
    torch.cuda.synchronize()
    got = {"scales": to_np_u8(sc), "bits": to_np_u8(bt), "codes": to_np_u8(cd),
           "y_g": to_np_u16(yg), "m_g": to_np_u8(mg), "q_g": to_np_u8(qg),
           "y_f": to_np_u16(yf), "m_f": to_np_u8(mf), "q_f": to_np_u8(qf)}
    compare_variant_every_element(name, kind, to_np_u16(x_roll), to_np_u16(x_train), got)


def _lowbits_site(name, x_roll, x_train, nbits):
    import fp4_rollout_guided_amd as tr
    rows, cols = x_roll.shape
    _say(f"case {name}: b = {nbits} low bits {rows}x{cols}, every element")
    ts = tr.tensor_scale(x_roll)
    sc, pl, _ = tr.capture_lowbits(x_roll, ts, nbits)
    y, m, q = tr.lowbits_fakequant_fwd(x_train, sc, ts, nbits, pl, want_codes=True)
    torch.cuda.synchronize()
    xr = to_np_u16(x_roll)
    ts_oracle = np.float32(oracle.tensor_scale(xr))   # the oracle's own tensor scale, never the GPU's
    assert ts.cpu().numpy().view(np.uint32)[0] == ts_oracle.view(np.uint32), name
    got = {"scales": to_np_u8(sc), "planes": to_np_u8(pl), "y": to_np_u16(y), "mask": to_np_u8(m),
           "codes": to_np_u8(q)}
    compare_variant_every_element(name, "lowbits", xr, to_np_u16(x_train), got, extra=(ts_oracle, nbits))


@pytest.fixture(scope="module")
def large_hidden(device):
    x_roll = workloads.large_hidden_rollout(device)
    _, s_block = oracle_block_scales(x_roll)
    return x_roll, place_near_midpoints(x_roll, s_block)


def test_mx_large_hidden(device, large_hidden):
    _mx_site("large hidden", *large_hidden, kind="mx")


def test_mx8_large_hidden(device, large_hidden):
    _mx_site("large hidden", *large_hidden, kind="mx8")


@pytest.mark.parametrize("nbits", [2, 3])
def test_lowbits_large_hidden(device, large_hidden, nbits):
    _lowbits_site("large hidden", *large_hidden, nbits=nbits)


@pytest.mark.parametrize("which", ["k", "v"])
def test_variants_kv_cache(device, which):
    x_roll = workloads.kv_cache_rollout(device, which)
    _, s_block = oracle_block_scales(x_roll)
    x_train = place_kv(x_roll, which, s_block)
    shape2d = (x_roll.shape[0], x_roll.shape[1] * x_roll.shape[2])
    _mx_site(f"KV cache {which}", x_roll.reshape(shape2d), x_train.reshape(shape2d), kind="mx")
    _mx_site(f"KV cache {which}", x_roll.reshape(shape2d), x_train.reshape(shape2d), kind="mx8")
    _lowbits_site(f"KV cache {which}", x_roll.reshape(shape2d), x_train.reshape(shape2d), nbits=2)
