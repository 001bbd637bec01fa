"""Helpers shared by the GPU parity tests: run the whole path through the
C ABI (via the binding) and run the oracle on the same inputs."""
import numpy as np
import torch

import oracle


def to_np_u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)


def to_np_u8(t):
    return t.contiguous().cpu().numpy().reshape(-1)


def from_np_u16(a, device, shape=None):
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return t.reshape(shape) if shape is not None else t


def gpu_path(x_roll, x_train, grad, ts=None, want_codes=True):
    """Run tensor scale, capture, guided and RNE forward and STE backward (on
    the guided mask) on device tensors; return host copies."""
    import fp4_rollout_guided_amd as tr
    ts_gpu = tr.tensor_scale(x_roll) if ts is None else ts
    scales, bits, codes = tr.capture(x_roll, ts_gpu, want_codes=want_codes)
    y_g, m_g, q_g = tr.guided_fakequant_fwd(x_train, scales, ts_gpu, bits, want_codes=True)
    y_r, m_r, q_r = tr.rne_fakequant_fwd(x_train, scales, ts_gpu, want_codes=True)
    if want_codes:
        y_f, m_f, q_f = tr.full_info_fakequant_fwd(x_train, scales, ts_gpu, codes, want_codes=True)
    gin = tr.ste_bwd(grad, m_g)
    torch.cuda.synchronize()
    out = {
        "ts": ts_gpu.cpu().numpy().view(np.uint32)[0],
        "scales": to_np_u8(scales), "bits": to_np_u8(bits),
        "y_g": to_np_u16(y_g), "mask_g": to_np_u8(m_g), "q_g": to_np_u8(q_g),
        "y_r": to_np_u16(y_r), "mask_r": to_np_u8(m_r), "q_r": to_np_u8(q_r),
        "gin": to_np_u16(gin),
    }
    if want_codes:
        out["codes"] = to_np_u8(codes)
        out.update({"y_f": to_np_u16(y_f), "mask_f": to_np_u8(m_f), "q_f": to_np_u8(q_f)})
    return out


def oracle_path(xr, xt, g, ts=None, want_codes=True):
    """The same path on host arrays of bf16 bits."""
    ts = oracle.tensor_scale(xr) if ts is None else np.float32(ts)
    cap = oracle.capture(xr, ts, with_codes=want_codes)
    gd = oracle.guided_fwd(xt, cap["scales"], ts, cap["bits"])
    rn = oracle.rne_fwd(xt, cap["scales"], ts)
    out = {
        "ts": np.float32(ts).view(np.uint32),
        "scales": cap["scales"], "bits": cap["bits"],
        "y_g": gd["y"], "mask_g": gd["mask"], "q_g": gd["codes"],
        "y_r": rn["y"], "mask_r": rn["mask"], "q_r": rn["codes"],
        "gin": oracle.ste_bwd(g, gd["mask"], xt.size),
    }
    if want_codes:
        out["codes"] = cap["codes"]
        fi = oracle.full_info_fwd(xt, cap["scales"], ts, cap["codes"])
        out.update({"y_f": fi["y"], "mask_f": fi["mask"], "q_f": fi["codes"]})
    return out


def assert_same(got, want, keys=None, ctx=""):
    keys = keys or [k for k in want if k in got]
    for k in keys:
        a, b = np.asarray(got[k]), np.asarray(want[k])
        assert a.shape == b.shape, (ctx, k, a.shape, b.shape)
        if not np.array_equal(a, b):
            bad = np.flatnonzero(a.reshape(-1) != b.reshape(-1))
            raise AssertionError(f"{ctx}: {k} differs at {bad.size} of {b.size} positions; first {bad[:8].tolist()} "
                                 f"got {a.reshape(-1)[bad[:8]].tolist()} want {b.reshape(-1)[bad[:8]].tolist()}")
