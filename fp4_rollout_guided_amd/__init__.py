"""Python binding for libtrace (rollout-guided FP4 rounding on MI355X).

Argument marshalling only: every step of the path runs in the HIP kernels of
``libtrace.so`` (built by ``python fp4_rollout_guided_amd/build.py``).  PyTorch
supplies device memory and the current stream.  There is no CPU fallback:
importing this package fails if the library has not been built.

Functions mirror the C ABI in ``include/trace.h``:

    tensor_scale(x)                                  -> ts (fp32[1])
    tensor_scale_noalloc(x)                          -> ts, without a workspace
    capture(x_roll, ts, want_codes=False)            -> (scales, bits, codes)
    guided_fakequant_fwd(x_train, scales, ts, bits)  -> (y, mask, qcodes)
    rne_fakequant_fwd(x_train, scales, ts)           -> (y, mask, qcodes)
    full_info_fakequant_fwd(x_train, scales, ts, codes) -> (y, mask, qcodes)
    gather_records(bits, scales, codes, cols, row_index) -> (bits, scales, codes)
    grouped_tensor_scale(x, offsets)                 -> ts (fp32[groups])
    grouped_capture / grouped_guided_fakequant_fwd / grouped_rne_fakequant_fwd /
    grouped_full_info_fakequant_fwd: as above, with one tensor scale per group
    of rows (per-expert scales of packed MoE rows; offsets int64[groups + 1])
    mx_capture / mx_guided_fakequant_fwd / mx_rne_fakequant_fwd /
    mx_full_info_fakequant_fwd: the MXFP4 variant (32-element blocks, E8M0
    scales, no tensor scale)
    mx8_capture / mx8_guided_fakequant_fwd / mx8_rne_fakequant_fwd /
    mx8_full_info_fakequant_fwd: the MXFP8 (E4M3) activation grid of the W4A8
    setting (32-element blocks, E8M0 scales, one code byte per element)
    tensor_scale_batch(xs)                           -> [ts, ...] (up to 8 sites, one pass)
    capture_batch(xs, tss, want_codes=False)         -> [(scales, bits, codes), ...] (one launch)
    capture_lowbits(x_roll, ts, nbits)               -> (scales, planes, codes)
    lowbits_fakequant_fwd(x_train, scales, ts, nbits, planes) -> (y, mask, qcodes)
    ste_bwd(grad_out, mask)                          -> grad_in
    mismatch_stats(x_train, scales, ts, bits, codes, stats=None) -> stats (int64[20], added to)

and ``GuidedFakeQuant`` wraps the forward/backward pair as an autograd
function.
"""
import ctypes
import os

import torch

__all__ = [
    "TraceError", "LIB_PATH", "SMALLGRID_LIB_PATH", "lib", "load_library", "abi_version", "tensor_scale",
    "tensor_scale_noalloc", "capture",
    "guided_fakequant_fwd", "rne_fakequant_fwd", "full_info_fakequant_fwd", "ste_bwd", "gather_records",
    "gathered_guided_fakequant_fwd", "gathered_rne_fakequant_fwd", "gathered_full_info_fakequant_fwd",
    "grouped_tensor_scale", "grouped_capture", "grouped_guided_fakequant_fwd", "grouped_rne_fakequant_fwd",
    "grouped_full_info_fakequant_fwd", "mx_capture", "mx_guided_fakequant_fwd", "mx_rne_fakequant_fwd",
    "mx_full_info_fakequant_fwd", "mx8_capture", "mx8_guided_fakequant_fwd", "mx8_rne_fakequant_fwd",
    "mx8_full_info_fakequant_fwd", "capture_lowbits", "lowbits_fakequant_fwd", "mismatch_stats", "STAT_FIELDS",
    "GuidedFakeQuant", "tensor_scale_batch", "capture_batch", "MAX_BATCH_SITES",
    "STATUS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtrace.so")
# the same sources with tiny grid caps, for the tests of the grid-stride paths
SMALLGRID_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtrace_smallgrid.so")

STATUS = {0: "TRACE_OK", 1: "TRACE_E_NULL", 2: "TRACE_E_SHAPE", 3: "TRACE_E_ALIGN",
          4: "TRACE_E_ALIAS", 5: "TRACE_E_HIP"}


class TraceError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        msg = lib.trace_status_string(status).decode()
        if status == 5:
            msg += f" (hipError_t {lib.trace_last_hip_error()})"
        super().__init__(f"{what}: {msg}")


def load_library(path):
    """Load a libtrace build and declare its entry points' signatures."""
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python fp4_rollout_guided_amd/build.py` "
            "(libtrace has no CPU fallback)")
    L = ctypes.CDLL(path)
    p, i64, st, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    sig = {
        "trace_abi_version": ([], ctypes.c_int),
        "trace_status_string": ([st], ctypes.c_char_p),
        "trace_last_hip_error": ([], ctypes.c_int),
        "trace_tensor_scale_workspace_bytes": ([i64], sz),
        "trace_tensor_scale": ([p, i64, p, sz, p, p], st),
        "trace_tensor_scale_noalloc": ([p, i64, p, p], st),
        "trace_capture": ([p, i64, i64, p, p, p, p, p], st),
        "trace_guided_fakequant_fwd": ([p, i64, i64, p, p, p, p, p, p, p], st),
        "trace_rne_fakequant_fwd": ([p, i64, i64, p, p, p, p, p, p], st),
        "trace_full_info_fakequant_fwd": ([p, i64, i64, p, p, p, p, p, p, p], st),
        "trace_ste_bwd": ([p, p, i64, p, p], st),
        "trace_gather_records": ([p, p, p, i64, i64, p, i64, p, p, p, p], st),
        "trace_gathered_guided_fakequant_fwd": ([p, i64, i64, p, i64, p, i64, p, p, p, p, p, p, p], st),
        "trace_gathered_full_info_fakequant_fwd": ([p, i64, i64, p, i64, p, i64, p, p, p, p, p, p, p], st),
        "trace_gathered_rne_fakequant_fwd": ([p, i64, i64, p, i64, p, i64, p, p, p, p, p, p], st),
        "trace_grouped_tensor_scale_workspace_bytes": ([i64], sz),
        "trace_grouped_tensor_scale": ([p, i64, i64, p, i64, p, sz, p, p], st),
        "trace_grouped_capture": ([p, i64, i64, p, i64, p, p, p, p, p], st),
        "trace_grouped_guided_fakequant_fwd": ([p, i64, i64, p, i64, p, p, p, p, p, p, p], st),
        "trace_grouped_rne_fakequant_fwd": ([p, i64, i64, p, i64, p, p, p, p, p, p], st),
        "trace_grouped_full_info_fakequant_fwd": ([p, i64, i64, p, i64, p, p, p, p, p, p, p], st),
        "trace_mx_capture": ([p, i64, i64, p, p, p, p], st),
        "trace_capture_lowbits": ([p, i64, i64, p, ctypes.c_int32, p, p, p, p], st),
        "trace_lowbits_fakequant_fwd": ([p, i64, i64, p, p, ctypes.c_int32, p, p, p, p, p], st),
        "trace_mx_guided_fakequant_fwd": ([p, i64, i64, p, p, p, p, p, p], st),
        "trace_mx_rne_fakequant_fwd": ([p, i64, i64, p, p, p, p, p], st),
        "trace_mx_full_info_fakequant_fwd": ([p, i64, i64, p, p, p, p, p, p], st),
        "trace_mx8_capture": ([p, i64, i64, p, p, p, p], st),
        "trace_mismatch_stats": ([p, i64, i64, p, p, p, p, p, p], st),
        "trace_mx8_guided_fakequant_fwd": ([p, i64, i64, p, p, p, p, p, p], st),
        "trace_mx8_rne_fakequant_fwd": ([p, i64, i64, p, p, p, p, p], st),
        "trace_mx8_full_info_fakequant_fwd": ([p, i64, i64, p, p, p, p, p, p], st),
        "trace_tensor_scale_batch_workspace_bytes": ([p, ctypes.c_int32], sz),
        "trace_tensor_scale_batch": ([p, ctypes.c_int32, p, sz, p], st),
        "trace_capture_batch": ([p, ctypes.c_int32, p], st),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    return L


lib = load_library(LIB_PATH)


def abi_version() -> int:
    return lib.trace_abi_version()


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _bf16(t, name):
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must be bf16 (or its raw 16-bit pattern), got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


_U8 = (torch.uint8,)
_F32 = (torch.float32,)
_I64 = (torch.int64,)
_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _arg(t, name, like, dtypes, numel):
    """Check a tensor argument before its pointer reaches the C ABI (which
    sees no sizes or devices): on ``like``'s device, contiguous, of one of
    ``dtypes``, and holding at least ``numel`` elements.  A host tensor
    beside device data, or a short buffer, would otherwise be read or
    written out of bounds by a kernel."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor, got {type(t).__name__}")
    if t.device != like.device:
        raise ValueError(f"{name} must be on {like.device} (the data's device), got {t.device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must be {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} needs at least {numel} elements, got {t.numel()}")
    return t


def _rows_cols(t):
    cols = t.shape[-1] if t.dim() > 0 else 1
    rows = t.numel() // cols if cols else 0
    return rows, cols


def _u8(n, like, out, name):
    if out is None:
        return torch.empty(n, dtype=torch.uint8, device=like.device)
    return _arg(out, name, like, _U8, n)


def _bf16_out(out, like, n, name):
    if out is None:
        return torch.empty_like(like)
    return _arg(out, name, like, _BF16, n)


def _check(status, what):
    if status != 0:
        raise TraceError(status, what)


# --------------------------------------------------------------------------
# entry points
# --------------------------------------------------------------------------

def tensor_scale(x, out=None, workspace=None):
    """ts = fl32(max|x| / 2688) as a float32[1] device tensor."""
    _bf16(x, "x")
    n = x.numel()
    need = lib.trace_tensor_scale_workspace_bytes(n)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    _arg(workspace, "workspace", x, _U8, need)
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=x.device)
    _arg(out, "out", x, _F32, 1)
    _check(lib.trace_tensor_scale(_ptr(x), n, _ptr(workspace), workspace.numel(), _ptr(out), _stream(x)),
           "trace_tensor_scale")
    return out


def tensor_scale_noalloc(x, out=None):
    """``tensor_scale`` without a workspace: the library's per-GPU scratch
    array holds the partial maxima (for callers that cannot allocate; calls
    that overlap on one GPU race)."""
    _bf16(x, "x")
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=x.device)
    _arg(out, "out", x, _F32, 1)
    _check(lib.trace_tensor_scale_noalloc(_ptr(x), x.numel(), _ptr(out), _stream(x)), "trace_tensor_scale_noalloc")
    return out


def capture(x_roll, ts, want_codes=False, scales=None, bits=None, codes=None):
    """Compact rollout record of one site tensor: (scales u8[n/16],
    bits u8[n/8], codes u8[n/2] or None)."""
    _bf16(x_roll, "x_roll")
    rows, cols = _rows_cols(x_roll)
    n = rows * cols
    _arg(ts, "ts", x_roll, _F32, 1)
    scales = _u8(n // 16, x_roll, scales, "scales")
    bits = _u8(n // 8, x_roll, bits, "bits")
    if want_codes or codes is not None:
        codes = _u8(n // 2, x_roll, codes, "codes")
    _check(lib.trace_capture(_ptr(x_roll), rows, cols, _ptr(ts), _ptr(scales), _ptr(bits), _ptr(codes),
                             _stream(x_roll)), "trace_capture")
    return scales, bits, codes


class _Site(ctypes.Structure):
    """trace_site of include/trace.h."""
    _fields_ = [("x", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("ts", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("bits", ctypes.c_void_p),
                ("codes", ctypes.c_void_p)]


MAX_BATCH_SITES = 8


def _sites(xs, tss, records=None):
    if len(xs) > MAX_BATCH_SITES:
        raise ValueError(f"at most {MAX_BATCH_SITES} sites per batch, got {len(xs)}")
    arr = (_Site * max(1, len(xs)))()
    if len(tss) != len(xs) or (records is not None and len(records) != len(xs)):
        raise ValueError("one tensor scale (and record) per site is required")
    for i, x in enumerate(xs):
        _bf16(x, f"xs[{i}]")
        rows, cols = _rows_cols(x)
        n = rows * cols
        _arg(tss[i], f"ts[{i}]", x, _F32, 1)
        sc, bt, cd = records[i] if records is not None else (None, None, None)
        if records is not None:
            _arg(sc, f"scales[{i}]", x, _U8, n // 16)
            _arg(bt, f"bits[{i}]", x, _U8, n // 8)
            if cd is not None:
                _arg(cd, f"codes[{i}]", x, _U8, n // 2)
        arr[i] = _Site(x.data_ptr() if x.numel() else None, rows, cols, tss[i].data_ptr(),
                       None if sc is None else sc.data_ptr(), None if bt is None else bt.data_ptr(),
                       None if cd is None else cd.data_ptr())
    return arr


def tensor_scale_batch(xs, outs=None, workspace=None):
    """Tensor scales of up to 8 site tensors in one pass: a list of
    float32[1] device tensors, each equal to tensor_scale(x)."""
    if not xs:
        return []
    dev = xs[0].device
    outs = outs if outs is not None else [torch.empty(1, dtype=torch.float32, device=dev) for _ in xs]
    arr = _sites(xs, outs)
    need = lib.trace_tensor_scale_batch_workspace_bytes(arr, len(xs))
    if workspace is None:
        workspace = torch.empty(max(4, need), dtype=torch.uint8, device=dev)
    _arg(workspace, "workspace", xs[0], _U8, need)
    _check(lib.trace_tensor_scale_batch(arr, len(xs), _ptr(workspace), workspace.numel(), _stream(xs[0])),
           "trace_tensor_scale_batch")
    return outs


def capture_batch(xs, tss, want_codes=False, records=None):
    """Compact records of up to 8 site tensors in one launch: a list of
    (scales, bits, codes or None), each equal to capture(x, ts)."""
    if not xs:
        return []
    if records is None:
        records = []
        for x in xs:
            n = x.numel()
            records.append((_u8(n // 16, x, None, "scales"), _u8(n // 8, x, None, "bits"),
                            _u8(n // 2, x, None, "codes") if want_codes else None))
    arr = _sites(xs, tss, records)
    _check(lib.trace_capture_batch(arr, len(xs), _stream(xs[0])), "trace_capture_batch")
    return records


def _fwd(mode, x, scales, ts, side, y, mask, want_codes, qcodes):
    _bf16(x, "x_train")
    rows, cols = _rows_cols(x)
    n = rows * cols
    _arg(scales, "scales", x, _U8, n // 16)
    _arg(ts, "ts", x, _F32, 1)
    if mode != "rne":
        _arg(side, "bits" if mode == "guided" else "codes", x, _U8, n // 8 if mode == "guided" else n // 2)
    y = _bf16_out(y, x, n, "y")
    mask = _u8(n // 8, x, mask, "mask")
    if want_codes or qcodes is not None:
        qcodes = _u8(n // 2, x, qcodes, "qcodes")
    if mode == "guided":
        st = lib.trace_guided_fakequant_fwd(_ptr(x), rows, cols, _ptr(scales), _ptr(ts), _ptr(side), _ptr(y),
                                            _ptr(mask), _ptr(qcodes), _stream(x))
    elif mode == "full":
        st = lib.trace_full_info_fakequant_fwd(_ptr(x), rows, cols, _ptr(scales), _ptr(ts), _ptr(side), _ptr(y),
                                               _ptr(mask), _ptr(qcodes), _stream(x))
    else:
        st = lib.trace_rne_fakequant_fwd(_ptr(x), rows, cols, _ptr(scales), _ptr(ts), _ptr(y), _ptr(mask),
                                         _ptr(qcodes), _stream(x))
    _check(st, {"guided": "trace_guided_fakequant_fwd", "full": "trace_full_info_fakequant_fwd",
                "rne": "trace_rne_fakequant_fwd"}[mode])
    return y, mask, qcodes


def guided_fakequant_fwd(x_train, scales, ts, bits, y=None, mask=None, want_codes=False, qcodes=None):
    """Rollout-guided fake-quant forward: (y bf16, mask u8[n/8], qcodes)."""
    return _fwd("guided", x_train, scales, ts, bits, y, mask, want_codes, qcodes)


def rne_fakequant_fwd(x_train, scales, ts, y=None, mask=None, want_codes=False, qcodes=None):
    """Plain round-to-nearest-even fake-quant forward: (y, mask, qcodes)."""
    return _fwd("rne", x_train, scales, ts, None, y, mask, want_codes, qcodes)


def full_info_fakequant_fwd(x_train, scales, ts, codes, y=None, mask=None, want_codes=False, qcodes=None):
    """Full-information guided forward from the rollout's 4-bit codes: (y, mask, qcodes)."""
    return _fwd("full", x_train, scales, ts, codes, y, mask, want_codes, qcodes)


def ste_bwd(grad_out, mask, grad_in=None):
    """Straight-through estimator backward: grad_out where mask is set."""
    _bf16(grad_out, "grad_out")
    n = grad_out.numel()
    _arg(mask, "mask", grad_out, _U8, n // 8)
    grad_in = _bf16_out(grad_in, grad_out, n, "grad_in")
    _check(lib.trace_ste_bwd(_ptr(grad_out), _ptr(mask), grad_out.numel(), _ptr(grad_in), _stream(grad_out)),
           "trace_ste_bwd")
    return grad_in


def gather_records(bits, scales, codes, cols, row_index):
    """Records in the trainer's row order: row r of the result is source row
    row_index[r] (int64 device tensor); out-of-range indices give zero rows."""
    if not row_index.is_cuda or row_index.dtype != torch.int64 or not row_index.is_contiguous():
        raise ValueError("row_index must be a contiguous int64 device tensor")
    src_rows = scales.numel() * 16 // cols if cols else 0
    dst_rows = row_index.numel()
    n = dst_rows * cols
    n_src = src_rows * cols
    _arg(scales, "scales", row_index, _U8, n_src // 16)
    _arg(bits, "bits", row_index, _U8, n_src // 8)
    if codes is not None:
        _arg(codes, "codes", row_index, _U8, n_src // 2)
    bits_d = torch.empty(n // 8, dtype=torch.uint8, device=bits.device)
    scales_d = torch.empty(n // 16, dtype=torch.uint8, device=bits.device)
    codes_d = torch.empty(n // 2, dtype=torch.uint8, device=bits.device) if codes is not None else None
    _check(lib.trace_gather_records(_ptr(bits), _ptr(scales), _ptr(codes), src_rows, cols, _ptr(row_index),
                                    dst_rows, _ptr(bits_d), _ptr(scales_d), _ptr(codes_d), _stream(bits)),
           "trace_gather_records")
    return bits_d, scales_d, codes_d


def _gathered_fwd(mode, x, row_index, scales, ts, side, offsets, y, mask, want_codes, qcodes):
    _bf16(x, "x_train")
    rows, cols = _rows_cols(x)
    _arg(row_index, "row_index", x, _I64, rows)
    if row_index.numel() != rows:
        raise ValueError(f"row_index needs one entry per row of x_train ({rows}), got {row_index.numel()}")
    _arg(scales, "scales", x, _U8, 0)
    src_rows = scales.numel() * 16 // cols if cols else 0
    n, n_src = rows * cols, src_rows * cols
    groups = 0
    if offsets is not None:
        groups = _offsets(offsets, x)
    _arg(ts, "ts", x, _F32, max(groups, 1))
    if mode != "rne":
        _arg(side, "bits" if mode == "guided" else "codes", x, _U8, n_src // 8 if mode == "guided" else n_src // 2)
    y = _bf16_out(y, x, n, "y")
    mask = _u8(n // 8, x, mask, "mask")
    if want_codes or qcodes is not None:
        qcodes = _u8(n // 2, x, qcodes, "qcodes")
    head = (_ptr(x), rows, cols, _ptr(row_index), src_rows, _ptr(offsets), groups, _ptr(scales), _ptr(ts))
    tail = (_ptr(y), _ptr(mask), _ptr(qcodes), _stream(x))
    name = {"guided": "trace_gathered_guided_fakequant_fwd", "full": "trace_gathered_full_info_fakequant_fwd",
            "rne": "trace_gathered_rne_fakequant_fwd"}[mode]
    fn = getattr(lib, name)
    _check(fn(*head, *tail) if mode == "rne" else fn(*head, _ptr(side), *tail), name)
    return y, mask, qcodes


def gathered_guided_fakequant_fwd(x_train, row_index, scales, ts, bits, offsets=None, y=None, mask=None,
                                  want_codes=False, qcodes=None):
    """``guided_fakequant_fwd`` of x_train row r on source row row_index[r]
    of the record (scales, bits; the source's row count is
    scales.numel() * 16 / cols) without a gathered copy; ts is one tensor
    scale, or one per group of source rows when ``offsets`` is given.
    Out-of-range indices give zero-scale blocks."""
    return _gathered_fwd("guided", x_train, row_index, scales, ts, bits, offsets, y, mask, want_codes, qcodes)


def gathered_rne_fakequant_fwd(x_train, row_index, scales, ts, offsets=None, y=None, mask=None, want_codes=False,
                               qcodes=None):
    """``rne_fakequant_fwd`` on source rows row_index[r] of the record's
    scale bytes, as ``gathered_guided_fakequant_fwd``."""
    return _gathered_fwd("rne", x_train, row_index, scales, ts, None, offsets, y, mask, want_codes, qcodes)


def gathered_full_info_fakequant_fwd(x_train, row_index, scales, ts, codes, offsets=None, y=None, mask=None,
                                     want_codes=False, qcodes=None):
    """``full_info_fakequant_fwd`` on source rows row_index[r] of the record
    (scales, codes), as ``gathered_guided_fakequant_fwd``."""
    return _gathered_fwd("full", x_train, row_index, scales, ts, codes, offsets, y, mask, want_codes, qcodes)


def _offsets(offsets, x):
    _arg(offsets, "offsets", x, _I64, 2)
    if offsets.dim() != 1:
        raise ValueError("offsets must be a 1-D int64 device tensor of groups + 1 entries")
    groups = offsets.numel() - 1
    if groups < 1:
        raise ValueError("at least one group is required")
    return groups


def grouped_tensor_scale(x, offsets, out=None, workspace=None):
    """One tensor scale per group of rows: ts[g] = fl32(amax over rows
    [offsets[g], offsets[g+1]) / 2688), as a float32[groups] device tensor."""
    _bf16(x, "x")
    rows, cols = _rows_cols(x)
    groups = _offsets(offsets, x)
    need = lib.trace_grouped_tensor_scale_workspace_bytes(rows)
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=x.device)
    _arg(workspace, "workspace", x, _U8, need)
    if out is None:
        out = torch.empty(groups, dtype=torch.float32, device=x.device)
    _arg(out, "out", x, _F32, groups)
    _check(lib.trace_grouped_tensor_scale(_ptr(x), rows, cols, _ptr(offsets), groups, _ptr(workspace),
                                          workspace.numel(), _ptr(out), _stream(x)), "trace_grouped_tensor_scale")
    return out


def grouped_capture(x_roll, offsets, ts, want_codes=False, scales=None, bits=None, codes=None):
    """``capture`` with ts[group of the row] as each row's tensor scale."""
    _bf16(x_roll, "x_roll")
    rows, cols = _rows_cols(x_roll)
    groups = _offsets(offsets, x_roll)
    n = rows * cols
    _arg(ts, "ts", x_roll, _F32, groups)
    scales = _u8(n // 16, x_roll, scales, "scales")
    bits = _u8(n // 8, x_roll, bits, "bits")
    if want_codes or codes is not None:
        codes = _u8(n // 2, x_roll, codes, "codes")
    _check(lib.trace_grouped_capture(_ptr(x_roll), rows, cols, _ptr(offsets), groups, _ptr(ts), _ptr(scales),
                                     _ptr(bits), _ptr(codes), _stream(x_roll)), "trace_grouped_capture")
    return scales, bits, codes


def _grouped_fwd(mode, x, offsets, scales, ts, side, y, mask, want_codes, qcodes):
    _bf16(x, "x_train")
    rows, cols = _rows_cols(x)
    groups = _offsets(offsets, x)
    n = rows * cols
    _arg(scales, "scales", x, _U8, n // 16)
    _arg(ts, "ts", x, _F32, groups)
    if mode != "rne":
        _arg(side, "bits" if mode == "guided" else "codes", x, _U8, n // 8 if mode == "guided" else n // 2)
    y = _bf16_out(y, x, n, "y")
    mask = _u8(n // 8, x, mask, "mask")
    if want_codes or qcodes is not None:
        qcodes = _u8(n // 2, x, qcodes, "qcodes")
    head = (_ptr(x), rows, cols, _ptr(offsets), groups, _ptr(scales), _ptr(ts))
    tail = (_ptr(y), _ptr(mask), _ptr(qcodes), _stream(x))
    if mode == "guided":
        st, name = lib.trace_grouped_guided_fakequant_fwd(*head, _ptr(side), *tail), "trace_grouped_guided_fakequant_fwd"
    elif mode == "full":
        st, name = (lib.trace_grouped_full_info_fakequant_fwd(*head, _ptr(side), *tail),
                    "trace_grouped_full_info_fakequant_fwd")
    else:
        st, name = lib.trace_grouped_rne_fakequant_fwd(*head, *tail), "trace_grouped_rne_fakequant_fwd"
    _check(st, name)
    return y, mask, qcodes


def grouped_guided_fakequant_fwd(x_train, offsets, scales, ts, bits, y=None, mask=None, want_codes=False,
                                 qcodes=None):
    """``guided_fakequant_fwd`` with one tensor scale per group of rows."""
    return _grouped_fwd("guided", x_train, offsets, scales, ts, bits, y, mask, want_codes, qcodes)


def grouped_rne_fakequant_fwd(x_train, offsets, scales, ts, y=None, mask=None, want_codes=False, qcodes=None):
    """``rne_fakequant_fwd`` with one tensor scale per group of rows."""
    return _grouped_fwd("rne", x_train, offsets, scales, ts, None, y, mask, want_codes, qcodes)


def grouped_full_info_fakequant_fwd(x_train, offsets, scales, ts, codes, y=None, mask=None, want_codes=False,
                                    qcodes=None):
    """``full_info_fakequant_fwd`` with one tensor scale per group of rows."""
    return _grouped_fwd("full", x_train, offsets, scales, ts, codes, y, mask, want_codes, qcodes)


def capture_lowbits(x_roll, ts, nbits, want_codes=False, scales=None, planes=None, codes=None):
    """Capture keeping b = nbits low bits per element: (scales u8[n/16],
    planes u8[nbits * n/8], codes or None)."""
    _bf16(x_roll, "x_roll")
    rows, cols = _rows_cols(x_roll)
    n = rows * cols
    _arg(ts, "ts", x_roll, _F32, 1)
    scales = _u8(n // 16, x_roll, scales, "scales")
    planes = _u8(max(0, nbits) * (n // 8), x_roll, planes, "planes")
    if want_codes or codes is not None:
        codes = _u8(n // 2, x_roll, codes, "codes")
    _check(lib.trace_capture_lowbits(_ptr(x_roll), rows, cols, _ptr(ts), nbits, _ptr(scales), _ptr(planes),
                                     _ptr(codes), _stream(x_roll)), "trace_capture_lowbits")
    return scales, planes, codes


def lowbits_fakequant_fwd(x_train, scales, ts, nbits, planes, y=None, mask=None, want_codes=False, qcodes=None):
    """Guided forward from b = nbits cached low bits: (y, mask, qcodes)."""
    _bf16(x_train, "x_train")
    rows, cols = _rows_cols(x_train)
    n = rows * cols
    _arg(scales, "scales", x_train, _U8, n // 16)
    _arg(ts, "ts", x_train, _F32, 1)
    _arg(planes, "planes", x_train, _U8, max(0, nbits) * (n // 8))
    y = _bf16_out(y, x_train, n, "y")
    mask = _u8(n // 8, x_train, mask, "mask")
    if want_codes or qcodes is not None:
        qcodes = _u8(n // 2, x_train, qcodes, "qcodes")
    _check(lib.trace_lowbits_fakequant_fwd(_ptr(x_train), rows, cols, _ptr(scales), _ptr(ts), nbits, _ptr(planes),
                                           _ptr(y), _ptr(mask), _ptr(qcodes), _stream(x_train)),
           "trace_lowbits_fakequant_fwd")
    return y, mask, qcodes


def mx_capture(x_roll, want_codes=False, scales=None, bits=None, codes=None):
    """MXFP4 capture: (scales u8[n/32] E8M0, bits u8[n/8], codes u8[n/2] or None)."""
    _bf16(x_roll, "x_roll")
    rows, cols = _rows_cols(x_roll)
    n = rows * cols
    scales = _u8(n // 32, x_roll, scales, "scales")
    bits = _u8(n // 8, x_roll, bits, "bits")
    if want_codes or codes is not None:
        codes = _u8(n // 2, x_roll, codes, "codes")
    _check(lib.trace_mx_capture(_ptr(x_roll), rows, cols, _ptr(scales), _ptr(bits), _ptr(codes), _stream(x_roll)),
           "trace_mx_capture")
    return scales, bits, codes


def _mx_fwd(mode, x, scales, side, y, mask, want_codes, qcodes):
    _bf16(x, "x_train")
    rows, cols = _rows_cols(x)
    n = rows * cols
    _arg(scales, "scales", x, _U8, n // 32)
    if mode != "rne":
        _arg(side, "bits" if mode == "guided" else "codes", x, _U8, n // 8 if mode == "guided" else n // 2)
    y = _bf16_out(y, x, n, "y")
    mask = _u8(n // 8, x, mask, "mask")
    if want_codes or qcodes is not None:
        qcodes = _u8(n // 2, x, qcodes, "qcodes")
    tail = (_ptr(y), _ptr(mask), _ptr(qcodes), _stream(x))
    if mode == "guided":
        st, name = lib.trace_mx_guided_fakequant_fwd(_ptr(x), rows, cols, _ptr(scales), _ptr(side), *tail), \
            "trace_mx_guided_fakequant_fwd"
    elif mode == "full":
        st, name = lib.trace_mx_full_info_fakequant_fwd(_ptr(x), rows, cols, _ptr(scales), _ptr(side), *tail), \
            "trace_mx_full_info_fakequant_fwd"
    else:
        st, name = lib.trace_mx_rne_fakequant_fwd(_ptr(x), rows, cols, _ptr(scales), *tail), \
            "trace_mx_rne_fakequant_fwd"
    _check(st, name)
    return y, mask, qcodes


def mx_guided_fakequant_fwd(x_train, scales, bits, y=None, mask=None, want_codes=False, qcodes=None):
    """Rollout-guided forward on MXFP4 scales: (y, mask, qcodes)."""
    return _mx_fwd("guided", x_train, scales, bits, y, mask, want_codes, qcodes)


def mx_rne_fakequant_fwd(x_train, scales, y=None, mask=None, want_codes=False, qcodes=None):
    """Round-to-nearest-even forward on MXFP4 scales: (y, mask, qcodes)."""
    return _mx_fwd("rne", x_train, scales, None, y, mask, want_codes, qcodes)


def mx_full_info_fakequant_fwd(x_train, scales, codes, y=None, mask=None, want_codes=False, qcodes=None):
    """Full-information guided forward on MXFP4 scales: (y, mask, qcodes)."""
    return _mx_fwd("full", x_train, scales, codes, y, mask, want_codes, qcodes)


def mx8_capture(x_roll, want_codes=False, scales=None, bits=None, codes=None):
    """MXFP8 capture: (scales u8[n/32] E8M0, bits u8[n/8], codes u8[n] E4M3FN or None)."""
    _bf16(x_roll, "x_roll")
    rows, cols = _rows_cols(x_roll)
    n = rows * cols
    scales = _u8(n // 32, x_roll, scales, "scales")
    bits = _u8(n // 8, x_roll, bits, "bits")
    if want_codes or codes is not None:
        codes = _u8(n, x_roll, codes, "codes")
    _check(lib.trace_mx8_capture(_ptr(x_roll), rows, cols, _ptr(scales), _ptr(bits), _ptr(codes), _stream(x_roll)),
           "trace_mx8_capture")
    return scales, bits, codes


def _mx8_fwd(mode, x, scales, side, y, mask, want_codes, qcodes):
    _bf16(x, "x_train")
    rows, cols = _rows_cols(x)
    n = rows * cols
    _arg(scales, "scales", x, _U8, n // 32)
    if mode != "rne":
        _arg(side, "bits" if mode == "guided" else "codes", x, _U8, n // 8 if mode == "guided" else n)
    y = _bf16_out(y, x, n, "y")
    mask = _u8(n // 8, x, mask, "mask")
    if want_codes or qcodes is not None:
        qcodes = _u8(n, x, qcodes, "qcodes")
    tail = (_ptr(y), _ptr(mask), _ptr(qcodes), _stream(x))
    if mode == "guided":
        name = "trace_mx8_guided_fakequant_fwd"
        st = lib.trace_mx8_guided_fakequant_fwd(_ptr(x), rows, cols, _ptr(scales), _ptr(side), *tail)
    elif mode == "full":
        name = "trace_mx8_full_info_fakequant_fwd"
        st = lib.trace_mx8_full_info_fakequant_fwd(_ptr(x), rows, cols, _ptr(scales), _ptr(side), *tail)
    else:
        name = "trace_mx8_rne_fakequant_fwd"
        st = lib.trace_mx8_rne_fakequant_fwd(_ptr(x), rows, cols, _ptr(scales), *tail)
    _check(st, name)
    return y, mask, qcodes


def mx8_guided_fakequant_fwd(x_train, scales, bits, y=None, mask=None, want_codes=False, qcodes=None):
    """Rollout-guided forward on the MXFP8 grid: (y, mask, qcodes u8[n])."""
    return _mx8_fwd("guided", x_train, scales, bits, y, mask, want_codes, qcodes)


def mx8_rne_fakequant_fwd(x_train, scales, y=None, mask=None, want_codes=False, qcodes=None):
    """Round-to-nearest-even forward on the MXFP8 grid: (y, mask, qcodes u8[n])."""
    return _mx8_fwd("rne", x_train, scales, None, y, mask, want_codes, qcodes)


def mx8_full_info_fakequant_fwd(x_train, scales, codes, y=None, mask=None, want_codes=False, qcodes=None):
    """Full-information forward on the MXFP8 grid (codes: rollout E4M3FN bytes,
    u8[n]): (y, mask, qcodes u8[n])."""
    return _mx8_fwd("full", x_train, scales, codes, y, mask, want_codes, qcodes)


# Layout of the agreement statistics: hist[0..14], then these counters.
STAT_FIELDS = ("straddle", "crossed", "recovered", "violations", "elements")


def mismatch_stats(x_train, scales, ts, bits, codes, stats=None):
    """Agreement statistics of x_train's RNE / guided / full-information
    codes with the rollout codes, ADDED to ``stats`` (an int64[20] device
    tensor, zeroed here when not given): [0..14] histogram of signed grid
    steps between rollout and RNE codes, then straddle, crossed, recovered,
    violations, elements (the counts are below 2^63)."""
    _bf16(x_train, "x_train")
    rows, cols = _rows_cols(x_train)
    n = rows * cols
    _arg(scales, "scales", x_train, _U8, n // 16)
    _arg(ts, "ts", x_train, _F32, 1)
    _arg(bits, "bits", x_train, _U8, n // 8)
    _arg(codes, "codes", x_train, _U8, n // 2)
    if stats is None:
        stats = torch.zeros(20, dtype=torch.int64, device=x_train.device)
    _arg(stats, "stats", x_train, _I64, 20)
    _check(lib.trace_mismatch_stats(_ptr(x_train), rows, cols, _ptr(scales), _ptr(ts), _ptr(bits), _ptr(codes),
                                    _ptr(stats), _stream(x_train)), "trace_mismatch_stats")
    return stats


class GuidedFakeQuant(torch.autograd.Function):
    """y = s * q* in the forward, straight-through (clip-masked) gradient in
    the backward; the rollout record (scales, ts, bits) is not differentiated."""

    @staticmethod
    def forward(ctx, x_train, scales, ts, bits):
        y, mask, _ = guided_fakequant_fwd(x_train.contiguous(), scales, ts, bits)
        ctx.save_for_backward(mask)
        return y

    @staticmethod
    def backward(ctx, grad_out):
        (mask,) = ctx.saved_tensors
        return ste_bwd(grad_out.contiguous(), mask), None, None, None
