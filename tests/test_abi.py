"""C-ABI checks that need no GPU: the library loads, exports every entry
point declared in include/trace.h, and rejects bad arguments before making
any HIP call (the fake device addresses below are never dereferenced)."""
import ctypes
import os
import re

import pytest

import fp4_rollout_guided_amd as tr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
L = tr.lib
A = 0x7F0000000000          # fake, 256-byte aligned "device" addresses
OK, E_NULL, E_SHAPE, E_ALIGN, E_ALIAS = 0, 1, 2, 3, 4


def P(v):
    return ctypes.c_void_p(v)


def declared_symbols():
    with open(os.path.join(ROOT, "include", "trace.h")) as fh:
        text = fh.read()
    return sorted(set(re.findall(r"TRACE_API\s+[\w\s\*]+?\b(trace_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_symbols()
    assert len(names) >= 10
    raw = ctypes.CDLL(tr.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_version_and_status_strings():
    assert tr.abi_version() == 10
    for code in range(6):
        assert L.trace_status_string(code).decode().startswith("TRACE")
    assert b"unknown" in L.trace_status_string(99)
    assert L.trace_last_hip_error() == 0


def test_workspace_size():
    assert L.trace_tensor_scale_workspace_bytes(0) == 4
    assert L.trace_tensor_scale_workspace_bytes(16) == 4
    assert L.trace_tensor_scale_workspace_bytes(4096 * 2) == 8
    big = L.trace_tensor_scale_workspace_bytes(1 << 34)
    assert 4 <= big <= 4 * 4096


def test_tensor_scale_noalloc_validation():
    f = L.trace_tensor_scale_noalloc
    assert f(None, 4096, P(A + 0x200000), None) == E_NULL
    assert f(P(A), 4096, None, None) == E_NULL
    assert f(P(A), -16, P(A + 0x200000), None) == E_SHAPE
    assert f(P(A), 4095, P(A + 0x200000), None) == E_SHAPE
    assert f(P(A + 8), 4096, P(A + 0x200000), None) == E_ALIGN
    assert f(P(A), 4096, P(A + 0x200002), None) == E_ALIGN
    assert f(P(A), 4096, P(A + 0x100), None) == E_ALIAS      # ts_out inside x
    assert L.trace_tensor_scale_workspace_bytes(1 << 40) <= 6144  # every size fits the 6 KiB scratch


def test_tensor_scale_validation():
    f = L.trace_tensor_scale
    ws = L.trace_tensor_scale_workspace_bytes(4096)
    assert f(None, 4096, P(A + 0x100000), ws, P(A + 0x200000), None) == E_NULL
    assert f(P(A), 4096, None, ws, P(A + 0x200000), None) == E_NULL
    assert f(P(A), 4096, P(A + 0x100000), ws, None, None) == E_NULL
    assert f(P(A), -16, P(A + 0x100000), ws, P(A + 0x200000), None) == E_SHAPE
    assert f(P(A), 4095, P(A + 0x100000), ws, P(A + 0x200000), None) == E_SHAPE
    assert f(P(A), 1 << 20, P(A + 0x100000), 3, P(A + 0x200000), None) == E_SHAPE
    assert f(P(A + 2), 4096, P(A + 0x100000), ws, P(A + 0x200000), None) == E_ALIGN
    assert f(P(A), 4096, P(A + 0x100001), ws, P(A + 0x200000), None) == E_ALIGN
    assert f(P(A), 4096, P(A + 0x100000), ws, P(A + 0x200002), None) == E_ALIGN
    # ts_out inside x
    assert f(P(A), 4096, P(A + 0x100000), ws, P(A + 64), None) == E_ALIAS


def test_capture_validation():
    f = L.trace_capture
    x, ts, sc, bt, cd = A, A + 0x100000, A + 0x200000, A + 0x300000, A + 0x400000
    assert f(None, 4, 32, P(ts), P(sc), P(bt), None, None) == E_NULL
    assert f(P(x), 4, 32, None, P(sc), P(bt), None, None) == E_NULL
    assert f(P(x), 4, 32, P(ts), None, P(bt), None, None) == E_NULL
    assert f(P(x), 4, 32, P(ts), P(sc), None, None, None) == E_NULL
    assert f(P(x), 4, 24, P(ts), P(sc), P(bt), None, None) == E_SHAPE
    assert f(P(x), -1, 32, P(ts), P(sc), P(bt), None, None) == E_SHAPE
    assert f(P(x), 1 << 62, 1 << 4, P(ts), P(sc), P(bt), None, None) == E_SHAPE
    assert f(P(x + 8), 4, 32, P(ts), P(sc), P(bt), None, None) == E_ALIGN
    assert f(P(x), 4, 32, P(ts), P(sc), P(bt + 1), None, None) == E_ALIGN
    assert f(P(x), 4, 32, P(ts), P(sc), P(bt), P(cd + 4), None) == E_ALIGN
    assert f(P(x), 4, 32, P(ts), P(x + 16), P(bt), None, None) == E_ALIAS      # scales inside x
    assert f(P(x), 4, 32, P(ts), P(sc), P(sc + 4), None, None) == E_ALIAS     # bits over scales
    assert f(P(x), 4, 32, P(ts), P(sc), P(bt), P(bt + 8), None) == E_ALIAS    # codes over bits
    assert f(P(x), 4, 32, P(sc + 4), P(sc), P(bt), None, None) == E_ALIAS     # scales over ts
    # empty tensors are a no-op that makes no HIP call and accepts NULL buffers
    assert f(P(x), 0, 32, P(ts), P(sc), P(bt), None, None) == OK
    assert f(P(x), 7, 0, P(ts), P(sc), P(bt), None, None) == OK
    assert f(None, 0, 32, None, None, None, None, None) == OK
    assert f(None, 0, 24, None, None, None, None, None) == E_SHAPE


@pytest.mark.parametrize("mode", ["guided", "rne", "full"])
def test_fakequant_validation(mode):
    guided = mode != "rne"
    x, sc, ts, bt, y, mk, qc = (A, A + 0x100000, A + 0x200000, A + 0x300000, A + 0x400000,
                                A + 0x500000, A + 0x600000)

    def call(x=x, rows=4, cols=32, sc=sc, ts=ts, bt=bt, y=y, mk=mk, qc=None):
        args = [P(x) if x is not None else None, rows, cols, P(sc) if sc is not None else None,
                P(ts) if ts is not None else None]
        if guided:
            args.append(P(bt) if bt is not None else None)
        args += [P(y) if y is not None else None, P(mk) if mk is not None else None,
                 P(qc) if qc is not None else None, None]
        fn = {"guided": L.trace_guided_fakequant_fwd, "rne": L.trace_rne_fakequant_fwd,
              "full": L.trace_full_info_fakequant_fwd}[mode]
        return fn(*args)

    assert call(x=None) == E_NULL
    assert call(sc=None) == E_NULL
    assert call(ts=None) == E_NULL
    assert call(y=None) == E_NULL
    assert call(mk=None) == E_NULL
    if guided:
        assert call(bt=None) == E_NULL
        assert call(bt=bt + 1) == E_ALIGN
    if mode == "full":
        assert call(bt=bt + 2) == E_ALIGN          # codes need 8-byte alignment
        assert call(bt=y + 64) == E_ALIAS         # codes inside y
    assert call(cols=40) == E_SHAPE
    assert call(rows=-2) == E_SHAPE
    assert call(x=x + 4) == E_ALIGN
    assert call(y=y + 8) == E_ALIGN
    assert call(mk=mk + 1) == E_ALIGN
    assert call(qc=qc + 2) == E_ALIGN
    assert call(y=x + 32) == E_ALIAS          # partial overlap with x
    assert call(mk=sc) == E_ALIAS             # mask over scales
    assert call(qc=y + 64) == E_ALIAS         # qcodes inside y
    assert call(mk=y + 16) == E_ALIAS
    assert call(rows=0) == OK
    assert call(rows=0, x=None, y=None, mk=None, sc=None) == OK
    assert call(rows=0, y=x) == OK            # exact in-place is allowed


def test_ste_validation():
    f = L.trace_ste_bwd
    g, m, gi = A, A + 0x100000, A + 0x200000
    assert f(None, P(m), 64, P(gi), None) == E_NULL
    assert f(P(g), None, 64, P(gi), None) == E_NULL
    assert f(P(g), P(m), 64, None, None) == E_NULL
    assert f(P(g), P(m), 60, P(gi), None) == E_SHAPE
    assert f(P(g), P(m), -16, P(gi), None) == E_SHAPE
    assert f(P(g + 2), P(m), 64, P(gi), None) == E_ALIGN
    assert f(P(g), P(m + 1), 64, P(gi), None) == E_ALIGN
    assert f(P(g), P(m), 64, P(g + 16), None) == E_ALIAS
    assert f(P(g), P(m), 64, P(m - 32), None) == E_ALIAS
    assert f(P(g), P(m), 0, P(gi), None) == OK
    assert f(P(g), P(m), 0, P(g), None) == OK
    assert f(None, None, 0, None, None) == OK


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros(4, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        tr.capture(x, torch.zeros(1))
    with pytest.raises(TypeError):
        tr.ste_bwd(torch.zeros(32), torch.zeros(4, dtype=torch.uint8))


def test_gather_records_validation():
    f = L.trace_gather_records
    bs, ss, cs, idx, bd, sd, cd = (A, A + 0x100000, A + 0x200000, A + 0x300000, A + 0x400000, A + 0x500000,
                                   A + 0x600000)

    def call(bs=bs, ss=ss, cs=None, src_rows=8, cols=64, idx=idx, dst_rows=5, bd=bd, sd=sd, cd=None):
        q = lambda v: P(v) if v is not None else None
        return f(q(bs), q(ss), q(cs), src_rows, cols, q(idx), dst_rows, q(bd), q(sd), q(cd), None)

    assert call(idx=None) == E_NULL
    assert call(bd=None) == E_NULL
    assert call(cs=cs) == E_NULL          # codes source without a destination
    assert call(cd=cd) == E_NULL          # codes destination without a source
    assert call(cols=40) == E_SHAPE
    assert call(dst_rows=-1) == E_SHAPE
    assert call(idx=idx + 4) == E_ALIGN
    assert call(bd=bd + 1) == E_ALIGN
    assert call(cs=cs, cd=cd + 4) == E_ALIGN
    assert call(bd=bs + 8) == E_ALIAS     # destination over source plane
    assert call(sd=idx + 8) == E_ALIAS    # destination over the index array
    assert call(dst_rows=0) == OK


def test_gathered_fwd_validation():
    """Every call below is rejected before any HIP call, or is a no-op."""
    x, idx, off, sc, ts, sd, y, mk, qc = (A + k * 0x1000000 for k in range(9))

    def call(f=L.trace_gathered_guided_fakequant_fwd, x=x, rows=8, cols=64, idx=idx, src_rows=6, off=None, groups=0,
             sc=sc, ts=ts, sd=sd, y=y, mk=mk, qc=None):
        q = lambda v: P(v) if v is not None else None
        return f(q(x), rows, cols, q(idx), src_rows, q(off), groups, q(sc), q(ts), q(sd), q(y), q(mk), q(qc), None)

    full = L.trace_gathered_full_info_fakequant_fwd
    assert call(idx=None) == E_NULL
    assert call(ts=None) == E_NULL
    assert call(sd=None) == E_NULL
    assert call(groups=3) == E_NULL                    # groups without offsets
    assert call(off=off, groups=0) == E_SHAPE
    assert call(cols=40) == E_SHAPE
    assert call(rows=-1) == E_SHAPE
    assert call(src_rows=-1) == E_SHAPE
    assert call(rows=1 << 40, cols=1 << 16) == E_SHAPE  # rows * (cols/8)^2 reaches 2^64
    assert call(idx=idx + 4) == E_ALIGN
    assert call(x=x + 8) == E_ALIGN
    assert call(mk=mk + 1) == E_ALIGN
    assert call(off=off + 4, groups=2) == E_ALIGN
    assert call(f=full, sd=sd + 4) == E_ALIGN          # codes 8-byte aligned
    assert call(y=idx + 16) == E_ALIAS                 # output over the index array
    assert call(mk=sc) == E_ALIAS                      # mask over the source scale bytes
    assert call(qc=off, off=off, groups=2) == E_ALIAS  # qcodes over the offsets
    assert call(rows=0) == OK
    # the RNE forward reads no side plane (its signature has none)
    rne = L.trace_gathered_rne_fakequant_fwd
    q = lambda v: P(v) if v is not None else None

    def call_rne(x=x, rows=8, cols=64, idx=idx, src_rows=6, off=None, groups=0, sc=sc, ts=ts, y=y, mk=mk):
        return rne(q(x), rows, cols, q(idx), src_rows, q(off), groups, q(sc), q(ts), q(y), q(mk), None, None)

    assert call_rne(sc=None) == E_NULL
    assert call_rne(idx=None) == E_NULL
    assert call_rne(groups=2) == E_NULL
    assert call_rne(cols=24) == E_SHAPE
    assert call_rne(idx=idx + 2) == E_ALIGN
    assert call_rne(mk=sc) == E_ALIAS
    assert call_rne(rows=0) == OK


def test_build_script_loads_without_the_library():
    """build() must work on a fresh tree (no libtrace.so yet): the build
    script is loaded by path and does not import the binding."""
    import subprocess, sys, os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import sys, __graft_entry__ as g; m = g._build_module(); "
            "assert 'fp4_rollout_guided_amd' not in sys.modules; assert m.LIB.endswith('libtrace.so')")
    subprocess.run([sys.executable, "-c", code], cwd=root, check=True)


def test_grouped_validation():
    x, off, ts, sc, bi, cd, y, mk = (A + k * 0x1000000 for k in range(8))
    cap = L.trace_grouped_capture
    assert cap(P(x), 64, 32, None, 4, P(ts), P(sc), P(bi), None, None) == E_NULL
    assert cap(P(x), 64, 32, P(off), 0, P(ts), P(sc), P(bi), None, None) == E_SHAPE
    assert cap(P(x), 64, 32, P(off), (1 << 20) + 1, P(ts), P(sc), P(bi), None, None) == E_SHAPE
    assert cap(P(x), 64, 32, P(off + 4), 4, P(ts), P(sc), P(bi), None, None) == E_ALIGN
    assert cap(P(x), 64, 40, P(off), 4, P(ts), P(sc), P(bi), None, None) == E_SHAPE
    assert cap(P(x), 0, 32, P(off), 4, P(ts), P(sc), P(bi), None, None) == OK
    assert cap(P(x), 0, 32, P(off), 0, P(ts), P(sc), P(bi), None, None) == E_SHAPE  # groups checked first
    # outputs over the ts array or the offsets are aliasing errors
    assert cap(P(x), 64, 32, P(off), 4, P(ts), P(ts), P(bi), None, None) == E_ALIAS
    assert cap(P(x), 64, 32, P(off), 4, P(ts), P(sc), P(off + 8), None, None) == E_ALIAS
    for fn, side in ((L.trace_grouped_guided_fakequant_fwd, P(bi)), (L.trace_grouped_full_info_fakequant_fwd, P(cd))):
        assert fn(P(x), 64, 32, None, 4, P(sc), P(ts), side, P(y), P(mk), None, None) == E_NULL
        assert fn(P(x), 64, 32, P(off), 4, P(sc), P(ts), None, P(y), P(mk), None, None) == E_NULL
        assert fn(P(x), 64, 32, P(off), -1, P(sc), P(ts), side, P(y), P(mk), None, None) == E_SHAPE
        assert fn(P(x), 64, 32, P(off), 4, P(sc), P(ts), side, P(ts), P(mk), None, None) == E_ALIAS
        assert fn(P(x), 64, 32, P(off), 4, P(sc), P(ts), side, P(y), P(off + 16), None, None) == E_ALIAS
    rne = L.trace_grouped_rne_fakequant_fwd
    assert rne(P(x), 64, 32, P(off), 4, P(sc), P(ts), P(y + 2), P(mk), None, None) == E_ALIGN
    ts_fn = L.trace_grouped_tensor_scale
    ws = L.trace_grouped_tensor_scale_workspace_bytes(64)
    assert ws == 256 and L.trace_grouped_tensor_scale_workspace_bytes(0) == 0
    assert ts_fn(P(x), 64, 32, P(off), 4, P(A + 0x9000000), ws - 4, P(ts), None) == E_SHAPE
    assert ts_fn(P(x), 64, 32, P(off), 4, None, ws, P(ts), None) == E_NULL
    assert ts_fn(P(x), 64, 32, P(off), 4, P(A + 0x9000000), ws, None, None) == E_NULL
    assert ts_fn(P(x), 64, 32, P(off), 4, P(A + 0x9000000), ws, P(ts + 2), None) == E_ALIGN
    assert ts_fn(P(x), 64, 32, P(off), 4, P(x + 64), ws, P(ts), None) == E_ALIAS
    assert ts_fn(P(x), 64, 32, P(off), 4, P(A + 0x9000000), ws, P(off + 24), None) == E_ALIAS


def test_mx_validation():
    x, sc, bi, cd, y, mk = (A + k * 0x1000000 for k in range(6))
    cap = L.trace_mx_capture
    assert cap(P(x), 4, 48, P(sc), P(bi), None, None) == E_SHAPE      # cols % 32
    assert cap(P(x), 4, 64, None, P(bi), None, None) == E_NULL
    assert cap(P(x), 4, 64, P(sc), P(bi + 1), None, None) == E_ALIGN   # bits need 2 bytes
    assert cap(P(x), 4, 64, P(sc), P(bi), P(cd + 4), None) == E_ALIGN  # codes need 8 bytes
    assert cap(P(x), 4, 64, P(sc), P(x + 64), None, None) == E_ALIAS
    assert cap(P(x), 0, 64, None, None, None, None) == OK
    g = L.trace_mx_guided_fakequant_fwd
    assert g(P(x), 4, 64, P(sc), None, P(y), P(mk), None, None) == E_NULL
    assert g(P(x), 4, 64, P(sc), P(bi), P(y), P(mk + 1), None, None) == E_ALIGN
    assert g(P(x), 4, 64, P(sc), P(bi), P(sc), P(mk), None, None) == E_ALIAS
    f = L.trace_mx_full_info_fakequant_fwd
    assert f(P(x), 4, 64, P(sc), P(cd + 4), P(y), P(mk), None, None) == E_ALIGN
    r = L.trace_mx_rne_fakequant_fwd
    assert r(P(x), 4, 80, P(sc), P(y), P(mk), None, None) == E_SHAPE


def test_mx8_validation():
    x, sc, bi, cd, y, mk = (A + k * 0x1000000 for k in range(6))
    cap = L.trace_mx8_capture
    assert cap(P(x), 4, 48, P(sc), P(bi), None, None) == E_SHAPE      # cols % 32
    assert cap(P(x), 4, 64, P(sc), None, None, None) == E_NULL
    assert cap(P(x + 8), 4, 64, P(sc), P(bi), None, None) == E_ALIGN   # bf16 needs 16 bytes
    assert cap(P(x), 4, 64, P(sc), P(bi), P(cd + 8), None) == E_ALIGN  # codes need 16 bytes
    assert cap(P(x), 4, 64, P(sc), P(bi), P(x + 256), None) == E_ALIAS  # 256 code bytes end at x + 512
    assert cap(P(x), 0, 64, None, None, None, None) == OK
    g = L.trace_mx8_guided_fakequant_fwd
    assert g(P(x), 4, 64, P(sc), None, P(y), P(mk), None, None) == E_NULL
    assert g(P(x), 4, 64, P(sc), P(bi), P(y), P(mk), P(cd + 8), None) == E_ALIGN
    assert g(P(x), 4, 64, P(sc), P(bi), P(y), P(mk), P(y + 496), None) == E_ALIAS   # qcodes over y
    f = L.trace_mx8_full_info_fakequant_fwd
    assert f(P(x), 4, 64, P(sc), P(cd + 8), P(y), P(mk), None, None) == E_ALIGN
    assert f(P(x), 4, 64, P(sc), P(cd), P(cd + 240), P(mk), None, None) == E_ALIAS  # y over the rollout codes
    r = L.trace_mx8_rne_fakequant_fwd
    assert r(P(x), 4, 80, P(sc), P(y), P(mk), None, None) == E_SHAPE
    assert r(P(x), -1, 64, P(sc), P(y), P(mk), None, None) == E_SHAPE


def test_mismatch_stats_validation():
    x, sc, ts, bi, cd, st = (A + k * 0x1000000 for k in range(6))
    f = L.trace_mismatch_stats
    assert f(P(x), 4, 40, P(sc), P(ts), P(bi), P(cd), P(st), None) == E_SHAPE
    assert f(P(x), 4, 64, P(sc), P(ts), P(bi), None, P(st), None) == E_NULL
    assert f(P(x), 4, 64, P(sc), P(ts), P(bi), P(cd), None, None) == E_NULL
    assert f(P(x), 4, 64, P(sc), P(ts), P(bi), P(cd), P(st + 4), None) == E_ALIGN
    assert f(P(x), 4, 64, P(sc), P(ts), P(bi), P(cd + 4), P(st), None) == E_ALIGN
    assert f(P(x), 4, 64, P(sc), P(ts), P(bi), P(cd), P(x + 8), None) == E_ALIAS
    assert f(P(x), 4, 64, P(sc), P(ts), P(bi), P(cd), P(cd + 120), None) == E_ALIAS   # codes are 128 bytes
    assert f(P(x), 0, 64, None, None, None, None, None, None) == OK


def test_lowbits_validation():
    x, ts, sc, pl, cd, y, mk = (A + k * 0x1000000 for k in range(7))
    cap = L.trace_capture_lowbits
    assert cap(P(x), 4, 64, P(ts), 0, P(sc), P(pl), None, None) == E_SHAPE
    assert cap(P(x), 4, 64, P(ts), 5, P(sc), P(pl), None, None) == E_SHAPE
    assert cap(P(x), 4, 64, P(ts), 2, P(sc), None, None, None) == E_NULL
    assert cap(P(x), 4, 64, P(ts), 2, P(sc), P(pl + 1), None, None) == E_ALIGN
    assert cap(P(x), 4, 64, P(ts), 3, P(pl + 64), P(pl), None, None) == E_ALIAS   # 3 * 32 bytes > 64
    assert cap(P(x), 0, 64, P(ts), 3, None, None, None, None) == OK
    f = L.trace_lowbits_fakequant_fwd
    assert f(P(x), 4, 64, P(sc), P(ts), 9, P(pl), P(y), P(mk), None, None) == E_SHAPE
    assert f(P(x), 4, 64, P(sc), P(ts), 2, None, P(y), P(mk), None, None) == E_NULL
    assert f(P(x), 4, 64, P(sc), P(ts), 2, P(pl), P(pl + 32), P(mk), None, None) == E_ALIAS  # y over plane 1


def test_header_is_c99_and_links(tmp_path):
    """include/trace.h is a C header: a strict C99 translation unit that
    includes it compiles without warnings, links against libtrace.so and
    reads the ABI version (no GPU call)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "use_trace.c"
    src.write_text('#include "trace.h"\n'
                   "int main(void) { return trace_abi_version() == TRACE_ABI_VERSION ? 0 : 1; }\n")
    exe = tmp_path / "use_trace"
    libdir = os.path.dirname(tr.LIB_PATH)
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    str(src), "-L", libdir, "-l:libtrace.so", f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True)
    assert subprocess.run([str(exe)]).returncode == 0


def _batch(*sites):
    arr = (tr._Site * max(1, len(sites)))()
    for i, s in enumerate(sites):
        arr[i] = tr._Site(*s)
    return arr


def test_batch_validation():
    """trace_tensor_scale_batch / trace_capture_batch: every per-site rule,
    the batch size limit and aliasing across sites, all before any HIP call."""
    ts_b, cap_b, ws_b = L.trace_tensor_scale_batch, L.trace_capture_batch, L.trace_tensor_scale_batch_workspace_bytes
    # site = (x, rows, cols, ts, scales, bits, codes); 4 x 4096 elements each
    good = [(A + k * 0x1000000, 4, 4096, A + 0x8000000 + 16 * k, A + 0x9000000 + k * 0x100000,
             A + 0xA000000 + k * 0x100000, None) for k in range(3)]
    ws = A + 0xB000000
    need = ws_b(_batch(*good), 3)
    assert need == 4 * 3 * 4  # one workgroup per 4096-element tile, 4 tiles per site
    assert ws_b(_batch(*good), 9) == 0  # an invalid batch needs no workspace
    assert ts_b(_batch(), 0, None, 0, None) == OK and cap_b(_batch(), 0, None) == OK
    assert ts_b(None, 2, P(ws), need, None) == E_NULL
    assert cap_b(None, 1, None) == E_NULL
    assert ts_b(_batch(*good), 9, P(ws), need, None) == E_SHAPE
    assert ts_b(_batch(*good), -1, P(ws), need, None) == E_SHAPE
    assert cap_b(_batch(*good), 9, None) == E_SHAPE
    assert ts_b(_batch(*good), 3, P(ws), need - 4, None) == E_SHAPE
    assert ts_b(_batch(*good), 3, None, need, None) == E_NULL
    assert ts_b(_batch(*good), 3, P(ws + 2), need, None) == E_ALIGN
    bad = list(good)
    bad[1] = (good[1][0], 4, 4095) + good[1][3:]
    assert ts_b(_batch(*bad), 3, P(ws), need, None) == E_SHAPE
    bad[1] = (None,) + good[1][1:]
    assert ts_b(_batch(*bad), 3, P(ws), need, None) == E_NULL
    bad[1] = (good[1][0] + 8,) + good[1][1:]
    assert cap_b(_batch(*bad), 3, None) == E_ALIGN
    bad[1] = good[1][:5] + (good[1][5] + 1, None)
    assert cap_b(_batch(*bad), 3, None) == E_ALIGN
    bad[1] = good[1][:4] + (None,) + good[1][5:]
    assert cap_b(_batch(*bad), 3, None) == E_NULL
    # empty sites: NULL data is fine; the tensor scale pass still writes ts
    empty = (None, 0, 4096, A + 0x8000100, None, None, None)
    assert cap_b(_batch(empty, (None, 0, 16, None, None, None, None)), 2, None) == OK
    assert ws_b(_batch(empty), 1) == 0
    assert ts_b(_batch((None, 0, 16, None, None, None, None)), 1, P(ws), 4, None) == E_NULL
    # aliasing across sites: site 2's ts inside site 0's tensor; site 1's bits
    # overlapping site 0's scales; the workspace over a ts; two ts the same
    bad = list(good)
    bad[2] = good[2][:3] + (good[0][0] + 64,) + good[2][4:]
    assert ts_b(_batch(*bad), 3, P(ws), need, None) == E_ALIAS
    bad = list(good)
    bad[1] = good[1][:5] + (good[0][4],) + good[1][6:]
    assert cap_b(_batch(*bad), 3, None) == E_ALIAS
    assert ts_b(_batch(*good), 3, P(good[1][3]), need, None) == E_ALIAS
    bad = list(good)
    bad[1] = good[1][:3] + (good[0][3],) + good[1][4:]
    assert ts_b(_batch(*bad), 3, P(ws), need, None) == E_ALIAS


def test_binding_argument_checks():
    """The binding's check of every tensor argument (the C ABI sees neither
    sizes nor devices): another device than the data's, wrong dtype,
    non-contiguous and short buffers are refused with an exception."""
    import torch
    x = torch.zeros(4, 32, dtype=torch.bfloat16)
    ok = torch.zeros(16, dtype=torch.uint8)
    assert tr._arg(ok, "bits", x, tr._U8, 16) is ok
    with pytest.raises(ValueError, match="must be on"):
        tr._arg(torch.zeros(16, dtype=torch.uint8, device="meta"), "bits", x, tr._U8, 16)
    with pytest.raises(TypeError, match="must be"):
        tr._arg(torch.zeros(16, dtype=torch.int8), "bits", x, tr._U8, 16)
    with pytest.raises(ValueError, match="at least 16"):
        tr._arg(torch.zeros(15, dtype=torch.uint8), "bits", x, tr._U8, 16)
    with pytest.raises(ValueError, match="contiguous"):
        tr._arg(torch.zeros(32, dtype=torch.uint8)[::2], "bits", x, tr._U8, 16)
    with pytest.raises(TypeError, match="tensor"):
        tr._arg(None, "ts", x, tr._F32, 1)
    with pytest.raises(TypeError):
        tr._arg(torch.zeros(1, dtype=torch.float64), "ts", x, tr._F32, 1)
