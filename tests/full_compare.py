"""Every element of a full-size site against the oracle.

The GPU runs the path; its inputs and outputs are copied once into files
under /dev/shm (memory-backed; the system temp directory when /dev/shm is
missing or too small), and a pool of worker processes maps them read-only:
each worker takes a chunk, recomputes it with the oracle and compares it
with the GPU's bytes itself, returning only whether they are equal (and the
first differences when not).  No array passes through the parent process,
which is what limited the workers before.  The workers are started with the
forkserver method: fresh interpreters that import only NumPy and the oracle,
never the GPU runtime."""
import os
import shutil
import sys
import tempfile
import time

import numpy as np

CPU_SHARE = 16          # host cores granted to a process driving one GPU
CHUNK_ELEMS = 1 << 17   # elements per worker task (a multiple of 32; small chunks keep the oracle's temporaries in cache)

_POOL = None


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _warm(_):
    import oracle  # noqa: F401
    return 0


def pool():
    """A process pool of up to CPU_SHARE oracle workers, created once."""
    global _POOL
    if _POOL is None:
        import multiprocessing as mp
        try:
            cores = len(os.sched_getaffinity(0))
        except AttributeError:
            cores = os.cpu_count() or 1
        cores = max(1, min(cores, CPU_SHARE))
        p = mp.get_context("forkserver").Pool(cores)
        p.map(_warm, range(cores))
        _POOL = (p, cores)
    return _POOL


# --------------------------------------------------------------------------
# shared files
# --------------------------------------------------------------------------

def _nbytes(a):
    return int(a.numel() * a.element_size()) if hasattr(a, "numel") else int(np.asarray(a).nbytes)


class Shared:
    """Flat arrays in files the workers map read-only.  Values are device
    tensors (copied straight into the file) or host arrays; 2-byte elements
    are kept as uint16 bit patterns, everything else as bytes."""

    def __init__(self, arrays):
        need = sum(_nbytes(a) for a in arrays.values())
        self.dir = None
        for base in ("/dev/shm", tempfile.gettempdir()):
            try:
                st = os.statvfs(base)
            except OSError:
                continue
            if st.f_bavail * st.f_frsize >= need + (1 << 30):
                self.dir = tempfile.mkdtemp(prefix="trace_cmp_", dir=base)
                break
        if self.dir is None:
            raise RuntimeError(f"no room for {need} bytes of comparison data in /dev/shm or the temp directory")
        self.specs = {}
        for k, a in arrays.items():
            self.put(k, a)

    def put(self, key, a):
        path = os.path.join(self.dir, key)
        if hasattr(a, "numel"):            # a torch tensor (device or host)
            import torch
            t = a.contiguous().reshape(-1)
            wide = t.element_size() == 2
            t = t.view(torch.int16) if wide else t.view(torch.uint8)
            dt = np.uint16 if wide else np.uint8
            mm = np.memmap(path, dtype=dt, mode="w+", shape=(max(1, t.numel()),))
            if t.numel():
                torch.from_numpy(mm.view(np.int16) if wide else mm).narrow(0, 0, t.numel()).copy_(t)
            n = t.numel()
        else:
            arr = np.ascontiguousarray(a).reshape(-1)
            dt = arr.dtype
            mm = np.memmap(path, dtype=dt, mode="w+", shape=(max(1, arr.size),))
            mm[:arr.size] = arr
            n = arr.size
        mm.flush()
        del mm
        self.specs[key] = (path, np.dtype(dt).str, n)

    def close(self):
        if self.dir:
            shutil.rmtree(self.dir, ignore_errors=True)
            self.dir = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def _read(spec, lo, hi):
    """Elements [lo, hi) of a shared array, copied out of the mapping."""
    path, dt, n = spec
    mm = np.memmap(path, dtype=np.dtype(dt), mode="r", shape=(max(1, n),))
    out = np.array(mm[lo:hi])
    del mm
    return out


# --------------------------------------------------------------------------
# oracle outputs of one chunk, per kind of path
# --------------------------------------------------------------------------

# elements per byte of each output (bytes = elements / per); bf16 outputs and
# outputs not listed are one uint16 per element
_PER = {
    "nvfp4": {"scales": 16, "bits": 8, "codes": 2, "mask_g": 8, "q_g": 2, "mask_r": 8, "q_r": 2, "mask_f": 8,
              "q_f": 2},
    "mx": {"scales": 32, "bits": 8, "codes": 2, "m_g": 8, "q_g": 2, "m_f": 8, "q_f": 2, "m_r": 8, "q_r": 2},
    "mx8": {"scales": 32, "bits": 8, "codes": 1, "m_g": 8, "q_g": 1, "m_f": 8, "q_f": 1, "m_r": 8, "q_r": 1},
    "lowbits": {"scales": 16, "mask": 8, "codes": 2},
}
_PER["grouped"] = _PER["nvfp4"]
_PER["gathered"] = _PER["nvfp4"]


def _oracle_nvfp4(xr, xt, g, ts):
    import oracle
    cap = oracle.capture(xr, ts, with_codes=True)
    gd = oracle.guided_fwd(xt, cap["scales"], ts, cap["bits"])
    rn = oracle.rne_fwd(xt, cap["scales"], ts)
    fi = oracle.full_info_fwd(xt, cap["scales"], ts, cap["codes"])
    return {"scales": cap["scales"], "bits": cap["bits"], "codes": cap["codes"],
            "y_g": gd["y"], "mask_g": gd["mask"], "q_g": gd["codes"],
            "y_r": rn["y"], "mask_r": rn["mask"], "q_r": rn["codes"],
            "y_f": fi["y"], "mask_f": fi["mask"], "q_f": fi["codes"],
            "gin": oracle.ste_bwd(g, gd["mask"], xt.size)}


def _oracle_variant(kind, xr, xt, g, extra):
    import oracle
    if kind in ("mx", "mx8"):
        cap_f, gd_f, rn_f, fi_f = (
            (oracle.mx_capture, oracle.mx_guided_fwd, oracle.mx_rne_fwd, oracle.mx_full_info_fwd) if kind == "mx" else
            (oracle.mx8_capture, oracle.mx8_guided_fwd, oracle.mx8_rne_fwd, oracle.mx8_full_info_fwd))
        cap = cap_f(xr, with_codes=True)
        gd = gd_f(xt, cap["scales"], cap["bits"])
        fi = fi_f(xt, cap["scales"], cap["codes"])
        out = {"scales": cap["scales"], "bits": cap["bits"], "codes": cap["codes"], "y_g": gd["y"],
               "m_g": gd["mask"], "q_g": gd["codes"], "y_f": fi["y"], "m_f": fi["mask"], "q_f": fi["codes"]}
        if extra == "with_rne":
            rn = rn_f(xt, cap["scales"])
            out.update({"y_r": rn["y"], "m_r": rn["mask"], "q_r": rn["codes"]})
        if g is not None:
            out["gin"] = oracle.ste_bwd(g, gd["mask"], xt.size)
        return out
    ts, nbits = extra
    cap = oracle.capture_lowbits(xr, ts, nbits)
    out = oracle.lowbits_fwd(xt, cap["scales"], ts, cap["planes"], nbits)
    return {"scales": cap["scales"], "planes": cap["planes"], "y": out["y"], "mask": out["mask"],
            "codes": out["codes"]}


def _oracle_grouped(xr, xt, rows, cols, off, ts):
    import oracle
    cap = oracle.grouped_capture(xr, rows, cols, off, ts, with_codes=True)
    gd = oracle.grouped_guided_fwd(xt, rows, cols, off, cap["scales"], ts, cap["bits"])
    rn = oracle.grouped_rne_fwd(xt, rows, cols, off, cap["scales"], ts)
    fi = oracle.grouped_full_info_fwd(xt, rows, cols, off, cap["scales"], ts, cap["codes"])
    return {"scales": cap["scales"], "bits": cap["bits"], "codes": cap["codes"],
            "y_g": gd["y"], "mask_g": gd["mask"], "q_g": gd["codes"],
            "y_r": rn["y"], "mask_r": rn["mask"], "q_r": rn["codes"],
            "y_f": fi["y"], "mask_f": fi["mask"], "q_f": fi["codes"]}


def _oracle_gathered(xt, idx, xr_rows_of, cols, src_rows, off, ts):
    """Guided and full-information forwards of destination rows xt (their
    source rows idx) on records read back in place, all from the oracle: the
    record of the distinct source rows the chunk refers to (in ascending
    order, so every group's rows stay together) is the oracle's capture of
    those rows with their groups' scales; the indices are mapped into it."""
    import oracle
    valid = (idx >= 0) & (idx < src_rows)
    u = np.unique(idx[valid])
    xr = xr_rows_of(u)
    if off is None:
        cap = oracle.capture(xr, ts, with_codes=True)
        sub = None
    else:
        group = np.searchsorted(off, u, side="right") - 1
        sub = np.r_[0, np.cumsum(np.bincount(group, minlength=len(off) - 1))].astype(np.int64)
        cap = oracle.grouped_capture(xr, u.size, cols, sub, ts, with_codes=True)
    local = np.full(idx.size, -1, dtype=np.int64)
    local[valid] = np.searchsorted(u, idx[valid])
    gd = oracle.gathered_fwd("guided", xt, cols, cap, u.size, local, ts, sub)
    fi = oracle.gathered_fwd("full", xt, cols, cap, u.size, local, ts, sub)
    rn = oracle.gathered_fwd("rne", xt, cols, cap, u.size, local, ts, sub)
    return {"y_g": gd["y"], "mask_g": gd["mask"], "q_g": gd["codes"],
            "y_f": fi["y"], "mask_f": fi["mask"], "q_f": fi["codes"],
            "y_r": rn["y"], "mask_r": rn["mask"], "q_r": rn["codes"]}


# --------------------------------------------------------------------------
# worker tasks
# --------------------------------------------------------------------------

def _ts_task(args):
    import oracle
    spec, a, b = args
    return np.float32(oracle.tensor_scale(_read(spec, a, b)))


def _check_task(args):
    """Recompute elements [a, b) of a site with the oracle and compare them
    with the GPU's outputs in the shared files.  Returns None when every
    byte is equal, else a description of the first differences."""
    kind, specs, a, b, extra = args
    if kind == "gathered":
        cols, src_rows, off, ts = extra
        r0, r1 = a // cols, b // cols
        idx = _read(specs["idx"], r0, r1)
        path, dt, nx = specs["xr"]

        def rows_of(u):
            mm = np.memmap(path, dtype=np.dtype(dt), mode="r", shape=(max(1, nx),))
            out = np.array(mm[: src_rows * cols].reshape(src_rows, cols)[u]).reshape(-1)
            del mm
            return out

        want = _oracle_gathered(_read(specs["xt"], a, b), idx, rows_of, cols, src_rows, off, ts)
    elif kind == "grouped":
        cols, off, ts = extra
        r0, r1 = a // cols, b // cols
        sub = np.clip(np.asarray(off, dtype=np.int64) - r0, 0, r1 - r0).astype(np.int64)
        want = _oracle_grouped(_read(specs["xr"], a, b), _read(specs["xt"], a, b), r1 - r0, cols, sub, ts)
    else:
        xr, xt = _read(specs["xr"], a, b), _read(specs["xt"], a, b)
        g = _read(specs["g"], a, b) if "g" in specs else None
        want = _oracle_nvfp4(xr, xt, g, extra) if kind == "nvfp4" else _oracle_variant(kind, xr, xt, g, extra)
    per = _PER[kind]
    n = specs["xr"][2]
    for k, w in want.items():
        if k not in specs:
            continue
        if k == "planes":   # b planes: plane j of the chunk sits at j * n / 8 + a / 8 in the whole array
            nb = extra[1]
            m = (b - a) // 8
            parts = [(j * (n // 8) + a // 8, w[j * m:(j + 1) * m]) for j in range(nb)]
        else:
            d = per.get(k, 1)
            parts = [(a // d, w)]
        for lo, ww in parts:
            have = _read(specs[k], lo, lo + ww.size)
            if not np.array_equal(have, ww):
                bad = np.flatnonzero(have != ww)
                return (f"{k} differs from the oracle at {bad.size} positions of elements [{a}, {b}); first "
                        f"offsets {(lo + bad[:6]).tolist()} got {have[bad[:6]].tolist()} want {ww[bad[:6]].tolist()}")
    return None


def _run_checks(name, kind, sh, n, extra, chunk, progress=8):
    p, cores = pool()
    t0 = time.perf_counter()
    starts = list(range(0, n, chunk))
    tasks = ((kind, sh.specs, a, min(a + chunk, n), extra) for a in starts)
    step = max(1, len(starts) // progress)
    for i, err in enumerate(p.imap(_check_task, tasks, chunksize=1)):
        if err is not None:
            raise AssertionError(f"{name} ({kind}): {err}")
        if (i + 1) % step == 0 or i + 1 == len(starts):
            _say(f"  {name}: {min(starts[i] + chunk, n)} of {n} elements equal to the oracle "
                 f"({time.perf_counter() - t0:.1f} s, {cores} workers)")
    return n


# --------------------------------------------------------------------------
# entry points of the tests
# --------------------------------------------------------------------------

def tensor_scale_of(sh, key="xr"):
    """The oracle's tensor scale of a shared input: the maximum of the
    scales of its chunks, which equals the whole tensor's scale exactly
    (dividing by 2688 and rounding are monotone; pinned in
    test_oracle_arith.py)."""
    p, _ = pool()
    n = sh.specs[key][2]
    parts = p.map(_ts_task, [(sh.specs[key], a, min(a + (1 << 22), n)) for a in range(0, n, 1 << 22)])
    return np.float32(max(parts)) if parts else np.float32(0)


def compare_every_element(name, sh, outputs, ts):
    """The NVFP4 path on a whole site: sh holds the inputs xr, xt, g
    (``Shared``); outputs maps the GPU's outputs (tensors or host arrays:
    scales, bits, codes, y_g, mask_g, q_g, y_r, mask_r, q_r, y_f, mask_f,
    q_f, gin) to be compared; ts is the oracle's tensor scale."""
    for k, v in outputs.items():
        sh.put(k, v)
    return _run_checks(name, "nvfp4", sh, sh.specs["xr"][2], np.float32(ts), CHUNK_ELEMS)


def compare_variant_every_element(name, kind, xr, xt, got, extra=None, g=None):
    """The MXFP4 (kind "mx"), MXFP8 ("mx8") or b-low-bits ("lowbits", extra =
    (the oracle's tensor scale, b)) path on a whole site: xr, xt (and g) the
    inputs, got the GPU's outputs (tensors or host arrays; the low-bits
    planes as one array of b planes of n / 8 bytes each).  For mx and mx8,
    extra = "with_rne" also compares the RNE forward (y_r, m_r, q_r), and a
    gradient g the STE backward on the guided mask (gin)."""
    ins = {"xr": xr, "xt": xt}
    if g is not None:
        ins["g"] = g
    with Shared(ins) as sh:
        n = sh.specs["xr"][2]
        assert n % 32 == 0
        for k, v in got.items():
            sh.put(k, v)
        return _run_checks(name, kind, sh, n, extra, CHUNK_ELEMS, progress=4)


def compare_gathered_every_element(name, xr, src_rows, xt, idx, cols, off, ts, got):
    """The forwards on records read back in place: xr the source site
    (src_rows x cols), xt the destination rows, idx their source rows
    (int64, out-of-range allowed), off the source's row groups (None: one
    tensor scale ts) and the oracle's tensor scale(s) ts; got the GPU's
    y_g, mask_g, q_g, y_f, mask_f, q_f (and y_r, mask_r, q_r of the RNE
    forward).  Chunks of whole destination rows."""
    with Shared({"xr": xr, "xt": xt, "idx": np.asarray(idx, dtype=np.int64)}) as sh:
        for k, v in got.items():
            sh.put(k, v)
        n = sh.specs["xt"][2]
        chunk = max(1, CHUNK_ELEMS // cols) * cols
        extra = (cols, src_rows, None if off is None else np.asarray(off, dtype=np.int64),
                 np.float32(ts) if off is None else np.asarray(ts, dtype=np.float32))
        return _run_checks(name, "gathered", sh, n, extra, chunk, progress=4)


def compare_grouped_every_element(name, xr, xt, rows, cols, off, ts, got):
    """The per-expert path on a whole rows x cols site with row groups off
    (int64[G + 1]) and the oracle's per-group tensor scales ts: chunks of
    whole rows, each with the group offsets clipped to its rows, so every row
    keeps its group's scale."""
    with Shared({"xr": xr, "xt": xt}) as sh:
        for k, v in got.items():
            sh.put(k, v)
        chunk = max(1, CHUNK_ELEMS // cols) * cols
        return _run_checks(name, "grouped", sh, rows * cols, (cols, np.asarray(off, dtype=np.int64), ts), chunk,
                           progress=4)
