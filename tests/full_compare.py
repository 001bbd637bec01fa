"""Every element of a full-size site against the oracle.

The GPU runs the whole path (tensor scale, capture with codes, guided, RNE
and full-information forwards, STE backward); every output comes back to the
host, and the oracle recomputes the same outputs chunk by chunk in a pool of
worker processes, with the tensor scale the oracle computed over the whole
tensor.  Each chunk's outputs are compared with the GPU's bit for bit.  The
workers are started with the forkserver method: they are fresh interpreters
that import only NumPy and the oracle, never the GPU runtime."""
import os
import sys
import time

import numpy as np

CPU_SHARE = 16          # host cores granted to a process driving one GPU
CHUNK_ELEMS = 1 << 17   # elements per worker task (a multiple of 16; small chunks keep the oracle's temporaries in cache)

_POOL = None


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _oracle_chunk(args):
    import oracle
    xr, xt, g, ts = args
    cap = oracle.capture(xr, ts, with_codes=True)
    gd = oracle.guided_fwd(xt, cap["scales"], ts, cap["bits"])
    rn = oracle.rne_fwd(xt, cap["scales"], ts)
    fi = oracle.full_info_fwd(xt, cap["scales"], ts, cap["codes"])
    return {"scales": cap["scales"], "bits": cap["bits"], "codes": cap["codes"],
            "y_g": gd["y"], "mask_g": gd["mask"], "q_g": gd["codes"],
            "y_r": rn["y"], "mask_r": rn["mask"], "q_r": rn["codes"],
            "y_f": fi["y"], "mask_f": fi["mask"], "q_f": fi["codes"],
            "gin": oracle.ste_bwd(g, gd["mask"], xt.size)}


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


# elements per byte of each output (bytes = elements / per)
_PER = {"scales": 16, "bits": 8, "codes": 2, "mask_g": 8, "q_g": 2, "mask_r": 8, "q_r": 2, "mask_f": 8, "q_f": 2}
_BF16 = ("y_g", "y_r", "y_f", "gin")


def compare_every_element(name, xr, xt, g, ts, got):
    """xr, xt, g: host uint16 arrays of the whole site; ts: the oracle's
    tensor scale (np.float32); got: host arrays of the GPU's outputs (bytes
    for the record, masks and codes, uint16 for the bf16 outputs)."""
    n = xr.size
    assert n % 16 == 0
    p, cores = pool()
    t0 = time.perf_counter()
    starts = list(range(0, n, CHUNK_ELEMS))
    tasks = ((xr[a:a + CHUNK_ELEMS], xt[a:a + CHUNK_ELEMS], g[a:a + CHUNK_ELEMS], ts) for a in starts)
    step = max(1, len(starts) // 8)
    for i, want in enumerate(p.imap(_oracle_chunk, tasks, chunksize=1)):
        a = starts[i]
        b = min(a + CHUNK_ELEMS, n)
        for k, w in want.items():
            lo, hi = (a, b) if k in _BF16 else (a // _PER[k], b // _PER[k])
            have = got[k][lo:hi]
            if not np.array_equal(have, w):
                bad = np.flatnonzero(have != w)
                raise AssertionError(
                    f"{name}: {k} differs from the oracle at {bad.size} positions of chunk [{a}, {b}); first "
                    f"offsets {(lo + bad[:6]).tolist()} got {have[bad[:6]].tolist()} want {w[bad[:6]].tolist()}")
        if (i + 1) % step == 0 or i + 1 == len(starts):
            _say(f"  {name}: {b} of {n} elements equal to the oracle ({time.perf_counter() - t0:.1f} s, "
                 f"{cores} workers)")
    return n


def _oracle_variant_chunk(args):
    import oracle
    kind, xr, xt, extra, g = args
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


# elements per byte of each variant output; bf16 outputs are one uint16 per element
_VARIANT_PER = {
    "mx": {"scales": 32, "bits": 8, "codes": 2, "m_g": 8, "q_g": 2, "m_f": 8, "q_f": 2, "m_r": 8, "q_r": 2},
    "mx8": {"scales": 32, "bits": 8, "codes": 1, "m_g": 8, "q_g": 1, "m_f": 8, "q_f": 1, "m_r": 8, "q_r": 1},
    "lowbits": {"scales": 16, "mask": 8, "codes": 2},
}


def compare_variant_every_element(name, kind, xr, xt, got, extra=None, g=None):
    """The MXFP4 (kind "mx"), MXFP8 ("mx8") or b-low-bits ("lowbits", extra =
    (the oracle's tensor scale, b)) path on a whole site: got holds the GPU's
    outputs as host arrays (the low-bits planes as one array of b planes of
    n / 8 bytes each).  For mx and mx8, extra = "with_rne" also compares the
    RNE forward (y_r, m_r, q_r), and a gradient g (host uint16) the STE
    backward on the guided mask (gin)."""
    n = xr.size
    assert n % 32 == 0
    p, cores = pool()
    per = _VARIANT_PER[kind]
    t0 = time.perf_counter()
    starts = list(range(0, n, CHUNK_ELEMS))
    tasks = ((kind, xr[a:a + CHUNK_ELEMS], xt[a:a + CHUNK_ELEMS], extra,
              None if g is None else g[a:a + CHUNK_ELEMS]) for a in starts)
    step = max(1, len(starts) // 4)
    for i, want in enumerate(p.imap(_oracle_variant_chunk, tasks, chunksize=1)):
        a = starts[i]
        b = min(a + CHUNK_ELEMS, n)
        for k, w in want.items():
            if k == "planes":   # b planes: plane j of the chunk sits at j * n / 8 + a / 8 in the whole array
                nb = extra[1]
                m = (b - a) // 8
                pairs = [(got[k][j * (n // 8) + a // 8:j * (n // 8) + b // 8], w[j * m:(j + 1) * m], j * (n // 8) + a // 8)
                         for j in range(nb)]
            elif k in per:
                pairs = [(got[k][a // per[k]:b // per[k]], w, a // per[k])]
            else:
                pairs = [(got[k][a:b], w, a)]
            for have, ww, base in pairs:
                if not np.array_equal(have, ww):
                    bad = np.flatnonzero(have != ww)
                    raise AssertionError(
                        f"{name} ({kind}): {k} differs from the oracle at {bad.size} positions of chunk [{a}, {b}); "
                        f"first offsets {(base + bad[:6]).tolist()} got {have[bad[:6]].tolist()} "
                        f"want {ww[bad[:6]].tolist()}")
        if (i + 1) % step == 0 or i + 1 == len(starts):
            _say(f"  {name} ({kind}): {b} of {n} elements equal to the oracle ({time.perf_counter() - t0:.1f} s)")
    return n


def _oracle_grouped_chunk(args):
    import oracle
    xr, xt, rows, cols, off, ts = args
    cap = oracle.grouped_capture(xr, rows, cols, off, ts, with_codes=True)
    gd = oracle.grouped_guided_fwd(xt, rows, cols, off, cap["scales"], ts, cap["bits"])
    rn = oracle.grouped_rne_fwd(xt, rows, cols, off, cap["scales"], ts)
    fi = oracle.grouped_full_info_fwd(xt, rows, cols, off, cap["scales"], ts, cap["codes"])
    return {"scales": cap["scales"], "bits": cap["bits"], "codes": cap["codes"],
            "y_g": gd["y"], "mask_g": gd["mask"], "q_g": gd["codes"],
            "y_r": rn["y"], "mask_r": rn["mask"], "q_r": rn["codes"],
            "y_f": fi["y"], "mask_f": fi["mask"], "q_f": fi["codes"]}


def compare_grouped_every_element(name, xr, xt, rows, cols, off, ts, got):
    """The per-expert path on a whole rows x cols site with row groups off
    (int64[G + 1]) and the oracle's per-group tensor scales ts: chunks of
    whole rows, each with the group offsets clipped to its rows, so every row
    keeps its group's scale."""
    p, cores = pool()
    rows_per = max(1, CHUNK_ELEMS // cols)
    t0 = time.perf_counter()
    starts = list(range(0, rows, rows_per))
    off = np.asarray(off, dtype=np.int64)

    def task(r0):
        r1 = min(r0 + rows_per, rows)
        sub = np.clip(off - r0, 0, r1 - r0).astype(np.int64)
        return (xr[r0 * cols:r1 * cols], xt[r0 * cols:r1 * cols], r1 - r0, cols, sub, ts)

    step = max(1, len(starts) // 4)
    for i, want in enumerate(p.imap(_oracle_grouped_chunk, (task(r) for r in starts), chunksize=1)):
        a = starts[i] * cols
        b = min(starts[i] + rows_per, rows) * cols
        for k, w in want.items():
            lo, hi = (a, b) if k in _BF16 else (a // _PER[k], b // _PER[k])
            have = got[k][lo:hi]
            if not np.array_equal(have, w):
                bad = np.flatnonzero(have != w)
                raise AssertionError(
                    f"{name}: {k} differs from the oracle at {bad.size} positions of elements [{a}, {b}); first "
                    f"offsets {(lo + bad[:6]).tolist()} got {have[bad[:6]].tolist()} want {w[bad[:6]].tolist()}")
        if (i + 1) % step == 0 or i + 1 == len(starts):
            _say(f"  {name}: {b} of {rows * cols} elements equal to the oracle ({time.perf_counter() - t0:.1f} s)")
    return rows * cols
