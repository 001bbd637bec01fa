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
CHUNK_ELEMS = 1 << 20   # elements per worker task (a multiple of 16)

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
