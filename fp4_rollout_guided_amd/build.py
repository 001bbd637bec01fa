"""Build libtrace.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python fp4_rollout_guided_amd/build.py

(run as a script: importing the package would load the library first)

Flags that matter for exactness: no FP contraction (every fused multiply-add
in the kernels is written out), correctly rounded fp32 division, fp32
denormals kept, no fast-math.  Packed-fp32 instructions are disabled.  SLP
vectorization is off: it turns the per-element flag tests into vector-of-bool
packing code.
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libtrace.so")
SOURCES = ["kernels.hip", "mx_kernels.hip", "mx8_kernels.hip", "diag_kernels.hip", "api.cpp"]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-fno-slp-vectorize",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: libtrace needs ROCm's hipcc to build")


# The same sources with grids capped at 3 workgroups, so that every kernel's
# grid-stride loop runs several iterations on test-sized tensors (the
# production caps are reached only beyond 2^34 elements), and with the
# non-temporal stream threshold at 0 bytes, so that test-sized tensors run
# the instantiations that production uses for tensors past 256 MiB.  Loaded
# by the GPU tests only.
SMALLGRID_LIB = os.path.join(PKG, "libtrace_smallgrid.so")
SMALLGRID_DEFINES = ["-DTRACE_MAX_GROUPS=3u", "-DTRACE_AMAX_MAX_GROUPS=3u", "-DTRACE_NT_STREAM_BYTES=0ull"]


def _command(out, defines=()):
    return [hipcc(), *FLAGS, *defines, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            *[os.path.join(CSRC, s) for s in SOURCES], "-o", out]


# The bench's practical-ceiling probe (plain copy / read / fill streams).
CEILING_SRC = os.path.join(ROOT, "bench_ceiling.hip")
CEILING_BIN = os.path.join(ROOT, "_build", "bench_ceiling")

# A plain C caller of the library (tests/c/trace_c_smoke.c), built with the
# host C compiler against include/trace.h and libtrace.so; run by a GPU test.
C_SMOKE_SRC = os.path.join(ROOT, "tests", "c", "trace_c_smoke.c")
C_SMOKE_BIN = os.path.join(ROOT, "_build", "trace_c_smoke")


def _c_smoke_command(out):
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    return [os.environ.get("CC", "gcc"), "-std=c99", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"), C_SMOKE_SRC,
            "-L", PKG, "-l:libtrace.so", "-Wl,-rpath,$ORIGIN/../fp4_rollout_guided_amd",
            "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", out]


def build(verbose: bool = False) -> str:
    """Compile every source into fp4_rollout_guided_amd/libtrace.so (and the
    small-grid test build beside it), always rebuilding, and return the
    library's path."""
    jobs = [(LIB, _command(LIB + ".tmp")), (SMALLGRID_LIB, _command(SMALLGRID_LIB + ".tmp", SMALLGRID_DEFINES))]
    if os.path.exists(CEILING_SRC):
        os.makedirs(os.path.dirname(CEILING_BIN), exist_ok=True)
        jobs.append((CEILING_BIN, [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17",
                                   "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                                   CEILING_SRC, "-o", CEILING_BIN + ".tmp"]))
    procs = []
    for out, cmd in jobs:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((out, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    for out, p in procs:
        stdout, stderr = p.communicate()
        if p.returncode != 0:
            sys.stderr.write(stdout + stderr)
            raise RuntimeError(f"hipcc failed with exit code {p.returncode} building {os.path.basename(out)}")
        if verbose and stderr.strip():
            # the host pass does not know the packed-fp32 feature flag; that warning is expected
            lines = [l for l in stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
            if lines:
                print("\n".join(lines))
        os.replace(out + ".tmp", out)
    if os.path.exists(C_SMOKE_SRC):  # links against the library just built
        cmd = _c_smoke_command(C_SMOKE_BIN + ".tmp")
        if verbose:
            print(" ".join(cmd), flush=True)
        p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
        if p.returncode != 0:
            sys.stderr.write(p.stdout + p.stderr)
            raise RuntimeError(f"the C caller failed to build (exit code {p.returncode})")
        os.replace(C_SMOKE_BIN + ".tmp", C_SMOKE_BIN)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
