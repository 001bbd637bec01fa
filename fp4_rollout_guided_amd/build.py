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
SOURCES = ["kernels.hip", "mx_kernels.hip", "api.cpp"]
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


def build(verbose: bool = False) -> str:
    """Compile every source into fp4_rollout_guided_amd/libtrace.so (always
    rebuilds) and return its path."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    if verbose and res.stderr.strip():
        # the host pass does not know the packed-fp32 feature flag; that warning is expected
        lines = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
        if lines:
            print("\n".join(lines))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
