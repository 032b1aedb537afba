"""Build libmhc_seam.so (HIP for gfx950) in-tree with hipcc.

Flags: gfx950 only; -ffp-contract=off so that every fp32 rounding point in
the seam's elementwise chains is the one the source spells out with fmaf;
packed-fp32 instructions disabled.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmhc_seam.so")
SOURCES = [os.path.join(CSRC, "seam_kernels.hip"), os.path.join(CSRC, "head_kernels.hip"),
           os.path.join(CSRC, "gemm_kernels.hip"), os.path.join(CSRC, "seam_runtime.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False, extra_flags=()) -> str:
    out = LIB
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include"),
           "-x", "hip", *SOURCES, "-o", out + ".tmp", *extra_flags]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
