"""Build libmhc_seam.so (HIP for gfx950) in-tree with hipcc.

Each source compiles to its own object (in parallel, under _build/), then
one link.  Flags: gfx950 only; -ffp-contract=off so that every fp32 rounding point in
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
           os.path.join(CSRC, "gemm_kernels.hip"), os.path.join(CSRC, "measure_kernels.hip"),
           os.path.join(CSRC, "seam_runtime.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False, extra_flags=(), out: str = LIB) -> str:
    """Compile each source to an object in parallel (_build/), then link."""
    objdir = os.path.join(ROOT, "_build", os.path.basename(out) + ".obj")
    os.makedirs(objdir, exist_ok=True)
    flags = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include"),
             *extra_flags]
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [*flags, "-x", "hip", "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd), cmd))
        objs.append(obj)
    for p, cmd in procs:
        if p.wait() != 0:
            raise subprocess.CalledProcessError(p.returncode, cmd)
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
