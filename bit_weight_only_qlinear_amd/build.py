"""Builds libqlinear.so (the HIP kernels + C ABI) in-tree for gfx950.

Each translation unit is compiled by hipcc in parallel, then linked into one
shared library next to this file.  Packed fp32 instructions are disabled for
all device code, and the layout kernels (quant.hip) are compiled without FMA
contraction so that their fp32 arithmetic is one IEEE operation per step.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libqlinear.so")
BUILD = os.path.join(HERE, "_build")

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument", "-I", os.path.join(HERE, "..", "include")]
SOURCES = {
    "api.cpp": [],
    "quant.hip": ["-ffp-contract=off"],
    "gemv.hip": [],
    "gemm.hip": [],
    "gemm_aff2.hip": [],
    "gemm_aff4.hip": [],
    "gemm_aff8.hip": [],
    "gemm_kq.hip": [],
    "skinny.hip": [],
    "a8w4.hip": [],
    "noalloc.hip": [],
}


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libqlinear)")


def _compile(args):
    src, extra, defines = args
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc(), *lang, *COMMON, *extra, *defines, "-c", os.path.join(SRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(defines=(), out=OUT, verbose=True):
    """Compile every source and link `out`.  `defines` are extra -D flags
    (tuning constants); the default build uses none."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(s, e, list(defines)) for s, e in SOURCES.items()]
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(_compile, jobs))
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(defines=sys.argv[1:])
