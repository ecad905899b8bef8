"""Build the HIP library ``libamp.so`` for gfx950 in-tree.

Every ``csrc/*.hip`` and ``csrc/*.cpp`` is compiled by hipcc into ``_build/``
(in parallel) and linked into ``mixed_precision_numerics_amd/libamp.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libamp.so")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-ffp-contract=off",                         # FP32 op order is part of the contract
    "-fno-gpu-flush-denormals-to-zero",          # keep FP32 subnormals
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]
DEVICE = [
    "--offload-arch=" + ARCH,
    # packed FP32 instructions stay off (see the library notes)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

# Per-file additions.  The quantizer's register-resident cells are indexed by
# fully unrolled loops; the default unroll budget stops short on the
# stochastic-rounding variants and leaves the cell in scratch memory.
PER_FILE = {
    "nvfp4.hip": ["-mllvm", "-pragma-unroll-threshold=1000000"],
}


def hipcc() -> str:
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _headers_mtime() -> float:
    hs = glob.glob(os.path.join(CSRC, "*.hpp")) + glob.glob(os.path.join(ROOT, "include", "*.h"))
    return max((os.path.getmtime(h) for h in hs), default=0.0)


def _compile(src: str, incremental: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if incremental and os.path.exists(obj):
        newest = max(os.path.getmtime(src), _headers_mtime(), os.path.getmtime(__file__))
        if os.path.getmtime(obj) > newest:
            return obj
    extra = PER_FILE.get(os.path.basename(src), [])
    cmd = [hipcc(), "-c", src, "-o", obj] + COMMON + DEVICE + extra
    if src.endswith(".cpp"):
        cmd = [hipcc(), "-x", "hip", "-c", src, "-o", obj] + COMMON + DEVICE + extra
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False, jobs: int | None = None, incremental: bool = False) -> str:
    """Compile every source (``incremental``: reuse objects newer than their
    source, the headers and this script) and link the library."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    jobs = jobs or min(8, max(1, len(srcs)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, incremental), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-o", tmp] + objs + ["--offload-arch=" + ARCH, "-fPIC"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB, file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True, incremental="--incremental" in sys.argv)
