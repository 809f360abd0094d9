"""Compile libarcs.so (HIP kernels + C ABI) for gfx950, in-tree.

Flags: -O3, no fused multiply-add contraction (the penalty arithmetic is an
exact sequence of binary32 operations), packed-FP32 instruction selection
disabled, and a higher size limit for loops marked `#pragma unroll`: the
register-resident row is indexed by round number, so a round loop that is
only partly unrolled indexes it at run time and moves it to scratch memory.
hipcc's host pass warns that it does not know the packed-fp32 feature; the
warning is harmless.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libarcs.so")
BUILD_DIR = os.path.join(PKG, "_build")

SOURCES = ["api.hip", "argmax_kernel.hip", "sample_kernel.hip", "logprobs_kernel.hip", "commit_kernel.hip",
           "hybrid_kernel.hip"]
ARCH = os.environ.get("ARCS_OFFLOAD_ARCH", "gfx950")

COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-pragma-unroll-threshold=100000",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libarcs")


def _run(cmd, verbose):
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + p.stdout + p.stderr)
    if verbose:
        sys.stdout.write(p.stdout + p.stderr)


def build(verbose: bool = False) -> str:
    cc = hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        jobs.append([cc, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
