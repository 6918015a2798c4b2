"""Build libmoe.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree.

    python -m combine_grouped_gemm_amd.build      (or __graft_entry__.build())

Objects go to combine_grouped_gemm_amd/_build/; the library to
combine_grouped_gemm_amd/libmoe.so.  Always recompiles.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe.so")
SOURCES = ["router.hip", "route.hip", "layout.hip", "permute.hip", "combine.hip", "grouped_gemm.hip", "grouped_gemm_stream.hip",
           "grouped_gemm_wide.hip", "grouped_gemm_bwd.hip", "backward.hip",
           "moe_api.cpp"]
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe)")


def _flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-Wall",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            # packed fp32 VALU instructions are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# Per-source flags.  The wide GEMM takes its next tile with a single-lane atomicAdd whose result
# is used only at the tile boundary; the atomic optimizer would turn it into a wave reduction
# that reads the result at once (a wait for memory in the middle of a K loop stage).
EXTRA_FLAGS = {"grouped_gemm_wide.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + _flags() + EXTRA_FLAGS.get(src, []) + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libmoe.so failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
