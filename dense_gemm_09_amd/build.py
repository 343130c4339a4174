"""Build libgemm355.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m dense_gemm_09_amd.build   (or build() from Python)
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgemm355.so")
# (source, object name, extra defines). gemm_tile.hip is compiled once per
# (ragged flag, output part) and once for the split-K reduction, so that its
# kernel variants build in parallel.
SOURCES = [("api.cpp", "api", []), ("gemm_skinny.hip", "gemm_skinny", []),
           ("quant.hip", "quant", []), ("pack.hip", "pack", []),
           ("gemm_tile.hip", "gemm_reduce", ["-DG355_REDUCE=1"])]
SOURCES += [("gemm_tile.hip", f"gemm_tile_r{r}_p{p}", [f"-DG355_RAGGED={r}", f"-DG355_PART={p}"])
            for r in (0, 1) for p in range(5)]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # Packed FP32 VALU ops are kept out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(item) -> str:
    src, name, defines = item
    obj = os.path.join(BUILD, name + ".o")
    cmd = [HIPCC, *FLAGS, *defines]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every source and link the shared library. Returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = int(os.environ.get("MAX_JOBS", os.cpu_count() or 8))
    # the long compiles first
    order = sorted(SOURCES, key=lambda it: it[0] != "gemm_tile.hip")
    with cf.ThreadPoolExecutor(max_workers=max(1, min(16, jobs, len(order)))) as ex:
        objs = list(ex.map(_compile, order))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    shutil.move(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
