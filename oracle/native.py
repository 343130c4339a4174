"""Loader of the oracle's C triple loop (triple_loop.c). TEST INFRASTRUCTURE ONLY.

`build()` compiles triple_loop.c with gcc into oracle/_build/; `accumulate`
builds it on first use when the library is missing or older than its source,
so the oracle also works in a checkout where nothing was built. The compile
flags keep IEEE float64 semantics: no fused multiply-add contraction, no
fast-math reassociation.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "triple_loop.c")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(BUILD, "liboracle_f64.so")
CC = os.environ.get("CC", "gcc")
FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
         "-fno-fast-math"]

_lock = threading.Lock()
_lib = None


def build() -> str:
    """Compile triple_loop.c (always). Returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    tmp = f"{LIB}.{os.getpid()}.tmp"
    r = subprocess.run([CC, *FLAGS, SRC, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"oracle C build failed:\n{r.stderr}")
    os.replace(tmp, LIB)  # atomic: concurrent builders never see a half-written file
    return LIB


def _load() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
                build()
            L = ctypes.CDLL(LIB)
            L.oracle_gemm_f64.restype = ctypes.c_int
            L.oracle_gemm_f64.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_int]
            _lib = L
    return _lib


def accumulate(a: np.ndarray, b: np.ndarray, threads: int = 0, return_threads: bool = False):
    """acc = a b in float64 by the ascending-k triple loop. a: M x K, b: K x N.

    threads: 0 = the OpenMP default (OMP_NUM_THREADS, else all cores).
    """
    a = np.ascontiguousarray(a, dtype=np.float64)
    b = np.ascontiguousarray(b, dtype=np.float64)
    M, K = a.shape
    K2, N = b.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {a.shape} x {b.shape}")
    acc = np.empty((M, N), dtype=np.float64)
    used = 1
    if M > 0 and N > 0:
        used = _load().oracle_gemm_f64(M, N, K, a.ctypes.data, b.ctypes.data, acc.ctypes.data,
                                       int(threads))
    return (acc, used) if return_threads else acc
