"""MX (block-scaled) FP8 GEMM, written out in float64. TEST INFRASTRUCTURE ONLY.

What it computes: the FP8 GEMM with per-group scales instead of (or as the
finest case of) per-token x per-channel ones. The FP8 DeepGEMM page (sec. 3.2)
names the two granularities, per-GEMM/per-token-channel and per-group, and
warns that the scale convention has to be known. The reading taken here is the
group form of the OCP Microscaling (MX) formats: one power-of-two scale (E8M0
code c, value 2^(c-127), 255 = NaN) per 32 consecutive K elements of each row
of A and each column of B:

    a'(m, k) = e4m3(A[m, k]) * 2^(SA[m, k // 32] - 127)
    b'(k, n) = e4m3(B[n, k]) * 2^(SB[n, k // 32] - 127)
    acc      = sum_k a'(m, k) b'(k, n)     (float64, ascending k: the triple loop)
    then the same epilogue as the other GEMMs (alpha, beta * C_in, bias, act, cast)

A is row-major (K-major), B column-major (K-major): the layouts of the page's
FP8 path.

Parity status: pinned by tests/test_oracle_mx.py (the E8M0 decode table from
its definition; all scales 2^0 reduce to the FP8 GEMM with unit scales;
block-scaled integer data whose scaled values are themselves E4M3 values equal
the FP8 GEMM on those values, which fixes the block index k // 32, which
operand each scale belongs to and its sign; a uniform shift of all A scale
codes by d multiplies the result by 2^d exactly).
"""
from __future__ import annotations

import numpy as np

from .codecs import decode_e4m3
from .gemm import ROW, COL, _epilogue, _product, _select, logical_a, logical_b

MX_BLOCK = 32


def decode_e8m0(codes) -> np.ndarray:
    """uint8 E8M0 codes -> float64 scales 2^(c - 127); code 255 is NaN."""
    c = np.asarray(codes).astype(np.int64)
    out = np.ldexp(1.0, c - 127)
    return np.where(c == 255, np.nan, out)


def _block_scales(S: np.ndarray, rows, K: int) -> np.ndarray:
    """Per-element scale of K elements for the selected rows of a scale array."""
    kb = np.arange(K) // MX_BLOCK
    return decode_e8m0(np.asarray(S)[np.asarray(rows)][:, kb])


def gemm_mxfp8(M, N, K, alpha, A, B, scale_a, scale_b, beta, C, c_dtype, bias, act,
               rows=None, cols=None, with_z=False):
    """MX FP8 GEMM. A: E4M3 codes (M x lda), B: E4M3 codes (N x ldb, K-major),
    scale_a: E8M0 codes (M x ldsa), scale_b: (N x ldsb). Returns (y, out), or
    (y, out, z) with with_z."""
    r, c = _select(M, N, rows, cols)
    a = decode_e4m3(logical_a(A, ROW, M, K)[r, :])
    b = decode_e4m3(logical_b(B, COL, K, N)[:, c])
    if K > 0:
        a = a * _block_scales(scale_a, r, K)
        b = b * _block_scales(scale_b, c, K).T
    acc = _product(a, b)
    C_sel = C[np.ix_(r, c)] if beta != 0.0 else None
    bias_sel = None if bias is None else np.asarray(bias)[c]
    res = _epilogue(acc, alpha, beta, C_sel, c_dtype, bias_sel, act)
    return res if with_z else res[:2]
