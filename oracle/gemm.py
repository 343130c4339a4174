"""The GEMM definition, written out in float64. TEST INFRASTRUCTURE ONLY.

Argument conventions mirror the C ABI so a test can hand both sides the same
arrays: A is logically MxK, B KxN, C MxN (row-major, leading dimension ldc).
Layout 0 (ROW) / 1 (COL) says how an operand array is indexed:

* A ROW: a(m, k) = A[m, k] (array M x lda);  A COL: a(m, k) = A[k, m]
* B ROW: b(k, n) = B[k, n] (array K x ldb);  B COL: b(k, n) = B[n, k]

`rows` / `cols` restrict the computation to a subset of output rows and
columns (each output element depends only on its own row of A and column of
B), which is how full-size problems are checked on samples.

The accumulation is the plain i-k-j triple loop in float64 (triple_loop.c,
loaded by native.py): every acc[m, n] is the sum of its K products taken in
ascending k. For the FP8 variant every product of two E4M3 values is an
integer multiple of 2**-18 below 2**18 in magnitude, so for K <= 2**17 every
partial sum is exact in float64: the oracle's accumulator is then the exact
sum. For BF16 every product is exact in float64 (8-bit significands), so the
accumulator differs from the exact sum only by float64 rounding of the sums.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erfc

from .codecs import decode_bf16, decode_e4m3, round_to_bf16_bits, round_to_f32
from .native import accumulate

ROW, COL = 0, 1
OUT_F32, OUT_BF16 = 0, 1
ACT_NONE, ACT_RELU, ACT_GELU_ERF, ACT_GELU_TANH = 0, 1, 2, 3


def logical_a(A: np.ndarray, layout: int, M: int, K: int) -> np.ndarray:
    """The logical MxK view of operand A (codes, not values)."""
    return A[:M, :K] if layout == ROW else A[:K, :M].T


def logical_b(B: np.ndarray, layout: int, K: int, N: int) -> np.ndarray:
    """The logical KxN view of operand B (codes, not values)."""
    return B[:K, :N] if layout == ROW else B[:N, :K].T


def activation(z: np.ndarray, act: int) -> np.ndarray:
    """Epilogue activation (first DeepGEMM page, sec. 6.1: ReLU or GELU after the bias).

    GELU_ERF is the exact form z * Phi(z) = 0.5 z (1 + erf(z / sqrt 2)),
    evaluated as 0.5 z erfc(-z / sqrt 2) (the same function: 1 + erf(x) =
    erfc(-x)), which keeps its relative accuracy where Phi(z) is tiny; 1 + erf
    in float64 has no correct digits below z ~ -8.
    GELU_TANH is the usual tanh approximation 0.5 z (1 + tanh u), u =
    sqrt(2/pi) (z + 0.044715 z^3), evaluated as z / (1 + e^(-2u)) (the same
    function: 1 + tanh u = 2 / (1 + e^(-2u))), again free of cancellation.
    """
    if act == ACT_NONE:
        return z
    if act == ACT_RELU:
        return np.where(z > 0, z, 0.0)
    if act == ACT_GELU_ERF:
        return 0.5 * z * erfc(-z / math.sqrt(2.0))
    if act == ACT_GELU_TANH:
        c = math.sqrt(2.0 / math.pi)
        u = c * (z + 0.044715 * z * z * z)
        with np.errstate(over="ignore"):
            return z / (1.0 + np.exp(-2.0 * u))
    raise ValueError(f"unknown activation {act}")


def _decode_c(C: np.ndarray, c_dtype: int) -> np.ndarray:
    if c_dtype == OUT_F32:
        return np.asarray(C, dtype=np.float32).astype(np.float64)
    return decode_bf16(C)


def _epilogue(acc, alpha, beta, C_sel, c_dtype, bias_sel, act, row_scale=None,
              col_scale=None):
    """z = alpha * (scale_a[m] scale_b[n] acc) + beta * C_in + bias; y = act(z); cast.

    Order: scales after accumulation (FP8 page, sec. 3.2), then alpha*AB +
    beta*C (first page, sec. 1.1: alpha multiplies the product only, beta the
    old C only), then bias, activation, output (first page, sec. 6.1: the
    bias joins before the activation, and the activation sees the whole
    linear combination, beta*C included). With beta == 0, C_in is not read
    (its value, even NaN, does not matter). Returns (y, out, z).
    """
    dq = acc
    if row_scale is not None:
        dq = dq * np.asarray(row_scale, dtype=np.float64)[:, None]
    if col_scale is not None:
        dq = dq * np.asarray(col_scale, dtype=np.float64)[None, :]
    z = float(np.float32(alpha)) * dq
    if beta != 0.0:
        z = z + float(np.float32(beta)) * _decode_c(C_sel, c_dtype)
    if bias_sel is not None:
        z = z + decode_bf16(bias_sel)[None, :]
    y = activation(z, act)
    out = round_to_f32(y) if c_dtype == OUT_F32 else round_to_bf16_bits(y)
    return y, out, z


def _product(a, b):
    """acc = a b by the ascending-k float64 triple loop (an empty K gives zeros)."""
    if a.shape[1] == 0:
        return np.zeros((a.shape[0], b.shape[1]))
    return accumulate(a, b)


def _select(M, N, rows, cols):
    r = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    c = np.arange(N) if cols is None else np.asarray(cols, dtype=np.int64)
    return r, c


def gemm_bf16(M, N, K, alpha, A, layout_a, B, layout_b, beta, C, c_dtype, bias, act,
              rows=None, cols=None, with_z=False):
    """BF16 x BF16 GEMM with float64 accumulation and the fused epilogue.

    Returns (y, out): y is the float64 epilogue value before the output cast,
    out the rounded output (float32 array, or uint16 BF16 codes); with
    with_z, (y, out, z) with z the float64 value the activation was applied to.
    """
    r, c = _select(M, N, rows, cols)
    a = decode_bf16(logical_a(A, layout_a, M, K)[r, :])
    b = decode_bf16(logical_b(B, layout_b, K, N)[:, c])
    acc = _product(a, b)
    C_sel = C[np.ix_(r, c)] if beta != 0.0 else None
    bias_sel = None if bias is None else np.asarray(bias)[c]
    res = _epilogue(acc, alpha, beta, C_sel, c_dtype, bias_sel, act)
    return res if with_z else res[:2]


def gemm_fp8_scaled(M, N, K, alpha, A, layout_a, B, layout_b, scale_a, scale_b, beta, C,
                    c_dtype, bias, act, rows=None, cols=None, with_z=False):
    """E4M3 x E4M3 GEMM, per-row scale_a[M] and per-column scale_b[N], fused epilogue.

    Returns (y, out), or (y, out, z) with with_z, as gemm_bf16 does.
    """
    r, c = _select(M, N, rows, cols)
    a = decode_e4m3(logical_a(A, layout_a, M, K)[r, :])
    b = decode_e4m3(logical_b(B, layout_b, K, N)[:, c])
    acc = _product(a, b)
    C_sel = C[np.ix_(r, c)] if beta != 0.0 else None
    bias_sel = None if bias is None else np.asarray(bias)[c]
    res = _epilogue(acc, alpha, beta, C_sel, c_dtype, bias_sel, act,
                    row_scale=np.asarray(scale_a)[r], col_scale=np.asarray(scale_b)[c])
    return res if with_z else res[:2]
