"""CPU oracle for the GEMM hot path. TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package. The GPU library never calls it and shares no code with
it: the two meet only in the seeded inputs (package `synth`) they both read.

What it computes (in float64, the plain definition written out):

    acc[m, n] = sum_k a(m, k) * b(k, n)                 (float64, k ascending)
    dq        = scale_a[m] * scale_b[n] * acc           (FP8 variant only)
    z         = alpha * dq + beta * C_in[m, n] + bias[n]
    y         = act(z)
    out       = round_to_nearest_even(y) in FP32 or BF16 (single rounding)

The sum over k is a plain i-k-j triple loop in C (triple_loop.c, compiled by
native.py with gcc, no contraction into FMAs, OpenMP over output rows): each
acc[m, n] is accumulated in ascending k, one float64 add per term.

Sources: the GEMM definition C = alpha*A*B + beta*C with A MxK, B KxN (first
DeepGEMM page, sec. 1.1); FP32-or-better accumulation of 16-bit inputs (same
page, sec. 3.1); bias, then activation, then the output write, fused into the
epilogue (same page, sec. 6.1); per-token (row of A) and per-channel (column
of B) scales applied after accumulation and before the store (DeepGEMM: FP8
precision Tensor Core GEMM optimisation, sec. 1.2 and 3.2); the E4M3 format
(same page, sec. 1.2); element-by-element CPU comparison (the CUDA-tile GEMM
tutorial page, sec. 6).

The per-token FP8 quantiser that produces the FP8 GEMM's A operand (one
float32 scale amax/448 per row, E4M3 codes of x / scale) is in quant.py; the
quantising epilogue (per-row INT8 round(x * scale + zero_point) or E4M3 codes
of x * scale, first DeepGEMM page, sec. 6.2) is in qout.py; the block-scaled
(MX, one E8M0 scale per 32 K elements) FP8 GEMM is in mx.py.

Parity status: every function here is pinned by the `-m "not gpu"` tests in
tests/test_oracle.py, tests/test_oracle_quant.py, tests/test_oracle_qout.py and
tests/test_oracle_mx.py: codec tables against the formats' named values,
rounding ties, integer-valued products (exact), tiny dyadic operands against
rational arithmetic, the ascending-k order of the float64 sum, identity and
permutation matrices, alpha scaling the product only (alpha = 2, beta = 3,
C_in = AB, bias b gives exactly 5AB + b), the activation applied after
beta*C_in and the bias, GELU against tabulated normal-CDF values, a
high-precision (decimal) tanh form and the normal tail series, and planted
mistakes (a dropped K term, a transposed B, a flipped beta, a shifted bias,
alpha applied to the bias or to beta*C_in, the activation applied before
beta*C_in or the bias) rejected by the parity tolerance. No function is
"parity unpinned".
"""
from .codecs import (decode_bf16, decode_e4m3, round_to_bf16, round_to_bf16_bits,
                     round_to_f32)
from .gemm import activation, gemm_bf16, gemm_fp8_scaled, logical_a, logical_b
from .mx import decode_e8m0, gemm_mxfp8
from .qout import QOUT_E4M3, QOUT_INT8, quantize_output
from .quant import encode_e4m3, quantize_rows_e4m3

__all__ = [
    "decode_bf16", "decode_e4m3", "round_to_bf16", "round_to_bf16_bits", "round_to_f32",
    "activation", "gemm_bf16", "gemm_fp8_scaled", "logical_a", "logical_b",
    "encode_e4m3", "quantize_rows_e4m3", "quantize_output", "QOUT_INT8", "QOUT_E4M3",
    "decode_e8m0", "gemm_mxfp8",
]
