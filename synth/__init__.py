"""Seeded synthetic inputs for the GEMM workloads.

This module is shared by the tests, the benchmark and the smoke check. It
draws numbers and stores them in the storage formats of the operands (BF16 and
OCP FP8-E4M3 bit patterns, FP32). It holds none of the GEMM's arithmetic: it
never multiplies, accumulates, scales outputs or applies an epilogue. The
per-token / per-channel FP8 quantisation that turns a normally distributed
operand into E4M3 bytes plus FP32 scales is input preparation (it happens
before the GEMM; DeepGEMM: FP8 precision Tensor Core GEMM optimisation, sec.
1.2 and sec. 3.2 describe per-token A scales and per-channel B scales); both
the oracle and the GPU path consume the same bytes and the same scale vectors.

Operand storage conventions (the logical shapes are A: MxK, B: KxN, C: MxN):

* A, layout ROW: array (M, lda), element (m, k) at [m, k], lda >= K.
* A, layout COL: array (K, lda), element (m, k) at [k, m], lda >= M.
* B, layout ROW: array (K, ldb), element (k, n) at [k, n], ldb >= N.
* B, layout COL ("K-major"): array (N, ldb), element (k, n) at [n, k], ldb >= K.
* C: always row-major, array (M, ldc), ldc >= N.

Padding columns (beyond the logical extent of a row) are filled with NaN bit
patterns so that a kernel which reads padding into a product is caught.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

ROW = 0
COL = 1
OUT_F32 = 0
OUT_BF16 = 1
ACT_NONE = 0
ACT_RELU = 1
ACT_GELU_ERF = 2
ACT_GELU_TANH = 3

BF16_NAN_BITS = np.uint16(0x7FC0)
E4M3_NAN_BITS = np.uint8(0x7F)
E4M3_MAX = 448.0


def seed_for(config_index: int, tensor_index: int) -> int:
    """Per-tensor seed: A is tensor 0, B 1, C_in 2, bias 3."""
    return 0x5EED0000 + 16 * config_index + tensor_index


def normal(shape, std: float, seed: int) -> np.ndarray:
    """N(0, std^2) samples in float64 from a PCG64 stream."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal(size=shape, dtype=np.float64) * std


def small_ints(shape, lo: int, hi: int, seed: int) -> np.ndarray:
    """Uniform integers in [lo, hi] as float64 (exact in BF16 and E4M3 for |v| <= 16)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(lo, hi + 1, size=shape).astype(np.float64)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Store float64 values as BF16 bit patterns (uint16), via torch's cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Store values as OCP E4M3FN bit patterns (uint8), saturating at +-448."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).clamp(-E4M3_MAX, E4M3_MAX)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def quantize_rows_e4m3(x: np.ndarray):
    """Per-row FP8 quantisation: scale[r] = fp32(amax_r / 448), q = e4m3(x / scale).

    An all-zero row gets scale 1 and zero codes. Returns (codes uint8, scales float32).
    """
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    amax = t.abs().amax(dim=1)
    scale = amax / torch.tensor(E4M3_MAX, dtype=torch.float32)
    scale = torch.where(amax > 0, scale, torch.ones_like(scale))
    q = (t / scale[:, None]).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).numpy().copy(), scale.numpy().copy()


MX_BLOCK = 32
E4M3_EMAX = 8            # exponent of E4M3's largest normal value (448 = 1.75 * 2^8)
E8M0_NAN_BITS = np.uint8(0xFF)


def mx_quantize_rows(x: np.ndarray):
    """OCP Microscaling (MX) quantisation of each row in blocks of 32 elements.

    Per block: shared exponent e = floor(log2(amax)) - 8 (0 for an all-zero
    block), clamped to [-127, 127]; E8M0 code e + 127; elements are the E4M3
    codes of x / 2^e, saturating at +-448. Returns (codes uint8 [R, K], scale
    codes uint8 [R, ceil(K/32)]).
    """
    x = np.asarray(x, dtype=np.float64)
    R, K = x.shape
    nb = (K + MX_BLOCK - 1) // MX_BLOCK
    padded = np.zeros((R, nb * MX_BLOCK))
    padded[:, :K] = x
    blocks = padded.reshape(R, nb, MX_BLOCK)
    amax = np.abs(blocks).max(axis=2)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - E4M3_EMAX, 0.0)
    e = np.clip(e, -127, 127).astype(np.int64)
    scaled = blocks / np.ldexp(1.0, e)[:, :, None]
    codes = to_e4m3_bits(scaled.reshape(R, nb * MX_BLOCK)[:, :K])
    return codes, (e + 127).astype(np.uint8)


def mx_scale_ld(K: int) -> int:
    """Smallest valid scale-row length: ceil(K/32) rounded up to a multiple of 4 (>= 4)."""
    nb = (K + MX_BLOCK - 1) // MX_BLOCK
    return max(4, (nb + 3) // 4 * 4)


def make_mx_problem(M: int, N: int, K: int, *, seed_base: int, alpha: float = 1.0,
                    beta: float = 0.0, lda: Optional[int] = None, ldb: Optional[int] = None,
                    ldc: Optional[int] = None, ldsa: Optional[int] = None,
                    ldsb: Optional[int] = None, c_dtype: int = OUT_F32, act: int = ACT_NONE,
                    a_std: float = 1.0, b_std: float = 1.0, cin_std: float = 1.0,
                    bias_std: Optional[float] = None, int_data: Optional[tuple] = None,
                    scale_codes: Optional[tuple] = None, name: str = "") -> "Problem":
    """An MX FP8 problem: A ROW (M x lda), B COL (N x ldb), E8M0 scales per 32 K.

    Normal data are MX-quantised per row of A and per column of B. With
    int_data=(lo, hi) the elements are small integers (exact in E4M3) and the
    scale codes are drawn uniformly from scale_codes=(lo, hi). Scale bytes past
    ceil(K/32) in a row hold the NaN code 0xFF (they must never be used).
    """
    lda = max(1, K) if lda is None else lda
    ldb = max(1, K) if ldb is None else ldb
    ldc = max(1, N) if ldc is None else ldc
    ldsa = mx_scale_ld(K) if ldsa is None else ldsa
    ldsb = mx_scale_ld(K) if ldsb is None else ldsb
    nb = (K + MX_BLOCK - 1) // MX_BLOCK
    if int_data is not None:
        a_codes = to_e4m3_bits(small_ints((M, K), int_data[0], int_data[1], seed_base + 0))
        bt_codes = to_e4m3_bits(small_ints((N, K), int_data[0], int_data[1], seed_base + 1))
        lo, hi = scale_codes if scale_codes is not None else (127, 127)
        rng = np.random.Generator(np.random.PCG64(seed_base + 5))
        sa = rng.integers(lo, hi + 1, size=(M, nb)).astype(np.uint8)
        sb = rng.integers(lo, hi + 1, size=(N, nb)).astype(np.uint8)
    else:
        a_codes, sa = mx_quantize_rows(normal((M, K), a_std, seed_base + 0))
        bt_codes, sb = mx_quantize_rows(normal((K, N), b_std, seed_base + 1).T)
    A = _pad(a_codes, lda, E4M3_NAN_BITS)
    B = _pad(bt_codes, ldb, E4M3_NAN_BITS)
    mx_a = np.full((M, ldsa), E8M0_NAN_BITS, np.uint8)
    mx_a[:, :nb] = sa
    mx_b = np.full((N, ldsb), E8M0_NAN_BITS, np.uint8)
    mx_b[:, :nb] = sb
    cin = normal((M, N), cin_std, seed_base + 2)
    if c_dtype == OUT_F32:
        C = np.full((M, ldc), np.nan, dtype=np.float32)
        C[:, :N] = cin.astype(np.float32)
    else:
        C = np.full((M, ldc), BF16_NAN_BITS, dtype=np.uint16)
        C[:, :N] = to_bf16_bits(cin)
    bias = None
    if bias_std is not None:
        bias = to_bf16_bits(normal((N,), bias_std, seed_base + 3))
    return Problem("mxfp8", M, N, K, alpha, beta, ROW, COL, lda, ldb, ldc, c_dtype, act, A, B, C,
                   bias, None, None, name or f"mxfp8_{M}x{N}x{K}", mx_a, mx_b, ldsa, ldsb)


def _pad(bits: np.ndarray, ld: int, pad_value) -> np.ndarray:
    rows, cols = bits.shape
    if ld == cols:
        return np.ascontiguousarray(bits)
    out = np.full((rows, ld), pad_value, dtype=bits.dtype)
    out[:, :cols] = bits
    return out


def store_a(logical_bits: np.ndarray, layout: int, ld: int, pad_value) -> np.ndarray:
    """Lay a logical MxK bit matrix out as operand A with the given layout and ld."""
    mat = logical_bits if layout == ROW else np.ascontiguousarray(logical_bits.T)
    return _pad(mat, ld, pad_value)


def store_b(logical_bits: np.ndarray, layout: int, ld: int, pad_value) -> np.ndarray:
    """Lay a logical KxN bit matrix out as operand B with the given layout and ld."""
    mat = logical_bits if layout == ROW else np.ascontiguousarray(logical_bits.T)
    return _pad(mat, ld, pad_value)


@dataclasses.dataclass
class Problem:
    """One GEMM call: shapes, layouts, epilogue and the operand arrays (bit patterns)."""

    kind: str  # "bf16" or "fp8"
    M: int
    N: int
    K: int
    alpha: float
    beta: float
    layout_a: int
    layout_b: int
    lda: int
    ldb: int
    ldc: int
    c_dtype: int
    act: int
    A: np.ndarray
    B: np.ndarray
    C: np.ndarray  # C_in (row-major, ldc); float32 or uint16 (bf16 bits)
    bias: Optional[np.ndarray]  # uint16 bf16 bits [N] or None
    scale_a: Optional[np.ndarray] = None  # float32 [M] (fp8 only)
    scale_b: Optional[np.ndarray] = None  # float32 [N] (fp8 only)
    name: str = ""
    # MX FP8 (kind "mxfp8"): E8M0 block-scale codes, one per 32 K elements.
    mx_a: Optional[np.ndarray] = None     # uint8 [M, ldsa]
    mx_b: Optional[np.ndarray] = None     # uint8 [N, ldsb]
    ldsa: int = 0
    ldsb: int = 0

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


def default_ld(rows_or_cols: int, pad: int = 0) -> int:
    return rows_or_cols + pad


def make_problem(
    kind: str,
    M: int,
    N: int,
    K: int,
    *,
    seed_base: int,
    alpha: float = 1.0,
    beta: float = 0.0,
    layout_a: int = ROW,
    layout_b: int = COL,
    lda: Optional[int] = None,
    ldb: Optional[int] = None,
    ldc: Optional[int] = None,
    c_dtype: int = OUT_F32,
    act: int = ACT_NONE,
    a_std: float = 1.0,
    b_std: float = 1.0,
    cin_std: float = 1.0,
    bias_std: Optional[float] = None,
    int_range: Optional[tuple] = None,
    name: str = "",
) -> Problem:
    """Build a seeded problem. seed_base = seed_for(config, 0); tensors use +0..+3.

    With int_range=(lo, hi), A and B hold small integers (exactly representable)
    instead of normal samples; for fp8 the scales are then 1.
    """
    if lda is None:
        lda = max(1, K if layout_a == ROW else M)
    if ldb is None:
        ldb = max(1, N if layout_b == ROW else K)
    if ldc is None:
        ldc = max(1, N)
    if int_range is not None:
        a_val = small_ints((M, K), int_range[0], int_range[1], seed_base + 0)
        b_val = small_ints((K, N), int_range[0], int_range[1], seed_base + 1)
    else:
        a_val = normal((M, K), a_std, seed_base + 0)
        b_val = normal((K, N), b_std, seed_base + 1)
    scale_a = scale_b = None
    if kind == "bf16":
        a_bits = to_bf16_bits(a_val)
        b_bits = to_bf16_bits(b_val)
        pad = BF16_NAN_BITS
    elif kind == "fp8":
        if int_range is not None:
            a_bits = to_e4m3_bits(a_val)
            b_bits = to_e4m3_bits(b_val)
            scale_a = np.ones(M, dtype=np.float32)
            scale_b = np.ones(N, dtype=np.float32)
        else:
            a_bits, scale_a = quantize_rows_e4m3(a_val) if M > 0 and K > 0 else (
                np.zeros((M, K), np.uint8), np.ones(M, np.float32))
            bt_bits, scale_b = quantize_rows_e4m3(b_val.T) if N > 0 and K > 0 else (
                np.zeros((N, K), np.uint8), np.ones(N, np.float32))
            b_bits = np.ascontiguousarray(bt_bits.T)
        pad = E4M3_NAN_BITS
    else:
        raise ValueError(kind)
    A = store_a(a_bits, layout_a, lda, pad)
    B = store_b(b_bits, layout_b, ldb, pad)
    cin = normal((M, N), cin_std, seed_base + 2)
    if c_dtype == OUT_F32:
        C = np.full((M, ldc), np.nan, dtype=np.float32)
        C[:, :N] = cin.astype(np.float32)
    else:
        C = np.full((M, ldc), BF16_NAN_BITS, dtype=np.uint16)
        C[:, :N] = to_bf16_bits(cin)
    bias = None
    if bias_std is not None:
        bias = to_bf16_bits(normal((N,), bias_std, seed_base + 3))
    return Problem(kind, M, N, K, alpha, beta, layout_a, layout_b, lda, ldb, ldc, c_dtype,
                   act, A, B, C, bias, scale_a, scale_b, name)
