"""Roofline and tiling arithmetic for GEMM (host-side bookkeeping, no GPU work).

The traffic model is the one worked through on the "GEMM (matrix multiply)"
tiling page: with A (MxK), B (KxN) and C (MxN) in HBM, an untiled GEMM reads
2MNK elements; with square output tiles of edge T each operand is re-read
N/T (resp. M/T) times, giving 2MNK/T element reads, i.e. 2K/T reads per
output element; one K step of length k costs a tile 2 T^2 k flops against
2 T k elements fetched, so its HBM arithmetic intensity is T / (bytes per
element) -- T/2 for 16-bit operands. The ridge point is peak FLOP/s over
HBM bytes/s.
"""
from __future__ import annotations

import math

# MI355X published dense peaks (no sparsity) and HBM3E bandwidth.
MI355X_PEAK_TFLOPS = {"bf16": 2516.6, "fp16": 2516.6, "fp8": 5033.2, "fp32": 157.3,
                      "fp64": 78.6}
MI355X_HBM_GBPS = 8000.0
MI355X_CUS = 256
MI355X_XCDS = 8


def gemm_flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


def naive_element_reads(M: int, N: int, K: int) -> int:
    """Element reads of the untiled GEMM: a row of A and a column of B per output."""
    return 2 * M * N * K


def tiled_element_reads(M: int, N: int, K: int, T: int) -> float:
    """Element reads with square output tiles of edge T (HBM worst case, no cache reuse)."""
    return 2 * M * N * K / T


def reads_per_output(K: int, T: int) -> float:
    return 2 * K / T


def tile_intensity(T: int, elem_bytes: float) -> float:
    """FLOP per HBM byte of one output tile: 2 T^2 k / (2 T k elem_bytes)."""
    return T / elem_bytes


def ridge_point(peak_flops: float, bandwidth_bytes: float) -> float:
    return peak_flops / bandwidth_bytes


def tile_edge_for_ridge(peak_flops: float, bandwidth_bytes: float, elem_bytes: float) -> float:
    return ridge_point(peak_flops, bandwidth_bytes) * elem_bytes


def bandwidth_bound_flops(T: int, elem_bytes: float, bandwidth_bytes: float) -> float:
    return tile_intensity(T, elem_bytes) * bandwidth_bytes


def grid_tiles(M: int, N: int, BM: int, BN: int) -> int:
    return math.ceil(M / BM) * math.ceil(N / BN)


def tile_operand_bytes(rows: int, bk: int, elem_bytes: float) -> float:
    return rows * bk * elem_bytes


def accumulators_per_thread(BM: int, BN: int, threads: int) -> float:
    return BM * BN / threads


def compulsory_bytes(M: int, N: int, K: int, a_bytes: float, b_bytes: float,
                     c_out_bytes: float, c_in_bytes: float = 0.0, bias_bytes: float = 0.0,
                     scale_bytes: float = 0.0) -> float:
    """Bytes a GEMM must move at least once: read A, B, C_in, bias, scales; write C."""
    return (M * K * a_bytes + K * N * b_bytes + M * N * (c_out_bytes + c_in_bytes)
            + N * bias_bytes + (M + N) * scale_bytes)
