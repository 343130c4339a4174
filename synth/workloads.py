"""The named synthetic workloads (shapes, layouts, value distributions, epilogues).

Shapes follow the pages' workloads: square 4096^3 GEMMs (the tiling example of
the first DeepGEMM page, sec. 2.2, and the H100 roofline arithmetic of the
"GEMM (matrix multiply)" tiling page), FP8 transformer projections with
per-token / per-channel scales (DeepGEMM: FP8 precision Tensor Core GEMM
optimisation, sec. 1.2 and 3.2), FFN projection shapes, decode-sized M (the
1 x 4096 x 4096 row of the first page's sec. 5.1 table) and ragged sizes that
are not multiples of any tile (first page, sec. 4.2-4.3).

`N(0, s)` below means standard deviation s. All values are drawn from
seeded PCG64 streams; nothing is read from disk.
"""
from __future__ import annotations

from typing import List

from . import (ACT_GELU_ERF, ACT_NONE, COL, OUT_BF16, OUT_F32, ROW, Problem,
               make_problem)

BASE = 0x5EED0000


def seed_base(config: int, sub: int = 0) -> int:
    """Seed of tensor 0 of a workload; tensors A, B, C_in, bias use +0..+3."""
    return BASE + 16 * config + 4096 * sub


def small_square(n: int = 256) -> Problem:
    """M=N=K=256 bf16, A and B ~N(0,1), C fp32 zero-init, alpha 1, beta 0, A and B row-major."""
    return make_problem("bf16", n, n, n, seed_base=seed_base(0), alpha=1.0, beta=0.0,
                        layout_a=ROW, layout_b=ROW, c_dtype=OUT_F32, cin_std=0.0,
                        name=f"bf16_{n}^3_rowB")


def square_bf16(n: int = 4096) -> Problem:
    """M=N=K=n bf16, A,B ~N(0,1/sqrt(K)), C_in fp32 ~N(0,1), alpha 1, beta 0.5, A row-major, B col-major."""
    return make_problem("bf16", n, n, n, seed_base=seed_base(1), alpha=1.0, beta=0.5,
                        layout_a=ROW, layout_b=COL, c_dtype=OUT_F32,
                        a_std=n ** -0.5, b_std=n ** -0.5, cin_std=1.0,
                        name=f"bf16_{n}^3_beta0.5")


def fp8_projection(M: int = 4096, N: int = 7168, K: int = 2048, sub: int = 0) -> Problem:
    """FP8 E4M3 per-token/per-channel scaled, bias bf16 ~N(0,0.1), GELU, bf16 out."""
    return make_problem("fp8", M, N, K, seed_base=seed_base(2, sub), alpha=1.0, beta=0.0,
                        layout_a=ROW, layout_b=COL, c_dtype=OUT_BF16, act=ACT_GELU_ERF,
                        bias_std=0.1, name=f"fp8_{M}x{N}x{K}_bias_gelu")


FFN_SHAPES = [(14336, 4096), (4096, 14336)]
FFN_M = [512, 2048, 8192]


def ffn(M: int, N: int, K: int) -> Problem:
    """FFN projection: bf16 K-major, activations ~N(0,1), weights ~N(0,0.02), bias, bf16 out."""
    sub = FFN_M.index(M) * 2 + FFN_SHAPES.index((N, K))
    return make_problem("bf16", M, N, K, seed_base=seed_base(3, sub), alpha=1.0, beta=0.0,
                        layout_a=ROW, layout_b=COL, c_dtype=OUT_BF16, act=ACT_NONE,
                        a_std=1.0, b_std=0.02, bias_std=0.02,
                        name=f"ffn_bf16_{M}x{N}x{K}")


DECODE_M = [1, 4, 16, 64]
DECODE_N = [4096, 11008, 18432]


def decode(kind: str, M: int, N: int, K: int = 4096) -> Problem:
    """Decode-shaped skinny GEMM: activations ~N(0,1), weights ~N(0,0.02), bf16 out, no epilogue."""
    sub = DECODE_M.index(M) * 3 + DECODE_N.index(N) + (0 if kind == "bf16" else 100)
    return make_problem(kind, M, N, K, seed_base=seed_base(4, sub), alpha=1.0, beta=0.0,
                        layout_a=ROW, layout_b=COL, c_dtype=OUT_BF16, act=ACT_NONE,
                        a_std=1.0, b_std=0.02, name=f"decode_{kind}_{M}x{N}x{K}")


def ragged(kind: str, n: int = 4093, padded: bool = False) -> Problem:
    """M=N=K=4093: bf16 with fp32 out, or fp8 with bf16 out; tight or padded (4096) leading dims."""
    ld = 4096 if padded else n
    sub = (0 if kind == "bf16" else 1) + (2 if padded else 0)
    if kind == "bf16":
        return make_problem("bf16", n, n, n, seed_base=seed_base(4, 1000 + sub), alpha=1.0,
                            beta=0.0, layout_a=ROW, layout_b=COL, lda=ld, ldb=ld, ldc=ld,
                            c_dtype=OUT_F32, a_std=n ** -0.5, b_std=n ** -0.5,
                            name=f"ragged_bf16_{n}^3_ld{ld}")
    return make_problem("fp8", n, n, n, seed_base=seed_base(4, 1000 + sub), alpha=1.0,
                        beta=0.0, layout_a=ROW, layout_b=COL, lda=ld, ldb=ld, ldc=ld,
                        c_dtype=OUT_BF16, name=f"ragged_fp8_{n}^3_ld{ld}")


def all_decode() -> List[tuple]:
    return [(kind, M, N) for kind in ("bf16", "fp8") for M in DECODE_M for N in DECODE_N]
