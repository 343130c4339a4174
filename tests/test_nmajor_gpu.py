"""BF16 GEMM with B stored N-contiguous (row-major K x N) on the DMA path.

Such a B is copied into an N-major LDS tile and its MFMA fragments are read
with the transposing LDS read; the K-major path reads fragments directly.
Both put the same K indices in the same register slots, so for the same plan
the two layouts must give the same bits: B given row-major equals the same
logical B given column-major. Each case is also checked against the oracle,
and NaN in the padding columns of a row-major B (ldb > N) must not reach C.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

from synth import (ACT_GELU_ERF, ACT_NONE, ACT_RELU, COL, OUT_BF16, OUT_F32, ROW,
                   make_problem)
from tests.common import compare

pytestmark = pytest.mark.gpu


def run_both(p):
    """Run p (B row-major) and the same logical B column-major; return both outputs."""
    import copy
    import torch
    from tests.gpu_util import run
    import oracle
    assert p.layout_b == ROW
    q = copy.copy(p)
    q.layout_b, q.ldb = COL, p.K
    q.B = np.ascontiguousarray(oracle.logical_b(p.B, ROW, p.K, p.N).T)   # N x K, same bits
    out_row = run(p)
    out_col = run(q)
    return out_row, out_col


CASES = [
    # M, N, K, c_dtype, act, beta
    (256, 256, 256, OUT_F32, ACT_NONE, 0.0),
    (300, 264, 200, OUT_F32, ACT_GELU_ERF, 0.5),       # ragged M and N (N % 8 == 0), bias
    (512, 512, 4096, OUT_BF16, ACT_RELU, 0.0),         # 256x256 tiles, long K
    (384, 640, 1024, OUT_BF16, ACT_NONE, 0.0),
    (64, 4096, 2048, OUT_F32, ACT_NONE, 0.0),          # split-K plan
]


@pytest.mark.parametrize("M,N,K,c_dtype,act,beta", CASES)
def test_row_major_b_matches_k_major_bitwise(M, N, K, c_dtype, act, beta):
    import dense_gemm_09_amd as g
    pl = g.plan(M, N, K, False)
    print(f"[plan] tile={pl.tile_m}x{pl.tile_n} split={pl.split_k}", flush=True)
    p = make_problem("bf16", M, N, K, seed_base=0x5EEDE100 + M + N + K, layout_a=ROW,
                     layout_b=ROW, c_dtype=c_dtype, act=act, beta=beta,
                     bias_std=0.1 if act != ACT_NONE else None, a_std=1.0, b_std=K ** -0.5,
                     name=f"rowB_{M}x{N}x{K}")
    out_row, out_col = run_both(p)
    assert np.array_equal(out_row.view(np.uint8), out_col.view(np.uint8)), \
        f"{int((out_row != out_col).sum())} elements differ between B layouts"
    compare(p, out_row)


def test_row_major_b_nan_padding_and_square_4096():
    p = make_problem("bf16", 4096, 4096, 4096, seed_base=0x5EEDE200, layout_a=ROW, layout_b=ROW,
                     ldb=4096 + 8, c_dtype=OUT_F32, a_std=4096 ** -0.5, b_std=4096 ** -0.5,
                     name="rowB_4096_padded")
    assert (p.B[:, 4096:] == 0x7FC0).all()      # BF16 NaN in the padding columns
    out_row, out_col = run_both(p)
    assert np.all(np.isfinite(out_row))
    assert np.array_equal(out_row.view(np.uint8), out_col.view(np.uint8))
    rows = np.array([0, 1, 255, 256, 2047, 4095])
    cols = np.array([0, 7, 8, 255, 256, 4088, 4095])
    compare(p, out_row[np.ix_(rows, cols)], rows=rows, cols=cols)


def test_row_major_b_integer_exact():
    p = make_problem("bf16", 200, 136, 328, seed_base=0x5EEDE300, layout_a=ROW, layout_b=ROW,
                     c_dtype=OUT_F32, int_range=(-4, 4), name="rowB_int")
    out_row, _ = run_both(p)
    from tests.common import reference
    _, ref = reference(p)
    assert np.array_equal(out_row, ref)


def test_row_major_b_decode_sized_m():
    """M <= 16 with row-major B takes the tile path (the skinny kernel reads
    K-major B only), so it is checked against the oracle, not against the
    column-major run (which takes the skinny kernel)."""
    from tests.gpu_util import run
    p = make_problem("bf16", 5, 1000, 512, seed_base=0x5EEDE400, layout_a=ROW, layout_b=ROW,
                     c_dtype=OUT_F32, a_std=1.0, b_std=0.05, name="rowB_decode")
    compare(p, run(p))
