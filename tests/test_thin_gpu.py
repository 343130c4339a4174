"""The 64-row tiles for few rows (M <= 64), against the oracle.

Row counts up to 64 run on 64x256 tiles (four waves of 64x64, a four-slice
LDS ring) or 64x128 tiles (two waves of 64x64, a six-slice ring), split over
K so that tiles x splits fill the CUs once. Integer
operands make every summation order exact, so FP32 outputs must equal the
oracle bit for bit: M below and at the tile height, N ragged and a multiple
of the tile, split and unsplit K, the N-contiguous B path, FP8, ragged K and
the epilogue with beta, bias and activation (tolerance path).
"""
from __future__ import annotations

import numpy as np
import pytest

import dense_gemm_09_amd as g
import synth
from synth import ACT_GELU_ERF, ACT_RELU, OUT_BF16, OUT_F32, ROW
from tests.common import compare, reference
from tests.gpu_util import run

pytestmark = pytest.mark.gpu


def _exact(p):
    pl = g.plan(p.M, p.N, p.K, p.kind != "bf16")
    print(f"[plan] {p.kind} M={p.M} N={p.N} K={p.K} tile={pl.tile_m}x{pl.tile_n} "
          f"split={pl.split_k}", flush=True)
    _, ref = reference(p)
    out = run(p)
    bad = np.argwhere(out != ref)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
@pytest.mark.parametrize("M,N,K", [(17, 300, 512), (40, 256, 1024), (64, 4096, 4096),
                                   (64, 520, 8192), (33, 1000, 203), (64, 257, 64)])
def test_thin_tile_exact(kind, M, N, K):
    lo, hi = (-4, 4) if kind == "bf16" else (-16, 16)
    p = synth.make_problem(kind, M, N, K, seed_base=0x770000 + M + N + K, int_range=(lo, hi),
                           c_dtype=OUT_F32)
    _exact(p)


@pytest.mark.parametrize("N", [264, 4096])
def test_thin_tile_row_major_b_exact(N):
    p = synth.make_problem("bf16", 64, N, 1000, seed_base=0x780000 + N, layout_b=ROW,
                           int_range=(-4, 4), c_dtype=OUT_F32)
    _exact(p)


@pytest.mark.parametrize("la,lb", [(1, 1), (1, 0), (0, 0)])
def test_few_rows_register_loaded_operands_exact(la, lb):
    """M <= 64 with an operand the DMA path cannot read (A column-major, or a
    row-major B whose N is not a multiple of 8): the 128x128 register-loader
    tile runs with the K split planned for the 64-row tile."""
    M, N, K = 40, 300 if lb == 1 else 301, 3001
    p = synth.make_problem("bf16", M, N, K, seed_base=0x7A0000 + la * 2 + lb, layout_a=la,
                           layout_b=lb, int_range=(-4, 4), c_dtype=OUT_F32)
    assert g.plan(M, N, K, False).split_k > 1
    _exact(p)


@pytest.mark.parametrize("kind,c_dtype,act", [("bf16", OUT_BF16, ACT_GELU_ERF),
                                              ("bf16", OUT_F32, ACT_RELU),
                                              ("fp8", OUT_BF16, ACT_GELU_ERF)])
def test_thin_tile_epilogue(kind, c_dtype, act):
    M, N, K = 48, 1100, 2048
    p = synth.make_problem(kind, M, N, K, seed_base=0x790000 + c_dtype + act, beta=0.5,
                           bias_std=0.1, act=act, c_dtype=c_dtype, a_std=K ** -0.5)
    compare(p, run(p))


def test_thin_plans():
    for fp8 in (False, True):
        for M, N in ((64, 4096), (64, 18432), (20, 11008)):
            p = g.plan(M, N, 4096, fp8)
            assert p.tile_m == 64 and p.tile_n in (128, 256)
            assert p.grid <= 256 or p.split_k == 1
