"""Seeded random configurations through the C ABI against the float64 oracle.

Each case draws, from a fixed seed, a shape (M, N up to 700 with a share of
decode-sized M <= 16 and of M, N in the 17..64 band, K up to 1200 including
0 and values that end inside a 16-byte chunk), the input kind (BF16 or FP8
E4M3 with per-token / per-channel scales), the layouts of A and B (any for
BF16, K-major for FP8), padded leading dimensions (NaN padding), alpha,
beta, a bias, the activation and the output type. Together they reach the
skinny kernel, the 64-row tiles, the 128x128 and 256x256 tiles, split-K with
its reduction, the DMA, N-major and register loaders and the ragged-K patch
in combinations the targeted tests do not list one by one.
"""
from __future__ import annotations

import numpy as np
import pytest

import dense_gemm_09_amd as g
import synth
from synth import (ACT_GELU_ERF, ACT_GELU_TANH, ACT_NONE, ACT_RELU, COL, OUT_BF16, OUT_F32,
                   ROW)
from tests.common import compare
from tests.gpu_util import run

pytestmark = pytest.mark.gpu

N_CASES = 48


def _dim(rng, small_share=0.25, band_share=0.2, hi=700):
    u = rng.random()
    if u < small_share:
        return int(rng.integers(1, 17))
    if u < small_share + band_share:
        return int(rng.integers(17, 65))
    return int(rng.integers(65, hi + 1))


def _case(i):
    rng = np.random.default_rng(0xC0FFEE00 + i)
    kind = "bf16" if rng.random() < 0.55 else "fp8"
    M, N = _dim(rng), _dim(rng, small_share=0.05)
    u = rng.random()
    if u < 0.05:
        K = 0
    elif u < 0.35:
        K = int(rng.integers(1, 1201))                       # any K: ragged tails
    else:
        K = 16 * int(rng.integers(1, 76))                    # whole 16-element chunks
    if kind == "bf16":
        la, lb = int(rng.integers(0, 2)), int(rng.integers(0, 2))
    else:
        la, lb = ROW, COL
    pad = lambda: int(rng.choice([0, 0, 1, 8, 16, 37]))      # noqa: E731
    lda = (K if la == ROW else M) + pad()
    ldb = (N if lb == ROW else K) + pad()
    ldc = N + pad()
    alpha = float(rng.choice([1.0, -1.5, 0.5]))
    beta = float(rng.choice([0.0, 0.0, 0.75]))
    bias = float(rng.choice([0.0, 0.1])) or None
    act = int(rng.choice([ACT_NONE, ACT_RELU, ACT_GELU_ERF, ACT_GELU_TANH]))
    c_dtype = int(rng.choice([OUT_F32, OUT_BF16]))
    return dict(kind=kind, M=M, N=N, K=K, layout_a=la, layout_b=lb, lda=max(1, lda),
                ldb=max(1, ldb), ldc=max(1, ldc), alpha=alpha, beta=beta, bias_std=bias,
                act=act, c_dtype=c_dtype)


CASES = [_case(i) for i in range(N_CASES)]


def _id(c):
    return (f"{c['kind']}-{c['M']}x{c['N']}x{c['K']}-l{c['layout_a']}{c['layout_b']}"
            f"-ld{c['lda']},{c['ldb']},{c['ldc']}-a{c['alpha']}-b{c['beta']}"
            f"-act{c['act']}-out{c['c_dtype']}")


def test_cases_reach_every_kernel():
    """The draw covers the skinny kernel, the 64-row tiles, larger tiles,
    split-K, K = 0 and ragged K (a property of the seeded draw itself)."""
    plans = [g.plan(c["M"], c["N"], c["K"], c["kind"] == "fp8") for c in CASES]
    assert any(p.kernel == 1 for p in plans)
    assert any(p.kernel == 0 and p.tile_m == 64 for p in plans)
    assert any(p.kernel == 0 and p.tile_m >= 128 for p in plans)
    assert any(p.split_k > 1 for p in plans)
    assert any(c["K"] == 0 for c in CASES)
    assert any(c["K"] % 16 != 0 for c in CASES)
    assert {c["kind"] for c in CASES} == {"bf16", "fp8"}


@pytest.mark.parametrize("i", range(N_CASES), ids=[_id(c) for c in CASES])
def test_random_configuration(i):
    c = CASES[i]
    kind = c["kind"]
    p = synth.make_problem(kind, c["M"], c["N"], c["K"], seed_base=0x5A5A0000 + 16 * i,
                           alpha=c["alpha"], beta=c["beta"], layout_a=c["layout_a"],
                           layout_b=c["layout_b"], lda=c["lda"], ldb=c["ldb"], ldc=c["ldc"],
                           c_dtype=c["c_dtype"], act=c["act"], a_std=1.0,
                           b_std=max(1, c["K"]) ** -0.5, bias_std=c["bias_std"],
                           name=_id(c))
    pl = g.plan(p.M, p.N, p.K, kind == "fp8")
    print(f"[plan] kernel={pl.kernel} tile={pl.tile_m}x{pl.tile_n} split={pl.split_k}",
          flush=True)
    compare(p, run(p))
