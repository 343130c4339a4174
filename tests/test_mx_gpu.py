"""Parity of the MX (E8M0 block-scaled) FP8 GEMM, gemm_mxfp8, on the GPU.

Exact cases: integer E4M3 data in [-4, 4] and scale exponents in [-1, 2]
give products that are multiples of 2^-2 below 2^8 and sums below 2^21, so
FP32 accumulation (and the FP8 MFMA's 13-bit alignment window) is exact in any
order: the FP32 output must equal the oracle bit for bit. They cover the
128x128 tiles with ragged M and N, K that is not a multiple of
the 128-element slice (the last slice holds fewer than four scale blocks and
the caller's padding bytes are the NaN code 0xFF, which must not be used),
split-K with its reduction, decode-sized M (which takes the tile path here),
and K = 0.

Random cases: MX-quantised normal data with bias, GELU and BF16 or FP32
output, checked with the FP8 tolerances (section of tests/tolerance.py), on
full size at the 4096^3 shape by sampled rows and columns.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

from synth import ACT_GELU_ERF, ACT_NONE, ACT_RELU, OUT_BF16, OUT_F32, make_mx_problem
from tests.common import compare, reference

pytestmark = pytest.mark.gpu


def run(p, repeat=1, rows=None, cols=None):
    import torch
    from tests.gpu_util import call, to_device
    print(f"[gpu] mxfp8 {p.name} M={p.M} N={p.N} K={p.K} ldsa={p.ldsa} c_dtype={p.c_dtype}",
          flush=True)
    sys.stdout.flush()
    d = to_device(p)
    c0 = d["C"].clone()
    outs = []
    for _ in range(repeat):
        d["C"].copy_(c0)
        call(p, d)
        torch.cuda.synchronize()
        o = d["C"].cpu().numpy()
        outs.append(o.view(np.uint16) if p.c_dtype == OUT_BF16 else o)
    for o in outs[1:]:  # bitwise (the padding columns hold NaN)
        assert np.array_equal(o.view(np.uint8), outs[0].view(np.uint8)), "run-to-run difference"
    out = outs[0]
    if p.ldc > p.N:  # padding columns of C are never written
        pad = out[:, p.N:]
        assert (np.isnan(pad).all() if p.c_dtype == OUT_F32 else (pad == 0x7FC0).all())
    out = out[:, :p.N]
    if rows is not None:
        out = out[np.ix_(rows, cols)]
    return out


EXACT = [
    (256, 256, 256),     # 128x128 tiles, two per CU
    (300, 260, 160),     # ragged M, N; K = 160: five blocks, the last slice holds one
    (129, 70, 96),       # 128x128 tiles, K below one slice
    (64, 4096, 2048),    # split-K + reduction
    (5, 384, 512),       # decode-sized M on the tile path
]


@pytest.mark.parametrize("M,N,K", EXACT)
def test_exact_integer_problems(M, N, K):
    import dense_gemm_09_amd as g
    pl = g.plan(M, N, K, True)
    print(f"[plan] tile={pl.tile_m}x{pl.tile_n} split={pl.split_k}", flush=True)
    p = make_mx_problem(M, N, K, seed_base=0x5EEDB000 + M + N + K, int_data=(-4, 4),
                        scale_codes=(126, 129), c_dtype=OUT_F32, ldc=N + 3, beta=0.0)
    out = run(p, repeat=2)
    y, ref = reference(p)
    assert np.array_equal(y, np.round(y * 4) / 4), "exact case must be a multiple of 1/4"
    mism = np.argwhere(out != ref)
    assert mism.size == 0, f"{len(mism)} mismatches, first {mism[0]}: {out[tuple(mism[0])]} vs {ref[tuple(mism[0])]}"


def test_exact_with_epilogue_beta_bias_relu():
    p = make_mx_problem(192, 136, 224, seed_base=0x5EEDB100, int_data=(-4, 4),
                        scale_codes=(126, 129), c_dtype=OUT_F32, beta=0.5, alpha=2.0,
                        act=ACT_RELU, bias_std=4.0)
    # bias and C_in are arbitrary BF16 / FP32 values: y is then rounded once
    out = run(p)
    compare(p, out)


def test_k_zero():
    p = make_mx_problem(33, 40, 0, seed_base=0x5EEDB200, c_dtype=OUT_F32, beta=1.5,
                        bias_std=1.0, act=ACT_RELU)
    out = run(p)
    compare(p, out)


@pytest.mark.parametrize("M,N,K,c_dtype,act", [
    (512, 1024, 1024, OUT_BF16, ACT_GELU_ERF),
    (384, 640, 2048, OUT_F32, ACT_NONE),
    (16, 2048, 4096, OUT_BF16, ACT_NONE),      # split-K
])
def test_random_mx_quantised(M, N, K, c_dtype, act):
    p = make_mx_problem(M, N, K, seed_base=0x5EEDB300 + M + K, c_dtype=c_dtype, act=act,
                        a_std=1.0, b_std=0.05, bias_std=0.1)
    out = run(p)
    compare(p, out)


def test_square_4096_sampled():
    p = make_mx_problem(4096, 4096, 4096, seed_base=0x5EEDB400, c_dtype=OUT_BF16, act=ACT_NONE,
                        a_std=1.0, b_std=4096 ** -0.5, name="mxfp8_4096^3")
    rng = np.random.default_rng(4)
    rows = np.unique(np.concatenate([[0, 127, 128, 255, 4095], rng.integers(0, 4096, 27)]))
    cols = np.unique(np.concatenate([[0, 127, 128, 4095], rng.integers(0, 4096, 28)]))
    out = run(p, rows=rows, cols=cols)
    compare(p, out, rows=rows, cols=cols)
