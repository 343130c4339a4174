"""Parity of the quantising epilogue (gemm_bf16_quant / gemm_fp8_scaled_quant) on the GPU.

Exact cases: integer-valued A, B and bias, ReLU or no activation, power-of-two
output scales and integer zero points. y, y * s + zp and y * s are then exact
in FP32 whatever the accumulation order, so every code must equal the
oracle's bit for bit. These cases cover each kernel path the plan can take:
the 256- and 128-wide tiles with ragged edges, split-K with its reduction
kernel, the skinny decode kernel, and the register loader (row-major B).

Random cases: the kernel's FP32 y differs from the oracle's by at most the
parity bound of the FP32 path (1e-4 |alpha| ||a_m|| ||b_n||, times the
activation's largest slope near z, plus a few FP32 ulps and the activation's
FP32 evaluation error; tests/tolerance.py), so each code must lie
between the oracle's codes for y - e and y + e (the quantiser is monotone for
positive scales). That bound is conservative (Cauchy-Schwarz on the worst
case); the actual error of a BF16 GEMM is near 1e-6 relative, so the test
also requires that at least 99.9% of its codes equal the oracle's code for y
itself. FP8 sums carry more: each FP8 MFMA drops product bits below 2^-13 of
its K group's largest product (tests/test_parity_gpu.py pins that window),
about 1e-4 relative, i.e. ~0.01 of an INT8 step at full scale, so there the
requirement is 98%.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from oracle import QOUT_E4M3, QOUT_INT8
from synth import ACT_GELU_ERF, ACT_NONE, ACT_RELU, COL, ROW, make_problem
from tests.common import operand_norms, reference
from tests import tolerance
from tests.tolerance import ulp_f32

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A


def bf16_bits_of_ints(v):
    return (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def run_quant(p, out_scale, out_zero, q_dtype, ldq=None, repeat=1):
    """Run the quantising GEMM for problem p; return (Q[:, :N], raw Q) as numpy uint8."""
    import torch
    import dense_gemm_09_amd as g
    from tests.gpu_util import to_device
    ldq = p.N if ldq is None else ldq
    print(f"[gpu] quant {p.name} M={p.M} N={p.N} K={p.K} ldq={ldq} q_dtype={q_dtype} "
          f"zp={'yes' if out_zero is not None else 'no'}", flush=True)
    sys.stdout.flush()
    d = to_device(p)
    Q = torch.full((max(p.M, 1) * ldq,), SENTINEL, dtype=torch.uint8, device="cuda")
    osc = torch.from_numpy(np.asarray(out_scale, np.float32)).cuda()
    ozp = None if out_zero is None else torch.from_numpy(np.asarray(out_zero, np.int32)).cuda()
    outs = []
    for _ in range(repeat):
        if p.kind == "bf16":
            g.gemm_bf16_quant(p.M, p.N, p.K, p.alpha, d["A"], p.lda, p.layout_a, d["B"], p.ldb,
                              p.layout_b, d["bias"], p.act, osc, ozp, Q, ldq, q_dtype)
        else:
            g.gemm_fp8_scaled_quant(p.M, p.N, p.K, p.alpha, d["A"], p.lda, p.layout_a, d["B"],
                                    p.ldb, p.layout_b, d["scale_a"], d["scale_b"], d["bias"],
                                    p.act, osc, ozp, Q, ldq, q_dtype)
        torch.cuda.synchronize()
        outs.append(Q.cpu().numpy().reshape(max(p.M, 1), ldq)[:p.M].copy())
    for o in outs[1:]:
        assert np.array_equal(o, outs[0]), "run-to-run difference"
    raw = outs[0]
    assert np.all(raw[:, p.N:] == SENTINEL), "columns N..ldq-1 were written"
    return raw[:, :p.N], raw


def as_codes(q_u8, q_dtype):
    return q_u8.view(np.int8).astype(np.int64) if q_dtype == QOUT_INT8 else q_u8


def exact_problem(kind, M, N, K, seed, layout_b=COL, act=ACT_RELU, bias=True):
    p = make_problem(kind, M, N, K, seed_base=0x5EED9000 + 16 * seed, layout_a=ROW,
                     layout_b=layout_b, act=act, int_range=(-4, 4) if kind == "bf16" else (-8, 8),
                     name=f"exact_{kind}_{M}x{N}x{K}")
    if bias:
        rng = np.random.default_rng(seed)
        p.bias = bf16_bits_of_ints(rng.integers(-64, 64, size=N))
    return p


EXACT_CASES = [
    # kind, M, N, K, layout_b: the plan's tile / split / kernel differ across these
    ("bf16", 300, 260, 200, COL),      # 128-wide tiles, ragged M, N and K
    ("bf16", 512, 512, 256, COL),      # 256x256 tiles
    ("bf16", 64, 4096, 2048, COL),     # split-K + reduction kernel
    ("bf16", 5, 300, 512, COL),        # skinny decode kernel
    ("bf16", 130, 70, 96, ROW),        # register loader for B
    ("fp8", 300, 260, 256, COL),
    ("fp8", 64, 4096, 2048, COL),      # split-K
    ("fp8", 3, 520, 1024, COL),        # skinny
]


@pytest.mark.parametrize("q_dtype", [QOUT_INT8, QOUT_E4M3])
@pytest.mark.parametrize("case", EXACT_CASES, ids=lambda c: f"{c[0]}_{c[1]}x{c[2]}x{c[3]}_{'col' if c[4] else 'row'}B")
def test_exact_codes(case, q_dtype):
    import dense_gemm_09_amd as g
    kind, M, N, K, lb = case
    p = exact_problem(kind, M, N, K, seed=M + N + K, layout_b=lb)
    pl = g.plan(M, N, K, kind == "fp8")
    print(f"[plan] kernel={pl.kernel} tile={pl.tile_m}x{pl.tile_n} split={pl.split_k}", flush=True)
    y, _ = reference(p)
    assert np.all(y == np.rint(y)), "exact case must have integer y"
    rng = np.random.default_rng(M * 7 + N)
    amax = np.maximum(np.abs(y).max(axis=1), 1.0)
    if q_dtype == QOUT_INT8:
        # power-of-two scale per row (some rows saturate), integer zero points
        s = np.exp2(np.round(np.log2(100.0 / amax)) + rng.integers(-1, 2, size=M)).astype(np.float32)
        zp = rng.integers(-20, 21, size=M).astype(np.int32)
    else:
        s = np.exp2(np.round(np.log2(400.0 / amax)) + rng.integers(-1, 2, size=M)).astype(np.float32)
        zp = None
    q, _ = run_quant(p, s, zp, q_dtype, ldq=N + 4, repeat=2)
    ref = oracle.quantize_output(y, s, zp, q_dtype)
    got = as_codes(q, q_dtype)
    if q_dtype == QOUT_E4M3:
        # -0 and +0 are both exact zeros: compare values there, codes elsewhere
        vz = oracle.decode_e4m3(ref) == 0
        assert np.array_equal(oracle.decode_e4m3(got)[vz], np.zeros(vz.sum()))
        got, ref = got[~vz], ref[~vz]
    mism = np.argwhere(got != ref)
    assert mism.size == 0, f"{len(mism)} code mismatches, first {mism[0]}"
    if q_dtype == QOUT_INT8:
        assert (got == 127).any() or (got == -128).any() or M < 8  # saturation exercised


def bracket_check(p, q_u8, s, zp, q_dtype, rows=None, cols=None, min_exact=None):
    if min_exact is None:
        min_exact = 0.999 if p.kind == "bf16" else 0.98
    y, _, z = reference(p, rows, cols, with_z=True)
    rn, cn = operand_norms(p, rows, cols)
    e = 1e-4 * abs(p.alpha) * np.outer(rn, cn)
    e = e * tolerance.slope_bound(z, e, p.act) + tolerance.ACT_REL[p.act] * np.abs(y)
    e = e + 4 * ulp_f32(y)
    r = np.arange(p.M) if rows is None else np.asarray(rows)
    s_sel = np.asarray(s)[r]
    zp_sel = None if zp is None else np.asarray(zp)[r]
    lo = oracle.quantize_output(y - e, s_sel, zp_sel, q_dtype)
    hi = oracle.quantize_output(y + e, s_sel, zp_sel, q_dtype)
    mid = oracle.quantize_output(y, s_sel, zp_sel, q_dtype)
    got = as_codes(q_u8, q_dtype)
    if q_dtype == QOUT_E4M3:
        lo, hi, mid, got = (oracle.decode_e4m3(x) for x in (lo, hi, mid, got))
    ok = (lo <= got) & (got <= hi)
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{int((~ok).sum())} codes outside the bracket, first {i}: "
                             f"got={got[i]} lo={lo[i]} hi={hi[i]} y={y[i]!r}")
    frac = float((got == mid).mean())
    assert frac >= min_exact, f"only {frac:.5f} of the codes equal the oracle's code for y"
    return frac


@pytest.mark.parametrize("q_dtype", [QOUT_INT8, QOUT_E4M3])
@pytest.mark.parametrize("kind,M,N,K,act", [
    ("fp8", 384, 1024, 1024, ACT_GELU_ERF),
    ("bf16", 256, 640, 1024, ACT_NONE),
    ("bf16", 40, 2048, 4096, ACT_GELU_ERF),   # split-K
    ("fp8", 16, 1000, 2048, ACT_NONE),        # skinny
])
def test_random_codes_within_bracket(kind, M, N, K, act, q_dtype):
    p = make_problem(kind, M, N, K, seed_base=0x5EED9800 + M + N, layout_a=ROW, layout_b=COL,
                     act=act, a_std=1.0, b_std=0.05, bias_std=0.1,
                     name=f"rand_{kind}_{M}x{N}x{K}")
    y, _ = reference(p)
    rng = np.random.default_rng(N)
    amax = np.maximum(np.abs(y).max(axis=1), 1e-3)
    if q_dtype == QOUT_INT8:
        s = (120.0 / amax).astype(np.float32)
        zp = rng.integers(-10, 11, size=M).astype(np.int32)
    else:
        s = (440.0 / amax).astype(np.float32)
        zp = None
    q, _ = run_quant(p, s, zp, q_dtype, ldq=N + 1)   # odd ldq: element stores
    q2, _ = run_quant(p, s, zp, q_dtype)             # ldq = N: vector stores where aligned
    assert np.array_equal(q, q2)
    bracket_check(p, q, s, zp, q_dtype)


def test_fp8_projection_full_size_sampled():
    """The FP8 projection shape (4096 x 7168 x 2048, bias, GELU) with INT8 output, sampled."""
    from synth import workloads
    p = workloads.fp8_projection()
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 2047, 4095],
                                     np.random.default_rng(1).integers(0, p.M, 26)]))
    cols = np.unique(np.concatenate([[0, 1, 255, 256, 7167],
                                     np.random.default_rng(2).integers(0, p.N, 59)]))
    s = np.full(p.M, 24.0, np.float32)
    zp = np.full(p.M, -3, np.int32)
    q, _ = run_quant(p, s, zp, QOUT_INT8)
    bracket_check(p, q[np.ix_(rows, cols)], s, zp, QOUT_INT8, rows=rows, cols=cols)


def test_k_zero_quantises_bias():
    p = make_problem("bf16", 7, 33, 0, seed_base=0x5EED9F00, act=ACT_RELU, bias_std=4.0,
                     name="k0_quant")
    s = np.full(7, 8.0, np.float32)
    zp = np.arange(7, dtype=np.int32) - 3
    q, _ = run_quant(p, s, zp, QOUT_INT8)
    y, _ = reference(p)
    assert np.array_equal(as_codes(q, QOUT_INT8), oracle.quantize_output(y, s, zp, QOUT_INT8))
