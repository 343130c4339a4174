"""Parity tolerances for comparing a GEMM result with the float64 oracle.

FP32 output:
  * relative Frobenius error ||out - y||_F / ||y||_F <= 1e-5, and
  * per element |out - y| <= 1e-4 * |alpha| * ||a_m||_2 * ||b_n||_2 + ulp_f32(y),
    where a_m is row m of A and b_n column n of B (dequantised for FP8).

FP8 inputs with FP32 output: the same per-element bound, and relative
Frobenius error <= 1e-4. One gfx950 FP8 MFMA instruction aligns the products
of its K group to the largest product's exponent E and drops bits below
2^(E-13) (tests/test_parity_gpu.py::test_fp8_mfma_alignment_window pins
this), so its sums are not FP32-exact; 1e-5 is out of reach for any FP8 MFMA
on this chip, while the per-element bound still holds.

BF16 output (at most one BF16 ulp after the epilogue cast): element (m, n)
passes if |out - RNE_bf16(y)| <= ulp_bf16(y); where cancellation makes y much
smaller than the terms it came from, an FP32 accumulator cannot be expected
to land in the right BF16 ulp, so the element also passes if
|out - y| <= ulp_bf16(y) + e_mn, with e_mn = 1e-4 * |alpha| * ||a_m|| ||b_n||
(x 1.13, the largest slope of GELU, when the activation is a GELU).
"""
from __future__ import annotations

import numpy as np

ACT_GELU = (2, 3)


def ulp_bf16(y: np.ndarray) -> np.ndarray:
    a = np.abs(np.asarray(y, dtype=np.float64))
    _, e2 = np.frexp(a)
    lead = np.maximum(e2 - 1, -126)
    return np.ldexp(1.0, lead - 7)


def ulp_f32(y: np.ndarray) -> np.ndarray:
    a = np.abs(np.asarray(y, dtype=np.float64))
    _, e2 = np.frexp(a)
    lead = np.maximum(e2 - 1, -126)
    return np.ldexp(1.0, lead - 23)


def check_f32(out, y, row_norm, col_norm, alpha=1.0, what="", frob=1e-5):
    out = np.asarray(out, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    assert out.shape == y.shape, (out.shape, y.shape)
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    err = np.abs(out - y)
    bound = 1e-4 * abs(alpha) * np.outer(row_norm, col_norm) + ulp_f32(y)
    bad = err > bound
    denom = np.linalg.norm(y)
    rel = np.linalg.norm(out - y) / denom if denom > 0 else np.linalg.norm(out - y)
    info = dict(rel_frob=float(rel), max_abs=float(err.max(initial=0.0)),
                n_bad=int(bad.sum()), worst_ratio=float((err / bound).max(initial=0.0)))
    assert rel <= frob, f"{what}: relative Frobenius error {rel:.3e} > {frob:g} ({info})"
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {info['n_bad']} elements above bound, first {tuple(i)}: "
                             f"out={out[tuple(i)]!r} ref={y[tuple(i)]!r} bound={bound[tuple(i)]!r}")
    return info


def check_bf16(out_vals, y, ref_vals, row_norm, col_norm, alpha=1.0, act=0, what=""):
    """out_vals: decoded GPU BF16 values; ref_vals: decoded RNE_bf16(y) from the oracle."""
    out = np.asarray(out_vals, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref_vals, dtype=np.float64)
    assert out.shape == y.shape == ref.shape
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    u = ulp_bf16(y)
    strict = np.abs(out - ref) <= u
    e_mn = 1e-4 * abs(alpha) * np.outer(row_norm, col_norm)
    if act in ACT_GELU:
        e_mn = e_mn * 1.13
    loose = np.abs(out - y) <= u + e_mn
    ok = strict | loose
    info = dict(n=int(out.size), exact=int((out == ref).sum()), one_ulp=int((strict & (out != ref)).sum()),
                cancellation=int((~strict & loose).sum()), n_bad=int((~ok).sum()))
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{what}: {info['n_bad']} elements beyond 1 bf16 ulp, first {i}: "
                             f"out={out[i]!r} ref={ref[i]!r} y={y[i]!r} ulp={u[i]!r} ({info})")
    return info
