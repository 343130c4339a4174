"""Parity tolerances for comparing a GEMM result with the float64 oracle.

Let e_mn = 1e-4 * |alpha| * ||a_m||_2 * ||b_n||_2 (a_m row m of A, b_n column n
of B, dequantised for FP8): the bound on the FP32 accumulation error in the
pre-activation value z[m, n]. The GPU's z' = z + d with |d| <= e_mn, so after
the activation its value is off by at most e_mn * L(z), where L(z) is the
largest |act'| on [z - e_mn, z + e_mn] (`slope_bound`): 1 without activation,
0 or 1 for ReLU, and for GELU the largest |GELU'| on the interval (tiny far
into the negative range, where GELU's output is tiny too).

FP32 output:
  * relative Frobenius error ||out - y||_F / ||y||_F <= 1e-5, and
  * per element |out - y| <= e_mn * L(z) + ulp_f32(y) + ACT_REL[act] * |y|.
    ACT_REL is the relative accuracy the kernels' activation evaluation
    promises in FP32 (GELU 2^-19, measured on the GPU over a dense sweep of z by
    tests/test_act_gpu.py; exact for ReLU and none).

FP8 inputs with FP32 output: the same per-element bound, and relative
Frobenius error <= 1e-4. One gfx950 FP8 MFMA instruction aligns the products
of its K group to the largest product's exponent E and drops bits below
2^(E-13) (tests/test_parity_gpu.py::test_fp8_mfma_alignment_window pins
this), so its sums are not FP32-exact; 1e-5 is out of reach for any FP8 MFMA
on this chip, while the per-element bound still holds.

BF16 output (at most one BF16 ulp after the epilogue cast): element (m, n)
passes if |out - RNE_bf16(y)| <= ulp_bf16(y) ("strict"); where cancellation
makes y much smaller than the terms it came from, an FP32 accumulator cannot
be expected to land in the right BF16 ulp, so the element also passes if
|out - y| <= ulp_bf16(y) + e_mn * L(z) ("cancellation"). Elements that pass
only through the second test are counted in the returned info.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import ndtr

ACT_NONE, ACT_RELU, ACT_GELU_ERF, ACT_GELU_TANH = 0, 1, 2, 3
ACT_GELU = (ACT_GELU_ERF, ACT_GELU_TANH)
ACT_REL = {ACT_NONE: 0.0, ACT_RELU: 0.0, ACT_GELU_ERF: 2.0 ** -19, ACT_GELU_TANH: 2.0 ** -19}
# |d/dz tanh-GELU - d/dz erf-GELU| over all z stays below this (checked by
# tests/test_oracle.py::test_tanh_gelu_slope_margin).
TANH_SLOPE_MARGIN = 0.03
_SQRT2 = math.sqrt(2.0)


def gelu_slope(z):
    """d/dz z*Phi(z) = Phi(z) + z*phi(z)."""
    z = np.asarray(z, dtype=np.float64)
    return ndtr(z) + z * np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)


def slope_bound(z, e, act):
    """Largest |act'(t)| for t in [z - e, z + e] (elementwise)."""
    z = np.asarray(z, dtype=np.float64)
    e = np.broadcast_to(np.asarray(e, dtype=np.float64), z.shape)
    if act == ACT_NONE:
        return np.ones_like(z)
    if act == ACT_RELU:
        return np.where(z + e > 0, 1.0, 0.0)
    lo, hi = z - e, z + e
    # GELU' has its extrema at +-sqrt(2) (GELU''(t) = phi(t) (2 - t^2)) and is
    # monotone between them, so the maximum of |GELU'| on an interval is at an
    # endpoint or at one of those two points inside it.
    L = np.maximum(np.abs(gelu_slope(lo)), np.abs(gelu_slope(hi)))
    for c in (-_SQRT2, _SQRT2):
        inside = (lo <= c) & (c <= hi)
        L = np.where(inside, np.maximum(L, abs(float(gelu_slope(c)))), L)
    if act == ACT_GELU_TANH:
        L = L + TANH_SLOPE_MARGIN
    return L


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


def _slope(z, e_mn, act, shape):
    if act == ACT_NONE:
        return np.ones(shape)
    if z is None:
        raise ValueError("an activation needs the oracle's pre-activation values z")
    return slope_bound(z, e_mn, act)


def check_f32(out, y, row_norm, col_norm, alpha=1.0, what="", frob=1e-5, z=None, act=ACT_NONE):
    out = np.asarray(out, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    assert out.shape == y.shape, (out.shape, y.shape)
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    err = np.abs(out - y)
    e_mn = 1e-4 * abs(alpha) * np.outer(row_norm, col_norm)
    bound = e_mn * _slope(z, e_mn, act, y.shape) + ulp_f32(y) + ACT_REL[act] * np.abs(y)
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


def check_bf16(out_vals, y, ref_vals, row_norm, col_norm, alpha=1.0, act=ACT_NONE, what="",
               z=None):
    """out_vals: decoded GPU BF16 values; ref_vals: decoded RNE_bf16(y) from the oracle;
    z: the oracle's pre-activation values (needed when act is not ACT_NONE)."""
    out = np.asarray(out_vals, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref_vals, dtype=np.float64)
    assert out.shape == y.shape == ref.shape
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    u = ulp_bf16(y)
    strict = np.abs(out - ref) <= u
    e_mn = 1e-4 * abs(alpha) * np.outer(row_norm, col_norm)
    loose = np.abs(out - y) <= u + e_mn * _slope(z, e_mn, act, y.shape)
    ok = strict | loose
    info = dict(n=int(out.size), exact=int((out == ref).sum()), one_ulp=int((strict & (out != ref)).sum()),
                cancellation=int((~strict & loose).sum()), n_bad=int((~ok).sum()))
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{what}: {info['n_bad']} elements beyond 1 bf16 ulp, first {i}: "
                             f"out={out[i]!r} ref={ref[i]!r} y={y[i]!r} ulp={u[i]!r} ({info})")
    return info
