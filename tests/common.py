"""Test helpers: run the oracle on a synth.Problem and compare results with it."""
from __future__ import annotations

import numpy as np

import oracle
from tests import tolerance


def reference(p, rows=None, cols=None, with_z=False):
    """(y, out) from the oracle for problem p, optionally on a row/column sample;
    (y, out, z) with with_z (z: the pre-activation values)."""
    if p.kind == "bf16":
        return oracle.gemm_bf16(p.M, p.N, p.K, p.alpha, p.A, p.layout_a, p.B, p.layout_b,
                                p.beta, p.C, p.c_dtype, p.bias, p.act, rows=rows, cols=cols,
                                with_z=with_z)
    if p.kind == "mxfp8":
        return oracle.gemm_mxfp8(p.M, p.N, p.K, p.alpha, p.A, p.B, p.mx_a, p.mx_b, p.beta, p.C,
                                 p.c_dtype, p.bias, p.act, rows=rows, cols=cols, with_z=with_z)
    return oracle.gemm_fp8_scaled(p.M, p.N, p.K, p.alpha, p.A, p.layout_a, p.B, p.layout_b,
                                  p.scale_a, p.scale_b, p.beta, p.C, p.c_dtype, p.bias, p.act,
                                  rows=rows, cols=cols, with_z=with_z)


def operand_norms(p, rows=None, cols=None):
    """||a_m||_2 per selected row and ||b_n||_2 per selected column (dequantised)."""
    dec = oracle.decode_bf16 if p.kind == "bf16" else oracle.decode_e4m3
    r = np.arange(p.M) if rows is None else np.asarray(rows)
    c = np.arange(p.N) if cols is None else np.asarray(cols)
    a = dec(oracle.logical_a(p.A, p.layout_a, p.M, p.K)[r, :])
    b = dec(oracle.logical_b(p.B, p.layout_b, p.K, p.N)[:, c])
    if p.kind == "mxfp8" and p.K > 0:
        kb = np.arange(p.K) // 32
        a = a * oracle.decode_e8m0(np.asarray(p.mx_a)[r][:, kb])
        b = b * oracle.decode_e8m0(np.asarray(p.mx_b)[c][:, kb]).T
    rn = np.sqrt((a * a).sum(axis=1))
    cn = np.sqrt((b * b).sum(axis=0))
    if p.kind == "fp8":
        rn = rn * np.asarray(p.scale_a, dtype=np.float64)[r]
        cn = cn * np.asarray(p.scale_b, dtype=np.float64)[c]
    return rn, cn


def compare(p, out, rows=None, cols=None, what=""):
    """Check a result (M'xN' array: float32, or uint16 BF16 codes) against the oracle."""
    y, ref, z = reference(p, rows, cols, with_z=True)
    rn, cn = operand_norms(p, rows, cols)
    what = what or p.name
    if p.c_dtype == 0:
        info = tolerance.check_f32(out, y, rn, cn, p.alpha, what,
                                   frob=1e-5 if p.kind == "bf16" else 1e-4, z=z, act=p.act)
    else:
        info = tolerance.check_bf16(oracle.decode_bf16(out), y, oracle.decode_bf16(ref), rn, cn,
                                    p.alpha, p.act, what, z=z)
    print(f"[parity] {what}: {info}", flush=True)
    return info
