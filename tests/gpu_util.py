"""Run a synth.Problem through the C ABI on the GPU (tests only)."""
from __future__ import annotations

import sys

import numpy as np


def _dev(arr, torch):
    if arr is None:
        return None
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def to_device(p):
    import torch
    return dict(A=_dev(p.A, torch), B=_dev(p.B, torch), C=_dev(p.C, torch),
                bias=_dev(p.bias, torch),
                scale_a=_dev(p.scale_a, torch), scale_b=_dev(p.scale_b, torch),
                mx_a=_dev(p.mx_a, torch), mx_b=_dev(p.mx_b, torch))


def call(p, d, workspace=None, stream=None):
    import dense_gemm_09_amd as g
    if p.kind == "bf16":
        g.gemm_bf16(p.M, p.N, p.K, p.alpha, d["A"], p.lda, p.layout_a, d["B"], p.ldb, p.layout_b,
                    p.beta, d["C"], p.ldc, p.c_dtype, d["bias"], p.act, workspace=workspace,
                    stream=stream)
    elif p.kind == "mxfp8":
        g.gemm_mxfp8(p.M, p.N, p.K, p.alpha, d["A"], p.lda, p.layout_a, d["B"], p.ldb, p.layout_b,
                     d["mx_a"], p.ldsa, d["mx_b"], p.ldsb, p.beta, d["C"], p.ldc, p.c_dtype,
                     d["bias"], p.act, workspace=workspace, stream=stream)
    else:
        g.gemm_fp8_scaled(p.M, p.N, p.K, p.alpha, d["A"], p.lda, p.layout_a, d["B"], p.ldb,
                          p.layout_b, d["scale_a"], d["scale_b"], p.beta, d["C"], p.ldc,
                          p.c_dtype, d["bias"], p.act, workspace=workspace, stream=stream)


def run(p, rows=None, cols=None, log=True):
    """Copy p to the GPU, run it, return the output (selected rows/cols) as numpy."""
    import torch
    if log:
        print(f"[gpu] {p.name or p.kind} M={p.M} N={p.N} K={p.K} lda={p.lda} ldb={p.ldb} "
              f"ldc={p.ldc} layouts=({p.layout_a},{p.layout_b})", flush=True)
        sys.stdout.flush()
    d = to_device(p)
    call(p, d)
    torch.cuda.synchronize()
    out = d["C"].cpu().numpy()
    if p.c_dtype == 1:
        out = out.view(np.uint16)
    out = out[:, :p.N]
    if rows is not None:
        out = out[np.asarray(rows)]
    if cols is not None:
        out = out[:, np.asarray(cols)]
    return out
