"""Pre-laid-out weights (gemm_pack_b) and N-concatenated projections on the GPU.

The pack is a permutation of elements: its output must equal the oracle's
logical K x N view of B, transposed, bit for bit, and must not touch the
padding of each packed row. A GEMM on the packed weight (which takes the DMA
path) is checked against the oracle on the original operands. An
N-concatenated weight ([Wq | Wk | Wv], the fused projection of the FP8 page's
interface discussion) run as one launch must match the three separate
launches: bit for bit on integer-valued data, where every order of summation
is exact.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from synth import COL, OUT_BF16, OUT_F32, ROW, make_problem
from tests.common import compare

pytestmark = pytest.mark.gpu


def dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


@pytest.mark.parametrize("K,N,layout,es", [
    (200, 130, ROW, 2), (64, 64, ROW, 2), (1000, 77, ROW, 1), (129, 300, COL, 2), (96, 5, COL, 1),
])
def test_pack_is_the_k_major_view(K, N, layout, es):
    import torch
    import dense_gemm_09_amd as g
    print(f"[gpu] pack K={K} N={N} layout={layout} es={es}", flush=True)
    sys.stdout.flush()
    rng = np.random.default_rng(K + N)
    dt = np.uint16 if es == 2 else np.uint8
    ldb = (N + 3) if layout == ROW else (K + 5)
    B = rng.integers(0, 1 << (8 * es), size=(K if layout == ROW else N, ldb)).astype(dt)
    ldbp = (K + 15) // 16 * 16 + 16
    sentinel = 0x5A5A if es == 2 else 0x5A
    Bp = dev(np.full((N, ldbp), sentinel, dt))
    g.pack_b(K, N, dev(B), ldb, layout, es, Bp, ldbp)
    torch.cuda.synchronize()
    got = Bp.cpu().numpy().view(dt)
    want = oracle.logical_b(B, layout, K, N).T            # N x K
    assert np.array_equal(got[:, :K], want)
    assert (got[:, K:] == sentinel).all()


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_gemm_on_packed_weight(kind):
    import torch
    import dense_gemm_09_amd as g
    from tests.gpu_util import to_device, call
    M, N, K = 384, 520, 768
    lb = ROW if kind == "bf16" else COL
    ldb = None if kind == "bf16" else K + 3          # fp8: unaligned K-major rows
    p = make_problem(kind, M, N, K, seed_base=0x5EEDD000 + (kind == "fp8"), layout_b=lb, ldb=ldb,
                     c_dtype=OUT_BF16, bias_std=0.1, a_std=1.0, b_std=0.05, name=f"packed_{kind}")
    es = 2 if kind == "bf16" else 1
    ldbp = (K * es + 15) // 16 * 16 // es
    print(f"[gpu] gemm on packed B {kind} {M}x{N}x{K} layout_b={lb} ldb={p.ldb} -> ldbp={ldbp}",
          flush=True)
    d = to_device(p)
    Bp = torch.empty((N, ldbp), dtype=d["B"].dtype, device="cuda")
    g.pack_b(K, N, d["B"], p.ldb, lb, es, Bp, ldbp)
    d["B"] = Bp
    import copy
    q = copy.copy(p)
    q.layout_b, q.ldb = COL, ldbp
    call(q, d)
    torch.cuda.synchronize()
    out = d["C"].cpu().numpy().view(np.uint16)[:, :N]
    compare(p, out)   # against the oracle on the original operands


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_concatenated_projection_matches_separate_launches(kind):
    import torch
    import dense_gemm_09_amd as g
    from tests.gpu_util import to_device, call
    M, K, parts = 256, 1024, (512, 256, 384)
    N = sum(parts)
    p = make_problem(kind, M, N, K, seed_base=0x5EEDD100 + (kind == "fp8"), layout_b=COL,
                     c_dtype=OUT_F32, int_range=(-4, 4), name=f"qkv_{kind}")
    print(f"[gpu] fused projection {kind} M={M} N={parts} K={K}", flush=True)
    d = to_device(p)
    call(p, d)
    fused = d["C"].cpu().numpy()[:, :N].copy()
    n0 = 0
    for n in parts:
        C = torch.zeros((M, n), dtype=torch.float32, device="cuda")
        Bn = d["B"][n0:n0 + n]                         # rows n0.. of the K-major weight
        if kind == "bf16":
            g.gemm_bf16(M, n, K, 1.0, d["A"], p.lda, ROW, Bn, p.ldb, COL, 0.0, C, n, OUT_F32)
        else:
            g.gemm_fp8_scaled(M, n, K, 1.0, d["A"], p.lda, ROW, Bn, p.ldb, COL, d["scale_a"],
                              d["scale_b"][n0:n0 + n], 0.0, C, n, OUT_F32)
        torch.cuda.synchronize()
        assert np.array_equal(C.cpu().numpy(), fused[:, n0:n0 + n]), f"part at column {n0}"
        n0 += n
