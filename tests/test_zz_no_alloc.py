"""gemm_bf16_noalloc, the entry point that allocates nothing, against gemm_bf16.

Both calls run the same plan and kernels; gemm_bf16_noalloc only takes its
split-K partials from the library's per-GPU scratch array instead of a caller
workspace. So its output must equal gemm_bf16's bit for bit (and both pass the
oracle's tolerance). Two calls in a row, the second smaller than the first,
show that the scratch array's contents from one call do not leak into the
next; a shape whose workspace exceeds the array is refused before anything is
launched. Under HIP graph capture (the callers the entry point is for) every
replay recomputes the partials before reading them, also when other calls
have used the scratch array in between, and the very first call of a process
may be the captured one.
"""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np
import pytest

import dense_gemm_09_amd as g
import synth
from synth import ACT_GELU_ERF, OUT_BF16, OUT_F32
from tests.common import compare
from tests.gpu_util import to_device

pytestmark = pytest.mark.gpu


def _both(p):
    import torch
    pl = g.plan(p.M, p.N, p.K, False)
    print(f"[gpu] noalloc vs gemm_bf16 M={p.M} N={p.N} K={p.K} split={pl.split_k} "
          f"workspace={pl.workspace_bytes}", flush=True)
    d = to_device(p)
    c_ref = d["C"].clone()
    ws = torch.empty(max(1, pl.workspace_bytes), dtype=torch.uint8, device="cuda")
    g.gemm_bf16(p.M, p.N, p.K, p.alpha, d["A"], p.lda, p.layout_a, d["B"], p.ldb, p.layout_b,
                p.beta, c_ref, p.ldc, p.c_dtype, d["bias"], p.act, workspace=ws)
    g.gemm_bf16_noalloc(p.M, p.N, p.K, p.alpha, d["A"], p.lda, p.layout_a, d["B"], p.ldb,
                        p.layout_b, p.beta, d["C"], p.ldc, p.c_dtype, d["bias"], p.act)
    torch.cuda.synchronize()
    assert torch.equal(d["C"], c_ref), "gemm_bf16_noalloc differs from gemm_bf16"
    out = d["C"].cpu().numpy()
    return out.view(np.uint16) if p.c_dtype == OUT_BF16 else out


def test_noalloc_two_calls_second_smaller():
    big = synth.make_problem("bf16", 64, 4096, 4096, seed_base=0xD00000, beta=0.5, bias_std=0.1,
                             act=ACT_GELU_ERF, c_dtype=OUT_BF16, a_std=1.0, b_std=0.02)
    small = synth.make_problem("bf16", 40, 1024, 2048, seed_base=0xD01000, beta=0.5,
                               bias_std=0.1, c_dtype=OUT_F32, a_std=1.0, b_std=0.02)
    assert g.plan(64, 4096, 4096, False).split_k > 1 and g.plan(40, 1024, 2048, False).split_k > 1
    for p in (big, small):
        out = _both(p)
        compare(p, out[:, :p.N])


def test_noalloc_largest_workspace_and_unsplit():
    # exactly the scratch size (32 MiB of partials), then a plan with no split
    p = synth.make_problem("bf16", 512, 4096, 14336, seed_base=0xD02000, c_dtype=OUT_BF16,
                           bias_std=0.1, a_std=1.0, b_std=0.02)
    assert g.plan(512, 4096, 14336, False).workspace_bytes == 32 << 20
    _both(p)
    q = synth.make_problem("bf16", 300, 260, 192, seed_base=0xD03000, beta=0.5, c_dtype=OUT_F32)
    assert g.plan(300, 260, 192, False).workspace_bytes == 0
    compare(q, _both(q)[:, :q.N])


def test_noalloc_refuses_workspace_beyond_scratch():
    import torch
    M, N, K = 1024, 4096, 14336
    assert g.plan(M, N, K, False).workspace_bytes > 32 << 20
    A = torch.zeros((M, K), dtype=torch.int16, device="cuda")
    B = torch.zeros((N, K), dtype=torch.int16, device="cuda")
    C = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(g.GemmError) as e:
        g.gemm_bf16_noalloc(M, N, K, 1.0, A, K, synth.ROW, B, K, synth.COL, 0.0, C, N, OUT_F32)
    assert e.value.status == 6  # GEMM_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert bool((C == 7.0).all()), "a refused call must not touch C"


def test_noalloc_graph_replays_with_other_calls_between():
    import torch
    M, N, K = 64, 4096, 4096
    p = synth.make_problem("bf16", M, N, K, seed_base=0xD04000, beta=0.5, bias_std=0.1,
                           act=ACT_GELU_ERF, c_dtype=OUT_BF16, a_std=1.0, b_std=0.02)
    q = synth.make_problem("bf16", 40, 1024, 2048, seed_base=0xD05000, c_dtype=OUT_F32,
                           a_std=1.0, b_std=0.02)
    assert g.plan(M, N, K, False).split_k > 1 and g.plan(40, 1024, 2048, False).split_k > 1
    print(f"[gpu] noalloc graph capture M={M} N={N} K={K}", flush=True)
    d, e = to_device(p), to_device(q)
    c0 = d["C"].clone()
    ref = d["C"].clone()
    ws = torch.empty(g.workspace_size(M, N, K, False), dtype=torch.uint8, device="cuda")
    g.gemm_bf16(M, N, K, p.alpha, d["A"], p.lda, p.layout_a, d["B"], p.ldb, p.layout_b, p.beta,
                ref, p.ldc, p.c_dtype, d["bias"], p.act, workspace=ws)
    torch.cuda.synchronize()
    compare(p, ref.cpu().numpy().view(np.uint16))
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        g.gemm_bf16_noalloc(M, N, K, p.alpha, d["A"], p.lda, p.layout_a, d["B"], p.ldb,
                            p.layout_b, p.beta, d["C"], p.ldc, p.c_dtype, d["bias"], p.act,
                            stream=s)
    for _ in range(3):
        # an eager call of another split-K shape overwrites the scratch array
        g.gemm_bf16_noalloc(q.M, q.N, q.K, q.alpha, e["A"], q.lda, q.layout_a, e["B"], q.ldb,
                            q.layout_b, q.beta, e["C"], q.ldc, q.c_dtype, None, q.act)
        d["C"].copy_(c0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(d["C"], ref)


def test_noalloc_first_call_of_a_process_under_capture():
    child = os.path.join(os.path.dirname(os.path.abspath(__file__)), "noalloc_capture_child.py")
    r = subprocess.run([sys.executable, "-u", child], capture_output=True, text=True, timeout=600)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count("equal True") == 3
