"""Child process of tests/test_zz_no_alloc.py: the first gemm_bf16_noalloc call
of a fresh process (so the scratch address is looked up inside the capture)
is made under HIP graph capture; every replay must equal gemm_bf16's eager
result. Prints one line per step; exits 0 only if all replays are equal."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

import dense_gemm_09_amd as g  # noqa: E402
import synth  # noqa: E402
from tests.gpu_util import to_device  # noqa: E402


def main():
    M, N, K = 64, 4096, 4096
    assert g.plan(M, N, K, False).split_k > 1
    p = synth.make_problem("bf16", M, N, K, seed_base=0xD10000, c_dtype=synth.OUT_F32,
                           a_std=1.0, b_std=0.02)
    d = to_device(p)
    ref = d["C"].clone()
    ws = torch.empty(g.workspace_size(M, N, K, False), dtype=torch.uint8, device="cuda")
    g.gemm_bf16(M, N, K, 1.0, d["A"], p.lda, p.layout_a, d["B"], p.ldb, p.layout_b, 0.0, ref,
                p.ldc, p.c_dtype, None, 0, workspace=ws)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        g.gemm_bf16_noalloc(M, N, K, 1.0, d["A"], p.lda, p.layout_a, d["B"], p.ldb, p.layout_b,
                            0.0, d["C"], p.ldc, p.c_dtype, None, 0, stream=s)
    print("[child] captured", flush=True)
    ok = True
    for i in range(3):
        d["C"].zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eq = bool(torch.equal(d["C"], ref))
        print(f"[child] replay {i} equal {eq}", flush=True)
        ok = ok and eq
    sys.exit(0 if ok else 1)


if __name__ == "__main__":
    main()
