"""Operands past 2 GiB: the register-loader path at the DMA extent boundary.

The DMA loader addresses an operand with 32-bit byte offsets, so an operand
spanning 2 GiB or more is read by the register loader instead (the host
switches per operand). These tests build an A of just over 2 GiB on the GPU
(seeded torch generator, small integers, so every summation order is exact),
run the GEMM, and compare sampled rows (first, last, around the 2 GiB byte
offset, and random) with the oracle bit for bit.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_operand_spanning_more_than_2gib(kind):
    import torch
    import dense_gemm_09_amd as g
    K, N = 4096, 64
    es = 2 if kind == "bf16" else 1
    M = (1 << 31) // (es * K) + 3          # A spans just over 2 GiB
    print(f"[gpu] large A {kind} M={M} N={N} K={K} ({M * K * es / 2**30:.3f} GiB)", flush=True)
    sys.stdout.flush()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0x5EEDE000 + es)
    a_int = torch.randint(-4, 5, (M, K), device="cuda", generator=gen, dtype=torch.int8)
    b_int = torch.randint(-4, 5, (N, K), device="cuda", generator=gen, dtype=torch.int8)
    if kind == "bf16":
        A = a_int.to(torch.bfloat16).view(torch.int16)
        B = b_int.to(torch.bfloat16).view(torch.int16)
    else:
        A = a_int.to(torch.float8_e4m3fn).view(torch.uint8)
        B = b_int.to(torch.float8_e4m3fn).view(torch.uint8)
    del a_int, b_int
    C = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    if kind == "bf16":
        g.gemm_bf16(M, N, K, 1.0, A, K, 0, B, K, 1, 0.0, C, N, 0)
    else:
        ones_m = torch.ones(M, dtype=torch.float32, device="cuda")
        ones_n = torch.ones(N, dtype=torch.float32, device="cuda")
        g.gemm_fp8_scaled(M, N, K, 1.0, A, K, 0, B, K, 1, ones_m, ones_n, 0.0, C, N, 0)
    torch.cuda.synchronize()
    row_2g = (1 << 31) // (es * K)          # first row at or past the 2 GiB byte offset
    rng = np.random.default_rng(es)
    rows = np.unique(np.concatenate([[0, 1, row_2g - 1, row_2g, row_2g + 1, M - 2, M - 1],
                                     rng.integers(0, M, 25)]))
    idx = torch.from_numpy(rows).cuda()
    a_rows = A.index_select(0, idx).cpu().numpy()
    b_all = B.cpu().numpy()
    out = C.index_select(0, idx).cpu().numpy()
    if kind == "bf16":
        y, ref = oracle.gemm_bf16(len(rows), N, K, 1.0, a_rows.view(np.uint16), 0,
                                  b_all.view(np.uint16), 1, 0.0, None, 0, None, 0)
    else:
        y, ref = oracle.gemm_fp8_scaled(len(rows), N, K, 1.0, a_rows, 0, b_all, 1,
                                        np.ones(len(rows), np.float32), np.ones(N, np.float32),
                                        0.0, None, 0, None, 0)
    assert np.array_equal(out, ref), f"{int((out != ref).sum())} mismatches on sampled rows"
