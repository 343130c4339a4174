"""C ABI checks that need no GPU: exports, status strings, plans, argument validation.

Every call here fails validation (or returns early) before anything touches
the HIP runtime, so nothing is launched.
"""
import ctypes
import os
import re

import pytest

import dense_gemm_09_amd as g
from dense_gemm_09_amd import ACT_GELU_TANH, COL, OUT_BF16, OUT_F32, ROW

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm355.h")

OK, NULLP, BAD_DIM, BAD_LD, BAD_ENUM, UNSUP, WS_SMALL, HIPERR = range(8)
FAKE = 0x7F0000000000  # a non-NULL address that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = g.lib()
    names = declared_functions()
    assert set(names) == set(g.EXPORTS)
    for n in names:
        assert hasattr(L, n), n
        assert ctypes.cast(getattr(L, n), ctypes.c_void_p).value


def test_status_strings():
    for code, name in enumerate(g.STATUS):
        assert g.status_string(code) == name
    assert g.status_string(99) == "GEMM_ERR_UNKNOWN"


def bf16(M=64, N=64, K=64, alpha=1.0, A=FAKE, lda=None, la=ROW, B=FAKE, ldb=None, lb=COL,
         beta=0.0, C=FAKE, ldc=None, cd=OUT_F32, bias=None, act=0, ws=None, wsb=0):
    lda = (K if la == ROW else M) if lda is None else lda
    ldb = (N if lb == ROW else K) if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return g.lib().gemm_bf16(M, N, K, alpha, A, lda, la, B, ldb, lb, beta, C, ldc, cd, bias, act,
                             ws, wsb, None)


def fp8(M=64, N=64, K=64, A=FAKE, lda=None, la=ROW, B=FAKE, ldb=None, lb=COL, sa=FAKE, sb=FAKE,
        C=FAKE, ldc=None, cd=OUT_BF16, ws=None, wsb=0):
    lda = (K if la == ROW else M) if lda is None else lda
    ldb = (N if lb == ROW else K) if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return g.lib().gemm_fp8_scaled(M, N, K, 1.0, A, lda, la, B, ldb, lb, sa, sb, 0.0, C, ldc, cd,
                                   None, 0, ws, wsb, None)


def test_bad_enums():
    assert bf16(la=2) == BAD_ENUM
    assert bf16(lb=-1) == BAD_ENUM
    assert bf16(cd=2) == BAD_ENUM
    assert bf16(act=4) == BAD_ENUM
    assert bf16(act=-1) == BAD_ENUM
    assert fp8(cd=7) == BAD_ENUM


def test_bad_dims():
    assert bf16(M=-1) == BAD_DIM
    assert bf16(N=-5) == BAD_DIM
    assert bf16(K=-1) == BAD_DIM
    assert bf16(M=(1 << 30) + 1) == BAD_DIM
    assert fp8(K=-2) == BAD_DIM


def test_bad_leading_dimensions():
    assert bf16(M=8, N=16, K=32, lda=31) == BAD_LD
    assert bf16(M=8, N=16, K=32, la=COL, lda=7) == BAD_LD
    assert bf16(M=8, N=16, K=32, lb=ROW, ldb=15) == BAD_LD
    assert bf16(M=8, N=16, K=32, lb=COL, ldb=31) == BAD_LD
    assert bf16(M=8, N=16, K=32, ldc=15) == BAD_LD
    assert bf16(M=8, N=16, K=0, lda=0) == BAD_LD  # ld must be >= 1 even when K == 0
    assert fp8(M=8, N=16, K=32, lda=16) == BAD_LD


def test_fp8_layouts_other_than_k_major_unsupported():
    assert fp8(la=COL) == UNSUP
    assert fp8(lb=ROW) == UNSUP


def test_null_pointers():
    assert bf16(C=None) == NULLP
    assert bf16(A=None) == NULLP
    assert bf16(B=None) == NULLP
    assert fp8(sa=None) == NULLP
    assert fp8(sb=None) == NULLP


def test_quick_returns_launch_nothing():
    # M == 0 or N == 0: OK without touching any pointer
    assert bf16(M=0, A=None, B=None, C=None) == OK
    assert bf16(N=0, A=None, B=None, C=None, ldc=1, ldb=64) == OK
    assert fp8(M=0, A=None, B=None, C=None, sa=None, sb=None) == OK


def test_workspace_checked_before_launch():
    M, N, K = 1, 1024, 8192
    need = g.workspace_size(M, N, K, False)
    info = g.plan(M, N, K, False)
    assert need == info.workspace_bytes
    if need > 0:
        assert bf16(M=M, N=N, K=K, ws=None, wsb=0) == NULLP
        assert bf16(M=M, N=N, K=K, ws=FAKE, wsb=need - 1) == WS_SMALL


def test_workspace_size_of_bad_sizes_is_zero():
    assert g.workspace_size(-1, 5, 5, False) == 0
    assert g.workspace_size(0, 5, 5, True) == 0


@pytest.mark.parametrize("fp8_", [False, True])
@pytest.mark.parametrize("M,N,K", [(4096, 4096, 4096), (4096, 7168, 2048), (512, 4096, 14336),
                                   (8192, 14336, 4096), (1, 4096, 4096), (64, 18432, 4096),
                                   (4093, 4093, 4093), (256, 256, 256), (1, 1, 1), (5, 7, 0),
                                   (64, 4096, 4096), (33, 11008, 4096), (17, 100, 333),
                                   (64, 65536, 4096)])
def test_plans_are_consistent(M, N, K, fp8_):
    p = g.plan(M, N, K, fp8_)
    assert p.split_k >= 1
    assert g.workspace_size(M, N, K, fp8_) == p.workspace_bytes
    if p.kernel == 1:  # skinny: M <= 16, 16 columns per workgroup, no split
        assert M <= 16 and p.tile_n == 16 and p.split_k == 1
        assert p.grid == -(-N // 16) and p.tile_m == 16 * -(-M // 16)
        return
    assert M > 16
    assert p.tile_k == (128 if fp8_ else 64)
    assert (p.tile_m, p.tile_n) in ((128, 128), (256, 128), (256, 256), (64, 256), (64, 128))
    tiles = -(-M // p.tile_m) * -(-N // p.tile_n)
    assert p.grid == tiles * p.split_k
    if M <= 64:  # a 64-row tile, split to fill the 256 CUs at most once
        assert p.tile_m == 64 and p.tile_n in (128, 256)
        assert p.split_k == 1 or p.grid <= 256
    assert p.workspace_bytes == (p.split_k * M * N * 4 if p.split_k > 1 else 0)
    if K == 0:
        assert p.split_k == 1
    # every K partition is non-empty
    if p.split_k > 1:
        per = -(-K // (p.split_k * p.tile_k)) * p.tile_k
        assert (p.split_k - 1) * per < K


def test_square_4096_uses_one_full_wave_of_256_tiles():
    p = g.plan(4096, 4096, 4096, False)
    assert (p.tile_m, p.tile_n, p.split_k, p.grid) == (256, 256, 1, 256)


# Plans chosen by the tile ranking, each measured on the GPU as the fastest (or
# within noise of it) among the forced alternatives of tile shape and split.
@pytest.mark.parametrize("M,N,K,fp8_,want", [
    (4096, 4096, 4096, True, (256, 256, 1)),
    (4096, 7168, 2048, True, (256, 256, 1)),
    (4093, 4093, 4093, False, (256, 256, 1)),
    (8192, 14336, 4096, False, (256, 256, 1)),
    (2048, 4096, 14336, False, (256, 256, 2)),
    (512, 12288, 4096, False, (128, 128, 1)),
    (512, 4096, 14336, False, (128, 128, 4)),
    (1024, 4096, 4096, True, (128, 128, 1)),
    (2048, 4096, 14336, True, (128, 128, 1)),
])
def test_measured_plans(M, N, K, fp8_, want):
    p = g.plan(M, N, K, fp8_)
    assert (p.tile_m, p.tile_n, p.split_k) == want


def test_plan_null_out():
    assert g.lib().gemm_plan(4, 4, 4, 0, None) == NULLP


def test_binding_rejects_short_tensors_before_calling():
    import torch
    A = torch.zeros(10, dtype=torch.int16)
    with pytest.raises(ValueError):
        g._need(A, 1000, "A")  # CPU tensor is rejected as well


def quant(M=64, K=64, X=FAKE, ldx=None, Q=FAKE, ldq=None, scale=FAKE):
    ldx = K if ldx is None else ldx
    ldq = K if ldq is None else ldq
    return g.lib().gemm_quantize_fp8_rows(M, K, X, ldx, Q, ldq, scale, None)


def test_quantizer_validation_before_launch():
    assert quant(M=-1) == BAD_DIM
    assert quant(K=-1) == BAD_DIM
    assert quant(M=1 << 31) == BAD_DIM
    assert quant(ldx=63) == BAD_LD
    assert quant(ldq=63) == BAD_LD
    assert quant(scale=None) == NULLP
    assert quant(X=None) == NULLP
    assert quant(Q=None) == NULLP
    # M == 0: nothing to do, no pointer is touched
    assert quant(M=0, X=None, Q=None, scale=None) == OK


def qgemm(fp8_=False, M=64, N=64, K=64, A=FAKE, la=ROW, B=FAKE, lb=COL, sa=FAKE, sb=FAKE,
          act=0, osc=FAKE, ozp=None, Q=FAKE, ldq=None, qd=g.QOUT_INT8, ws=None, wsb=0):
    lda = K if la == ROW else M
    ldb = N if lb == ROW else K
    ldq = N if ldq is None else ldq
    if fp8_:
        return g.lib().gemm_fp8_scaled_quant(M, N, K, 1.0, A, lda, la, B, ldb, lb, sa, sb, None,
                                             act, osc, ozp, Q, ldq, qd, ws, wsb, None)
    return g.lib().gemm_bf16_quant(M, N, K, 1.0, A, lda, la, B, ldb, lb, None, act, osc, ozp, Q,
                                   ldq, qd, ws, wsb, None)


@pytest.mark.parametrize("fp8_", [False, True])
def test_quantising_gemm_validation_before_launch(fp8_):
    assert qgemm(fp8_, qd=2) == BAD_ENUM
    assert qgemm(fp8_, qd=-1) == BAD_ENUM
    assert qgemm(fp8_, act=9) == BAD_ENUM
    assert qgemm(fp8_, qd=g.QOUT_E4M3, ozp=FAKE) == UNSUP
    assert qgemm(fp8_, osc=None) == NULLP
    assert qgemm(fp8_, Q=None) == NULLP
    assert qgemm(fp8_, ldq=63) == BAD_LD
    assert qgemm(fp8_, M=-1) == BAD_DIM
    if fp8_:
        assert qgemm(True, sa=None) == NULLP
        assert qgemm(True, lb=ROW) == UNSUP
    # a split-K plan needs its workspace
    ws = g.workspace_size(64, 4096, 4096, fp8_)
    if ws:
        assert qgemm(fp8_, M=64, N=4096, K=4096) == NULLP
        assert qgemm(fp8_, M=64, N=4096, K=4096, ws=FAKE, wsb=ws - 1) == WS_SMALL
    # M == 0 or N == 0: nothing is launched or read
    assert qgemm(fp8_, M=0, A=None, B=None, osc=None, Q=None) == OK
    assert qgemm(fp8_, N=0, ldq=1, A=None, B=None, osc=None, Q=None) == OK


def mx(M=64, N=64, K=256, A=FAKE, lda=None, la=ROW, B=FAKE, ldb=None, lb=COL, sa=FAKE, ldsa=8,
       sb=FAKE, ldsb=8, C=FAKE, ldc=None, cd=OUT_BF16, act=0, ws=None, wsb=0):
    lda = K if lda is None else lda
    ldb = K if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return g.lib().gemm_mxfp8(M, N, K, 1.0, A, lda, la, B, ldb, lb, sa, ldsa, sb, ldsb, 0.0, C,
                              ldc, cd, None, act, ws, wsb, None)


def test_mx_validation_before_launch():
    assert mx(cd=2) == BAD_ENUM
    assert mx(act=7) == BAD_ENUM
    assert mx(la=COL) == UNSUP
    assert mx(lb=ROW) == UNSUP
    assert mx(ldsa=7) == BAD_LD            # ceil(256/32) = 8 blocks
    assert mx(ldsb=6) == BAD_LD
    assert mx(ldsa=10) == BAD_LD           # not a multiple of 4
    assert mx(K=32, ldsa=2, ldsb=4) == BAD_LD   # at least 4 bytes per row
    assert mx(sa=None) == NULLP
    assert mx(sb=None) == NULLP
    assert mx(sa=FAKE + 2) == UNSUP        # scale rows must be 4-byte aligned
    assert mx(M=1 << 24, ldsa=1 << 8) == BAD_DIM   # scale offsets past 2^31
    assert mx(M=0, A=None, B=None, sa=None, sb=None) == OK
    ws = g.workspace_size(64, 4096, 2048, True)
    assert ws > 0
    assert mx(N=4096, K=2048, ldsa=64, ldsb=64) == NULLP
    assert mx(N=4096, K=2048, ldsa=64, ldsb=64, ws=FAKE, wsb=ws - 1) == WS_SMALL


def pack(K=64, N=48, B=FAKE, ldb=None, lb=ROW, es=2, Bp=FAKE, ldbp=None):
    ldb = (N if lb == ROW else K) if ldb is None else ldb
    ldbp = K if ldbp is None else ldbp
    return g.lib().gemm_pack_b(K, N, B, ldb, lb, es, Bp, ldbp, None)


def test_pack_validation_before_launch():
    assert pack(lb=2) == BAD_ENUM
    assert pack(es=4) == BAD_ENUM
    assert pack(K=-1) == BAD_DIM
    assert pack(N=1 << 31) == BAD_DIM
    assert pack(ldb=47) == BAD_LD            # ROW: ldb >= N
    assert pack(lb=COL, ldb=63) == BAD_LD    # COL: ldb >= K
    assert pack(ldbp=63) == BAD_LD
    assert pack(B=None) == NULLP
    assert pack(Bp=None) == NULLP
    assert pack(K=0, B=None, Bp=None, ldbp=1) == OK
