"""K that is not a multiple of the 16-byte chunk, on the DMA-fed tile kernels.

K-major operands reach LDS by DMA also when K ends inside a 16-byte chunk
(8 BF16 / 16 E4M3 elements) and when rows are not 16-byte aligned (tight
leading dimension such as lda = K = 4093, or a base pointer a few bytes off;
BF16 at 2-byte, E4M3 at any byte alignment). The DMA copies only chunks that
lie wholly below the end of K; in the last K slice the kernel writes each
row's straddling chunk itself (its valid elements, then zeros). These tests
pin that path against the oracle:

* integer operands, so every summation order is exact and the FP32 output
  must equal the oracle bit for bit;
* padded leading dimensions whose padding holds NaN codes, so an element past
  K that reached the MFMA shows up as NaN; tight ones, where the elements
  past K of a row are the next row's (nonzero) values;
* K below one slice (the patched slice is the first), K a few elements past
  a slice, split-K (only the last split ends inside a chunk), the 256x256
  and 128x128 tiles (the last also with one register-loaded operand),
  N-contiguous B with a DMA-fed ragged A, unaligned base pointers, and MX.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import dense_gemm_09_amd as g
import synth
from synth import COL, OUT_BF16, OUT_F32, ROW, ACT_GELU_ERF, make_mx_problem
from tests.common import compare, reference
from tests.gpu_util import call, run, to_device

pytestmark = pytest.mark.gpu


def _exact(p, rows=None):
    _, ref = reference(p, rows=rows)
    out = run(p, rows=rows)
    bad = np.argwhere(~((out == ref) | (np.isnan(out) & np.isnan(ref))))
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"


BF16_CASES = [
    # M, N, K, lda, ldb            tile / what
    (300, 260, 5, 5, 5),           # 128x128, K inside the first chunk, tight
    (300, 260, 37, 37, 37),        # K inside the first slice, tight (odd row pitch)
    (300, 260, 37, 48, 56),        # ... padded (NaN after K)
    (512, 512, 203, 203, 203),     # 128x128, four slices, tight
    (512, 512, 203, 216, 208),     # ... padded
    (520, 600, 65, 65, 72),        # one element past a slice
    (3000, 3000, 203, 203, 203),   # 256x256
    (64, 4096, 2053, 2053, 2056),  # split-K: only the last split is ragged
    (130, 260, 4093, 4093, 4096),  # split-K 16
]


@pytest.mark.parametrize("M,N,K,lda,ldb", BF16_CASES)
def test_bf16_ragged_k_exact(M, N, K, lda, ldb):
    p = synth.make_problem("bf16", M, N, K, seed_base=0x710000 + M + K + lda, lda=lda, ldb=ldb,
                           int_range=(-4, 4), c_dtype=OUT_F32)
    rows = None if M * N <= 600 * 600 else np.unique(np.r_[0:8, M - 8:M, 1000:1016])
    _exact(p, rows)


FP8_CASES = [
    (300, 260, 5, 16, 32),         # K inside the first chunk, padded
    (300, 260, 5, 5, 5),           # ... tight: byte-aligned rows
    (300, 260, 77, 80, 96),        # K inside the first slice
    (300, 260, 77, 77, 77),
    (512, 512, 203, 208, 224),     # 128x128
    (512, 512, 203, 203, 203),
    (520, 600, 129, 144, 144),     # one element past a slice
    (3000, 3000, 203, 208, 208),   # 256x256
    (3000, 3000, 203, 203, 203),
    (64, 4096, 2053, 2064, 2064),  # split-K
    (64, 4096, 2053, 2053, 2053),
]


@pytest.mark.parametrize("M,N,K,lda,ldb", FP8_CASES)
def test_fp8_ragged_k_exact(M, N, K, lda, ldb):
    p = synth.make_problem("fp8", M, N, K, seed_base=0x720000 + M + K, lda=lda, ldb=ldb,
                           int_range=(-16, 16), c_dtype=OUT_F32)
    rows = None if M * N <= 600 * 600 else np.unique(np.r_[0:8, M - 8:M, 1000:1016])
    _exact(p, rows)


@pytest.mark.parametrize("la,lb,N", [(ROW, ROW, 264),   # N-contiguous B by DMA, ragged A
                                     (ROW, ROW, 261),   # B by registers (N % 8 != 0), A by DMA
                                     (COL, COL, 260)])  # A by registers, B by DMA
def test_bf16_ragged_k_layouts_exact(la, lb, N):
    M, K = 300, 203
    p = synth.make_problem("bf16", M, N, K, seed_base=0x730000 + la * 2 + lb + N, layout_a=la,
                           layout_b=lb, int_range=(-4, 4), c_dtype=OUT_F32)
    _exact(p)


@pytest.mark.parametrize("c_dtype", [OUT_F32, OUT_BF16])
def test_bf16_ragged_k_random_epilogue(c_dtype):
    """Normal data with beta, bias and GELU: the tolerance path, tight rows."""
    M, N, K = 700, 520, 333
    p = synth.make_problem("bf16", M, N, K, seed_base=0x740000 + c_dtype, beta=0.5,
                           bias_std=0.1, act=ACT_GELU_ERF, c_dtype=c_dtype, a_std=K ** -0.5)
    compare(p, run(p))


def _shifted(t, elems, torch):
    """A copy of device tensor t starting `elems` elements into a fresh buffer."""
    buf = torch.zeros(t.numel() + 16, dtype=t.dtype, device="cuda")
    buf[elems:elems + t.numel()] = t.reshape(-1)
    return buf, buf.data_ptr() + elems * t.element_size()


@pytest.mark.parametrize("kind,shift", [("bf16", 1), ("fp8", 1), ("fp8", 3), ("mxfp8", 5)])
def test_unaligned_base_ragged_k(kind, shift):
    """Base pointers `shift` elements past 16-byte alignment and odd row pitches."""
    import torch
    M, N, K = 150, 140, 203
    if kind == "mxfp8":
        p = make_mx_problem(M, N, K, seed_base=0x750000, int_data=(-4, 4),
                            scale_codes=(126, 129), name="mx_unaligned")
    else:
        p = synth.make_problem(kind, M, N, K, seed_base=0x750000 + shift,
                               int_range=(-4, 4) if kind == "bf16" else (-16, 16),
                               c_dtype=OUT_F32)
    d = to_device(p)
    keep_a, d["A"] = _shifted(d["A"], shift, torch)
    keep_b, d["B"] = _shifted(d["B"], shift + 2, torch)
    print(f"[gpu] unaligned ragged {kind} M={M} N={N} K={K} shift={shift}", flush=True)
    sys.stdout.flush()
    call(p, d)
    torch.cuda.synchronize()
    _, ref = reference(p)
    out = d["C"].cpu().numpy()[:, :N]
    assert np.array_equal(out, ref), f"{int((out != ref).sum())} mismatches"


@pytest.mark.parametrize("M,N,K,lda", [(300, 260, 100, 112), (300, 260, 100, 100),
                                       (256, 256, 4093, 4096), (256, 256, 4093, 4093)])
def test_mx_ragged_k_exact(M, N, K, lda):
    ldsa = max(4, -(-((K + 31) // 32) // 4) * 4)
    p = make_mx_problem(M, N, K, seed_base=0x760000 + K, lda=lda, ldb=lda, ldsa=ldsa, ldsb=ldsa,
                        int_data=(-4, 4), scale_codes=(126, 129), name=f"mx_ragged_{K}_{lda}")
    _exact(p)


def test_plans_cover_split_and_both_tiles():
    """The shapes above reach the tiles and the split they are meant to."""
    assert g.plan(64, 4096, 2053, False).split_k > 1
    assert g.plan(130, 260, 4093, False).split_k > 1
    assert g.plan(64, 4096, 2053, True).split_k > 1
    assert (g.plan(3000, 3000, 203, False).tile_m, g.plan(3000, 3000, 203, False).tile_n) == (256, 256)
    assert (g.plan(512, 512, 203, False).tile_m, g.plan(512, 512, 203, False).tile_n) == (128, 128)
    assert (g.plan(512, 512, 203, True).tile_m, g.plan(512, 512, 203, True).tile_n) == (128, 128)
