"""GPU parity of the per-token FP8 quantiser (gemm_quantize_fp8_rows) against
the oracle (oracle/quant.py). Codes and scales are integer/bitwise decisions:
the comparison is exact. Inputs are seeded BF16 rows shaped like the FP8
GEMM's A operand (token rows of activations)."""
import numpy as np
import pytest
import torch

import dense_gemm_09_amd as g
import oracle
import synth

pytestmark = pytest.mark.gpu


def run_quant(x_bits, K, ldq=None, q_fill=0xA5):
    M, ldx = x_bits.shape
    ldq = K if ldq is None else ldq
    X = torch.from_numpy(x_bits.view(np.int16).copy()).cuda()
    Q = torch.full((max(M, 1), max(ldq, 1)), q_fill, dtype=torch.uint8, device="cuda")
    S = torch.full((max(M, 1),), float("nan"), dtype=torch.float32, device="cuda")
    g.quantize_fp8_rows(M, K, X, ldx, Q, ldq, S)
    torch.cuda.synchronize()
    return Q.cpu().numpy()[:M], S.cpu().numpy()[:M]


def rows(M, K, std, seed, ld=None):
    ld = K if ld is None else ld
    x = np.full((M, ld), synth.BF16_NAN_BITS, np.uint16)
    x[:, :K] = synth.to_bf16_bits(synth.normal((M, K), std, seed))
    return x


def check(x_bits, K, ldq=None):
    q, s = run_quant(x_bits, K, ldq)
    q_ref, s_ref = oracle.quantize_rows_e4m3(x_bits, K)
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(q[:, :K], q_ref)
    if ldq is not None and ldq > K:
        assert np.all(q[:, K:] == 0xA5)  # padding untouched


@pytest.mark.parametrize("M,K", [(1, 1), (1, 8), (3, 7), (5, 1000), (300, 2048), (257, 4104),
                                 (64, 2048 + 8 * 3), (2, 20000)])
def test_random_rows(M, K):
    check(rows(M, K, 1.0, 0xC00000 + M + K), K)


def test_token_rows_of_the_fp8_projection():
    """The FP8 projection's A operand: 4096 tokens x K=2048, N(0,1) activations."""
    check(rows(4096, 2048, 1.0, 0xC10000), 2048)


def test_padded_leading_dimensions():
    x = rows(100, 520, 2.0, 0xC20000, ld=520 + 24)
    check(x, 520, ldq=520 + 40)


def test_every_bf16_value_at_scale_one():
    """Rows whose amax is 448 have scale exactly 1, so each code is the E4M3
    rounding of the BF16 value itself: this covers every BF16 value in
    [-448, 448], all E4M3 ties and the subnormal range."""
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = oracle.decode_bf16(codes)
    keep = np.isfinite(vals) & (np.abs(vals) <= 448)
    v = codes[keep]
    K = 1024
    v = np.concatenate([v, np.zeros((-len(v)) % (K - 1), np.uint16)])
    body = v.reshape(-1, K - 1)
    x = np.concatenate([np.full((body.shape[0], 1), 0x43E0, np.uint16), body], axis=1)  # 448
    q, s = run_quant(x, K)
    assert np.all(s == 1.0)
    q_ref, _ = oracle.quantize_rows_e4m3(x, K)
    assert np.array_equal(q, q_ref)


def test_zero_rows_and_wide_dynamic_range():
    rng = np.random.default_rng(5)
    x = np.zeros((6, 777), np.float64)
    x[1] = rng.standard_normal(777) * np.exp2(rng.uniform(-30, 10, 777))
    x[2, 100] = -3e-5
    x[3] = 1e-35 * rng.standard_normal(777)
    x[4] = rng.standard_normal(777) * 1e30
    bits = synth.to_bf16_bits(x)
    check(bits, 777)
    q, s = run_quant(bits, 777)
    assert s[0] == 1.0 and s[5] == 1.0 and not q[0].any()


def test_k_zero_writes_unit_scales():
    q, s = run_quant(np.zeros((7, 1), np.uint16), 0, ldq=1)
    assert np.all(s == 1.0)


def test_deterministic():
    x = rows(512, 2048, 1.0, 0xC30000)
    a = run_quant(x, 2048)
    b = run_quant(x, 2048)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


def test_quantised_rows_feed_the_fp8_gemm():
    """Quantise activations on the GPU, run the FP8 GEMM on the result, and
    compare with the oracle GEMM on the oracle's codes and scales."""
    from tests.common import compare
    from tests.gpu_util import run
    M, N, K = 256, 384, 512
    p = synth.make_problem("fp8", M, N, K, seed_base=0xC40000, c_dtype=synth.OUT_BF16,
                           bias_std=0.1, act=synth.ACT_GELU_ERF)
    x = rows(M, K, 1.0, 0xC50000)
    q, s = run_quant(x, K)
    q_ref, s_ref = oracle.quantize_rows_e4m3(x, K)
    assert np.array_equal(q, q_ref)
    p.A = q.copy()
    p.scale_a = s.copy()
    compare(p, run(p))
