"""Pins of the oracle's MX (block-scaled) FP8 GEMM (CPU only).

The E8M0 table is checked against its definition (2^(c-127), 255 = NaN).
The block-scaled GEMM is pinned against the FP8 GEMM with unit scales, which
is itself pinned (tests/test_oracle.py): with every scale 2^0 the two must
agree exactly, and with small integer data and small scale exponents every
scaled element a * 2^e is itself an E4M3 value, so the MX product must equal
the FP8 product of those values. That second check fails for a wrong block
index (k // 32), for scales applied to the wrong operand, row or column, or
with the wrong sign of the exponent. A uniform shift of the A scale codes
scales the result by an exact power of two.
"""
import numpy as np
import pytest

import oracle
from synth import ACT_NONE, OUT_F32, make_mx_problem


def test_e8m0_table():
    c = np.arange(256, dtype=np.uint8)
    v = oracle.decode_e8m0(c)
    assert np.isnan(v[255])
    assert np.array_equal(v[:255], np.array([2.0 ** (i - 127) for i in range(255)]))
    assert v[127] == 1.0 and v[0] == 2.0 ** -127 and v[254] == 2.0 ** 127


def fp8_on(p, a_codes, b_codes):
    """The FP8 oracle with unit per-token / per-channel scales on given codes."""
    return oracle.gemm_fp8_scaled(p.M, p.N, p.K, p.alpha, a_codes, 0, b_codes, 1,
                                  np.ones(p.M, np.float32), np.ones(p.N, np.float32), p.beta,
                                  p.C, p.c_dtype, p.bias, p.act)


def test_unit_scales_equal_the_fp8_gemm():
    p = make_mx_problem(37, 45, 200, seed_base=0x5EEDA000, int_data=(-16, 16),
                        scale_codes=(127, 127), bias_std=0.5, beta=0.5, act=2)
    y_mx, out_mx = oracle.gemm_mxfp8(p.M, p.N, p.K, p.alpha, p.A, p.B, p.mx_a, p.mx_b, p.beta,
                                     p.C, p.c_dtype, p.bias, p.act)
    y_fp8, out_fp8 = fp8_on(p, p.A, p.B)
    assert np.array_equal(y_mx, y_fp8)
    assert np.array_equal(out_mx, out_fp8)


@pytest.mark.parametrize("M,N,K", [(9, 11, 96), (16, 8, 130), (5, 33, 257)])
def test_block_scales_fold_into_the_data(M, N, K):
    # data in [-4, 4] and exponents in [-3, 3]: every a * 2^e is an E4M3 value
    p = make_mx_problem(M, N, K, seed_base=0x5EEDA100 + K, int_data=(-4, 4),
                        scale_codes=(124, 130), act=ACT_NONE, c_dtype=OUT_F32)
    kb = np.arange(K) // 32
    a_val = oracle.decode_e4m3(p.A[:, :K]) * oracle.decode_e8m0(p.mx_a[:, kb])
    b_val = oracle.decode_e4m3(p.B[:, :K]) * oracle.decode_e8m0(p.mx_b[:, kb])   # N x K
    a_codes = oracle.encode_e4m3(a_val.astype(np.float32))
    b_codes = oracle.encode_e4m3(b_val.astype(np.float32))
    assert np.array_equal(oracle.decode_e4m3(a_codes), a_val)   # folding is exact
    assert np.array_equal(oracle.decode_e4m3(b_codes), b_val)
    y_mx, _ = oracle.gemm_mxfp8(p.M, p.N, p.K, 1.0, p.A, p.B, p.mx_a, p.mx_b, 0.0, p.C,
                                p.c_dtype, None, ACT_NONE)
    y_fp8, _ = oracle.gemm_fp8_scaled(M, N, K, 1.0, a_codes, 0, b_codes, 1,
                                      np.ones(M, np.float32), np.ones(N, np.float32), 0.0, p.C,
                                      p.c_dtype, None, ACT_NONE)
    assert np.array_equal(y_mx, y_fp8)
    # and a wrong block index would not have matched: shifting the scale
    # columns by one block changes the result
    shifted = np.roll(p.mx_a[:, :(K + 31) // 32], 1, axis=1)
    mx_a2 = p.mx_a.copy()
    mx_a2[:, :shifted.shape[1]] = shifted
    y_bad, _ = oracle.gemm_mxfp8(p.M, p.N, p.K, 1.0, p.A, p.B, mx_a2, p.mx_b, 0.0, p.C,
                                 p.c_dtype, None, ACT_NONE)
    assert not np.array_equal(y_bad, y_fp8)


def test_uniform_scale_shift_is_a_power_of_two():
    p = make_mx_problem(20, 24, 160, seed_base=0x5EEDA200, a_std=1.0, b_std=0.5)
    y0, _ = oracle.gemm_mxfp8(p.M, p.N, p.K, 1.0, p.A, p.B, p.mx_a, p.mx_b, 0.0, p.C, p.c_dtype,
                              None, ACT_NONE)
    nb = (p.K + 31) // 32
    for d in (-3, 2):
        mx_a = p.mx_a.copy()
        mx_a[:, :nb] = (mx_a[:, :nb].astype(np.int64) + d).astype(np.uint8)
        y, _ = oracle.gemm_mxfp8(p.M, p.N, p.K, 1.0, p.A, p.B, mx_a, p.mx_b, 0.0, p.C,
                                 p.c_dtype, None, ACT_NONE)
        assert np.array_equal(y, y0 * 2.0 ** d)


def test_padding_scale_bytes_are_not_used():
    p = make_mx_problem(6, 7, 70, seed_base=0x5EEDA300)
    assert (p.mx_a[:, 3:] == 0xFF).all()       # ceil(70/32) = 3 blocks, rest NaN code
    y, _ = oracle.gemm_mxfp8(p.M, p.N, p.K, 1.0, p.A, p.B, p.mx_a, p.mx_b, 0.0, p.C, p.c_dtype,
                             None, ACT_NONE)
    assert np.all(np.isfinite(y))
