"""Pins of the float64 oracle against facts that do not come from the oracle itself.

* codec tables: every BF16 and E4M3 code against the format definitions'
  named values and against torch's own decoders (a library cross-check);
* round-to-nearest-even ties, single rounding from float64, overflow and
  subnormals, worked out by hand;
* exact answers: integer-valued operands (checked against integer matmul of
  the drawn integers), tiny operands with hand-chosen dyadic values (checked
  against rational arithmetic), identity and permutation matrices, closed
  forms for the scales and the bias, alpha/beta linearity;
* the epilogue's order in closed form: alpha scales the product only (not
  beta*C_in, not the bias), and the activation sees beta*C_in and the bias
  (first DeepGEMM page, sec. 1.1 and 6.1);
* the accumulation order: ascending k in float64, shown by a sum whose float64
  value depends on the order;
* GELU against tabulated values of the standard normal CDF;
* a planted-mistake check: oracles with a dropped term, a transposed
  operand, a wrong sign, a misplaced alpha or an activation applied too early
  fail the parity tolerance.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import ACT_GELU_ERF, ACT_GELU_TANH, ACT_NONE, ACT_RELU, COL, OUT_BF16, OUT_F32, ROW
from tests import tolerance
from tests.common import compare, operand_norms, reference


# ---------------------------------------------------------------- codecs

def test_bf16_decode_named_values():
    d = lambda c: float(oracle.decode_bf16(np.uint16(c)))
    assert d(0x3F80) == 1.0
    assert d(0xC000) == -2.0
    assert d(0x3F00) == 0.5
    assert d(0x4049) == 3.140625
    assert d(0x7F7F) == (2 - 2 ** -7) * 2.0 ** 127
    assert d(0x0080) == 2.0 ** -126
    assert d(0x0001) == 2.0 ** -133
    assert d(0x007F) == 127 * 2.0 ** -133
    assert d(0x7F80) == np.inf and d(0xFF80) == -np.inf
    assert np.isnan(d(0x7FC0)) and np.isnan(d(0x7F81))
    z = oracle.decode_bf16(np.uint16(0x8000))
    assert z == 0.0 and np.signbit(z)


def test_bf16_decode_all_codes_match_torch():
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    mine = oracle.decode_bf16(codes)
    theirs = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(theirs)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], theirs[~nan])
    assert np.array_equal(np.signbit(mine[~nan]), np.signbit(theirs[~nan]))


def test_e4m3_decode_named_values():
    d = lambda c: float(oracle.decode_e4m3(np.uint8(c)))
    assert d(0x38) == 1.0 and d(0xB8) == -1.0
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert d(0x08) == 2.0 ** -6
    assert d(0x01) == 2.0 ** -9
    assert d(0x07) == 7 * 2.0 ** -9
    assert d(0x40) == 2.0 and d(0x44) == 3.0 and d(0x3C) == 1.5
    assert d(0x77) == 240.0
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    vals = oracle.decode_e4m3(np.arange(256, dtype=np.uint8))
    assert int(np.isnan(vals).sum()) == 2
    assert np.nanmax(vals) == 448.0
    # positive finite codes are strictly increasing in their bit pattern
    pos = vals[:127]
    assert np.all(np.diff(pos) > 0)


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.decode_e4m3(codes)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(theirs)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], theirs[~nan])


def test_round_bf16_ties_and_single_rounding():
    r = lambda x: float(oracle.round_to_bf16(np.float64(x)))
    assert r(1 + 2 ** -8) == 1.0                       # tie -> even (fraction 0)
    assert r(1 + 3 * 2 ** -8) == 1 + 2 ** -6           # tie -> even (fraction 2)
    assert r(1 + 2 ** -8 + 2 ** -30) == 1 + 2 ** -7    # just above the tie: rounds up
    # a detour through float32 would first drop 2**-30 and then round the tie down:
    assert float(np.float32(1 + 2 ** -8 + 2 ** -30)) == 1 + 2 ** -8
    assert r(-(1 + 2 ** -8 + 2 ** -30)) == -(1 + 2 ** -7)
    assert r(2.0 ** -134) == 0.0                       # half the smallest subnormal -> even (0)
    assert r(3 * 2.0 ** -134) == 2.0 ** -132           # 1.5 quanta -> 2 quanta
    big = (2 - 2 ** -7) * 2.0 ** 127
    assert r(big) == big
    assert r((2 - 2 ** -8) * 2.0 ** 127) == np.inf     # tie at the overflow threshold
    assert r(3.39e38) == big
    assert np.isnan(r(np.nan))
    assert oracle.round_to_bf16_bits(np.float64(1.0)) == 0x3F80
    assert oracle.round_to_bf16_bits(np.float64(-448.0)) == 0xC3E0


def test_round_bf16_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(200000) * 10.0 ** rng.integers(-30, 30, 200000),
                        rng.standard_normal(1000) * 1e-39]).astype(np.float32)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    mine = oracle.round_to_bf16_bits(x.astype(np.float64))
    assert np.array_equal(mine, theirs)


def test_round_f32_ties():
    assert float(oracle.round_to_f32(1 + 2 ** -24)) == 1.0
    assert float(oracle.round_to_f32(1 + 3 * 2 ** -24)) == 1 + 2 ** -22
    assert float(oracle.round_to_f32(1 + 2 ** -24 + 2 ** -40)) == 1 + 2 ** -23


# ---------------------------------------------------------------- exact GEMMs

SHAPES = [(1, 1, 1), (3, 5, 7), (17, 9, 33), (64, 48, 40), (37, 130, 71)]


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("la,lb", [(ROW, ROW), (ROW, COL), (COL, ROW), (COL, COL)])
def test_integer_operands_exact(kind, M, N, K, la, lb):
    lo, hi = (-4, 4) if kind == "bf16" else (-16, 16)
    base = 0x1234000 + M * 7 + N * 3 + K
    p = synth.make_problem(kind, M, N, K, seed_base=base, layout_a=la, layout_b=lb,
                           int_range=(lo, hi), c_dtype=OUT_F32)
    a = synth.small_ints((M, K), lo, hi, base + 0).astype(np.int64)
    b = synth.small_ints((K, N), lo, hi, base + 1).astype(np.int64)
    exact = a @ b
    _, out = reference(p)
    assert out.dtype == np.float32
    assert np.array_equal(out, exact.astype(np.float32))


def test_fp8_integer_operands_exact_long_k():
    M, N, K = 8, 8, 2048
    base = 0x777000
    p = synth.make_problem("fp8", M, N, K, seed_base=base, int_range=(-16, 16))
    exact = (synth.small_ints((M, K), -16, 16, base).astype(np.int64)
             @ synth.small_ints((K, N), -16, 16, base + 1).astype(np.int64))
    _, out = reference(p)
    assert np.array_equal(out, exact.astype(np.float32))


def _dyadic(rng, shape):
    """Values i * 2**e with |i| < 256, e in [-4, 4]: exact in BF16."""
    i = rng.integers(-255, 256, size=shape)
    e = rng.integers(-4, 5, size=shape)
    return [[Fraction(int(i[r, c])) * Fraction(2) ** int(e[r, c]) for c in range(shape[1])]
            for r in range(shape[0])]


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (2, 3, 4), (5, 4, 3), (4, 4, 8), (8, 7, 6)])
def test_tiny_bruteforce_rational(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    a = _dyadic(rng, (M, K))
    b = _dyadic(rng, (K, N))
    A = synth.to_bf16_bits(np.array([[float(v) for v in row] for row in a]))
    B = synth.to_bf16_bits(np.array([[float(v) for v in row] for row in b]))
    C = np.zeros((M, N), np.float32)
    _, out = oracle.gemm_bf16(M, N, K, 1.0, A, ROW, B, ROW, 0.0, C, OUT_F32, None, ACT_NONE)
    for m in range(M):
        for n in range(N):
            s = sum(a[m][k] * b[k][n] for k in range(K))
            assert out[m, n] == np.float32(float(s)), (m, n)


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
@pytest.mark.parametrize("lb", [ROW, COL])
def test_identity_and_permutation(kind, lb):
    M, K = 23, 19
    base = 0x4242000
    p = synth.make_problem(kind, M, K, K, seed_base=base, layout_b=lb, int_range=(-9, 9))
    one = 0x3F80 if kind == "bf16" else 0x38
    dt = np.uint16 if kind == "bf16" else np.uint8
    dec = oracle.decode_bf16 if kind == "bf16" else oracle.decode_e4m3
    a_vals = dec(p.A[:M, :K])
    for perm in (np.arange(K), np.random.default_rng(3).permutation(K)):
        eye = np.zeros((K, K), dt)
        eye[perm, np.arange(K)] = one  # b(k, n) = 1 iff k = perm[n]
        B = synth.store_b(eye, lb, K, 0)
        if kind == "bf16":
            _, out = oracle.gemm_bf16(M, K, K, 1.0, p.A, ROW, B, lb, 0.0, p.C, OUT_F32, None, 0)
        else:
            ones = np.ones(K, np.float32)
            _, out = oracle.gemm_fp8_scaled(M, K, K, 1.0, p.A, ROW, B, lb, np.ones(M, np.float32),
                                            ones, 0.0, p.C, OUT_F32, None, 0)
        assert np.array_equal(out, a_vals[:, perm].astype(np.float32))


def test_layouts_agree():
    M, N, K = 29, 31, 37
    base = 0x5151000
    outs = []
    for la in (ROW, COL):
        for lb in (ROW, COL):
            p = synth.make_problem("bf16", M, N, K, seed_base=base, layout_a=la, layout_b=lb,
                                   lda=(K + 5 if la == ROW else M + 3),
                                   ldb=(N + 2 if lb == ROW else K + 1))
            outs.append(reference(p)[1])
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_alpha_linearity_and_beta_cancellation():
    M, N, K = 40, 24, 56
    base = 0x6161000
    p = synth.make_problem("bf16", M, N, K, seed_base=base, int_range=(-4, 4))
    _, out1 = reference(p)
    p.alpha = 2.0
    _, out2 = reference(p)
    assert np.array_equal(out2, 2 * out1)
    p.alpha = -0.25
    _, out3 = reference(p)
    assert np.array_equal(out3, -0.25 * out1)
    # beta * C_in with C_in = -A B (exact integers) cancels to zero
    p.alpha, p.beta = 1.0, 1.0
    p.C = -out1.copy()
    _, out4 = reference(p)
    assert np.array_equal(out4, np.zeros_like(out4))
    # beta = 3, C_in = A B  ->  4 A B
    p.beta = 3.0
    p.C = out1.copy()
    _, out5 = reference(p)
    assert np.array_equal(out5, 4 * out1)


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_alpha_scales_product_only(kind):
    """alpha = 2, beta = 3, C_in = A B, integer bias b: out = 2 AB + 3 AB + b = 5 AB + b
    exactly. A reading where alpha also scaled beta*C_in (8 AB + b) or the bias
    (5 AB + 2b) gives another integer."""
    M, N, K = 12, 10, 24
    base = 0x6262000
    lo, hi = (-4, 4) if kind == "bf16" else (-16, 16)
    p = synth.make_problem(kind, M, N, K, seed_base=base, int_range=(lo, hi), c_dtype=OUT_F32)
    ab = (synth.small_ints((M, K), lo, hi, base).astype(np.int64)
          @ synth.small_ints((K, N), lo, hi, base + 1).astype(np.int64))
    bias_vals = np.arange(N, dtype=np.float64) * 3 - 13   # nonzero integers, exact in BF16
    p.bias = synth.to_bf16_bits(bias_vals)
    p.alpha, p.beta = 2.0, 3.0
    p.C = ab.astype(np.float32)
    _, out = reference(p)
    assert np.array_equal(out, (5 * ab + bias_vals[None, :]).astype(np.float32))


@pytest.mark.parametrize("act", [ACT_RELU, ACT_GELU_ERF])
def test_activation_sees_beta_c_and_bias(act):
    """A = 1, so A B has equal rows s_n = sum_k B[k, n] (integers). With
    beta*C_in = -s_n - 1 and bias +0.5 every z is exactly -0.5: ReLU gives 0 and
    GELU gives -0.5 Phi(-0.5) (normal-CDF table). Applying the activation before
    adding beta*C_in or the bias would give act(s_n) - s_n - 1 (+0.5) instead."""
    M, N, K = 6, 9, 16
    base = 0x6363000
    b = synth.small_ints((K, N), -4, 4, base + 1).astype(np.int64)
    s_n = b.sum(axis=0)
    A = synth.to_bf16_bits(np.ones((M, K)))
    B = synth.to_bf16_bits(b.astype(np.float64))
    C = np.tile((-s_n - 1).astype(np.float32), (M, 1))
    bias = synth.to_bf16_bits(np.full(N, 0.5))
    y, out = oracle.gemm_bf16(M, N, K, 1.0, A, ROW, B, ROW, 1.0, C, OUT_F32, bias, act)
    expect = 0.0 if act == ACT_RELU else -0.5 * (1.0 - PHI[0.5])
    assert np.all(np.abs(y - expect) <= 1e-15), (y, expect)
    assert np.any(s_n != -1)  # the mutant readings differ somewhere


def test_accumulation_is_ascending_k_in_float64():
    """Products 2^53, 1, -2^53 in this k order: (2^53 + 1) rounds to 2^53 in
    float64 (tie to even), so the ascending-k float64 sum is 0; in the reverse
    order it is (-2^53 + 1) + 2^53 = 1. Both are exact FP32 outputs."""
    A = synth.to_bf16_bits(np.array([[2.0 ** 26, 1.0, -(2.0 ** 26)]]))
    B = synth.to_bf16_bits(np.array([[2.0 ** 27], [1.0], [2.0 ** 27]]))
    C = np.zeros((1, 1), np.float32)
    _, out = oracle.gemm_bf16(1, 1, 3, 1.0, A, ROW, B, ROW, 0.0, C, OUT_F32, None, ACT_NONE)
    assert out[0, 0] == 0.0
    _, out = oracle.gemm_bf16(1, 1, 3, 1.0, A[:, ::-1].copy(), ROW, B[::-1].copy(), ROW, 0.0, C,
                              OUT_F32, None, ACT_NONE)
    assert out[0, 0] == 1.0


def test_beta_zero_does_not_read_c():
    p = synth.make_problem("bf16", 8, 8, 8, seed_base=0x7171000)
    p.C[:] = np.nan
    _, out = reference(p)
    assert np.all(np.isfinite(out))


def test_fp8_scale_closed_form():
    M, N, K = 6, 5, 64
    A = np.full((M, K), 0x38, np.uint8)      # every a = 1
    B = np.full((N, K), 0x40, np.uint8)      # every b = 2 (col-major)
    sa = np.array([2.0 ** m for m in range(M)], np.float32)
    sb = np.array([n + 1 for n in range(N)], np.float32)
    C = np.zeros((M, N), np.float32)
    _, out = oracle.gemm_fp8_scaled(M, N, K, 1.0, A, ROW, B, COL, sa, sb, 0.0, C, OUT_F32, None, 0)
    expect = np.array([[2 * K * 2.0 ** m * (n + 1) for n in range(N)] for m in range(M)])
    assert np.array_equal(out, expect.astype(np.float32))


@pytest.mark.parametrize("act", [ACT_NONE, ACT_RELU])
def test_bias_closed_form(act):
    M, N, K = 4, 9, 16
    A = np.zeros((M, K), np.uint16)
    B = synth.to_bf16_bits(np.ones((K, N)))
    vals = np.array([-3.0, -1.5, -0.25, 0.0, 0.5, 1.0, 2.0, 7.0, -8.0])
    bias = synth.to_bf16_bits(vals)
    C = np.zeros((M, N), np.uint16)
    _, out = oracle.gemm_bf16(M, N, K, 1.0, A, ROW, B, ROW, 0.0, C, OUT_BF16, bias, act)
    expect = vals if act == ACT_NONE else np.maximum(vals, 0)
    assert np.array_equal(oracle.decode_bf16(out), np.tile(expect, (M, 1)))


# Standard normal CDF, textbook table values.
PHI = {0.5: 0.6914624612740131, 1.0: 0.8413447460685429, 2.0: 0.9772498680518208,
       3.0: 0.9986501019683699}


def test_gelu_erf_against_normal_cdf_table():
    for x, phi in PHI.items():
        for sx, ph in ((x, phi), (-x, 1.0 - phi)):
            got = float(oracle.activation(np.float64(sx), ACT_GELU_ERF))
            assert abs(got - sx * ph) <= 1e-15 * max(1.0, abs(sx)), (sx, got)
    assert float(oracle.activation(np.float64(0.0), ACT_GELU_ERF)) == 0.0


def _normal_tail(x: float) -> float:
    """1 - Phi(x) for large x from the asymptotic series of Mills' ratio,
    phi(x)/x * sum_n (-1)^n (2n-1)!! / x^(2n) (alternating: the error is below
    the first omitted term)."""
    total, term = 0.0, 1.0
    for n in range(1, 12):
        total += term
        term *= -(2 * n - 1) / (x * x)
    return math.exp(-0.5 * x * x) / math.sqrt(2 * math.pi) / x * total


@pytest.mark.parametrize("x", [9.0, 10.0, 12.0, 20.0])
def test_gelu_erf_far_negative_tail(x):
    """GELU(-x) = -x (1 - Phi(x)): relative accuracy where Phi is tiny (the
    series' truncation error at these x is below 1e-11 relative)."""
    got = float(oracle.activation(np.float64(-x), ACT_GELU_ERF))
    want = -x * _normal_tail(x)
    assert want < 0 and abs(got - want) <= 1e-10 * abs(want), (x, got, want)


def _gelu_tanh_decimal(z: float) -> float:
    """0.5 z (1 + tanh u), u = sqrt(2/pi) (z + 0.044715 z^3), in 300-digit decimal
    arithmetic with tanh u = (e^(2u) - 1) / (e^(2u) + 1): the definition itself,
    evaluated far beyond float64 precision."""
    from decimal import Decimal, getcontext
    getcontext().prec = 300
    zd = Decimal(z)
    pi = Decimal("3.14159265358979323846264338327950288419716939937510582097494459")
    u = (Decimal(2) / pi).sqrt() * (zd + Decimal("0.044715") * zd ** 3)
    e2u = (2 * u).exp()
    return float(Decimal("0.5") * zd * (1 + (e2u - 1) / (e2u + 1)))


@pytest.mark.parametrize("z", [-15.0, -12.0, -9.0, -5.0, -1.0, -0.25, 0.5, 3.0, 8.0])
def test_gelu_tanh_against_high_precision_definition(z):
    got = float(oracle.activation(np.float64(z), ACT_GELU_TANH))
    want = _gelu_tanh_decimal(z)
    # float64 rounding of u alone moves e^(2u) by ~|2u| * 2^-52 relative
    u = math.sqrt(2 / math.pi) * (z + 0.044715 * z ** 3)
    assert abs(got - want) <= (1e-15 + 8 * abs(2 * u) * 2.0 ** -53) * abs(want), (z, got, want)


def test_gelu_tanh_properties():
    x = np.linspace(-8, 8, 20001)
    g = oracle.activation(x, ACT_GELU_TANH)
    ge = oracle.activation(x, ACT_GELU_ERF)
    assert np.max(np.abs(g - ge)) < 5e-4            # the approximation's known accuracy
    assert np.allclose(g - oracle.activation(-x, ACT_GELU_TANH), x, atol=1e-14)
    assert abs(float(oracle.activation(np.float64(1.0), ACT_GELU_TANH)) - 0.8411920) < 1e-6


def test_sampled_rows_match_full():
    p = synth.make_problem("fp8", 50, 40, 64, seed_base=0x8181000, bias_std=0.1,
                           act=ACT_GELU_ERF, c_dtype=OUT_BF16)
    y, out = reference(p)
    rows, cols = [0, 7, 49], [3, 39]
    ys, outs = reference(p, rows, cols)
    assert np.array_equal(outs, out[np.ix_(rows, cols)])
    assert np.array_equal(ys, y[np.ix_(rows, cols)])


# ---------------------------------------------------------------- planted mistakes

def _mutant(p, how):
    """The oracle with a planted mistake (CPU only)."""
    q = synth.Problem(**{f: getattr(p, f) for f in p.__dataclass_fields__})
    if how in ("alpha_scales_bias", "alpha_scales_beta_c", "act_before_beta_c", "act_before_bias"):
        # the product alone (alpha 1, no C_in, no bias, no activation), then
        # the epilogue terms combined in a wrong order
        acc, _ = reference(synth.Problem(**{**q.__dict__, "alpha": 1.0, "beta": 0.0, "bias": None,
                                            "act": ACT_NONE}))
        bc = p.beta * p.C.astype(np.float64)
        b = oracle.decode_bf16(p.bias)[None, :]
        act = lambda z: oracle.activation(z, p.act)
        if how == "alpha_scales_bias":
            return act(p.alpha * (acc + b) + bc)
        if how == "alpha_scales_beta_c":
            return act(p.alpha * (acc + bc) + b)
        if how == "act_before_beta_c":
            return act(p.alpha * acc + b) + bc
        return act(p.alpha * acc + bc) + b
    if how == "drop_last_k":
        y, _ = reference(synth.Problem(**{**q.__dict__, "K": p.K - 1}))
    elif how == "transpose_b":
        B = oracle.logical_b(p.B, p.layout_b, p.K, p.N)
        q.B = np.ascontiguousarray(B.T)  # b(k, n) read as b(n, k)
        q.layout_b = ROW
        y, _ = reference(q)
    elif how == "beta_sign":
        q.beta = -p.beta
        y, _ = reference(q)
    elif how == "bias_off_by_one":
        q.bias = np.roll(p.bias, 1)
        y, _ = reference(q)
    return y


@pytest.mark.parametrize("how", ["drop_last_k", "transpose_b", "beta_sign", "bias_off_by_one",
                                 "alpha_scales_bias", "alpha_scales_beta_c", "act_before_beta_c",
                                 "act_before_bias"])
@pytest.mark.parametrize("act", [ACT_RELU, ACT_GELU_ERF])
def test_tolerance_rejects_planted_mistakes(how, act):
    n = 64
    p = synth.make_problem("bf16", n, n, n, seed_base=0x9191000, alpha=1.5, beta=0.5,
                           bias_std=0.5, act=act, layout_b=COL, c_dtype=OUT_F32)
    y_true, _, z = reference(p, with_z=True)
    y_bad = _mutant(p, how)
    rn, cn = operand_norms(p)
    with pytest.raises(AssertionError):
        tolerance.check_f32(y_bad.astype(np.float32), y_true, rn, cn, p.alpha, z=z, act=act)
    with pytest.raises(AssertionError):
        tolerance.check_bf16(oracle.decode_bf16(oracle.round_to_bf16_bits(y_bad)), y_true,
                             oracle.round_to_bf16(y_true), rn, cn, p.alpha, act, z=z)
    # and the true oracle's own outputs pass
    tolerance.check_f32(y_true.astype(np.float32), y_true, rn, cn, p.alpha, z=z, act=act)
    tolerance.check_bf16(oracle.round_to_bf16(y_true), y_true, oracle.round_to_bf16(y_true), rn,
                         cn, p.alpha, act, z=z)


def test_slope_bound_against_sampling():
    """slope_bound(z, e) is the largest |GELU'| on [z - e, z + e]: compare with a
    dense sample of each interval (and the tanh form's margin above it)."""
    rng = np.random.default_rng(11)
    z = rng.uniform(-12, 12, 400)
    e = rng.uniform(0, 3, 400)
    L = tolerance.slope_bound(z, e, ACT_GELU_ERF)
    for zi, ei, Li in zip(z, e, L):
        t = np.linspace(zi - ei, zi + ei, 2001)
        sampled = np.abs(tolerance.gelu_slope(t)).max()
        assert sampled <= Li + 1e-12 and Li <= sampled + 1e-3, (zi, ei, Li, sampled)
    assert np.all(tolerance.slope_bound(z, e, ACT_RELU) == (z + e > 0))
    # far into the negative range the slope, and so the allowance, is tiny
    assert tolerance.slope_bound(np.float64(-8.0), 0.01, ACT_GELU_ERF) < 1e-12


def test_tanh_gelu_slope_margin():
    """|d/dz tanh-GELU - d/dz erf-GELU| < TANH_SLOPE_MARGIN everywhere (the
    tanh form's slope bound is the erf form's plus that margin)."""
    z = np.linspace(-12, 12, 240001)
    h = 1e-5
    d_tanh = (oracle.activation(z + h, ACT_GELU_TANH) - oracle.activation(z - h, ACT_GELU_TANH)) / (2 * h)
    d_erf = tolerance.gelu_slope(z)
    assert np.max(np.abs(d_tanh - d_erf)) < tolerance.TANH_SLOPE_MARGIN


def test_bf16_tolerance_rejects_two_ulp_error():
    p = synth.make_problem("bf16", 32, 32, 32, seed_base=0xA1A1000, c_dtype=OUT_BF16)
    y, ref = reference(p)
    rn, cn = operand_norms(p)
    vals = oracle.decode_bf16(ref)
    tolerance.check_bf16(vals, y, vals, rn, cn)
    bad = vals.copy()
    bad[5, 7] = vals[5, 7] + 2 * tolerance.ulp_bf16(y[5, 7]) + 1e-3 * abs(vals[5, 7])
    with pytest.raises(AssertionError):
        tolerance.check_bf16(bad, y, vals, rn, cn)


def test_compare_accepts_oracle_output():
    p = synth.make_problem("fp8", 33, 65, 96, seed_base=0xB1B1000, c_dtype=OUT_BF16,
                           bias_std=0.1, act=ACT_GELU_ERF)
    _, out = reference(p)
    compare(p, out)
