"""Pins of the oracle's quantising epilogue (CPU only).

INT8: round-half-even ties and the saturation bounds are fixed by the
definition q = clip(round(x * s + zp), -128, 127); the zero point shifts codes
exactly; an unsaturated code dequantises to within half a step of x. E4M3: a
value that is exactly a code (times a power-of-two scale) gives that code, and
magnitudes past 448 saturate. torch's round (half to even) and float8_e4m3fn
cast are cross-checks of the two rounding steps on random values, never used
inside the oracle.
"""
import numpy as np
import pytest
import torch

from oracle import QOUT_E4M3, QOUT_INT8, decode_e4m3, quantize_output


def q8(y, s=1.0, zp=None):
    y = np.atleast_2d(np.asarray(y, dtype=np.float64))
    zp_arr = None if zp is None else np.full(y.shape[0], zp, np.int32)
    return quantize_output(y, np.full(y.shape[0], s, np.float32), zp_arr, QOUT_INT8)[0]


def test_int8_ties_go_to_even():
    y = [0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, -3.5, 126.5]
    assert q8(y).tolist() == [0, 2, 2, 4, 0, -2, -2, -4, 126]


def test_int8_nearest_off_ties():
    y = [0.49, 0.51, 1.49, -0.51, -1.49, 2.0]
    assert q8(y).tolist() == [0, 1, 1, -1, -1, 2]


def test_int8_saturates():
    y = [127.0, 127.4, 127.5, 1000.0, 3.0e38, -128.0, -128.4, -128.5, -1000.0, -3.0e38]
    assert q8(y).tolist() == [127, 127, 127, 127, 127, -128, -128, -128, -128, -128]


def test_int8_zero_point_and_scale():
    # 3 * 0.5 + 10 = 11.5 -> 12 (tie to even); 0 -> zp; saturation after the shift
    assert q8([3.0, 0.0, -1.0, 200.0], s=0.5, zp=10).tolist() == [12, 10, 10, 110]
    assert q8([0.0, 240.0], s=0.5, zp=-10).tolist() == [-10, 110]
    assert q8([-300.0], s=1.0, zp=100).tolist() == [-128]


def test_int8_scale_is_a_multiplier_per_row():
    y = np.array([[1.0, 2.0], [1.0, 2.0]])
    q = quantize_output(y, np.array([4.0, 0.25], np.float32), np.array([0, 1], np.int32), QOUT_INT8)
    assert q.tolist() == [[4, 8], [1, 2]]  # row 1: 1*0.25+1 = 1.25 -> 1, 2*0.25+1 = 1.5 -> 2


def test_int8_dequantisation_error_bound():
    rng = np.random.default_rng(7)
    y = rng.normal(0.0, 3.0, size=(16, 512))
    s = rng.uniform(2.0, 30.0, size=16).astype(np.float32)
    zp = rng.integers(-20, 20, size=16).astype(np.int32)
    q = quantize_output(y, s, zp, QOUT_INT8)
    inside = (q > -128) & (q < 127)
    assert inside.mean() > 0.9
    deq = (q - zp[:, None]) / s.astype(np.float64)[:, None]
    err = np.abs(deq - y)[inside] * s.astype(np.float64)[:, None].repeat(512, 1)[inside]
    assert err.max() <= 0.5 + 1e-5


def test_int8_matches_torch_round_half_even():
    rng = np.random.default_rng(11)
    y = rng.normal(0.0, 40.0, size=(8, 1000))
    # include exact ties
    y[0, :200] = np.arange(-100, 100) + 0.5
    s = np.ones(8, np.float32)
    q = quantize_output(y, s, None, QOUT_INT8)
    t = torch.from_numpy(y.astype(np.float32)).round().clamp(-128, 127).to(torch.int64).numpy()
    assert np.array_equal(q, t)


def test_int8_monotone():
    y = np.sort(np.random.default_rng(3).normal(0.0, 50.0, size=4000))[None, :]
    q = quantize_output(y, np.array([1.7], np.float32), np.array([5], np.int32), QOUT_INT8)[0]
    assert np.all(np.diff(q) >= 0)


def test_e4m3_exact_codes_round_trip_through_scale():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = decode_e4m3(codes)
    for s in (0.125, 1.0, 16.0):
        y = (vals / s)[None, :]
        q = quantize_output(y, np.array([s], np.float32), None, QOUT_E4M3)[0]
        # -0 and +0 both decode to 0; compare values, and codes elsewhere
        assert np.array_equal(decode_e4m3(q), vals)
        nz = vals != 0
        assert np.array_equal(q[nz], codes[nz])


def test_e4m3_saturates_and_rejects_zero_point():
    y = np.array([[1.0e6, -1.0e6, 448.0, 449.0, 500.0, 3.0e38]])
    q = quantize_output(y, np.array([1.0], np.float32), None, QOUT_E4M3)[0]
    assert q.tolist() == [0x7E, 0xFE, 0x7E, 0x7E, 0x7E, 0x7E]
    with pytest.raises(ValueError):
        quantize_output(y, np.array([1.0], np.float32), np.array([0], np.int32), QOUT_E4M3)


def test_e4m3_matches_torch_cast_in_range():
    rng = np.random.default_rng(5)
    y = rng.normal(0.0, 2.0, size=(4, 2000))
    s = np.array([1.0, 10.0, 50.0, 0.01], np.float32)
    q = quantize_output(y, s, None, QOUT_E4M3)
    w = (y.astype(np.float32) * s[:, None]).astype(np.float32)
    ok = np.abs(w) <= 448
    t = torch.from_numpy(w).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert ok.mean() > 0.9
    assert np.array_equal(q[ok], t[ok])


def test_e4m3_monotone():
    y = np.sort(np.random.default_rng(9).normal(0.0, 100.0, size=4000))[None, :]
    q = quantize_output(y, np.array([3.0], np.float32), None, QOUT_E4M3)[0]
    assert np.all(np.diff(decode_e4m3(q)) >= 0)


def test_decision_is_taken_on_the_float32_output():
    # y just below a tie in float64 but equal to the tie after rounding to
    # float32: the code follows the float32 value (3.5 -> 4), not the float64
    # one (3.4999... -> 3).
    y = 3.5 - 2.0 ** -30
    assert np.float32(y) == np.float32(3.5)
    assert q8([y]).tolist() == [4]
