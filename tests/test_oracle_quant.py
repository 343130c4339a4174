"""Pins of the oracle's per-token FP8 quantiser (CPU only).

The E4M3 encoder is pinned by the format itself: every finite code must
round-trip through its exact value, every midpoint between two neighbouring
codes must go to the one with an even mantissa, magnitudes past 448 saturate,
and the subnormal range follows the 2^-9 quantum. torch's float8_e4m3fn cast
(a library routine the definition reduces to for in-range values) serves as a
cross-check on random float32 values, never inside the oracle. The row
quantiser is pinned by closed forms of its scale and by reconstruction bounds.
"""
import numpy as np
import pytest
import torch

from oracle import decode_e4m3, encode_e4m3, quantize_rows_e4m3

FINITE = [c for c in range(256) if c not in (0x7F, 0xFF)]


def test_every_finite_code_round_trips():
    v = decode_e4m3(np.array(FINITE, np.uint8)).astype(np.float32)
    assert np.array_equal(encode_e4m3(v), np.array(FINITE, np.uint8))


def test_midpoints_round_to_even_mantissa():
    pos = np.array([c for c in FINITE if c < 0x80], np.uint8)
    vals = decode_e4m3(pos)
    order = np.argsort(vals)
    pos, vals = pos[order], vals[order]
    for lo, hi, clo, chi in zip(vals[:-1], vals[1:], pos[:-1], pos[1:]):
        mid = np.float32((lo + hi) / 2)  # exact in float32: few significant bits
        assert float(mid) == (lo + hi) / 2
        even = clo if (clo & 1) == 0 else chi
        assert encode_e4m3([mid])[0] == even, (lo, hi)
        assert encode_e4m3([-mid])[0] == (even | 0x80)
        # just off the midpoint: nearest neighbour
        assert encode_e4m3([np.nextafter(mid, np.float32(0))])[0] == clo
        assert encode_e4m3([np.nextafter(mid, np.float32(1e9))])[0] == chi


def test_saturation_and_specials():
    assert list(encode_e4m3([448.0, 449.0, 463.9, 464.0, 1e6, -1e30])) == [0x7E, 0x7E, 0x7E, 0x7E,
                                                                          0x7E, 0xFE]
    assert list(encode_e4m3([0.0, -0.0])) == [0x00, 0x80]
    # subnormals: quantum 2^-9; 2^-10 is a tie between 0 and 2^-9 -> 0 (even)
    assert list(encode_e4m3([2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -9, 7 * 2.0 ** -9,
                             7.5 * 2.0 ** -9])) == [0x00, 0x02, 0x01, 0x07, 0x08]


def test_encoder_matches_torch_cast_on_random_values():
    rng = np.random.default_rng(7)
    y = np.concatenate([rng.standard_normal(100_000) * s for s in (1e-3, 0.1, 3.0, 100.0)])
    y = np.clip(y, -448, 448).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(encode_e4m3(y), ref)


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def test_row_scale_closed_forms():
    rows = np.array([[0.0, 0.0, 0.0, 0.0],
                     [448.0, -3.0, 1.0, 0.5],
                     [-1.0, 0.25, 0.125, 0.0],
                     [3.0, -7.0, 2.0, 1.0]])
    q, s = quantize_rows_e4m3(_bf16(rows))
    assert s.dtype == np.float32
    assert s[0] == 1.0 and not q[0].any()  # all-zero row: scale 1, zero codes
    assert s[1] == 1.0                      # amax 448 -> scale exactly 1
    assert list(q[1]) == list(encode_e4m3(np.float32([448.0, -3.0, 1.0, 0.5])))
    assert s[2] == np.float32(1.0) / np.float32(448.0)
    assert s[3] == np.float32(7.0) / np.float32(448.0)
    # the largest magnitude of a row always codes to +-448
    assert q[2][0] == 0xFE and q[3][1] == 0xFE


def test_reconstruction_bound_on_normal_rows():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 513)).astype(np.float32)
    xb = _bf16(x)
    xv = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).float().numpy().astype(np.float64)
    q, s = quantize_rows_e4m3(xb)
    back = decode_e4m3(q) * s[:, None].astype(np.float64)
    # E4M3 keeps 4 significant bits: half a unit is 2^-4 of the value in the
    # normal range; below 2^-6 * scale the error is at most half the 2^-9 quantum.
    err = np.abs(back - xv)
    bound = np.maximum(np.abs(xv) * 2.0 ** -4, 2.0 ** -10 * s[:, None]) * (1 + 1e-6)
    assert np.all(err <= bound)
    assert np.all(np.abs(decode_e4m3(q)) <= 448)


def test_planted_truncation_is_caught():
    """Rounding toward zero instead of to nearest even fails the midpoint pin."""
    def trunc_encode(y):
        y = np.asarray(y, np.float32)
        out = encode_e4m3(y)
        v = decode_e4m3(out)
        bad = np.abs(v) > np.abs(y)  # rounded away from zero: step one code down
        out[bad] = out[bad] - 1
        return out
    mids = np.float32([1.1875, 3.75, 1.5 * 2.0 ** -9])  # midpoints that round up under RNE
    assert not np.array_equal(trunc_encode(mids), encode_e4m3(mids))
