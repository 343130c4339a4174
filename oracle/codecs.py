"""Exact decoding of the storage formats and round-to-nearest-even encoding.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Decoding works from the bit fields, not from a library cast, so that what the
oracle believes a code means is written out here:

* BF16: sign (1 bit), exponent (8 bits, bias 127), fraction (7 bits); the
  upper half of an IEEE binary32.
* OCP FP8 E4M3FN: sign (1), exponent (4, bias 7), mantissa (3); no
  infinities; S.1111.111 is NaN; largest finite value 448 = S.1111.110. The
  DeepGEMM FP8 page (sec. 1.2) names E4M3 as 4 exponent bits and 3 mantissa
  bits; the bias, the subnormals and the NaN code are those of the OCP 8-bit
  floating point specification (E4M3FN variant), which is the FP8 format the
  gfx950 matrix cores read.
"""
from __future__ import annotations

import numpy as np


def decode_bf16(bits) -> np.ndarray:
    """uint16 BF16 codes -> exact float64 values."""
    b = np.asarray(bits).astype(np.uint32)
    s = (b >> 15) & 1
    e = ((b >> 7) & 0xFF).astype(np.int64)
    f = (b & 0x7F).astype(np.int64)
    sign = np.where(s == 1, -1.0, 1.0)
    normal = np.ldexp((128 + f).astype(np.float64), e - 127 - 7)
    subnormal = np.ldexp(f.astype(np.float64), -126 - 7)
    special = np.where(f == 0, np.inf, np.nan)
    mag = np.where(e == 0, subnormal, np.where(e == 255, special, normal))
    return sign * mag


def decode_e4m3(bits) -> np.ndarray:
    """uint8 OCP E4M3FN codes -> exact float64 values (NaN for S.1111.111)."""
    b = np.asarray(bits).astype(np.uint32)
    s = (b >> 7) & 1
    e = ((b >> 3) & 0xF).astype(np.int64)
    f = (b & 0x7).astype(np.int64)
    sign = np.where(s == 1, -1.0, 1.0)
    normal = np.ldexp((8 + f).astype(np.float64), e - 7 - 3)
    subnormal = np.ldexp(f.astype(np.float64), -6 - 3)
    mag = np.where(e == 0, subnormal, normal)
    mag = np.where((e == 15) & (f == 7), np.nan, mag)
    return sign * mag


def round_to_bf16(y) -> np.ndarray:
    """float64 -> nearest BF16 value (ties to even), returned as float64.

    One rounding straight from float64 (no detour through float32). Values at
    or beyond the overflow threshold become +-inf; NaN stays NaN.
    """
    y = np.asarray(y, dtype=np.float64)
    out = y.copy()
    a = np.abs(y)
    sel = np.isfinite(y) & (a > 0)
    av = a[sel]
    _, e2 = np.frexp(av)  # av = frac * 2**e2, 0.5 <= frac < 1
    lead = np.maximum(e2 - 1, -126)  # exponent of the leading bit; subnormal quantum below
    quantum = np.ldexp(1.0, lead - 7)  # 7 fraction bits
    r = np.rint(av / quantum) * quantum  # np.rint rounds half to even
    r = np.where(r >= 2.0 ** 128, np.inf, r)
    out[sel] = np.copysign(r, y[sel])
    return out


def round_to_bf16_bits(y) -> np.ndarray:
    """float64 -> uint16 BF16 codes of round_to_bf16(y)."""
    v = np.atleast_1d(round_to_bf16(y))
    nan = np.isnan(v)
    v32 = np.where(nan, 0.0, v).astype(np.float32)  # exact: v is representable in BF16
    bits = (v32.view(np.uint32) >> 16).astype(np.uint16)
    bits[nan] = 0x7FC0
    return bits.reshape(np.shape(y))


def round_to_f32(y) -> np.ndarray:
    """float64 -> nearest binary32 (IEEE round to nearest even), as float32."""
    return np.asarray(y, dtype=np.float64).astype(np.float32)
