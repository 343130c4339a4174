"""Per-token quantisation of the GEMM's output. TEST INFRASTRUCTURE ONLY.

What it computes (the reading of the quantising epilogue of the first DeepGEMM
page, sec. 6.2: the layer after the GEMM wants INT8, so each FP32 output x is
turned into round(x * scale + zero_point) before it is written, with one scale
per row (token) looked up by the row index):

    x  = float32(y)                           the FP32 epilogue value
    INT8: v = float32(x * s[m] + zp[m])       one rounding, as a fused multiply-add
          q = clip(round_half_even(v), -128, 127)
    E4M3: w = float32(x * s[m])
          q = E4M3 code of w (round to nearest even, saturating at +-448)

Readings where the page is silent: the zero point is per row like the scale
(absent = 0); "round" is round to nearest even, as every other cast on the
path; out-of-range values saturate; the E4M3 variant (the FP8 output the FP8
page's sec. 4.2 has the next layer read) has a scale and no zero point.

The quantised code is decided in float32 (the precision of the GEMM output the
page quantises), so for a given float32 x this function and the kernel reach
the same code; v is formed as x * s + zp in float64 and rounded once to
float32, which equals the fused multiply-add whenever the float64 sum is exact
(always for |zp| < 2**24 and x * s not far below 2**-29 in magnitude; below
that v rounds to zp either way).

Parity status: pinned by tests/test_oracle_qout.py (round-half-even ties,
saturation bounds, zero point, dequantisation error bound, E4M3 code round
trips and saturation, monotonicity, and torch's round / float8 cast as
cross-checks of the two rounding steps).
"""
from __future__ import annotations

import numpy as np

from .codecs import round_to_f32
from .quant import encode_e4m3

QOUT_INT8, QOUT_E4M3 = 0, 1


def quantize_output(y, out_scale, out_zero, q_dtype: int) -> np.ndarray:
    """float64 epilogue values (rows x cols) -> codes: int8 values (as int64) or E4M3 uint8.

    out_scale: per-row scales (rows,). out_zero: per-row zero points (rows,) or None.
    """
    x = round_to_f32(np.asarray(y, dtype=np.float64)).astype(np.float64)
    s = np.asarray(out_scale, dtype=np.float32).astype(np.float64)[:, None]
    if q_dtype == QOUT_INT8:
        zp = 0.0 if out_zero is None else np.asarray(out_zero, dtype=np.int64).astype(np.float64)[:, None]
        v = round_to_f32(x * s + zp).astype(np.float64)
        return np.clip(np.rint(v), -128, 127).astype(np.int64)
    if q_dtype == QOUT_E4M3:
        if out_zero is not None:
            raise ValueError("the E4M3 output has no zero point")
        w = round_to_f32(x * s)  # x * s is exact in float64 (24-bit significands)
        return encode_e4m3(w)
    raise ValueError(f"unknown q_dtype {q_dtype}")
