"""Per-token FP8 quantisation of BF16 rows. TEST INFRASTRUCTURE ONLY.

What it computes (the reading of the per-token scaling of DeepGEMM: FP8
precision Tensor Core GEMM optimisation, sec. 1.2, that the GEMM inputs also
follow):

    scale[m] = float32(amax_k |x(m,k)| / 448)         (1 for an all-zero row)
    q[m, k]  = E4M3 code of RNE(float32(x(m,k) / scale[m])), saturating at +-448

Both divisions are IEEE float32 divisions (numpy float32 arithmetic is
correctly rounded). The float32 -> E4M3 step is written out from the format
(OCP E4M3FN: sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals
below 2^-6, largest finite 448, no infinities) with round to nearest, ties to
even, and saturation to +-448 for larger magnitudes.

Parity status: pinned by tests/test_oracle_quant.py (every finite code
round-trips; every midpoint between neighbouring codes rounds to the even
one; saturation; subnormals; scale closed forms; torch's float8_e4m3fn cast
as a cross-check of the encoder on random values).
"""
from __future__ import annotations

import numpy as np

from .codecs import decode_bf16

E4M3_MAX = 448.0


def encode_e4m3(y) -> np.ndarray:
    """float32 values -> uint8 OCP E4M3FN codes (round to nearest even, saturating).

    NaN inputs are not handled (undefined in the quantiser's contract).
    """
    y = np.asarray(y, dtype=np.float32).astype(np.float64)  # exact widening
    sign = np.signbit(y).astype(np.uint8) << 7
    a = np.minimum(np.abs(y), E4M3_MAX)
    # Exponent of the leading bit, clamped to the normal range [-6, 8]; below
    # 2^-6 the quantum is the subnormal one, 2^-9.
    with np.errstate(divide="ignore"):
        lead = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    lead = np.clip(lead, -6, 8)
    quantum = np.ldexp(1.0, (lead - 3).astype(np.int64))
    r = np.rint(a / quantum) * quantum  # a / quantum is exact: quantum is a power of two
    # Rounding may carry into the next binade (e.g. 15.5 * 2^-3 -> 2^1); that
    # value is still exactly representable, so re-derive its fields from r.
    r = np.minimum(r, E4M3_MAX)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(r > 0, r, 1.0)))
    normal = r >= 2.0 ** -6
    e = np.where(normal, e, -6)
    mant = np.where(normal, r / np.ldexp(1.0, e.astype(np.int64)) * 8 - 8,
                    r / 2.0 ** -9)
    exp_field = np.where(normal, e + 7, 0)
    code = (exp_field.astype(np.int64) << 3) | np.rint(mant).astype(np.int64)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def quantize_rows_e4m3(x_bits, K: int | None = None):
    """BF16 codes (M x >=K, uint16) -> (E4M3 codes M x K uint8, scales float32[M])."""
    xb = np.asarray(x_bits)
    if K is None:
        K = xb.shape[1]
    x = decode_bf16(xb[:, :K]).astype(np.float32)  # exact: BF16 values are float32 values
    M = x.shape[0]
    amax = np.abs(x).max(axis=1) if K > 0 else np.zeros(M, np.float32)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = (x / scale[:, None]).astype(np.float32)
    return encode_e4m3(q).reshape(M, K), scale
