"""The epilogue's activations on the GPU against the oracle, value by value.

With K = 0 a GEMM is its epilogue alone: C = act(beta * C_in + bias). With
beta = 1 and no bias, C_in supplies the pre-activation values z exactly, so the
kernels' activations are compared with the oracle's float64 activation on every
z of a dense grid, with no accumulation error in the way:

* FP32 output: |out - act(z)| <= ulp_f32(y) + ACT_REL[act] * |y| for a dense
  float32 grid of z in [-16, 16] (the bound the FP32 parity tolerance allows
  for the activation), which includes the far negative range where GELU's
  value is a tiny number.
* BF16 output: every BF16 value z with |z| <= 16: within one BF16 ulp of
  RNE_bf16(act(z)) (the BF16 parity bound with no accumulation error), and in
  particular on [-12, -3], where an activation formed as z (1 - (1 - P)) has
  no correct digits.

Both the tile kernel's epilogue (M = 256) and the skinny kernel's (M = 16) run.
"""
from __future__ import annotations

import numpy as np
import pytest

import dense_gemm_09_amd as g
import oracle
from synth import ACT_GELU_ERF, ACT_GELU_TANH, ACT_NONE, ACT_RELU, COL, OUT_BF16, OUT_F32, ROW
from tests import tolerance

pytestmark = pytest.mark.gpu

ACTS = [ACT_NONE, ACT_RELU, ACT_GELU_ERF, ACT_GELU_TANH]


def _epilogue_only(z, c_dtype, act):
    """Run C = act(1 * C_in) with K = 0 on the GPU; z: (M, N) float32 values (or
    uint16 BF16 codes for BF16 output)."""
    import torch
    M, N = z.shape
    print(f"[gpu] epilogue-only act={act} c_dtype={c_dtype} M={M} N={N}", flush=True)
    if c_dtype == OUT_F32:
        C = torch.from_numpy(np.ascontiguousarray(z, dtype=np.float32)).cuda()
    else:
        C = torch.from_numpy(np.ascontiguousarray(z).view(np.int16)).cuda()
    g.gemm_bf16(M, N, 0, 1.0, None, 8, ROW, None, 8, COL, 1.0, C, N, c_dtype, None, act)
    torch.cuda.synchronize()
    out = C.cpu().numpy()
    return out if c_dtype == OUT_F32 else out.view(np.uint16)


@pytest.mark.parametrize("M", [256, 16], ids=["tile", "skinny"])
@pytest.mark.parametrize("act", ACTS)
def test_activation_fp32_output(act, M):
    N = 4096
    z = np.linspace(-16.0, 16.0, M * N, dtype=np.float64).astype(np.float32).reshape(M, N)
    z[0, :8] = [-12.0, -9.5, -7.25, -5.5, -3.0, -0.0, 0.0, 1.0]
    out = _epilogue_only(z, OUT_F32, act)
    zd = z.astype(np.float64)
    y = oracle.activation(zd, act)
    zeros_m, zeros_n = np.zeros(M), np.zeros(N)
    info = tolerance.check_f32(out, y, zeros_m, zeros_n, 1.0, f"act {act} fp32", z=zd, act=act)
    nz = y != 0
    rel = np.abs(out[nz].astype(np.float64) - y[nz]) / np.abs(y[nz])
    print(f"[act {act}] fp32: max relative error {rel.max(initial=0.0):.3e} "
          f"(allowed {tolerance.ACT_REL[act]:.3e} + 1 ulp) {info}", flush=True)


def _bf16_grid():
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = oracle.decode_bf16(codes)
    keep = np.isfinite(v) & (np.abs(v) <= 16.0)
    return codes[keep]


@pytest.mark.parametrize("M", [256, 16], ids=["tile", "skinny"])
@pytest.mark.parametrize("act", ACTS)
def test_activation_bf16_output(act, M):
    codes = _bf16_grid()
    N = 4096
    cap = M * N
    assert codes.size <= cap or M == 16
    rounds = [codes[i:i + cap] for i in range(0, codes.size, cap)]
    for part in rounds:
        z_codes = np.zeros(cap, np.uint16)
        z_codes[:part.size] = part
        z_codes = z_codes.reshape(M, N)
        out = _epilogue_only(z_codes, OUT_BF16, act)
        zd = oracle.decode_bf16(z_codes)
        y = oracle.activation(zd, act)
        ref = oracle.decode_bf16(oracle.round_to_bf16_bits(y))
        got = oracle.decode_bf16(out)
        info = tolerance.check_bf16(got, y, ref, np.zeros(M), np.zeros(N), 1.0, act,
                                    f"act {act} bf16", z=zd)
        far = (zd >= -12) & (zd <= -3)
        print(f"[act {act}] bf16: {info}; exact on [-12, -3]: "
              f"{int((got[far] == ref[far]).sum())} of {int(far.sum())}", flush=True)
        assert info["exact"] >= 0.99 * info["n"]
