"""The erfc fit table the kernels' GELU uses for BF16 and quantised outputs
(`erfc_log2_fit7` in csrc/common.hpp) against the function it approximates.

Q(t) = log2(e) log(erfc(x) e^(x^2) / t) + 63 with t = 1 / (1 + x/2): the
table, read from the source, must be what dense_gemm_09_amd/gelu_fit.py
produces and lie within 2e-6 of Q on t in [1/7, 1] (x <= 12), i.e. a
relative error below 1.4e-6 in the erfc it yields (most of it is the
float32 rounding of the constant term). The GPU side of the same
check is tests/test_act_gpu.py (every BF16 value in [-16, 16])."""
from __future__ import annotations

import os
import re

import numpy as np
import pytest

pytest.importorskip("scipy")
from dense_gemm_09_amd import gelu_fit  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _table():
    src = open(os.path.join(ROOT, "dense_gemm_09_amd", "csrc", "common.hpp")).read()
    body = src[src.index("float erfc_log2_fit7(float t)"):]
    body = body[:body.index("return q;")]
    return [float(x) for x in re.findall(r"(-?\d+\.\d+(?:e-?\d+)?)f", body)]


def test_table_is_the_fit():
    assert _table() == gelu_fit.fit()


def test_table_within_bound_of_target():
    c = _table()
    assert len(c) == 8
    t = np.linspace(1.0 / 7.0, 1.0, 200001)
    q = np.zeros_like(t)
    for a in c:
        q = q * t + a
    err = np.abs(q - gelu_fit.target(t))
    assert err.max() <= 2e-6, err.max()
