"""Coefficients of the erfc fit used by the kernels' GELU for BF16 and
quantised outputs (`erfc_log2_fit7` in csrc/common.hpp).

For x >= 0 and t = 1 / (1 + x/2), erfc(x) = t exp(-x^2 + P(t)) with P smooth
on (0, 1] (the form of the Chebyshev-fitted erfc of Numerical Recipes in C,
2nd ed., sec. 6.2). The kernels need Q(t) = log2(e) P(t) + 63 (the 2^63 keeps
the exponential's result normal far into GELU's negative tail; the kernel
scales by 2^-64, which also supplies GELU's factor 1/2). This script fits Q
with a degree-7 polynomial in t by least squares at Chebyshev nodes on
t in [1/7, 1] (x <= 12, |z| <= 17, past which GELU's value underflows FP32 or
equals z) and prints the coefficients, highest degree first, rounded to
float32. tests/test_gelu_fit_cpu.py checks the table in common.hpp against
the function it approximates. Needs numpy and scipy; the library does not
import it.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erfcx

LOG2E = 1.4426950408889634
DEGREE = 7
X_MAX = 12.0


def target(t):
    """Q(t) = log2(e) * log(erfc(x) e^(x^2) / t) + 63, x = 2 (1/t - 1)."""
    x = 2.0 * (1.0 / t - 1.0)
    return LOG2E * (np.log(erfcx(x)) - np.log(t)) + 63.0


def fit(degree=DEGREE, x_max=X_MAX, nodes=6000):
    tmin = 1.0 / (1.0 + x_max / 2.0)
    t = np.cos(np.linspace(0.0, np.pi, nodes)) * (1.0 - tmin) / 2.0 + (1.0 + tmin) / 2.0
    u = 2.0 * (t - tmin) / (1.0 - tmin) - 1.0
    c = np.polynomial.chebyshev.chebfit(u, target(t), degree)
    pu = np.polynomial.Polynomial(np.polynomial.chebyshev.cheb2poly(c))
    a, b = 2.0 / (1.0 - tmin), -2.0 * tmin / (1.0 - tmin) - 1.0
    pt = pu(np.polynomial.Polynomial([b, a]))
    return [float(np.float32(x)) for x in pt.coef[::-1]]


if __name__ == "__main__":
    for c in fit():
        print(f"{c!r}f,")
