"""CPU check of the polynomial the final-draw kernel uses for 1 - 2^-D.

For 0 < D < 1 the residual weight's factor 1 - 2^-D is computed as x * g(x)
with x = D ln 2 and g a degree-5 polynomial standing for (1 - e^-x)/x on
[0, ln 2]; from D = 1 up it is 1 - 2^-D directly.  The coefficients are read
from the kernel source, and the polynomial is checked against fp64 expm1 on
a dense grid: in exact arithmetic (its fp32 coefficients, fp64 evaluation)
its relative error stays under 2e-8 (1.83e-8 at most), and
evaluated the way the kernel does it (fp32 fused multiply-adds, emulated
here by rounding each exact fp64 step to fp32) the whole factor stays within
2e-7 relative of 1 - 2^-D for every D in (0, 1) (1.55e-7 at most, under 3
units in the last place, from the roundings of x, of each step and of x*g).
"""
import os
import re

import numpy as np

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "exact_draft_verification_amd", "csrc", "chain.hip")


def coefficients():
    text = open(SRC).read()
    body = re.search(r"one_minus_exp2_neg_small\(float D\) \{(.*?)\n\}", text, re.S).group(1)
    lead = re.search(r"float g = ([-0-9.e+]+)f;", body).group(1)
    rest = re.findall(r"g = fmaf\(g, x, ([-0-9.e+]+)f\);", body)
    ln2 = re.search(r"const float x = D \* ([0-9.]+)f;", body).group(1)
    return [np.float32(lead)] + [np.float32(c) for c in rest], np.float32(ln2)


def test_polynomial_relative_error_exact_arithmetic():
    c, _ = coefficients()
    assert len(c) == 6 and c[-1] == np.float32(1.0)
    x = np.linspace(1e-9, np.log(2.0), 200001)
    g = np.zeros_like(x)
    for k in c:
        g = g * x + np.float64(k)
    want = -np.expm1(-x) / x
    rel = np.abs(g - want) / want
    assert rel.max() < 2e-8, rel.max()


def test_kernel_evaluation_in_fp32():
    c, ln2 = coefficients()
    D = np.concatenate([np.linspace(1e-7, 1.0, 400001, endpoint=False),
                        np.geomspace(1e-30, 1e-7, 2001)]).astype(np.float32)
    D = D[(D > 0) & (D < 1)]
    f32 = np.float32
    x = (D.astype(np.float64) * np.float64(ln2)).astype(f32)
    g = np.full_like(x, c[0])
    for k in c[1:]:
        g = (g.astype(np.float64) * x.astype(np.float64) + np.float64(k)).astype(f32)
    got = (x.astype(np.float64) * g.astype(np.float64)).astype(f32).astype(np.float64)
    want = -np.expm1(-D.astype(np.float64) * np.log(2.0))
    rel = np.abs(got - want) / want
    assert rel.max() < 2e-7, rel.max()
