"""Constants of the HIP kernels checked on the host against the functions they
approximate (no GPU needed): the polynomial behind 1 - 2^-D for |D| < 1/4 in
the residual masses."""
import math
import os
import re

import numpy as np

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "draft_verification_amd", "csrc", "spec_verify.hip")


def _coefficients():
    text = open(SRC).read()
    i = text.index("(kernel-constant: one_minus_exp2_neg)")
    body = text[i:text.index("return", i)]
    lits = [float(x) for x in re.findall(r"([-+]?\d\.\d+e[-+]\d+)f", body)]
    assert len(lits) == 5, lits
    return lits[::-1]  # D^0 .. D^4 (Horner order in the source is D^4 first)


def test_series_polynomial_relative_error():
    c = [np.float32(x) for x in _coefficients()]
    D = np.linspace(-0.25, 0.25, 100001)
    exact = -np.expm1(-D * math.log(2.0))
    poly = np.zeros_like(D)
    for ck in c[::-1]:
        poly = poly * D + float(ck)
    approx = poly * D
    nz = D != 0.0
    rel = np.abs(approx[nz] / exact[nz] - 1.0)
    assert rel.max() < 2.5e-8, rel.max()
    # the leading coefficient is ln 2 to fp32 precision (the derivative at 0)
    assert abs(float(c[0]) - math.log(2.0)) < 1e-7


def test_series_meets_the_exponential_branch_continuously():
    # at |D| = 1/4 both branches agree to far better than the exp branch's own
    # error (~4e-7 relative)
    c = [float(np.float32(x)) for x in _coefficients()]
    for D in (0.25, -0.25):
        poly = 0.0
        for ck in c[::-1]:
            poly = poly * D + ck
        exact = -math.expm1(-D * math.log(2.0))
        assert abs(poly * D / exact - 1.0) < 2.5e-8
