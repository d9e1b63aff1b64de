"""The normal CDF of the cooperative scan's GELU (scan_coop.hip), against scipy.

The kernel takes Phi(a) = (1 + erf(a / sqrt 2)) / 2 with erf by Abramowitz and
Stegun's formula 7.1.26 (|error| <= 1.5e-7 for x >= 0) and reuses its factor
e^(-a^2/2) in GELU'(a) = Phi(a) + a e^(-a^2/2) / sqrt(2 pi).  The test reads the
formula's constants out of the kernel source, checks them against the printed
ones, evaluates the kernel's steps in float32 and checks the error of Phi,
GELU and GELU' everywhere on [-12, 12].
"""
import os
import re

import numpy as np
from scipy.special import ndtr

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "test_rnn_layer_amd", "csrc",
                   "scan_coop.hip")

# Abramowitz and Stegun, Handbook of Mathematical Functions, 7.1.26
AS_P = 0.3275911
AS_A = [0.254829592, -0.284496736, 1.421413741, -1.453152027, 1.061405429]


def _kernel_constants():
    txt = open(SRC).read()
    body = txt[txt.index("float normal_cdf(float a, float* e)"):]
    body = body[:body.index("\n}\n")]
    p = float(re.search(r"rcpf\(fmaf\(([-0-9.e]+)f, x, 1\.0f\)\)", body).group(1))
    first = float(re.search(r"float p = ([-0-9.e]+)f;", body).group(1))
    rest = [float(x) for x in re.findall(r"p = fmaf\(p, t, ([-0-9.e]+)f\);", body)]
    return p, [first] + rest  # a5, a4, ..., a1


def _phi_kernel(a):
    f = np.float32
    p, horner = _kernel_constants()
    a = a.astype(f)
    x = (np.abs(a) * f(0.7071067811865476)).astype(f)
    t = (f(1) / (f(p) * x + f(1))).astype(f)
    acc = f(horner[0])
    for c in horner[1:]:
        acc = (acc * t + f(c)).astype(f)
    e = np.exp2(a * (a * f(-0.7213475204444817))).astype(f)
    tail = (f(0.5) * (acc * t) * e).astype(f)
    return np.where(a >= 0, f(1) - tail, tail).astype(f), e


def test_constants_are_the_printed_ones():
    p, horner = _kernel_constants()
    assert p == AS_P
    assert horner == AS_A[::-1]


def test_normal_cdf_error_bound():
    a = np.linspace(-12.0, 12.0, 2_400_001).astype(np.float32)
    a64 = a.astype(np.float64)
    phi, e = _phi_kernel(a)
    ref = ndtr(a64)
    # the formula's 1.5e-7 on erf is 7.5e-8 on Phi; float32 evaluation adds a few ulp of 1
    assert np.abs(phi - ref).max() <= 3.5e-7
    assert np.abs(a64 * (phi - ref)).max() <= 5e-7
    dg = a * np.float32(0.3989422804014327) * e + phi
    dg_ref = ref + a64 * np.exp(-a64 ** 2 / 2) / np.sqrt(2 * np.pi)
    assert np.abs(dg - dg_ref).max() <= 3.5e-7


def test_normal_cdf_special_values():
    phi, e = _phi_kernel(np.array([0.0, 40.0, -40.0], dtype=np.float32))
    assert abs(float(phi[0]) - 0.5) <= 1e-7  # the formula's erf(0) is 1 - (a1 + ... + a5) = 1e-9
    assert phi[1] == np.float32(1.0) and phi[2] == np.float32(0.0)
    assert e[0] == np.float32(1.0)
