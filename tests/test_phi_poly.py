"""The normal-CDF polynomial of the MFMA scan (phi_poly.h), against scipy.

The scan's GELU is a * Phi(a) and GELU'(a) = Phi(a) + a phi(a), with Phi from
this polynomial.  The test evaluates the header's float32 coefficients the way
the kernel does (clamp, s = c^2, Horner in float32, 1/2 + c p(s)) and checks the
absolute error bound stated in the generator: 1.8e-4 on Phi, everywhere.
"""
import os
import re

import numpy as np
from scipy.special import ndtr

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "test_rnn_layer_amd", "csrc",
                   "phi_poly.h")


def _coefficients():
    txt = open(HDR).read()
    L = float(re.search(r"kPhiL = ([-0-9.e]+)f", txt).group(1))
    body = re.search(r"kPhiP\[kPhiDeg \+ 1\] = \{[^\n]*\n(.*?)\};", txt, re.S).group(1)
    p = [np.float32(x) for x in re.findall(r"([-0-9.e]+)f", body)]
    return np.float32(L), p


def _phi_kernel(a):
    L, p = _coefficients()
    c = np.clip(a.astype(np.float32), -L, L)
    s = (c * c).astype(np.float32)
    acc = p[-1]
    for coef in p[-2::-1]:
        acc = (acc * s + coef).astype(np.float32)
    return (c * acc + np.float32(0.5)).astype(np.float32)


def test_phi_poly_error_bound():
    a = np.linspace(-12.0, 12.0, 2_400_001).astype(np.float32)
    err = np.abs(_phi_kernel(a).astype(np.float64) - ndtr(a.astype(np.float64)))
    assert err.max() <= 1.8e-4, err.max()
    # GELU = a Phi(a): its error is |a| times Phi's, 1.8e-4 relative to |a|
    gelu_err = np.abs(a.astype(np.float64) * (_phi_kernel(a) - ndtr(a.astype(np.float64))))
    assert (gelu_err <= 1.8e-4 * np.abs(a.astype(np.float64)) + 1e-12).all()


def test_phi_poly_shape():
    L, p = _coefficients()
    assert len(p) == 6
    # p_0 approximates Phi'(0) = 1/sqrt(2 pi) (a minimax fit trades a little of it for the
    # tails); Phi(0) = 1/2 exactly; symmetry Phi(-a) = 1 - Phi(a)
    # (degree 5: 6.5e-4 off, an error of Phi of 6.5e-4 |a| near 0, inside the 1.8e-4 bound for |a| < 0.27)
    assert abs(float(p[0]) - 1 / np.sqrt(2 * np.pi)) < 1e-3
    assert _phi_kernel(np.zeros(1))[0] == np.float32(0.5)
    a = np.linspace(0, 6, 1001).astype(np.float32)
    np.testing.assert_allclose(_phi_kernel(-a), 1 - _phi_kernel(a), atol=1e-7)
