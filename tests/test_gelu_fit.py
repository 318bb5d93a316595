"""The GELU epilogue's erfc approximation, checked on the CPU.

The device computes Phi(-|z|) = t * exp2(Q2(t) - z^2 log2(e)/2) with the
constants of tiled_dense_gemm_bias_amd/gelu_fit.py. Here the same formula is
evaluated in float64 from those constants and compared with mpmath's normal
CDF; the fp32 rounding on the device is checked separately by the GPU
epilogue-probe test.
"""
import re

import mpmath
import numpy as np

from tiled_dense_gemm_bias_amd import gelu_fit

KERNELS_HPP = "tiled_dense_gemm_bias_amd/csrc/gba_kernels.hpp"


def test_fractional_error_of_phi_tail_is_below_1e5():
    mpmath.mp.dps = 30
    z = np.concatenate([np.linspace(0, 13.4, 3000), np.geomspace(1e-7, 13.4, 600)])
    got = gelu_fit.phi_neg_abs(z)
    ref = np.array([float(mpmath.ncdf(-v)) for v in z])
    frac = np.abs(got / ref - 1)
    assert frac.max() < 1e-5, frac.max()
    # and therefore GELU itself, z * Phi(z) = max(z,0) - |z| Phi(-|z|)
    for s in (1.0, -1.0):
        zz = s * z[z > 0]
        g = np.maximum(zz, 0) - np.abs(zz) * gelu_fit.phi_neg_abs(zz)
        gref = np.array([float(mpmath.mpf(v) * mpmath.ncdf(v)) for v in zz])
        assert np.all(np.abs(g - gref) <= 1e-5 * np.abs(gref) + 1e-300)


def test_kernel_constants_are_the_tested_ones():
    src = open(KERNELS_HPP).read()
    body = src[src.index("ACT == ACT_GELU"):src.index("} else {", src.index("ACT == ACT_GELU"))]
    consts = [float(v) for v in re.findall(r"(-?\d+\.\d+)f", body)]
    # t scale, five Horner coefficients after the leading one, -log2(e)/2
    assert consts[0] == gelu_fit.KERNEL_T_SCALE or abs(consts[0] - gelu_fit.KERNEL_T_SCALE) < 1e-15
    horner = consts[2:8]
    assert np.allclose(horner, gelu_fit.KERNEL_Q2, rtol=0, atol=0), horner
    assert abs(consts[8] + gelu_fit.KERNEL_HALF_LOG2E) < 1e-15


def test_fit_reproduces_kernel_constants():
    c, err = gelu_fit.fit()
    assert err < 1e-5
    assert np.allclose(gelu_fit.kernel_coefficients(c), gelu_fit.KERNEL_Q2, rtol=1e-6, atol=1e-7)
