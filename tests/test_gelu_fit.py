"""The GELU epilogue's normal-tail approximation, checked on the CPU.

The device computes Phi(-|z|) = 2^Q(|z|) with the degree-7 polynomial Q of
tiled_dense_gemm_bias_amd/gelu_fit.py. Here Q is evaluated in float64 from the
kernel's float32 constants and compared with mpmath's normal CDF; the fp32
rounding on the device is checked separately by the GPU epilogue-probe test.
"""
import re

import mpmath
import numpy as np

from tiled_dense_gemm_bias_amd import gelu_fit

KERNELS_HPP = "tiled_dense_gemm_bias_amd/csrc/gba_kernels.hpp"


def _gelu(z):
    z = np.asarray(z, dtype=np.float64)
    return np.maximum(z, 0) - np.abs(z) * gelu_fit.phi_neg_abs(z)


def _gelu_ref(z):
    mpmath.mp.dps = 30
    return np.array([float(mpmath.mpf(v) * mpmath.ncdf(v)) for v in z])


def test_fractional_error_of_phi_on_fit_range_is_below_1e5():
    mpmath.mp.dps = 30
    x = np.concatenate([np.linspace(0, gelu_fit.X_MAX, 3000), np.geomspace(1e-7, gelu_fit.X_MAX, 600)])
    got = gelu_fit.phi_neg_abs(x)
    ref = np.array([float(mpmath.ncdf(-v)) for v in x])
    frac = np.abs(got / ref - 1)
    assert frac.max() < 1e-5, frac.max()


def test_gelu_is_relatively_accurate_where_it_matters_and_tiny_elsewhere():
    zs = np.concatenate([np.linspace(-gelu_fit.X_MAX, gelu_fit.X_MAX, 4001),
                         np.geomspace(1e-7, gelu_fit.X_MAX, 400)])
    zs = np.concatenate([zs, -zs])
    err = np.abs(_gelu(zs) - _gelu_ref(zs))
    assert np.all(err <= 1e-5 * np.abs(_gelu_ref(zs)) + 1e-300)
    # past the fit range the correction term is below 1e-8 absolute
    zt = np.concatenate([np.linspace(gelu_fit.X_MAX, 40, 3000), np.geomspace(40, 1e6, 300)])
    zt = np.concatenate([zt, -zt])
    err = np.abs(_gelu(zt) - _gelu_ref(zt))
    assert err.max() < 1e-8, err.max()


def test_q_keeps_falling_past_the_fit_range_in_float32():
    # Horner in float32 (as on the device): no NaN anywhere up to the largest
    # finite float32, Q decreasing, |x| 2^Q(x) below 6e-9.
    c = [np.float32(v) for v in gelu_fit.KERNEL_Q]
    x = np.geomspace(gelu_fit.X_MAX, 3.0e38, 20000).astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        q = np.full_like(x, c[0])
        for cc in c[1:]:
            q = (q * x + cc).astype(np.float32)
    assert not np.isnan(q).any()
    assert np.all(q[1:] <= q[:-1])
    tail = x.astype(np.float64) * np.exp2(np.minimum(q.astype(np.float64), 0.0))
    assert tail.max() < 6e-9, tail.max()


def test_kernel_constants_are_the_tested_ones():
    src = open(KERNELS_HPP).read()
    start = src.index("ACT == ACT_GELU")
    body = src[start:src.index("} else", start)]
    consts = [float(v) for v in re.findall(r"(-?\d+\.\d+(?:e-?\d+)?)f", body)]
    # the eight Horner coefficients, then the clamp of the multiplier (3e38, for
    # z = +-inf) and the 0 of max(z, 0)
    assert consts[:8] == gelu_fit.KERNEL_Q and consts[8:] == [3.0e38, 0.0], consts


def test_fit_reproduces_kernel_constants():
    c, err = gelu_fit.fit()
    assert err < 1e-5
    assert np.allclose(gelu_fit.kernel_coefficients(c), gelu_fit.KERNEL_Q, rtol=1e-5, atol=1e-10)
