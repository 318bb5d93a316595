"""Fit of the erfc form used by the GELU epilogue (writes the kernel constants).

    python -m tiled_dense_gemm_bias_amd.gelu_fit

The epilogue needs Phi(-|z|) = erfc(x) / 2 with x = |z| / sqrt(2), accurate in
the *relative* sense so that z * Phi(z) stays accurate for large negative z.
It uses the form of Press, Teukolsky, Vetterling & Flannery, "Numerical
Recipes" (2nd ed., sec. 6.2):

    erfc(x) = t * exp(-x^2 + Q(t)),   t = 1 / (1 + x/2),   x >= 0,

whose exponent correction Q is smooth in t on (0, 1]; Numerical Recipes fits a
degree-9 Q. This script fits a degree-5 Q (fewer fused multiply-adds per output
element) by iteratively reweighted least squares on |log(approx/erfc)| over
x in [0, 9.5] -- far enough for bf16 outputs, whose smallest normal value
GELU reaches near z = -13.4 -- and reports the worst fractional error, which
the tests check. The kernel folds log2(e) and the factor 1/2 into the
coefficients so that Phi(-|z|) = t * exp2(-z^2 log2(e)/2 + Q2(t)) with
Q2 = log2(e) * Q - 1.
"""
from __future__ import annotations

import math

import numpy as np

DEGREE = 5
X_MAX = 9.5


def _erfc_log(x: np.ndarray) -> np.ndarray:
    import mpmath
    mpmath.mp.dps = 30
    return np.array([float(mpmath.log(mpmath.erfc(v))) for v in x])


def fit(degree: int = DEGREE, x_max: float = X_MAX):
    xs = np.unique(np.concatenate([np.linspace(0, x_max, 4000), np.geomspace(1e-6, x_max, 2000)]))
    t = 1.0 / (1.0 + xs / 2.0)
    target = _erfc_log(xs) - np.log(t) + xs * xs     # Q(t) that makes the form exact
    w = np.ones_like(t)
    V = np.vander(t, degree + 1)
    for _ in range(80):
        c, *_ = np.linalg.lstsq(V * w[:, None], target * w, rcond=None)
        err = V @ c - target
        w = w * (1 + 2 * np.abs(err) / np.abs(err).max())
        w /= w.mean()
    return c, float(np.abs(V @ c - target).max())


def kernel_coefficients(c: np.ndarray) -> list:
    """Q2 = log2(e) * Q - 1, highest degree first, rounded to float32."""
    q2 = np.array(c, dtype=np.float64) * math.log2(math.e)
    q2[-1] -= 1.0
    return [float(np.float32(v)) for v in q2]


# Coefficients compiled into act_fn<GELU> (gba_kernels.hpp), highest degree
# first: the output of kernel_coefficients(fit()[0]).
KERNEL_Q2 = [0.3300653100013733, -1.023119330406189, 0.6845195889472961,
             0.3670990467071533, 1.468679428100586, -2.827233076095581]
KERNEL_HALF_LOG2E = 0.7213475204444817    # log2(e) / 2
KERNEL_T_SCALE = 0.35355339059327373       # 1 / (2 sqrt 2): t = 1 / (1 + |z| / (2 sqrt 2))


def phi_neg_abs(z: np.ndarray) -> np.ndarray:
    """Phi(-|z|) evaluated in float64 from the kernel's float32 constants."""
    az = np.abs(np.asarray(z, dtype=np.float64))
    t = 1.0 / (1.0 + az * KERNEL_T_SCALE)
    q = np.zeros_like(t)
    for c in KERNEL_Q2:
        q = q * t + c
    return t * np.exp2(q - az * az * KERNEL_HALF_LOG2E)


def main() -> int:
    c, err = fit()
    print("degree %d on x in [0, %.1f]: max |log(approx/erfc)| = %.3e" % (DEGREE, X_MAX, err))
    print("Q2 (kernel) =", kernel_coefficients(c))
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
