"""Fit of the normal tail used by the GELU epilogue (writes the kernel constants).

    python -m tiled_dense_gemm_bias_amd.gelu_fit

The epilogue computes GELU(z) = z * Phi(z) as max(z, 0) - |z| * Phi(-|z|), which
needs Phi(-x), x = |z|, accurate in the *relative* sense wherever the result is
large enough to matter. It evaluates

    Phi(-x) = 2^Q(x),   Q a degree-7 polynomial in x,

which costs seven fused multiply-adds and one hardware exp2, with no division.
Q is fitted to log2 Phi(-x) on x in [0, 6] by iteratively reweighted least
squares (which approaches the minimax fit). The fit's leading coefficient is
negative, so Q keeps falling past x = 6 and |z| * 2^Q(|z|) stays below 6e-9 for
every |z| >= 6: GELU(z) for z <= -6 is then computed as a number below 6e-9 in
magnitude (the true value is below 6e-9 too), and for z >= 6 the correction is
below 6e-9 absolute. Both are far below the absolute floor of 2^-20 that the
element-wise check of the fused GEMM allows, and below every fp16 or bf16
rounding of |z| >= 6. On [0, 6] the fractional error of 2^Q is below 8e-6
(tests/test_gelu_fit.py pins it against mpmath).
"""
from __future__ import annotations

import numpy as np

DEGREE = 7
X_MAX = 6.0


def _log2_phi_neg(x: np.ndarray) -> np.ndarray:
    import mpmath
    mpmath.mp.dps = 40
    return np.array([float(mpmath.log(mpmath.erfc(v / mpmath.sqrt(2)) / 2, 2)) for v in x])


def fit(degree: int = DEGREE, x_max: float = X_MAX):
    """Coefficients of Q (highest degree first) and the max |Q - log2 Phi(-x)|."""
    xs = np.unique(np.concatenate([np.linspace(0, x_max, 4000), np.geomspace(1e-5, x_max, 800)]))
    target = _log2_phi_neg(xs)
    V = np.vander(xs, degree + 1)
    w = np.ones_like(xs)
    for _ in range(200):
        c, *_ = np.linalg.lstsq(V * w[:, None], target * w, rcond=None)
        err = V @ c - target
        w = w * (1 + 2 * np.abs(err) / np.abs(err).max())
        w /= w.mean()
    return c, float(np.abs(V @ c - target).max())


def kernel_coefficients(c: np.ndarray) -> list:
    """Q's coefficients rounded to float32, highest degree first."""
    return [float(np.float32(v)) for v in c]


# Coefficients compiled into act_fn<GELU> (gba_kernels.hpp), highest degree
# first: the output of kernel_coefficients(fit()[0]).
KERNEL_Q = [-1.8348076764596044e-06, 6.15982135059312e-05, -0.0009305241401307285,
            0.008507887832820415, -0.05396006256341934, -0.4584644138813019,
            -1.1512510776519775, -0.9999952912330627]


def q_poly(x: np.ndarray) -> np.ndarray:
    """Q(x) in float64 from the kernel's float32 constants (Horner, as the kernel)."""
    x = np.asarray(x, dtype=np.float64)
    q = np.full_like(x, KERNEL_Q[0])
    for c in KERNEL_Q[1:]:
        q = q * x + c
    return q


def phi_neg_abs(z: np.ndarray) -> np.ndarray:
    """Phi(-|z|) as the kernel approximates it, evaluated in float64."""
    return np.exp2(q_poly(np.abs(np.asarray(z, dtype=np.float64))))


def main() -> int:
    c, err = fit()
    print("degree %d on x in [0, %.1f]: max |Q - log2 Phi(-x)| = %.3e" % (DEGREE, X_MAX, err))
    print("Q (kernel) =", kernel_coefficients(c))
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
