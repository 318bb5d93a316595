"""Tolerance checks between a device result and the fp64 oracle.

TEST INFRASTRUCTURE ONLY (used by tests/, the smoke check and the benchmark's
correctness report). Holds no GEMM or epilogue arithmetic.

Criteria:
  * relative Frobenius error ||C - R||_F / ||R||_F <= 2e-2 -- the fp16 check of
    "TileLang: Write, Autotune, and Ship Fused Tensor-Core Kernels from Python",
    sections "Practical defaults" and "Numerical validation";
  * per element |C - R| <= atol_K + rtol * |R| with rtol = 1e-2 and
    atol_K = 1e-2 * sqrt(K) / 64: the elementwise rtol/atol of
    "writing-tilelang-kernels", Step-by-Step Workflow (validation step), with
    the absolute part scaled by sqrt(K)/64 as the fp32-accumulation error grows;
  * a stricter gate, used to catch small indexing mistakes that 2e-2 lets
    through: |C - R| <= ulp_out(R) + L_act * rel * S + 2^-20, where
    S = sum_k |A_ik B_kj| + |bias_j|, L_act bounds the activation's slope and
    rel is the fp32 accumulation error per unit of S: 2 sqrt(K+1) 2^-24 for
    16-bit inputs, fp8_sum_rel(K) for 8-bit ones.
"""
from __future__ import annotations

import math

import numpy as np

REL_FRO_TOL = 2e-2
RTOL = 1e-2

# Largest slope of each activation: identity/ReLU 1, logistic 1/4,
# z*Phi(z) has derivative Phi(z) + z*phi(z) <= 1.129 (max near z = 1.41),
# softplus' derivative is the logistic (< 1), the tanh form of GELU <= 1.129.
ACT_LIPSCHITZ = {0: 1.0, 1: 1.0, 2: 0.25, 3: 1.13, 4: 1.0, 5: 1.13}


def atol_k(K: int) -> float:
    return 1e-2 * math.sqrt(max(K, 1)) / 64.0


def ulp_out(x: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the fp16/bf16 grid at |x| (the spacing just above |x|)."""
    man, emin = (10, -14) if dtype in ("f16", 0) else (7, -126)
    ax = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 2.0 ** (emin - 1))))
    e = np.maximum(e, emin)
    return np.ldexp(1.0, (e - man).astype(np.int64))


def rel_frobenius(C: np.ndarray, R: np.ndarray) -> float:
    C = np.asarray(C, dtype=np.float64)
    R = np.asarray(R, dtype=np.float64)
    num = np.linalg.norm((C - R).ravel())
    den = np.linalg.norm(R.ravel())
    return float(num / den) if den > 0 else float(num)


def fp8_sum_rel(K: int) -> float:
    """Accumulation coefficient of the stricter gate for 8-bit inputs, per unit
    of S = sum |a w scale| (+ |bias|).

    Model: a 16x16x128 8-bit matrix instruction forms 128 exact products (two
    8-bit significands fit fp32) and sums them in fp32 in an order and with a
    rounding that are not published. Whatever the order, a partial sum passes
    through at most 127 additions; each result is taken to be a faithful fp32
    rounding (off by less than one ulp, 2^-23 of its magnitude <= S), which
    covers round-to-nearest and truncation alike. The instructions' results
    are accumulated in fp32, ceil(K/128) - 1 more additions along the chain (a
    split-K run's chains are no longer: its splits are summed in order after
    their slices), and the product is scaled once. First-order worst case:
    (127 + ceil(K/128) - 1 + 1) 2^-23, plus one more rounding for the split-K
    partial's scale: 1.9e-5 at K = 4096 (the largest error seen on random
    inputs there is 8.1e-6 per unit of S).
    """
    n_inst = max(1, -(-int(K) // 128))
    return (127 + (n_inst - 1) + 2) * 2.0 ** -23


def check(C, R, K: int, dtype: str, act: int = 0, S=None, sum_rel=None) -> dict:
    """Compare device output C (float64 values) against oracle R.

    Returns a report dict; report["ok"] is the official verdict and
    report["strict_ok"] the stricter gate (only when S is given). sum_rel is
    the gate's accumulation coefficient per unit of S; the default is the fp32
    summation bound 2 sqrt(K+1) 2^-24.
    """
    C = np.asarray(C, dtype=np.float64)
    R = np.asarray(R, dtype=np.float64)
    if C.shape != R.shape:
        raise ValueError("shape mismatch %s vs %s" % (C.shape, R.shape))
    err = np.abs(C - R)
    finite = bool(np.all(np.isfinite(C)))
    tol = atol_k(K) + RTOL * np.abs(R)
    rf = rel_frobenius(C, R) if C.size else 0.0
    rep = {
        "n": int(C.size),
        "finite": finite,
        "rel_frobenius": rf,
        "max_abs": float(err.max()) if C.size else 0.0,
        "elem_violations": int(np.count_nonzero(err > tol)),
        "max_ulp": float((err / ulp_out(R, dtype)).max()) if C.size else 0.0,
    }
    rep["ok"] = finite and rf <= REL_FRO_TOL and rep["elem_violations"] == 0
    if S is not None:
        L = ACT_LIPSCHITZ[int(act)]
        rel = 2.0 * math.sqrt(K + 1) * 2.0 ** -24 if sum_rel is None else sum_rel
        strict = ulp_out(R, dtype) + L * rel * np.asarray(S) + 2.0 ** -20
        bad = err > strict
        rep["strict_violations"] = int(np.count_nonzero(bad))
        if rep["strict_violations"]:
            idx = np.unravel_index(np.argmax(err - strict), err.shape)
            rep["worst"] = {"index": [int(i) for i in idx], "got": float(C[idx]),
                            "want": float(R[idx]), "bound": float(strict[idx])}
        rep["strict_ok"] = finite and rep["strict_violations"] == 0
    return rep
