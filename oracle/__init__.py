"""CPU oracle for C = act(A.B + bias) -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The HIP library never links, loads or
calls it, and it imports nothing from the HIP library's package.

The arithmetic lives in ``gemm_oracle.c`` (plain C, fp64): an i-k-j triple loop
with its own fp16/bf16 decoders and round-to-nearest-even encoders, followed by
the bias add and the activation written out from their definitions. See that
file's header for the pages and sections each step follows:
  - GEMM: "writing-tilelang-kernels", Kernel Anatomy / Step-by-Step Workflow
    (reference program A @ B, fp16 in, float accumulate).
  - Epilogue: "TileLang: Write, Autotune, and Ship Fused Tensor-Core Kernels
    from Python", Why tile-level control matters (bias add + GELU on the
    accumulator); ReLU / sigmoid from "writing-tilelang-kernels", Pre-flight
    Checklist and Key API Patterns; softplus from the same page's Elementwise
    (2D) template; the tanh form of GELU (Hendrycks and Gimpel, 2016).
  - transpose_B (same page, Key API Patterns): the second operand stored (N, K)
    and used as its transpose (``transpose_b=True``).
  - 8-bit inputs ("tilelang" (skillsmp.com), Documentation Structure: the type
    system lists float8_e4m3/e5m2, the GEMM examples an FP8 GEMM): OCP E4M3 /
    E5M2 A and (N, K) W, one fp32 scale on the product, fp16/bf16 bias and
    result (``gemm_bias_act_fp8``).

Every function here is pinned by ``tests/test_oracle_pins.py`` against facts
that do not come from the oracle itself (closed forms, exact rational brute
force, independent libraries, table values under ``tests/golden/``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gemm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F16, BF16 = 0, 1
ACT_NONE, ACT_RELU, ACT_SIGMOID, ACT_GELU, ACT_SOFTPLUS, ACT_GELU_TANH = 0, 1, 2, 3, 4, 5
ACTS = {"none": ACT_NONE, "relu": ACT_RELU, "sigmoid": ACT_SIGMOID, "gelu": ACT_GELU,
        "softplus": ACT_SOFTPLUS, "gelu_tanh": ACT_GELU_TANH}
DTYPES = {"f16": F16, "fp16": F16, "float16": F16, "bf16": BF16, "bfloat16": BF16}
FP8 = {"e4m3": 0, "e5m2": 1}


def build(force: bool = False, src: str = _SRC, out: str = _LIB) -> str:
    """Compile gemm_oracle.c with gcc (no fast-math: IEEE fp64 throughout)."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O3", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
             "-pthread", "-o", tmp, src, "-lm"])
        os.replace(tmp, out)
    return out


def _dt(dtype) -> int:
    return DTYPES[dtype] if isinstance(dtype, str) else int(dtype)


def _act(act) -> int:
    return ACTS[act] if isinstance(act, str) else int(act)


def _bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x)
    if x.dtype == np.float16:
        x = x.view(np.uint16)
    if x.dtype != np.uint16:
        raise TypeError("oracle inputs are fp16/bf16 bit patterns (uint16), got %s" % x.dtype)
    return x


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """The oracle's entry points bound to one compiled copy of gemm_oracle.c."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        ci = ctypes.c_int
        for name in ("oracle_gemm_bias_act", "oracle_gemm_bias_act_nt"):
            getattr(lib, name).argtypes = [p, p, p, p, p, i64, i64, i64, ci, ci, p, i64, ci]
            getattr(lib, name).restype = ci
        lib.oracle_gemm_bias_act_ex.argtypes = [p, p, p, p, p, i64, i64, i64, ci, ci, ci, ci, p,
                                                i64, ci]
        lib.oracle_gemm_bias_act_ex.restype = ci
        lib.oracle_gemm_bias_act_fp8_nt.argtypes = [p, p, p, p, p, i64, i64, i64,
                                                    ctypes.c_double, ci, ci, ci, p, i64, ci]
        lib.oracle_gemm_bias_act_fp8_nt.restype = ci
        lib.oracle_decode_fp8.argtypes = [ci, p, p, i64]
        lib.oracle_decode_fp8.restype = None
        lib.oracle_bias_act.argtypes = [p, p, p, i64, i64, ci, ci]
        lib.oracle_bias_act.restype = ci
        for name in ("oracle_decode", "oracle_encode", "oracle_act"):
            getattr(lib, name).argtypes = [ci, p, p, i64]
            getattr(lib, name).restype = None
        self._lib = lib
        self.path = path

    def gemm_bias_act(self, A, B, bias, act="none", dtype="f16", rows=None, nthreads=0,
                      with_abs=False, transpose_b=False, transpose_a=False):
        """fp64 act(A.B + bias) for the given rows (all rows when rows is None).

        A: uint16 bits [M, K], or [K, M] with transpose_a (the product is then
        A^T.B); B: uint16 bits [K, N], or [N, K] with transpose_b (the product
        is then A.B^T); bias: uint16 bits [N] or None.
        Returns out[len(rows) or M, N] float64, plus sum_k |A_ik B_kj| + |bias_j|
        when with_abs is set.
        """
        A, B = _bits(A), _bits(B)
        M, K = A.shape[::-1] if transpose_a else A.shape
        N, K2 = B.shape if transpose_b else B.shape[::-1]
        if K2 != K:
            raise ValueError("inner dimensions differ: A is %s, B is %s" % (A.shape, B.shape))
        if bias is not None:
            bias = _bits(bias)
            if bias.shape != (N,):
                raise ValueError("bias must have N=%d entries, got %s" % (N, bias.shape))
        r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
        nrows = M if r is None else r.shape[0]
        out = np.empty((nrows, N), dtype=np.float64)
        absout = np.empty((nrows, N), dtype=np.float64) if with_abs else None
        if transpose_a:
            rc = self._lib.oracle_gemm_bias_act_ex(
                _ptr(A), _ptr(B), _ptr(bias), _ptr(out), _ptr(absout), M, N, K, _act(act),
                _dt(dtype), 1, int(bool(transpose_b)), _ptr(r), 0 if r is None else nrows,
                int(nthreads))
        else:
            fn = self._lib.oracle_gemm_bias_act_nt if transpose_b else self._lib.oracle_gemm_bias_act
            rc = fn(_ptr(A), _ptr(B), _ptr(bias), _ptr(out), _ptr(absout), M, N, K, _act(act),
                    _dt(dtype), _ptr(r), 0 if r is None else nrows, int(nthreads))
        if rc != 0:
            raise ValueError("oracle_gemm_bias_act rejected its arguments")
        return (out, absout) if with_abs else out

    def gemm_bias_act_fp8(self, A, W, bias, scale=1.0, act="none", fmt="e4m3", dtype="bf16",
                          rows=None, nthreads=0, with_abs=False):
        """fp64 act(scale * A.W^T + bias) with 8-bit inputs.

        A: uint8 bits [M, K], W: uint8 bits [N, K], both in format fmt ("e4m3" or
        "e5m2"); bias: uint16 bits [N] of dtype, or None; scale: the fp32
        dequantization factor of the product. Returns out[len(rows) or M, N]
        float64 (plus |scale| sum_k |A_ik W_jk| + |bias_j| with with_abs).
        """
        A = np.ascontiguousarray(A)
        W = np.ascontiguousarray(W)
        if A.dtype != np.uint8 or W.dtype != np.uint8:
            raise TypeError("8-bit inputs are uint8 bit patterns")
        M, K = A.shape
        N, K2 = W.shape
        if K2 != K:
            raise ValueError("inner dimensions differ: A is %s, W is %s" % (A.shape, W.shape))
        if bias is not None:
            bias = _bits(bias)
            if bias.shape != (N,):
                raise ValueError("bias must have N=%d entries, got %s" % (N, bias.shape))
        r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
        nrows = M if r is None else r.shape[0]
        out = np.empty((nrows, N), dtype=np.float64)
        absout = np.empty((nrows, N), dtype=np.float64) if with_abs else None
        rc = self._lib.oracle_gemm_bias_act_fp8_nt(
            _ptr(A), _ptr(W), _ptr(bias), _ptr(out), _ptr(absout), M, N, K, float(scale),
            _act(act), FP8[fmt] if isinstance(fmt, str) else int(fmt), _dt(dtype), _ptr(r),
            0 if r is None else nrows, int(nthreads))
        if rc != 0:
            raise ValueError("oracle_gemm_bias_act_fp8_nt rejected its arguments")
        return (out, absout) if with_abs else out

    def decode_fp8(self, bits, fmt="e4m3"):
        bits = np.ascontiguousarray(np.asarray(bits, dtype=np.uint8))
        flat = bits.reshape(-1)
        out = np.empty(flat.shape, dtype=np.float64)
        self._lib.oracle_decode_fp8(FP8[fmt] if isinstance(fmt, str) else int(fmt), _ptr(flat),
                                    _ptr(out), flat.size)
        return out.reshape(bits.shape)

    def bias_act(self, X, bias, act="none", dtype="f16"):
        """fp64 act(X + bias) elementwise; X uint16 bits [M, N], bias [N] or None."""
        X = _bits(X)
        M, N = X.shape
        if bias is not None:
            bias = _bits(bias)
            if bias.shape != (N,):
                raise ValueError("bias must have N entries")
        out = np.empty((M, N), dtype=np.float64)
        rc = self._lib.oracle_bias_act(_ptr(X), _ptr(bias), _ptr(out), M, N, _act(act),
                                       _dt(dtype))
        if rc != 0:
            raise ValueError("oracle_bias_act rejected its arguments")
        return out

    def decode(self, bits, dtype="f16"):
        bits = _bits(np.asarray(bits))
        flat = np.ascontiguousarray(bits.reshape(-1))
        out = np.empty(flat.shape, dtype=np.float64)
        self._lib.oracle_decode(_dt(dtype), _ptr(flat), _ptr(out), flat.size)
        return out.reshape(bits.shape)

    def encode(self, x, dtype="f16"):
        """Round fp64 values to fp16/bf16 bit patterns, nearest-even."""
        x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
        flat = x.reshape(-1)
        out = np.empty(flat.shape, dtype=np.uint16)
        self._lib.oracle_encode(_dt(dtype), _ptr(flat), _ptr(out), flat.size)
        return out.reshape(x.shape)

    def act(self, z, act="none"):
        z = np.ascontiguousarray(np.asarray(z, dtype=np.float64))
        flat = z.reshape(-1)
        out = np.empty(flat.shape, dtype=np.float64)
        self._lib.oracle_act(_act(act), _ptr(flat), _ptr(out), flat.size)
        return out.reshape(z.shape)


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(_LIB):
            build()
        _default = Oracle(_LIB)
    return _default


def gemm_bias_act(*args, **kw):
    return default().gemm_bias_act(*args, **kw)


def bias_act(*args, **kw):
    return default().bias_act(*args, **kw)


def gemm_bias_act_fp8(*args, **kw):
    return default().gemm_bias_act_fp8(*args, **kw)


def decode_fp8(*args, **kw):
    return default().decode_fp8(*args, **kw)


def decode(*args, **kw):
    return default().decode(*args, **kw)


def encode(*args, **kw):
    return default().encode(*args, **kw)


def act(*args, **kw):
    return default().act(*args, **kw)
