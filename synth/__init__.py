"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and rounds them to fp16/bf16 (or OCP
8-bit float) bit patterns. It holds none of the GEMM or epilogue arithmetic, and it is the only
code that both the HIP path's callers and the oracle's callers use.

Recipe (one numpy PCG64 generator per workload, seeded from the workload):
  1. draw A, then B, then bias, in that order, as float32;
     N(0, v) means variance v (so std sqrt(v)); U(-1, 1) is uniform on [-1, 1);
  2. scale in float32;
  3. round to the storage type with round-to-nearest-even (numpy's float16
     cast for fp16; the top-16-bit RNE rule for bf16). 8-bit inputs are first
     divided by a per-tensor scale amax / (largest finite value), then rounded
     by torch's float8 conversion (nearest-even, saturated); the product of the
     two scales is the GEMM's dequantization factor.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def _draw(rng: np.random.Generator, shape, dist: str, scale: float) -> np.ndarray:
    if dist == "normal":
        x = rng.standard_normal(shape, dtype=np.float32)
    elif dist == "uniform":
        x = rng.random(shape, dtype=np.float32) * np.float32(2.0) - np.float32(1.0)
    else:
        raise ValueError(dist)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dtype: str              # "f16" | "bf16"
    act: str                # "none" | "relu" | "sigmoid" | "gelu"
    bias: bool
    seed: int
    a_dist: str = "normal"
    a_std: float = 1.0
    b_dist: str = "normal"
    b_std: float = 1.0
    bias_dist: str = "normal"
    bias_std: float = 1.0

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    def with_act(self, act: str) -> "Workload":
        return dataclasses.replace(self, act=act)


# The five workloads: shapes, dtypes, distributions and epilogues as stated for
# this library's validation and benchmark set.
WORKLOADS = {
    # 256^3 fp16, A,B ~ N(0,1); plain GEMM, then bias ~ N(0,1) + erf-GELU.
    "c1_plain": Workload("c1_plain", 256, 256, 256, "f16", "none", False, 1),
    "c1_gelu": Workload("c1_gelu", 256, 256, 256, "f16", "gelu", True, 1),
    # 1024^3 fp16 ~ N(0,1), no epilogue (the pages' demo GEMM shape).
    "c2_plain": Workload("c2_plain", 1024, 1024, 1024, "f16", "none", False, 2),
    # 4096^3 fp16 ~ N(0,1)/sqrt(2), bias ~ N(0,1), erf-GELU: the headline workload.
    "c3_gelu": Workload("c3_gelu", 4096, 4096, 4096, "f16", "gelu", True, 3,
                        a_std=1 / math.sqrt(2), b_std=1 / math.sqrt(2)),
    # Ragged 3000x5120x1000 fp16 ~ U(-1,1), bias ~ U(-1,1), ReLU and sigmoid.
    "c4_relu": Workload("c4_relu", 3000, 5120, 1000, "f16", "relu", True, 4,
                        a_dist="uniform", b_dist="uniform", bias_dist="uniform"),
    "c4_sigmoid": Workload("c4_sigmoid", 3000, 5120, 1000, "f16", "sigmoid", True, 4,
                           a_dist="uniform", b_dist="uniform", bias_dist="uniform"),
    # LLM-MLP shape, bf16: A ~ N(0,1), B ~ N(0,1/K), bias ~ N(0,0.02), erf-GELU.
    "c5_gelu": Workload("c5_gelu", 16384, 14336, 4096, "bf16", "gelu", True, 5,
                        b_std=1 / math.sqrt(4096), bias_std=math.sqrt(0.02)),
    # The same MLP's down projection for a batch of 128 tokens: few output tiles,
    # deep K (the split-K case); C5's distributions with K = 14336, bias, no act.
    "mlp_down_m128": Workload("mlp_down_m128", 128, 4096, 14336, "bf16", "none", True, 6,
                              b_std=1 / math.sqrt(14336), bias_std=math.sqrt(0.02)),
}


FP8_MAX = {"e4m3": 448.0, "e5m2": 57344.0}


def f32_to_fp8_bits(x: np.ndarray, fmt: str) -> np.ndarray:
    """float32 -> OCP 8-bit float bit patterns (torch's conversion: nearest, ties
    to even), saturated to the format's largest finite value first."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.clamp(-FP8_MAX[fmt], FP8_MAX[fmt])
    tdt = torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2
    return t.to(tdt).view(torch.uint8).numpy()


@dataclasses.dataclass(frozen=True)
class Fp8Workload:
    """A GEMM with 8-bit inputs: A [M,K] and W [N,K] in format fmt, each scaled
    per tensor onto the format's range (s = amax / largest finite value), bias
    and output in dtype; the product's dequantization factor is sA * sW."""
    name: str
    M: int
    N: int
    K: int
    fmt: str                # "e4m3" | "e5m2"
    dtype: str              # bias / output: "f16" | "bf16"
    act: str
    bias: bool
    seed: int
    a_std: float = 1.0
    b_std: float = 1.0
    bias_std: float = 1.0

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


# The 4096^3 and LLM-MLP workloads with E4M3 inputs (same draws as the 16-bit ones).
FP8_WORKLOADS = {
    "c3_fp8": Fp8Workload("c3_fp8", 4096, 4096, 4096, "e4m3", "f16", "gelu", True, 3,
                          a_std=1 / math.sqrt(2), b_std=1 / math.sqrt(2)),
    "c5_fp8": Fp8Workload("c5_fp8", 16384, 14336, 4096, "e4m3", "bf16", "gelu", True, 5,
                          b_std=1 / math.sqrt(4096), bias_std=math.sqrt(0.02)),
    # mlp_down_m128 with E4M3 inputs (the 8-bit split-K case).
    "mlp_down_m128_fp8": Fp8Workload("mlp_down_m128_fp8", 128, 4096, 14336, "e4m3", "bf16",
                                     "none", True, 6, b_std=1 / math.sqrt(14336),
                                     bias_std=math.sqrt(0.02)),
}


def make_inputs_fp8(w: Fp8Workload, M: Optional[int] = None, N: Optional[int] = None,
                    K: Optional[int] = None):
    """Return (A, W, bias, scale): A uint8 [M,K], W uint8 [N,K] (format w.fmt), bias
    uint16 [N] or None, scale the float32 product of the two per-tensor scales.
    Draw order A, W, bias from one generator seeded by the workload."""
    M = w.M if M is None else M
    N = w.N if N is None else N
    K = w.K if K is None else K
    rng = np.random.default_rng(w.seed)
    a = _draw(rng, (M, K), "normal", w.a_std)
    b = _draw(rng, (N, K), "normal", w.b_std)
    bias = to_bits(_draw(rng, (N,), "normal", w.bias_std), w.dtype) if w.bias else None
    fmax = np.float32(FP8_MAX[w.fmt])
    sa = np.float32(max(float(np.abs(a).max()), 1e-30)) / fmax
    sb = np.float32(max(float(np.abs(b).max()), 1e-30)) / fmax
    A = f32_to_fp8_bits(a / sa, w.fmt)
    W = f32_to_fp8_bits(b / sb, w.fmt)
    return A, W, bias, float(np.float32(sa * sb))


def make_inputs(w: Workload, M: Optional[int] = None, N: Optional[int] = None,
                K: Optional[int] = None):
    """Return (A, B, bias) as uint16 bit arrays; bias is None when w.bias is False.

    M/N/K override the workload's sizes (same distributions, same seed) for
    reduced-size parity cases.
    """
    M = w.M if M is None else M
    N = w.N if N is None else N
    K = w.K if K is None else K
    rng = np.random.default_rng(w.seed)
    A = to_bits(_draw(rng, (M, K), w.a_dist, w.a_std), w.dtype)
    B = to_bits(_draw(rng, (K, N), w.b_dist, w.b_std), w.dtype)
    bias = to_bits(_draw(rng, (N,), w.bias_dist, w.bias_std), w.dtype) if w.bias else None
    return A, B, bias


def random_bits(shape, dtype: str, seed: int, dist: str = "normal", scale: float = 1.0):
    rng = np.random.default_rng(seed)
    return to_bits(_draw(rng, shape, dist, scale), dtype)


def sample_rows(M: int, n: int = 64, seed: int = 0) -> np.ndarray:
    """n distinct rows in [0, M), always holding 0 and M-1, sorted."""
    if M <= n:
        return np.arange(M, dtype=np.int64)
    rng = np.random.default_rng(10_000 + seed)
    picked = set([0, M - 1])
    cand = rng.permutation(np.arange(1, M - 1))
    for c in cand:
        if len(picked) >= n:
            break
        picked.add(int(c))
    return np.array(sorted(picked), dtype=np.int64)
