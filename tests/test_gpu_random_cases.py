"""Seeded random cases across the whole call surface, against the fp64 oracle.

Each case draws its own shape (ragged M, N and K multiples of 8; a third of
them deep enough in K to split), activation, dtype, operand layouts
(transpose_A / transpose_B), bias or none, a split-K workspace or none, and
in 3 of 10 cases a forced schedule from the compiled-in table (skipped when
that kernel has no path for the layouts). Bar: the oracle's tolerance and the
strict accumulation gate on 48 sampled rows (always rows 0 and M-1), a NaN
sentinel in C that every element must overwrite, and a guard region past C
that must keep it. The 8-bit entry point
gets its own cases (format, output dtype, activation, bias, workspace). The
case lists are fixed by their seeds, so a failure names a reproducible case.
"""
import numpy as np
import pytest

import oracle
from oracle import compare
import synth
import tiled_dense_gemm_bias_amd as gba
from tests.gpu_util import empty, say, to_bits, to_dev

pytestmark = pytest.mark.gpu

ACTS = ["none", "relu", "sigmoid", "gelu", "softplus", "gelu_tanh"]
N_CASES = 96


def _cases():
    rng = np.random.default_rng(2024)
    out = []
    for i in range(N_CASES):
        ta = bool(rng.random() < 0.25)
        tb = bool(rng.random() < 0.4)
        M = int(rng.integers(1, 1500))
        if ta:
            M = max(8, M // 8 * 8)
        N = int(rng.integers(1, 190)) * 8
        K = int(rng.integers(1, 750)) * 8
        if rng.random() < 0.3:
            K = int(rng.integers(500, 2000)) * 8
        out.append(dict(i=i, M=M, N=N, K=K, ta=ta, tb=tb, act=ACTS[int(rng.integers(0, 6))],
                        dtype="f16" if rng.random() < 0.5 else "bf16",
                        ws=bool(rng.random() < 0.5), bias=bool(rng.random() < 0.8),
                        forced=bool(rng.random() < 0.3), pick=int(rng.integers(0, 1 << 30))))
    return out


GUARD = 8192   # elements past C that must keep their fill


def guarded(M, N, dtype):
    """A NaN-filled flat buffer and its leading (M, N) view."""
    flat = empty((M * N + GUARD,), dtype, fill_bits=0x7E00)
    return flat, flat[: M * N].view(M, N)


def check_guard(flat, M, N):
    g = to_bits(flat[M * N:])
    assert bool((g == 0x7E00).all()), "write past the end of C"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    gba.set_schedule(None)


@pytest.mark.parametrize("c", _cases(), ids=lambda c: "case%d" % c["i"])
def test_random_case(c):
    import torch
    M, N, K, dtype, act, ta, tb = c["M"], c["N"], c["K"], c["dtype"], c["act"], c["ta"], c["tb"]
    scheds = gba.list_schedules()
    sched = scheds[c["pick"] % len(scheds)] if c["forced"] else None
    A = synth.random_bits((K, M) if ta else (M, K), dtype, 1000 + c["i"])
    B = synth.random_bits((N, K) if tb else (K, N), dtype, 2000 + c["i"], scale=1.0 / np.sqrt(K))
    bias = synth.random_bits((N,), dtype, 3000 + c["i"]) if c["bias"] else None
    flat, out = guarded(M, N, dtype)
    say("random case", c, sched)
    gba.set_schedule(sched)
    try:
        ws = None
        if c["ws"]:
            nb = gba.workspace_size(M, N, K, act, dtype, transpose_b=tb, transpose_a=ta)
            ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda") if nb else None
        gba.gemm_bias_act(to_dev(A, dtype), to_dev(B, dtype), to_dev(bias, dtype), out, act,
                          transpose_b=tb, transpose_a=ta, workspace=ws)
    except gba.GbaError as e:
        if e.status == 9 and sched is not None:
            pytest.skip("the forced schedule's kernel has no path for these layouts")
        raise
    finally:
        gba.set_schedule(None)
    torch.cuda.synchronize()
    got = to_bits(out)
    rows = synth.sample_rows(M, 48, c["i"])
    R, S = oracle.gemm_bias_act(A, B, bias, act, dtype, rows=rows, with_abs=True,
                                transpose_b=tb, transpose_a=ta, nthreads=16)
    rep = compare.check(oracle.decode(got[rows], dtype), R, K=K, dtype=dtype,
                        act=oracle.ACTS[act], S=S)
    assert rep["ok"] and rep["strict_ok"], rep
    assert not (got == 0x7E00).any(), "an element of C was not written"
    check_guard(flat, M, N)


N_CASES_FP8 = 40


def _cases_fp8():
    rng = np.random.default_rng(2025)
    out = []
    for i in range(N_CASES_FP8):
        M = int(rng.integers(1, 1500))
        N = int(rng.integers(1, 190)) * 8
        K = int(rng.integers(1, 400)) * 16
        if rng.random() < 0.3:
            K = int(rng.integers(400, 1000)) * 16
        out.append(dict(i=i, M=M, N=N, K=K, fmt="e4m3" if rng.random() < 0.5 else "e5m2",
                        dtype="f16" if rng.random() < 0.5 else "bf16",
                        act=ACTS[int(rng.integers(0, 6))], bias=bool(rng.random() < 0.8),
                        ws=bool(rng.random() < 0.5)))
    return out


@pytest.mark.parametrize("c", _cases_fp8(), ids=lambda c: "fp8case%d" % c["i"])
def test_random_case_fp8(c):
    """8-bit inputs (per-tensor scaled onto the format's range), W stored [N,K]:
    the oracle's tolerance and the 8-bit strict gate on 48 sampled rows."""
    import torch
    M, N, K, fmt, dtype, act = c["M"], c["N"], c["K"], c["fmt"], c["dtype"], c["act"]
    w = synth.Fp8Workload("r%d" % c["i"], M, N, K, fmt, dtype, act, c["bias"], 5000 + c["i"])
    A, W, bias, scale = synth.make_inputs_fp8(w)
    flat, out = guarded(M, N, dtype)
    ws = None
    if c["ws"]:
        nb = gba.workspace_size(M, N, K, act, dtype, fp8=True)
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda") if nb else None
    say("random fp8 case", c)
    gba.gemm_bias_act_fp8(torch.from_numpy(A).cuda(), torch.from_numpy(W).cuda(),
                          to_dev(bias, dtype), out, scale, act, fmt, workspace=ws)
    torch.cuda.synchronize()
    got = to_bits(out)
    rows = synth.sample_rows(M, 48, c["i"])
    R, S = oracle.gemm_bias_act_fp8(A, W, bias, scale, act, fmt, dtype, rows=rows,
                                    with_abs=True, nthreads=16)
    rep = compare.check(oracle.decode(got[rows], dtype), R, K=K, dtype=dtype,
                        act=oracle.ACTS[act], S=S, sum_rel=compare.fp8_sum_rel(K))
    assert rep["ok"] and rep["strict_ok"], rep
    assert not (got == 0x7E00).any(), "an element of C was not written"
    check_guard(flat, M, N)
