"""8-bit-input path (gemm_bias_act_fp8_nt: A [M,K] and W [N,K] in OCP E4M3 or
E5M2, fp32 scale, fp16/bf16 bias and C) against the fp64 oracle, through the C
ABI.

Bars: bitwise on exact-integer inputs (every partial sum exact, power-of-two
scale) over ragged shapes and K tails, both formats, both output types; the
oracle's tolerance on random inputs at reduced and (64 sampled rows) full
workload sizes, plus an accumulation-aware gate sized for the 8-bit matrix
instruction (compare.fp8_sum_rel: the worst case of fp32 summation in any order
inside each 16x16x128 instruction, then in order across them).
"""
import numpy as np
import pytest

import oracle
from oracle import compare
import synth
import tiled_dense_gemm_bias_amd as gba
from tests.gpu_util import empty, say, to_bits

pytestmark = pytest.mark.gpu

ACTS = ["none", "relu", "sigmoid", "gelu", "softplus", "gelu_tanh"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dev8(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits)).to("cuda:0")


def dev16(bits, dtype):
    from tests.gpu_util import to_dev
    return to_dev(bits, dtype)


def run_fp8(A, W, bias, scale, act, fmt, dtype):
    import torch
    M, N = A.shape[0], W.shape[0]
    c = empty((M, N), dtype, fill_bits=0x7E00)   # NaN sentinel: every element must be written
    gba.gemm_bias_act_fp8(dev8(A), dev8(W), dev16(bias, dtype), c, scale, act, fmt)
    torch.cuda.synchronize()
    return to_bits(c)


def enc8(v, fmt):
    return synth.f32_to_fp8_bits(np.asarray(v, dtype=np.float32), fmt)


def int_inputs(M, N, K, fmt, dtype, seed):
    rng = np.random.default_rng(seed)
    A = enc8(rng.integers(-4, 5, (M, K)), fmt)
    W = enc8(rng.integers(-4, 5, (N, K)), fmt)
    bias = synth.to_bits(rng.integers(-8, 9, N).astype(np.float32), dtype)
    return A, W, bias


def check(A, W, bias, scale, act, fmt, dtype, got, rows=None, report=None):
    R, S = oracle.gemm_bias_act_fp8(A, W, bias, scale, act, fmt, dtype, rows=rows,
                                    with_abs=True, nthreads=16)
    C = oracle.decode(got if rows is None else got[rows], dtype)
    rep = compare.check(C, R, K=A.shape[1], dtype=dtype, act=oracle.ACTS[act], S=S,
                        sum_rel=compare.fp8_sum_rel(A.shape[1]))
    err = np.abs(C - R)
    rel = float((np.maximum(err - compare.ulp_out(R, dtype), 0) / np.maximum(S, 1e-30)).max())
    say("fp8 max (|C-R| - ulp) / S = %.3g" % rel, "rel_fro %.3g" % rep["rel_frobenius"])
    if report is not None:
        report.append(rel)
    assert rep["ok"] and rep["strict_ok"], rep
    return rep


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(256, 256, 256), (1, 8, 16), (37, 40, 48), (129, 136, 144),
                                   (300, 264, 1008), (520, 776, 128), (4100, 4200, 400)],
                         ids=lambda s: "x".join(map(str, s)))
def test_exact_integer_bitwise(shape, dtype, fmt):
    M, N, K = shape
    A, W, bias = int_inputs(M, N, K, fmt, dtype, seed=M + 3 * N + K)
    want = oracle.encode(oracle.gemm_bias_act_fp8(A, W, bias, 0.5, "relu", fmt, dtype,
                                                  nthreads=16), dtype)
    say("fp8 exact", shape, dtype, fmt)
    got = run_fp8(A, W, bias, 0.5, "relu", fmt, dtype)
    bad = np.argwhere(got != want)
    assert bad.size == 0, "%d mismatches, first %s" % (len(bad), bad[:3].tolist())


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("act", ACTS)
def test_random_every_act(act, fmt):
    w = synth.Fp8Workload("t", 300, 264, 1008, fmt, "bf16", act, True, 11)
    A, W, bias, scale = synth.make_inputs_fp8(w)
    say("fp8 random", act, fmt)
    got = run_fp8(A, W, bias, scale, act, fmt, "bf16")
    check(A, W, bias, scale, act, fmt, "bf16", got)


@pytest.mark.parametrize("name", ["c3_fp8", "c5_fp8"])
def test_full_size_sampled_rows(name):
    w = synth.FP8_WORKLOADS[name]
    A, W, bias, scale = synth.make_inputs_fp8(w)
    rows = synth.sample_rows(w.M, 64, seed=w.seed)
    say("fp8 full", name)
    got = run_fp8(A, W, bias, scale, w.act, w.fmt, w.dtype)
    check(A, W, bias, scale, w.act, w.fmt, w.dtype, got, rows=rows)
    expmask = 0x7C00 if w.dtype == "f16" else 0x7F80
    assert not np.any((got & expmask) == expmask)


def test_reduced_sizes_no_bias_and_short_k():
    for (M, N, K) in [(512, 768, 4096), (65, 72, 16), (257, 264, 272)]:
        w = synth.Fp8Workload("t", M, N, K, "e4m3", "f16", "gelu", False, 5)
        A, W, bias, scale = synth.make_inputs_fp8(w)
        say("fp8 reduced", M, N, K)
        check(A, W, None, scale, "gelu", "e4m3", "f16", run_fp8(A, W, None, scale, "gelu",
                                                                  "e4m3", "f16"))


def test_degenerate_shapes_and_determinism():
    import torch
    bias = synth.random_bits((16,), "f16", 5)
    for act in ("none", "gelu"):
        say("fp8 k0", act)
        got = run_fp8(np.zeros((5, 0), np.uint8), np.zeros((16, 0), np.uint8), bias, 1.0, act,
                      "e4m3", "f16")
        want = oracle.encode(np.broadcast_to(oracle.act(oracle.decode(bias), act), (5, 16)), "f16")
        assert np.array_equal(got, want), act
    c = torch.zeros(0, 16, dtype=torch.float16, device="cuda")
    gba.gemm_bias_act_fp8(dev8(np.zeros((0, 32), np.uint8)), dev8(np.zeros((16, 32), np.uint8)),
                          None, c, 1.0, "gelu", "e4m3")
    w = synth.FP8_WORKLOADS["c3_fp8"]
    A, W, b, s = synth.make_inputs_fp8(w, M=1000, N=1024, K=512)
    say("fp8 determinism")
    r1 = run_fp8(A, W, b, s, "gelu", "e4m3", "f16")
    r2 = run_fp8(A, W, b, s, "gelu", "e4m3", "f16")
    assert np.array_equal(r1, r2)


def test_float8_tensors_and_argument_errors():
    import torch
    M, N, K = 64, 64, 64
    A, W, bias = int_inputs(M, N, K, "e4m3", "f16", seed=3)
    a = dev8(A).view(torch.float8_e4m3fn)
    w = dev8(W).view(torch.float8_e4m3fn)
    c = empty((M, N), "f16")
    say("fp8 torch dtypes")
    gba.gemm_bias_act_fp8(a, w, dev16(bias, "f16"), c, 0.5, "relu")
    torch.cuda.synchronize()
    want = oracle.encode(oracle.gemm_bias_act_fp8(A, W, bias, 0.5, "relu", "e4m3", "f16"), "f16")
    assert np.array_equal(to_bits(c), want)
    with pytest.raises(gba.GbaError) as e:   # K not a multiple of 16
        gba.gemm_bias_act_fp8(dev8(np.zeros((8, 24), np.uint8)), dev8(np.zeros((8, 24), np.uint8)),
                              None, empty((8, 8), "f16"), 1.0, "none", "e4m3")
    assert e.value.status == 5
    with pytest.raises(gba.GbaError) as e:   # non-finite scale
        gba.gemm_bias_act_fp8(a, w, None, c, float("nan"), "none")
    assert e.value.status == 2


FP8_SPLIT_SHAPES = [(128, 1024, 8192), (200, 520, 4112), (300, 264, 2064)]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("shape", FP8_SPLIT_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_split_k_exact_integer_bitwise(shape, fmt):
    import torch
    M, N, K = shape
    A, W, bias = int_inputs(M, N, K, fmt, "bf16", seed=M + N + K)
    nb = gba.workspace_size(M, N, K, "relu", "bf16", fp8=True)
    assert nb > 0, "this shape is expected to split"
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    want = oracle.encode(oracle.gemm_bias_act_fp8(A, W, bias, 0.5, "relu", fmt, "bf16",
                                                  nthreads=16), "bf16")
    c = empty((M, N), "bf16", fill_bits=0x7E00)
    say("fp8 split exact", shape, fmt, nb)
    gba.gemm_bias_act_fp8(dev8(A), dev8(W), dev16(bias, "bf16"), c, 0.5, "relu", fmt, workspace=ws)
    torch.cuda.synchronize()
    got = to_bits(c)
    bad = np.argwhere(got != want)
    assert bad.size == 0, "%d mismatches, first %s" % (len(bad), bad[:3].tolist())
    assert np.array_equal(got, run_fp8(A, W, bias, 0.5, "relu", fmt, "bf16"))


@pytest.mark.parametrize("act", ["none", "gelu", "softplus"])
def test_split_k_random(act):
    import torch
    w = synth.Fp8Workload("t", 128, 1024, 8192, "e4m3", "bf16", act, True, 12,
                          b_std=1 / np.sqrt(8192), bias_std=np.sqrt(0.02))
    A, W, bias, scale = synth.make_inputs_fp8(w)
    nb = gba.workspace_size(w.M, w.N, w.K, act, "bf16", fp8=True)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    c = empty((w.M, w.N), "bf16", fill_bits=0x7E00)
    say("fp8 split random", act)
    gba.gemm_bias_act_fp8(dev8(A), dev8(W), dev16(bias, "bf16"), c, scale, act, "e4m3",
                          workspace=ws)
    torch.cuda.synchronize()
    check(A, W, bias, scale, act, "e4m3", "bf16", to_bits(c))
    assert gba.workspace_size(4096, 4096, 4096, "gelu", "f16", fp8=True) == 0
