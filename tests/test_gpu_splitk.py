"""Split-K path (gemm_bias_act_ex with a workspace) against the fp64 oracle,
through the C ABI.

Shapes whose tiles leave compute units idle split K: fp32 partial sums of K
ranges go to the workspace and a second kernel adds them in split order, then
applies bias, act and the rounding. Bars: bitwise on exact-integer inputs (and
equal to the one-kernel path there), the oracle's tolerance plus the strict
accumulation gate on random inputs, ragged shapes and K tails, both B layouts.
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def workspace(M, N, K, act, dtype, transpose_b=False, extra=0):
    import torch
    nb = gba.workspace_size(M, N, K, act, dtype, transpose_b=transpose_b)
    return nb, torch.empty(max(nb + extra, 16), dtype=torch.uint8, device="cuda")


def run(A, B, bias, act, dtype, transpose_b=False, ws=None):
    import torch
    M = A.shape[0]
    N = B.shape[0] if transpose_b else B.shape[1]
    c = empty((M, N), dtype, fill_bits=0x7E00)
    gba.gemm_bias_act(to_dev(A, dtype), to_dev(B, dtype), to_dev(bias, dtype), c, act,
                      transpose_b=transpose_b, workspace=ws)
    torch.cuda.synchronize()
    return to_bits(c)


def int_inputs(M, N, K, dtype, seed, transpose_b):
    rng = np.random.default_rng(seed)
    enc = (lambda v: v.astype(np.float16).view(np.uint16)) if dtype == "f16" else \
        (lambda v: synth.to_bits(v.astype(np.float32), "bf16"))
    A = enc(rng.integers(-1, 2, (M, K)).astype(np.float64))
    B = enc(rng.integers(-1, 2, (N, K) if transpose_b else (K, N)).astype(np.float64))
    bias = enc(rng.integers(-8, 9, N).astype(np.float64))
    return A, B, bias


# Deep K with few output tiles: the shapes the split is for (ragged M, N and K tails).
SPLIT_SHAPES = [(256, 256, 4096), (300, 264, 8008), (129, 136, 4104), (520, 776, 6000),
                (64, 1024, 6144)]


@pytest.mark.parametrize("transpose_b", [False, True], ids=["kn", "nk"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_exact_integer_bitwise_and_equal_to_one_kernel(shape, dtype, transpose_b):
    M, N, K = shape
    A, B, bias = int_inputs(M, N, K, dtype, M + N + K, transpose_b)
    nb, ws = workspace(M, N, K, "relu", dtype, transpose_b)
    assert nb > 0, "this shape is expected to split"
    want = oracle.encode(oracle.gemm_bias_act(A, B, bias, "relu", dtype, transpose_b=transpose_b,
                                              nthreads=16), dtype)
    say("splitk exact", shape, dtype, transpose_b, nb)
    got = run(A, B, bias, "relu", dtype, transpose_b, ws)
    bad = np.argwhere(got != want)
    assert bad.size == 0, "%d mismatches, first %s" % (len(bad), bad[:3].tolist())
    assert np.array_equal(got, run(A, B, bias, "relu", dtype, transpose_b))


@pytest.mark.parametrize("act", ACTS)
def test_random_every_act(act):
    M, N, K = 300, 264, 4000
    A = synth.random_bits((M, K), "bf16", 1)
    B = synth.random_bits((K, N), "bf16", 2, scale=0.25)
    bias = synth.random_bits((N,), "bf16", 3)
    _, ws = workspace(M, N, K, act, "bf16")
    say("splitk random", act)
    got = run(A, B, bias, act, "bf16", ws=ws)
    R, S = oracle.gemm_bias_act(A, B, bias, act, "bf16", with_abs=True)
    rep = compare.check(oracle.decode(got, "bf16"), R, K=K, dtype="bf16", act=oracle.ACTS[act], S=S)
    assert rep["ok"] and rep["strict_ok"], rep


@pytest.mark.parametrize("name", ["c2_plain", "c5_gelu"])
def test_deep_k_variants_of_the_workloads(name):
    # the workload's distributions at a split-K shape: few rows and columns, its K x 4
    w = synth.WORKLOADS[name]
    w = synth.Workload(w.name, 256, 384, 4 * w.K, w.dtype, w.act, w.bias, w.seed, w.a_dist,
                       w.a_std, w.b_dist, w.b_std, w.bias_dist, w.bias_std)
    A, B, bias = synth.make_inputs(w)
    nb, ws = workspace(w.M, w.N, w.K, w.act, w.dtype)
    assert nb > 0
    say("splitk workload", name, nb)
    got = run(A, B, bias, w.act, w.dtype, ws=ws)
    R, S = oracle.gemm_bias_act(A, B, bias, w.act, w.dtype, with_abs=True)
    rep = compare.check(oracle.decode(got, w.dtype), R, K=w.K, dtype=w.dtype,
                        act=oracle.ACTS[w.act], S=S)
    assert rep["ok"] and rep["strict_ok"], rep
    # determinism: the partials are added in split order
    assert np.array_equal(got, run(A, B, bias, w.act, w.dtype, ws=ws))


def test_small_workspace_falls_back_and_large_shapes_do_not_split():
    import torch
    M, N, K = 256, 256, 4096
    A, B, bias = int_inputs(M, N, K, "f16", 7, False)
    nb = gba.workspace_size(M, N, K, "gelu", "f16")
    assert nb > 0
    small = torch.empty(nb // 2, dtype=torch.uint8, device="cuda")
    say("splitk fallback")
    got = run(A, B, bias, "relu", "f16", ws=small)
    assert np.array_equal(got, run(A, B, bias, "relu", "f16"))
    assert gba.workspace_size(4096, 4096, 4096, "gelu", "f16") == 0
    assert gba.workspace_size(1024, 1024, 1024, "gelu", "f16") == 0   # the split would not pay
    assert gba.workspace_size(256, 256, 256, "gelu", "f16") == 0
    assert gba.workspace_size(1024, 1024, 64, "gelu", "f16") == 0     # too few K slices
    assert gba.workspace_size(0, 1024, 1024, "gelu", "f16") == 0


@pytest.mark.parametrize("shape,tile,split", [
    ((128, 4096, 14336), 128, True),    # 64x64 whole 60 us, 128x128 in 8 splits 31 us
    ((256, 256, 4096), 64, True),       # 64x64 split beats 128x128 split
    ((520, 776, 3000), 64, False),      # 64x64 whole beats either split
    ((4096, 4096, 4096), 256, False)])
def test_split_plan_agrees_with_workspace_size(shape, tile, split):
    M, N, K = shape
    s, S = gba.split_plan(M, N, K, "gelu", "bf16")
    nb = gba.workspace_size(M, N, K, "gelu", "bf16")
    assert (S > 1) == split and s["bm"] == tile
    assert nb == (S * M * N * 4 if S > 1 else 0)
    if S == 1:
        assert s == gba.get_schedule(M, N, K, "gelu", "bf16")
    say("split plan", shape, s["bm"], S)


def test_workspace_argument_errors():
    import torch
    a = torch.zeros(64, 64, dtype=torch.float16, device="cuda")
    c = torch.zeros(64, 64, dtype=torch.float16, device="cuda")
    with pytest.raises(gba.GbaError) as e:   # workspace overlapping C
        gba.gemm_bias_act(a, a, None, c, "none", workspace=c.view(torch.uint8).view(-1))
    assert e.value.status == 6
    with pytest.raises(gba.GbaError) as e:   # misaligned workspace
        ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
        gba.gemm_bias_act(a, a, None, c, "none", workspace=ws[8:])
    assert e.value.status == 5
