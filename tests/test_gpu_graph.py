"""The transpose_B, transpose_A, 8-bit and split-K entry points, and the
unfused gemm / bias_act pair, captured into HIP graphs.

None of them allocates, copies, fills or synchronises, so a caller can capture
them. Replays, with eager work and device synchronisation between them and the
captured inputs overwritten, must match eager calls bitwise.
"""
import numpy as np
import pytest

import synth
import tiled_dense_gemm_bias_amd as gba
from tests.gpu_util import empty, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_new_entry_points_replay_like_eager():
    import torch
    # transpose_B, bf16, 520 x 776 x 328
    A1 = [synth.random_bits((520, 328), "bf16", s) for s in (1, 2)]
    W1 = synth.random_bits((776, 328), "bf16", 3)
    b1 = synth.random_bits((776,), "bf16", 4)
    # 8-bit, 600 x 520 x 512
    w8 = synth.Fp8Workload("g", 600, 520, 512, "e4m3", "f16", "gelu", True, 5)
    A8a, W8, b8, sc = synth.make_inputs_fp8(w8)
    A8b = synth.make_inputs_fp8(synth.Fp8Workload("g", 600, 520, 512, "e4m3", "f16", "gelu",
                                                  True, 6))[0]
    # split-K, f16, 256 x 384 x 4096
    A3 = [synth.random_bits((256, 4096), "f16", s) for s in (7, 8)]
    B3 = synth.random_bits((4096, 384), "f16", 9, scale=1 / 64)
    b3 = synth.random_bits((384,), "f16", 10)
    nb = gba.workspace_size(256, 384, 4096, "softplus", "f16")
    assert nb > 0
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")

    a1 = [to_dev(x, "bf16") for x in A1]
    a8 = [torch.from_numpy(x).cuda() for x in (A8a, A8b)]
    a3 = [to_dev(x, "f16") for x in A3]
    w1, bb1 = to_dev(W1, "bf16"), to_dev(b1, "bf16")
    w8, bb8 = torch.from_numpy(W8).cuda(), to_dev(b8, "f16")
    bm3, bb3 = to_dev(B3, "f16"), to_dev(b3, "f16")

    def run_all(x1, x8, x3, c1, c8, c3):
        gba.gemm_bias_act(x1, w1, bb1, c1, "gelu_tanh", transpose_b=True)
        gba.gemm_bias_act_fp8(x8, w8, bb8, c8, sc, "gelu", "e4m3")
        gba.gemm_bias_act(x3, bm3, bb3, c3, "softplus", workspace=ws)

    refs = []
    for i in range(2):
        outs = (empty((520, 776), "bf16"), empty((600, 520), "f16"), empty((256, 384), "f16"))
        run_all(a1[i], a8[i], a3[i], *outs)
        refs.append(outs)
    torch.cuda.synchronize()

    src = (a1[0].clone(), a8[0].clone(), a3[0].clone())
    outs = (empty((520, 776), "bf16"), empty((600, 520), "f16"), empty((256, 384), "f16"))
    graph = torch.cuda.CUDAGraph()
    say("graph capture: transpose_B, 8-bit, split-K")
    with torch.cuda.graph(graph):
        run_all(*src, *outs)
    torch.cuda.synchronize()
    for r in range(4):
        i = r % 2
        src[0].copy_(a1[i])
        src[1].copy_(a8[i])
        src[2].copy_(a3[i])
        for o in outs:
            o.fill_(0.0)
        ws.fill_(255)   # the workspace carries nothing between calls
        say("graph replay", r)
        graph.replay()
        torch.cuda.synchronize()
        for o, ref in zip(outs, refs[i]):
            assert torch.equal(o.view(torch.int16), ref.view(torch.int16)), r


def test_transpose_a_replays_like_eager():
    import torch
    # transpose_A with B [K,N] (f16, 520 x 776 x 328) and with W [N,K] plus split-K
    # (bf16, 256 x 384 x 4096)
    At1 = [synth.random_bits((328, 520), "f16", s) for s in (11, 12)]
    B1 = synth.random_bits((328, 776), "f16", 13)
    b1 = synth.random_bits((776,), "f16", 14)
    At2 = [synth.random_bits((4096, 256), "bf16", s) for s in (15, 16)]
    W2 = synth.random_bits((384, 4096), "bf16", 17, scale=1 / 64)
    b2 = synth.random_bits((384,), "bf16", 18)
    nb = gba.workspace_size(256, 384, 4096, "gelu", "bf16", transpose_b=True, transpose_a=True)
    assert nb > 0
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    a1 = [to_dev(x, "f16") for x in At1]
    a2 = [to_dev(x, "bf16") for x in At2]
    bm1, bb1 = to_dev(B1, "f16"), to_dev(b1, "f16")
    w2, bb2 = to_dev(W2, "bf16"), to_dev(b2, "bf16")

    def run_all(x1, x2, c1, c2):
        gba.gemm_bias_act(x1, bm1, bb1, c1, "sigmoid", transpose_a=True)
        gba.gemm_bias_act(x2, w2, bb2, c2, "gelu", transpose_a=True, transpose_b=True,
                          workspace=ws)

    refs = []
    for i in range(2):
        outs = (empty((520, 776), "f16"), empty((256, 384), "bf16"))
        run_all(a1[i], a2[i], *outs)
        refs.append(outs)
    torch.cuda.synchronize()

    src = (a1[0].clone(), a2[0].clone())
    outs = (empty((520, 776), "f16"), empty((256, 384), "bf16"))
    graph = torch.cuda.CUDAGraph()
    say("graph capture: transpose_A, transpose_A + transpose_B + split-K")
    with torch.cuda.graph(graph):
        run_all(*src, *outs)
    torch.cuda.synchronize()
    for r in range(4):
        i = r % 2
        src[0].copy_(a1[i])
        src[1].copy_(a2[i])
        for o in outs:
            o.fill_(0.0)
        ws.fill_(255)
        say("graph replay transpose_A", r)
        graph.replay()
        torch.cuda.synchronize()
        for o, ref in zip(outs, refs[i]):
            assert torch.equal(o.view(torch.int16), ref.view(torch.int16)), r


def test_unfused_pair_and_plain_gemms_replay_like_eager():
    """gemm (B [K,N] and W [N,K]) and bias_act, the unfused pair, captured in
    one graph: the intermediate C of gemm feeds bias_act inside the graph."""
    import torch
    M, N, K = 392, 520, 264
    A = [synth.random_bits((M, K), "bf16", s) for s in (51, 52)]
    B = synth.random_bits((K, N), "bf16", 53)
    W = synth.random_bits((N, K), "bf16", 54)
    bias = synth.random_bits((N,), "bf16", 55)
    a = [to_dev(x, "bf16") for x in A]
    b, w, bb = to_dev(B, "bf16"), to_dev(W, "bf16"), to_dev(bias, "bf16")

    def run_all(x, mid, y, z):
        gba.gemm(x, b, mid)
        gba.bias_act(mid, bb, y, "softplus")
        gba.gemm(x, w, z, transpose_b=True)

    def bufs():
        return (empty((M, N), "bf16"), empty((M, N), "bf16"), empty((M, N), "bf16"))

    refs = []
    for i in range(2):
        outs = bufs()
        run_all(a[i], *outs)
        refs.append(outs)
    torch.cuda.synchronize()
    src, outs = a[0].clone(), bufs()
    graph = torch.cuda.CUDAGraph()
    say("graph capture: gemm, bias_act, gemm [N,K]")
    with torch.cuda.graph(graph):
        run_all(src, *outs)
    torch.cuda.synchronize()
    for r in range(4):
        i = r % 2
        src.copy_(a[i])
        for o in outs:
            o.fill_(0.0)
        say("graph replay unfused", r)
        graph.replay()
        torch.cuda.synchronize()
        for o, ref in zip(outs, refs[i]):
            assert torch.equal(o.view(torch.int16), ref.view(torch.int16)), r
