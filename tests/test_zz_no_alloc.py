"""gemm_bias_act_noalloc: the split-K path with the library's static scratch in
place of a caller's workspace, for callers that cannot allocate. Called through
the C ABI; its output must equal gemm_bias_act_ex's with a workspace bitwise
(same kernels, same split), on two calls in a row, the second smaller, and
agree with the oracle."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
import tiled_dense_gemm_bias_amd as gba
from oracle import compare
from tests.gpu_util import empty, say, to_bits, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


ACT = {"none": 0, "relu": 1, "sigmoid": 2, "gelu": 3, "softplus": 4, "gelu_tanh": 5}


def _run_pair(M, N, K, dtype, act, tb, seed):
    import torch
    A = synth.random_bits((M, K), dtype, seed)
    B = synth.random_bits((N, K) if tb else (K, N), dtype, seed + 1, scale=1 / 64)
    bias = synth.random_bits((N,), dtype, seed + 2)
    a, b, bb = to_dev(A, dtype), to_dev(B, dtype), to_dev(bias, dtype)
    dt = 0 if dtype == "f16" else 1
    flags = 1 if tb else 0
    nb = gba.workspace_size(M, N, K, act, dtype, transpose_b=tb)
    assert 0 < nb <= gba.lib().gba_noalloc_scratch_bytes(), nb   # the case splits K
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    ref = empty((M, N), dtype, fill_bits=0x7E00)
    got = empty((M, N), dtype, fill_bits=0x7C01)
    lib = gba.lib()
    lib.gba_set_stream(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    say("noalloc", M, N, K, dtype, act, "NK" if tb else "KN")
    st = lib.gemm_bias_act_ex(a.data_ptr(), b.data_ptr(), bb.data_ptr(), ref.data_ptr(), M, N, K,
                              ACT[act], dt, flags, ws.data_ptr(), nb)
    assert st == 0, st
    st = lib.gemm_bias_act_noalloc(a.data_ptr(), b.data_ptr(), bb.data_ptr(), got.data_ptr(), M, N,
                                   K, ACT[act], dt, flags)
    assert st == 0, gba.lib().gba_status_string(st)
    torch.cuda.synchronize()
    g, r = to_bits(got), to_bits(ref)
    assert np.array_equal(g, r)
    R, S = oracle.gemm_bias_act(A, B, bias, act, dtype, with_abs=True, transpose_b=tb)
    rep = compare.check(oracle.decode(g, dtype), R, K=K, dtype=dtype, act=oracle.ACTS[act], S=S)
    assert rep["ok"] and rep["strict_ok"], rep
    return g


def test_noalloc_equals_workspace_path_twice_second_smaller():
    first = _run_pair(256, 384, 16384, "f16", "softplus", False, 11)
    second = _run_pair(128, 256, 4096, "bf16", "gelu", True, 21)
    assert first.shape != second.shape


def test_noalloc_without_split_and_errors():
    import torch
    M, N, K = 512, 512, 256   # 256 tiles of 256^2 would not split; 16 of 128^2: no split at K=256
    A = synth.random_bits((M, K), "f16", 31)
    B = synth.random_bits((K, N), "f16", 32)
    a, b = to_dev(A, "f16"), to_dev(B, "f16")
    c = empty((M, N), "f16")
    ref = empty((M, N), "f16")
    say("noalloc no split")
    gba.gemm_bias_act_noalloc(a, b, None, c, "relu")
    gba.gemm_bias_act(a, b, None, ref, "relu")
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(c), to_bits(ref))
    lib = gba.lib()
    assert lib.gemm_bias_act_noalloc(a.data_ptr(), b.data_ptr(), None, c.data_ptr(), M, N, K, 1, 0,
                                     64) == 2   # unknown flag bit
    assert lib.gemm_bias_act_noalloc(a.data_ptr(), b.data_ptr(), None, c.data_ptr(), M, N, 12, 1, 0,
                                     0) == 5   # K % 8


def test_noalloc_in_a_graph_replays_like_eager():
    """Recorded under HIP graph capture, the use it exists for: a split-K call
    captured once and replayed four times with alternating inputs. Between
    replays an eager allocation-free call of another shape rewrites the shared
    scratch, with device synchronisation around it. Every replay and every
    eager call must equal its eager reference bitwise."""
    import torch
    M, N, K, dt, act = 256, 384, 4096, "f16", "gelu"
    A = [synth.random_bits((M, K), dt, s) for s in (41, 42)]
    B = synth.random_bits((K, N), dt, 43, scale=1 / 64)
    bias = synth.random_bits((N,), dt, 44)
    a = [to_dev(x, dt) for x in A]
    b, bb = to_dev(B, dt), to_dev(bias, dt)
    M2, N2, K2 = 128, 256, 8192
    assert gba.workspace_size(M, N, K, act, dt) > 0 and gba.workspace_size(M2, N2, K2, "relu", "bf16") > 0
    a2 = to_dev(synth.random_bits((M2, K2), "bf16", 45), "bf16")
    b2 = to_dev(synth.random_bits((K2, N2), "bf16", 46, scale=1 / 64), "bf16")
    refs = []
    for i in range(2):
        r = empty((M, N), dt, fill_bits=0x7E00)
        gba.gemm_bias_act_noalloc(a[i], b, bb, r, act)
        refs.append(r)
    ref2 = empty((M2, N2), "bf16", fill_bits=0x7E00)
    gba.gemm_bias_act_noalloc(a2, b2, None, ref2, "relu")
    torch.cuda.synchronize()
    for r in refs + [ref2]:
        assert not (to_bits(r) == 0x7E00).any()

    src, out, c2 = a[0].clone(), empty((M, N), dt), empty((M2, N2), "bf16")
    graph = torch.cuda.CUDAGraph()
    say("noalloc graph capture", M, N, K)
    with torch.cuda.graph(graph):
        gba.gemm_bias_act_noalloc(src, b, bb, out, act)
    torch.cuda.synchronize()
    for rep in range(4):
        i = rep % 2
        src.copy_(a[i])
        out.fill_(0.0)
        c2.fill_(0.0)
        gba.gemm_bias_act_noalloc(a2, b2, None, c2, "relu")   # eager, same scratch
        torch.cuda.synchronize()
        say("noalloc graph replay", rep)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), refs[i].view(torch.int16)), rep
        assert torch.equal(c2.view(torch.int16), ref2.view(torch.int16)), rep


def test_noalloc_first_call_under_capture():
    """In a fresh process, the device's first allocation-free call (which takes
    the scratch's address) made under graph capture: replays equal eager."""
    import os
    import subprocess
    import sys
    child = os.path.join(os.path.dirname(os.path.abspath(__file__)), "noalloc_capture_child.py")
    say("noalloc first call under capture (child process)")
    r = subprocess.run([sys.executable, child], capture_output=True, text=True, timeout=180)
    assert r.returncode == 0 and "replay equals eager: True" in r.stdout, (r.stdout[-2000:], r.stderr[-2000:])
