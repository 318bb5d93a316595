"""transpose_B path (gemm_bias_act_nt / gemm_nt: the second operand stored as
W [N, K]) against the fp64 oracle, through the C ABI.

Bars as in test_gpu_parity.py: bitwise on exact-integer inputs for every
schedule with this path (ragged shapes, both rasters), the oracle's tolerance
on random inputs, 64 sampled rows at full workload sizes; and bitwise equality
with the (K, N) path on the same schedule, since both feed the matrix cores the
same operands in the same order.
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
PERSISTENT = dict(bm=256, bn=256, bk=64, wm=2, wn=2, stages=2, raster=1, group_m=4, kernel=4,
                  loaders=4, spread=1)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    gba.set_schedule(None)


def tb_schedules():
    return [s for s in gba.list_schedules() if s["kernel"] in (3, 4)]


def sched_id(s):
    return "k%d_%dx%dx%d_s%d_p%d" % (s["kernel"], s["bm"], s["bn"], s["bk"], s["stages"],
                                     s["spread"])


def run_nt(A, W, bias, act, dtype, sched=None, transpose_b=True):
    import torch
    M = A.shape[0]
    N = W.shape[0] if transpose_b else W.shape[1]
    a, w, bb = to_dev(A, dtype), to_dev(W, dtype), to_dev(bias, dtype)
    c = empty((M, N), dtype, fill_bits=0x7E00)   # NaN sentinel: every element must be written
    gba.set_schedule(sched)
    try:
        gba.gemm_bias_act(a, w, bb, c, act, transpose_b=transpose_b)
    finally:
        gba.set_schedule(None)
    torch.cuda.synchronize()
    return to_bits(c)


def int_inputs(M, N, K, dtype, seed):
    rng = np.random.default_rng(seed)
    enc = (lambda v: v.astype(np.float16).view(np.uint16)) if dtype == "f16" else \
        (lambda v: synth.to_bits(v.astype(np.float32), "bf16"))
    A = enc(rng.integers(-1, 2, (M, K)).astype(np.float64))
    W = enc(rng.integers(-1, 2, (N, K)).astype(np.float64))
    bias = enc(rng.integers(-8, 9, N).astype(np.float64))
    return A, W, bias


def check_random(A, W, bias, act, dtype, got_bits, rows=None):
    R, S = oracle.gemm_bias_act(A, W, bias, act, dtype, rows=rows, with_abs=True,
                                transpose_b=True, nthreads=16)
    C = oracle.decode(got_bits if rows is None else got_bits[rows], dtype)
    rep = compare.check(C, R, K=A.shape[1], dtype=dtype, act=oracle.ACTS[act], S=S)
    assert rep["ok"] and rep["strict_ok"], rep
    return rep


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(256, 256, 256), (1, 8, 8), (37, 40, 24), (129, 136, 72),
                                   (300, 264, 1000), (520, 776, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_exact_integer_bitwise_every_schedule(shape, dtype):
    M, N, K = shape
    A, W, bias = int_inputs(M, N, K, dtype, seed=M + 2 * N + K)
    want = oracle.encode(oracle.gemm_bias_act(A, W, bias, "none", dtype, transpose_b=True), dtype)
    for s in tb_schedules():
        for raster in (0, 1):
            say("nt exact", shape, dtype, sched_id(s), "raster", raster)
            got = run_nt(A, W, bias, "none", dtype, sched=dict(s, raster=raster))
            bad = np.argwhere(got != want)
            assert bad.size == 0, "%s r%d: %d mismatches, first %s" % (
                sched_id(s), raster, len(bad), bad[:3].tolist())


@pytest.mark.parametrize("K", [128, 1000])
def test_persistent_many_tiles_bitwise(K):
    # 289 tiles of 256 x 256 on a 256-CU grid, ragged M, N (and K = 1000)
    M, N = 4100, 4200
    A, W, bias = int_inputs(M, N, K, "bf16", seed=K + 70)
    want = oracle.encode(oracle.gemm_bias_act(A, W, bias, "relu", "bf16", transpose_b=True,
                                              nthreads=16), "bf16")
    say("nt persistent exact", K)
    got = run_nt(A, W, bias, "relu", "bf16", sched=PERSISTENT)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("act", ACTS)
def test_random_every_schedule_and_same_bits_as_kn_layout(act, dtype):
    M, N, K = 300, 264, 136
    A = synth.random_bits((M, K), dtype, 1)
    W = synth.random_bits((N, K), dtype, 2, scale=0.25)
    bias = synth.random_bits((N,), dtype, 3)
    B = np.ascontiguousarray(W.T)
    R, S = oracle.gemm_bias_act(A, W, bias, act, dtype, with_abs=True, transpose_b=True)
    for s in tb_schedules():
        say("nt random", act, dtype, sched_id(s))
        got = run_nt(A, W, bias, act, dtype, sched=dict(s))
        rep = compare.check(oracle.decode(got, dtype), R, K=K, dtype=dtype,
                            act=oracle.ACTS[act], S=S)
        assert rep["ok"] and rep["strict_ok"], (sched_id(s), rep)
        kn = run_nt(A, B, bias, act, dtype, sched=dict(s), transpose_b=False)
        assert np.array_equal(got, kn), sched_id(s)


@pytest.mark.parametrize("name", ["c3_gelu", "c5_gelu"])
def test_full_size_sampled_rows(name):
    # the workload's B, stored transposed (a linear layer's [N, K] weight)
    w = synth.WORKLOADS[name]
    A, B, bias = synth.make_inputs(w)
    W = np.ascontiguousarray(B.T)
    del B
    rows = synth.sample_rows(w.M, 64, seed=w.seed)
    say("nt full", name, gba.get_schedule(w.M, w.N, w.K, w.act, w.dtype, transpose_b=True))
    got = run_nt(A, W, bias, w.act, w.dtype)
    check_random(A, W, bias, w.act, w.dtype, got, rows=rows)
    expmask = 0x7C00 if w.dtype == "f16" else 0x7F80
    assert not np.any((got & expmask) == expmask)


def test_reduced_c4_and_k_tail_and_no_bias():
    w = synth.WORKLOADS["c4_sigmoid"]
    A, B, bias = synth.make_inputs(w, M=1000, N=1280, K=1000)
    W = np.ascontiguousarray(B.T)
    say("nt c4 reduced")
    check_random(A, W, bias, "sigmoid", "f16", run_nt(A, W, bias, "sigmoid", "f16"))
    for (M, N, K) in [(64, 64, 8), (65, 72, 40), (257, 264, 264)]:
        A = synth.random_bits((M, K), "f16", M)
        W = synth.random_bits((N, K), "f16", N)
        say("nt nobias", M, N, K)
        check_random(A, W, None, "gelu", "f16", run_nt(A, W, None, "gelu", "f16"))


def test_short_k_runs_on_the_persistent_schedule():
    # K <= 64: one slice per tile, run by the non-persistent kernel with that tile
    A, W, bias = int_inputs(600, 520, 64, "f16", seed=5)
    want = oracle.encode(oracle.gemm_bias_act(A, W, bias, "none", "f16", transpose_b=True), "f16")
    say("nt persistent K=64")
    assert np.array_equal(run_nt(A, W, bias, "none", "f16", sched=PERSISTENT), want)


def test_gemm_nt_and_degenerate_shapes():
    import torch
    A, W, _ = int_inputs(77, 96, 200, "f16", seed=8)
    a, w = to_dev(A, "f16"), to_dev(W, "f16")
    c = empty((77, 96), "f16", fill_bits=0x7E00)
    say("gemm_nt")
    gba.gemm(a, w, c, transpose_b=True)
    torch.cuda.synchronize()
    want = oracle.encode(oracle.gemm_bias_act(A, W, None, "none", "f16", transpose_b=True), "f16")
    assert np.array_equal(to_bits(c), want)
    bias = synth.random_bits((16,), "f16", 5)
    for act in ACTS:
        say("nt k0", act)
        got = run_nt(np.zeros((5, 0), np.uint16), np.zeros((16, 0), np.uint16), bias, act, "f16")
        want = oracle.encode(np.broadcast_to(oracle.act(oracle.decode(bias), act), (5, 16)), "f16")
        assert np.array_equal(got, want), act
    gba.gemm_bias_act(torch.zeros(0, 8, dtype=torch.float16, device="cuda"),
                      torch.zeros(16, 8, dtype=torch.float16, device="cuda"), None,
                      torch.zeros(0, 16, dtype=torch.float16, device="cuda"), "gelu",
                      transpose_b=True)


def test_schedule_without_the_path_is_refused():
    import torch
    a = torch.zeros(64, 64, dtype=torch.float16, device="cuda")
    c = torch.zeros(64, 64, dtype=torch.float16, device="cuda")
    s0 = [s for s in gba.list_schedules() if s["kernel"] == 0][0]
    gba.set_schedule(s0)
    try:
        with pytest.raises(gba.GbaError) as e:
            gba.gemm_bias_act(a, a, None, c, "none", transpose_b=True)
        assert e.value.status == 9
    finally:
        gba.set_schedule(None)
    assert gba.get_schedule(4096, 4096, 4096, "gelu", "f16", transpose_b=True)["kernel"] == 4


def test_autotune_transpose_b_is_cached_under_its_own_key(tmp_path, monkeypatch):
    import json
    import torch
    monkeypatch.setenv("GBA_CACHE_DIR", str(tmp_path))
    M, N, K = 512, 512, 256
    A = synth.random_bits((M, K), "bf16", 1)
    W = synth.random_bits((N, K), "bf16", 2)
    bias = synth.random_bits((N,), "bf16", 3)
    a, w, bb = to_dev(A, "bf16"), to_dev(W, "bf16"), to_dev(bias, "bf16")
    c = empty((M, N), "bf16")
    say("nt autotune")
    best, ms = gba.autotune(a, w, bb, c, "relu", transpose_b=True)
    torch.cuda.synchronize()
    assert ms > 0 and best["kernel"] in (3, 4)
    check_random(A, W, bias, "relu", "bf16", to_bits(c))
    keys = [e["key"] for e in json.load(open(tmp_path / "schedules.json"))["entries"]]
    assert any(k.endswith("|bf16|relu|nt|512|512|256") for k in keys)
    assert gba.get_schedule(M, N, K, "relu", "bf16", transpose_b=True) == best
