"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle.

Bars:
  * exact-input cases (integer or short-mantissa entries whose every fp32
    partial sum is exact): bitwise equal to the oracle's rounded result, for
    every compiled-in schedule, ragged shapes included;
  * random cases: relative Frobenius <= 2e-2 and |C-R| <= 1e-2*sqrt(K)/64 +
    1e-2*|R| per element (oracle/compare.py), plus the stricter
    accumulation-aware 1-ulp gate;
  * full workload sizes: 64 sampled rows, in the launch configuration the
    benchmark times (the library's own schedule choice).
"""
import math

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
    yield
    gba.set_schedule(None)


def run_gpu(A, B, bias, act, dtype, sched=None):
    import torch
    M, K = A.shape
    N = B.shape[1]
    a, b, bb = to_dev(A, dtype), to_dev(B, dtype), to_dev(bias, dtype)
    c = empty((M, N), dtype, fill_bits=0x7E00)   # NaN sentinel: every element must be written
    gba.set_schedule(sched)
    try:
        gba.gemm_bias_act(a, b, bb, c, act)
    finally:
        gba.set_schedule(None)
    torch.cuda.synchronize()
    return to_bits(c)


def schedules():
    return gba.list_schedules()


def sched_id(s):
    return "k%d_%dx%dx%d_w%dx%d_s%d_l%d_p%d" % (s["kernel"], s["bm"], s["bn"], s["bk"], s["wm"],
                                                s["wn"], s["stages"], s["loaders"], s["spread"])


# ---------------------------------------------------------- bit-exact ----

def int_inputs(M, N, K, dtype, seed, lo=-1, hi=1, bias=True):
    rng = np.random.default_rng(seed)
    enc = (lambda v: v.astype(np.float16).view(np.uint16)) if dtype == "f16" else \
        (lambda v: synth.to_bits(v.astype(np.float32), "bf16"))
    A = enc(rng.integers(lo, hi + 1, (M, K)).astype(np.float64))
    B = enc(rng.integers(lo, hi + 1, (K, N)).astype(np.float64))
    bv = enc(rng.integers(-8, 9, N).astype(np.float64)) if bias else None
    return A, B, bv


EXACT_SHAPES = [(256, 256, 256), (1, 8, 8), (37, 40, 24), (129, 136, 72), (300, 264, 1000),
                (520, 776, 64)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", EXACT_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_exact_integer_gemm_is_bitwise_for_every_schedule(shape, dtype):
    M, N, K = shape
    A, B, bias = int_inputs(M, N, K, dtype, seed=M + N + K)
    R = oracle.gemm_bias_act(A, B, bias, "none", dtype)
    want = oracle.encode(R, dtype)
    for s in schedules():
        for raster in (0, 1):
            sch = dict(s, raster=raster)
            say("exact", shape, dtype, sched_id(s), "raster", raster)
            got = run_gpu(A, B, bias, "none", dtype, sched=sch)
            bad = np.argwhere(got != want)
            assert bad.size == 0, "%s %s: %d mismatches, first %s" % (
                sched_id(s), raster, len(bad), bad[:3].tolist())


PERSISTENT = dict(bm=256, bn=256, bk=64, wm=2, wn=2, stages=2, raster=1, group_m=4, kernel=4,
                  loaders=4, spread=1)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("K", [128, 192, 1000])
def test_persistent_kernel_streams_many_tiles_bitwise(K, dtype):
    # 17 x 17 = 289 tiles of 256 x 256 on a 256-CU grid: some workgroups run two
    # tiles, so the next tile's first slices are loaded inside the previous
    # tile's K loop. K = 128: two slices per tile (the shortest stream); K = 192:
    # an odd count, so the ring stage of slice 0 alternates from tile to tile;
    # K = 1000: a ragged last slice. Ragged M and N tiles too.
    M, N = 4100, 4200
    A, B, bias = int_inputs(M, N, K, dtype, seed=K + 7)
    want = oracle.encode(oracle.gemm_bias_act(A, B, bias, "none", dtype, nthreads=16), dtype)
    for raster in (0, 1):
        say("persistent exact", K, dtype, "raster", raster)
        got = run_gpu(A, B, bias, "none", dtype, sched=dict(PERSISTENT, raster=raster))
        bad = np.argwhere(got != want)
        assert bad.size == 0, "raster %d: %d mismatches, first %s" % (raster, len(bad),
                                                                      bad[:3].tolist())


def test_persistent_kernel_random_gelu_and_short_k():
    A = synth.random_bits((4100, 520), "bf16", 31)
    B = synth.random_bits((520, 4200), "bf16", 32, scale=1 / 16)
    bias = synth.random_bits((4200,), "bf16", 33)
    say("persistent random gelu")
    got = run_gpu(A, B, bias, "gelu", "bf16", sched=PERSISTENT)
    check_random(A, B, bias, "gelu", "bf16", got, rows=synth.sample_rows(4100, 64, seed=3))
    # K <= 64 (one slice per tile) runs as the non-persistent kernel with the same tile
    A, B, bias = int_inputs(600, 520, 64, "f16", seed=5)
    want = oracle.encode(oracle.gemm_bias_act(A, B, bias, "none", "f16"), "f16")
    say("persistent K=64")
    assert np.array_equal(run_gpu(A, B, bias, "none", "f16", sched=PERSISTENT), want)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_direct_to_lds_schedules_agree_bitwise_on_random_inputs(dtype):
    """Kernels 3 and 4 feed every output element the same 16x16x32 MFMAs in the
    same K order (64-deep slices of two 32-deep steps) and the same epilogue,
    whatever the tile, ring depth or persistence: on random inputs (inexact
    sums) every such schedule must give the same bits. Ragged M and N, a K tail
    (1000 = 15 x 64 + 40), and for the persistent kernel 17 x 17 = 289 tiles of
    256 x 256, so that some workgroups run two."""
    M, N, K = 4100, 4200, 1000
    A = synth.random_bits((M, K), dtype, 41)
    B = synth.random_bits((K, N), dtype, 42, scale=1 / 16)
    bias = synth.random_bits((N,), dtype, 43)
    scheds = [s for s in schedules() if s["kernel"] in (3, 4)]
    assert len(scheds) >= 5
    ref = None
    for s in scheds:
        for raster in (0, 1):
            say("agree", dtype, sched_id(s), "raster", raster)
            got = run_gpu(A, B, bias, "gelu", dtype, sched=dict(s, raster=raster))
            if ref is None:
                ref = got
                check_random(A, B, bias, "gelu", dtype, got, rows=synth.sample_rows(M, 64, seed=4))
            else:
                bad = np.argwhere(got != ref)
                assert bad.size == 0, (sched_id(s), raster, len(bad), bad[:3].tolist())


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_exact_relu_epilogue_bitwise(dtype):
    A, B, bias = int_inputs(200, 136, 520, dtype, seed=9)
    want = oracle.encode(oracle.gemm_bias_act(A, B, bias, "relu", dtype), dtype)
    say("exact relu", dtype)
    assert np.array_equal(run_gpu(A, B, bias, "relu", dtype), want)


def test_rounding_is_nearest_even_on_exact_sums():
    # A in {0, +-1, +-1/2, +-1/4}, B multiples of 2^-10 below 2 in magnitude (exact
    # in fp16): every product is a multiple of 2^-12 below 2, every partial sum of
    # 512 of them stays below 2^10 and so is exact in fp32, but the totals need
    # rounding to fp16 -- the result is unique.
    rng = np.random.default_rng(77)
    M, N, K = 160, 192, 512
    A = rng.choice([0.0, 1.0, -1.0, 0.5, -0.5, 0.25, -0.25], size=(M, K))
    B = rng.integers(-2047, 2048, size=(K, N)) / 1024.0
    Ab = A.astype(np.float16).view(np.uint16)
    Bb = B.astype(np.float16).view(np.uint16)
    assert np.array_equal(Bb.view(np.float16).astype(np.float64), B)
    want = oracle.encode(oracle.gemm_bias_act(Ab, Bb, None, "none", "f16"), "f16")
    for s in schedules():
        say("rne", sched_id(s))
        got = run_gpu(Ab, Bb, None, "none", "f16", sched=dict(s))
        assert np.array_equal(got, want), sched_id(s)


# ----------------------------------------------------- random parity ----

def check_random(A, B, bias, act, dtype, got_bits, rows=None):
    R, S = oracle.gemm_bias_act(A, B, bias, act, dtype, rows=rows, with_abs=True)
    C = oracle.decode(got_bits if rows is None else got_bits[rows], dtype)
    rep = compare.check(C, R, K=A.shape[1], dtype=dtype, act=oracle.ACTS[act], S=S)
    assert rep["ok"], rep
    assert rep["strict_ok"], rep
    return rep


@pytest.mark.parametrize("name", ["c1_plain", "c1_gelu", "c2_plain", "c4_relu", "c4_sigmoid"])
def test_workloads_full_check(name):
    w = synth.WORKLOADS[name]
    A, B, bias = synth.make_inputs(w)
    say("workload", name)
    got = run_gpu(A, B, bias, w.act, w.dtype)
    check_random(A, B, bias, w.act, w.dtype, got)


def test_c2_at_the_pages_default_tile():
    # 128x128x32 tiles, 4 waves: the pages' default GEMM starting point.
    w = synth.WORKLOADS["c2_plain"]
    A, B, bias = synth.make_inputs(w)
    sch = {"bm": 128, "bn": 128, "bk": 32, "wm": 2, "wn": 2, "stages": 2, "raster": 1,
           "group_m": 8, "kernel": 0, "loaders": 0, "spread": 0}
    say("c2 128x128x32")
    check_random(A, B, bias, "none", "f16", run_gpu(A, B, bias, "none", "f16", sched=sch))


@pytest.mark.parametrize("name,M,N,K", [("c3_gelu", 512, 768, 4096), ("c5_gelu", 384, 1024, 4096)])
def test_reduced_size_full_check(name, M, N, K):
    w = synth.WORKLOADS[name]
    A, B, bias = synth.make_inputs(w, M=M, N=N, K=K)
    say("reduced", name, M, N, K)
    check_random(A, B, bias, w.act, w.dtype, run_gpu(A, B, bias, w.act, w.dtype))


@pytest.mark.parametrize("name", ["c3_gelu", "c5_gelu"])
def test_full_size_sampled_rows(name):
    w = synth.WORKLOADS[name]
    A, B, bias = synth.make_inputs(w)
    rows = synth.sample_rows(w.M, 64, seed=w.seed)
    say("full", name, gba.get_schedule(w.M, w.N, w.K, w.act, w.dtype))
    got = run_gpu(A, B, bias, w.act, w.dtype)
    check_random(A, B, bias, w.act, w.dtype, got, rows=rows)
    # no element may be left unwritten (the NaN sentinel) or non-finite
    expmask = 0x7C00 if w.dtype == "f16" else 0x7F80
    assert not np.any((got & expmask) == expmask)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("act", ACTS)
def test_every_schedule_ragged_random(act, dtype):
    M, N, K = 300, 264, 136
    A = synth.random_bits((M, K), dtype, 1)
    B = synth.random_bits((K, N), dtype, 2, scale=0.25)
    bias = synth.random_bits((N,), dtype, 3)
    R, S = oracle.gemm_bias_act(A, B, bias, act, dtype, with_abs=True)
    for s in schedules():
        say("ragged", act, dtype, sched_id(s))
        got = run_gpu(A, B, bias, act, dtype, sched=dict(s))
        rep = compare.check(oracle.decode(got, dtype), R, K=K, dtype=dtype,
                            act=oracle.ACTS[act], S=S)
        assert rep["ok"] and rep["strict_ok"], (sched_id(s), rep)


def test_no_bias_and_k_tail():
    for (M, N, K) in [(64, 64, 8), (65, 72, 40), (257, 264, 264)]:
        A = synth.random_bits((M, K), "f16", M)
        B = synth.random_bits((K, N), "f16", N)
        say("nobias", M, N, K)
        check_random(A, B, None, "gelu", "f16", run_gpu(A, B, None, "gelu", "f16"))


# ----------------------------------------------------------- edges ----

def test_degenerate_shapes():
    import torch
    dt = "f16"
    bias = synth.random_bits((16,), dt, 5)
    # K == 0: the empty sum, C = act(bias)
    for act in ACTS:
        say("k0", act)
        got = run_gpu(np.zeros((5, 0), np.uint16), np.zeros((0, 16), np.uint16), bias, act, dt)
        want = oracle.encode(np.broadcast_to(oracle.act(oracle.decode(bias), act), (5, 16)), dt)
        assert np.array_equal(got, want), act
    # M == 0 / N == 0: no work, no error
    a = torch.zeros(0, 8, dtype=torch.float16, device="cuda")
    b = torch.zeros(8, 16, dtype=torch.float16, device="cuda")
    gba.gemm_bias_act(a, b, None, torch.zeros(0, 16, dtype=torch.float16, device="cuda"), "gelu")
    gba.gemm(b.t().contiguous()[:0], b, torch.zeros(0, 16, dtype=torch.float16, device="cuda"))
    # single row / column-chunk
    A = synth.random_bits((1, 8), dt, 1)
    B = synth.random_bits((8, 8), dt, 2)
    check_random(A, B, None, "none", dt, run_gpu(A, B, None, "none", dt))


@pytest.mark.parametrize("shape", [(133, 200, 96), (300, 264, 136)], ids=lambda s: "x".join(map(str, s)))
def test_writes_stay_inside_C(shape):
    # every schedule (the staged epilogues of kernels 3 and 4 mask rows and 16-byte
    # column chunks per wave block) and the 8-bit kernel: a guard band on both
    # sides of C keeps its fill
    import torch
    M, N, K = shape
    A = synth.random_bits((M, K), "f16", 1)
    B = synth.random_bits((K, N), "f16", 2)
    guard = 4096
    buf = torch.empty((M * N + 2 * guard,), dtype=torch.float16, device="cuda")
    c = buf[guard:guard + M * N].view(M, N)
    for s in [None] + gba.list_schedules():
        buf.fill_(7.0)
        say("guard band", shape, "heuristic" if s is None else s)
        gba.set_schedule(s)
        try:
            gba.gemm_bias_act(to_dev(A, "f16"), to_dev(B, "f16"), None, c, "none")
        finally:
            gba.set_schedule(None)
        torch.cuda.synchronize()
        assert bool((buf[:guard] == 7.0).all()) and bool((buf[guard + M * N:] == 7.0).all()), s
        check_random(A, B, None, "none", "f16", to_bits(c))
    # 8-bit inputs (K a multiple of 16)
    K8 = K // 16 * 16
    A8 = synth.f32_to_fp8_bits(np.random.default_rng(3).integers(-2, 3, (M, K8)).astype(np.float32), "e4m3")
    W8 = synth.f32_to_fp8_bits(np.random.default_rng(4).integers(-2, 3, (N, K8)).astype(np.float32), "e4m3")
    buf.fill_(7.0)
    say("guard band fp8", shape)
    gba.gemm_bias_act_fp8(torch.from_numpy(A8).cuda(), torch.from_numpy(W8).cuda(), None, c, 1.0,
                          "none", "e4m3")
    torch.cuda.synchronize()
    assert bool((buf[:guard] == 7.0).all()) and bool((buf[guard + M * N:] == 7.0).all())
    want = oracle.encode(oracle.gemm_bias_act_fp8(A8, W8, None, 1.0, "none", "e4m3", "f16"), "f16")
    assert np.array_equal(to_bits(c), want)


def test_run_to_run_bitwise_determinism():
    w = synth.WORKLOADS["c4_sigmoid"]
    A, B, bias = synth.make_inputs(w)
    say("determinism")
    r1 = run_gpu(A, B, bias, w.act, w.dtype)
    r2 = run_gpu(A, B, bias, w.act, w.dtype)
    assert np.array_equal(r1, r2)


def test_non_default_stream():
    import torch
    A = synth.random_bits((256, 512), "bf16", 1)
    B = synth.random_bits((512, 384), "bf16", 2)
    bias = synth.random_bits((384,), "bf16", 3)
    s = torch.cuda.Stream()
    a, b, bb = to_dev(A, "bf16"), to_dev(B, "bf16"), to_dev(bias, "bf16")
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        c = empty((256, 384), "bf16")
        say("stream")
        gba.gemm_bias_act(a, b, bb, c, "gelu")
    s.synchronize()
    check_random(A, B, bias, "gelu", "bf16", to_bits(c))


def test_graph_capture_replays_match_eager():
    # The launch path makes no allocation, copy, fill or synchronisation, so a
    # caller can capture it into a HIP graph. Replays, with eager work and
    # device synchronisation between them, must match eager calls bitwise --
    # also after the captured input buffer has been overwritten.
    import torch
    M, N, K = 520, 776, 328
    A = synth.random_bits((M, K), "f16", 21)
    A2 = synth.random_bits((M, K), "f16", 22)
    B = synth.random_bits((K, N), "f16", 23)
    bias = synth.random_bits((N,), "f16", 24)
    a, b, bb = to_dev(A, "f16"), to_dev(B, "f16"), to_dev(bias, "f16")
    a2 = to_dev(A2, "f16")
    ref1, ref2 = empty((M, N), "f16"), empty((M, N), "f16")
    gba.gemm_bias_act(a, b, bb, ref1, "gelu")
    gba.gemm_bias_act(a2, b, bb, ref2, "gelu")
    torch.cuda.synchronize()
    c = empty((M, N), "f16")
    src = a.clone()
    graph = torch.cuda.CUDAGraph()
    say("graph capture")
    with torch.cuda.graph(graph):
        gba.gemm_bias_act(src, b, bb, c, "gelu")
    torch.cuda.synchronize()
    for r in range(4):
        src.copy_(a if r % 2 == 0 else a2)
        c.fill_(0.0)
        say("graph replay", r)
        graph.replay()
        torch.cuda.synchronize()
        want = ref1 if r % 2 == 0 else ref2
        assert torch.equal(c.view(torch.int16), want.view(torch.int16)), r
    check_random(A2, B, bias, "gelu", "f16", to_bits(ref2))


# ---------------------------------------------------- unfused pair ----

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("act", ACTS)
def test_bias_act_against_oracle_on_its_input(act, dtype):
    import torch
    M, N = 333, 1032
    X = synth.random_bits((M, N), dtype, 11, scale=4.0)
    bias = synth.random_bits((N,), dtype, 12)
    x, bb = to_dev(X, dtype), to_dev(bias, dtype)
    y = empty((M, N), dtype, fill_bits=0x7E00)
    say("bias_act", act, dtype)
    gba.bias_act(x, bb, y, act)
    torch.cuda.synchronize()
    R = oracle.bias_act(X, bias, act, dtype)
    got = oracle.decode(to_bits(y), dtype)
    # one fp32 add, the activation, one rounding: within 1 ulp of the exact value
    err = np.abs(got - R)
    assert np.all(err <= compare.ulp_out(R, dtype) + 2.0 ** -22), float(err.max())
    # in place
    gba.bias_act(x, bb, x, act)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(x), to_bits(y))


def test_unfused_pair_matches_oracle_and_fused():
    import torch
    w = synth.WORKLOADS["c4_relu"]
    A, B, bias = synth.make_inputs(w, M=700, N=1024, K=1000)
    a, b, bb = to_dev(A, "f16"), to_dev(B, "f16"), to_dev(bias, "f16")
    for act in ("relu", "sigmoid", "gelu"):
        t = empty((700, 1024), "f16")
        y = empty((700, 1024), "f16")
        f = empty((700, 1024), "f16")
        say("unfused", act)
        gba.gemm(a, b, t)
        gba.bias_act(t, bb, y, act)
        gba.gemm_bias_act(a, b, bb, f, act)
        torch.cuda.synchronize()
        T = to_bits(t)
        check_random(A, B, None, "none", "f16", T)
        # second kernel pinned on the intermediate it actually read
        Ry = oracle.bias_act(T, bias, act, "f16")
        Y = oracle.decode(to_bits(y), "f16")
        assert np.all(np.abs(Y - Ry) <= compare.ulp_out(Ry, "f16") + 2.0 ** -22)
        # the unfused result carries one extra rounding of the intermediate
        check_random(A, B, bias, act, "f16", to_bits(f))
        rep = compare.check(Y, oracle.decode(to_bits(f), "f16"), K=1000, dtype="f16")
        assert rep["ok"], rep


# ------------------------------------------------------ epilogue code ----

@pytest.mark.parametrize("act", ACTS)
def test_epilogue_device_functions_on_dense_grid(act):
    import torch
    z = np.concatenate([np.linspace(-12, 12, 200001), np.geomspace(1e-6, 80, 4000)])
    z = np.concatenate([z, -z]).astype(np.float32)
    zt = torch.from_numpy(z).cuda()
    yt = torch.empty_like(zt)
    say("epilogue", act)
    gba.epilogue_probe(zt, yt, act)
    torch.cuda.synchronize()
    y = yt.cpu().numpy().astype(np.float64)
    ref = oracle.act(z.astype(np.float64), act)
    err = np.abs(y - ref)
    if act in ("none", "relu"):
        assert np.array_equal(y, ref)
    elif act == "sigmoid":
        # hardware exp2 and reciprocal, each within a couple of fp32 ulps, plus the
        # conditioning of exp: rounding z*log2(e) to fp32 moves e^-z by |z| 2^-24.
        bound = (1e-6 + np.abs(z) * 1.2e-7) * np.abs(ref) + 1e-37
        assert np.all(err <= bound), float((err / bound).max())
    elif act == "softplus":
        # max(z,0) + log1p(e^-|z|): hardware exp2 (conditioning |z| 2^-24 on e^-|z|),
        # log2 and reciprocal each within a few fp32 ulps, Kahan's log1p correction.
        t = np.exp(-np.abs(z.astype(np.float64)))
        bound = 2e-6 * np.abs(ref) + 1.2e-7 * np.abs(z) * t + 1e-37
        assert np.all(err <= bound), float((err / bound).max())
    elif act == "gelu_tanh":
        # z / (1 + 2^a), a = -2 y log2 e formed in fp32: two float32 constants and
        # three roundings (z^2, the fma, the product) give a relative error up to
        # 5 2^-24 = 3e-7 in a, so 2^a moves by |a| ln2 3e-7 relative; then the
        # hardware exp2 and reciprocal (a few ulp). Where 1 + 2^a passes 2^126 the
        # reciprocal is below the smallest normal float and flushes to zero, so
        # results below |z| 2^-126 (< 1e-36 on this grid) come out as -0.
        zz = z.astype(np.float64)
        a = 2 * np.sqrt(2 / np.pi) * np.log2(np.e) * np.abs(zz + 0.044715 * zz ** 3)
        bound = (2e-6 + a * 3.0e-7) * np.abs(ref) + 1e-36
        assert np.all(err <= bound), float((err / bound).max())
    else:
        # Phi(-|z|) = 2^Q(|z|) with fractional error < 8e-6 on |z| <= 6
        # (tests/test_gelu_fit.py); the fp32 Horner steps round Q (|Q| <= 30 there)
        # by a few ulp, which moves 2^Q by about 1e-6 per ulp relative. Past |z| = 6
        # the correction term is below 6e-9 absolute, far under the 2^-20 floor of
        # the fused GEMM's element-wise check.
        zz = np.abs(z.astype(np.float64))
        bound = 1.2e-5 * np.abs(ref) + np.where(zz > 6.0, 1e-8, 0.0) + 1e-37
        assert np.all(err <= bound), float((err / bound).max())


@pytest.mark.parametrize("act", ["none", "relu", "sigmoid", "gelu", "softplus", "gelu_tanh"])
def test_epilogue_non_finite(act):
    """An fp32 accumulator can overflow (bf16 operands reach 3.4e38): each
    activation gives its limit at +-inf (no inf * 0 NaN) and NaN for NaN, as the
    oracle does."""
    import torch
    z = np.array([np.inf, -np.inf, np.nan, 3.0e38, -3.0e38, 1e20, -1e20], dtype=np.float32)
    zt = torch.from_numpy(z).cuda()
    yt = torch.empty_like(zt)
    say("epilogue non-finite", act)
    gba.epilogue_probe(zt, yt, act)
    torch.cuda.synchronize()
    y = yt.cpu().numpy().astype(np.float64)
    ref = oracle.act(z.astype(np.float64), act)
    if act == "relu":
        assert y[2] == 0.0 and ref[2] == 0.0   # max(NaN, 0): IEEE maxNum on both sides
    else:
        assert np.isnan(y[2]) and np.isnan(ref[2])
    fin = [0, 1, 3, 4, 5, 6]
    assert np.array_equal(np.isinf(y[fin]), np.isinf(ref[fin])), (y, ref)
    assert np.allclose(y[fin], ref[fin], rtol=1e-5, atol=0.0), (y, ref)


# ------------------------------------------------------------ tuner ----

def test_autotune_writes_cache_and_is_used(tmp_path, monkeypatch):
    import json
    import torch
    monkeypatch.setenv("GBA_CACHE_DIR", str(tmp_path))
    M, N, K = 512, 512, 256
    A = synth.random_bits((M, K), "f16", 1)
    B = synth.random_bits((K, N), "f16", 2)
    bias = synth.random_bits((N,), "f16", 3)
    a, b, bb = to_dev(A, "f16"), to_dev(B, "f16"), to_dev(bias, "f16")
    c = empty((M, N), "f16")
    say("autotune")
    best, ms = gba.autotune(a, b, bb, c, "gelu")
    torch.cuda.synchronize()
    assert ms > 0
    check_random(A, B, bias, "gelu", "f16", to_bits(c))
    data = json.load(open(tmp_path / "schedules.json"))
    assert data["format"] == "gba-schedule-cache" and data["version"] == 1
    keys = [e["key"] for e in data["entries"]]
    assert any(k.endswith("|f16|gelu|nn|512|512|256") for k in keys)
    assert gba.get_schedule(M, N, K, "gelu", "f16") == best
