"""transpose_A path (gemm_bias_act_ex with GBA_TRANSPOSE_A: the first operand
stored as At [K, M]) against the fp64 oracle, through the C ABI.

Bars as in test_gpu_parity.py: bitwise on exact-integer inputs for every
schedule with this path (ragged shapes, both rasters, both B layouts), the
oracle's tolerance on random inputs, 64 sampled rows at full workload sizes;
and bitwise equality with the [M, K] path on the same schedule, since both feed
the matrix cores the same operands in the same order. M is a multiple of 8
throughout (16-byte rows of At).
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


def ta_schedules():
    """Compiled-in schedules with a transpose_A path: every kernel-3/4 schedule
    at the tiles the built-in heuristic picks (gba_get_schedule_ex refuses none
    of them); probed by forcing each and asking for a tiny product."""
    return [s for s in gba.list_schedules() if s["kernel"] in (3, 4) and _has_ta(s)]


_HAS_TA = {}


def _has_ta(s):
    import torch
    key = tuple(sorted(s.items()))
    if key not in _HAS_TA:
        a = torch.zeros(8, 8, dtype=torch.float16, device="cuda")
        c = torch.zeros(8, 8, dtype=torch.float16, device="cuda")
        gba.set_schedule(s)
        try:
            gba.gemm_bias_act(a, a, None, c, "none", transpose_a=True)
            _HAS_TA[key] = True
        except gba.GbaError as e:
            assert e.status == 9, e
            _HAS_TA[key] = False
        finally:
            gba.set_schedule(None)
    return _HAS_TA[key]


def sched_id(s):
    return "k%d_%dx%dx%d_s%d_p%d" % (s["kernel"], s["bm"], s["bn"], s["bk"], s["stages"],
                                     s["spread"])


def run(A, B, bias, act, dtype, sched=None, transpose_a=True, transpose_b=False, ws=None):
    import torch
    M = A.shape[1] if transpose_a else A.shape[0]
    N = B.shape[0] if transpose_b else B.shape[1]
    a, b, bb = to_dev(A, dtype), to_dev(B, dtype), to_dev(bias, dtype)
    c = empty((M, N), dtype, fill_bits=0x7E00)   # NaN sentinel: every element must be written
    gba.set_schedule(sched)
    try:
        gba.gemm_bias_act(a, b, bb, c, act, transpose_a=transpose_a, transpose_b=transpose_b,
                          workspace=ws)
    finally:
        gba.set_schedule(None)
    torch.cuda.synchronize()
    return to_bits(c)


def enc_fn(dtype):
    return (lambda v: v.astype(np.float16).view(np.uint16)) if dtype == "f16" else \
        (lambda v: synth.to_bits(v.astype(np.float32), "bf16"))


def int_inputs(M, N, K, dtype, seed, transpose_b=False):
    """At [K, M], B [K, N] (or [N, K]) and bias with entries in {-1, 0, 1} (bias
    in [-8, 8]): every partial sum is an exact fp32 integer."""
    rng = np.random.default_rng(seed)
    enc = enc_fn(dtype)
    At = enc(rng.integers(-1, 2, (K, M)).astype(np.float64))
    B = enc(rng.integers(-1, 2, (N, K) if transpose_b else (K, N)).astype(np.float64))
    bias = enc(rng.integers(-8, 9, N).astype(np.float64))
    return At, B, bias


@pytest.mark.parametrize("transpose_b", [False, True], ids=["kn", "nk"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(256, 256, 256), (8, 8, 8), (40, 40, 24), (136, 136, 72),
                                   (304, 264, 1000), (520, 776, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_exact_integer_bitwise_every_schedule(shape, dtype, transpose_b):
    M, N, K = shape
    At, B, bias = int_inputs(M, N, K, dtype, M + 2 * N + K, transpose_b)
    want = oracle.encode(oracle.gemm_bias_act(At, B, bias, "none", dtype, transpose_a=True,
                                              transpose_b=transpose_b), dtype)
    scheds = ta_schedules()
    assert len(scheds) >= 4   # kernel 4; kernel 3 at 256x128, 128x256, 128x128 s4
    for s in scheds:
        for raster in (0, 1):
            say("tn exact", shape, dtype, transpose_b, sched_id(s), "raster", raster)
            got = run(At, B, bias, "none", dtype, sched=dict(s, raster=raster),
                      transpose_b=transpose_b)
            bad = np.argwhere(got != want)
            assert bad.size == 0, "%s r%d: %d mismatches, first %s" % (
                sched_id(s), raster, len(bad), bad[:3].tolist())


@pytest.mark.parametrize("K", [128, 1000])
def test_persistent_many_tiles_bitwise(K):
    # 17 x 17 tiles of 256 x 256 on a 256-CU grid, ragged M, N (and K = 1000)
    M, N = 4104, 4200
    At, B, bias = int_inputs(M, N, K, "bf16", K + 90)
    want = oracle.encode(oracle.gemm_bias_act(At, B, bias, "relu", "bf16", transpose_a=True,
                                              nthreads=16), "bf16")
    say("tn persistent exact", K)
    got = run(At, B, bias, "relu", "bf16", sched=PERSISTENT)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("act", ACTS)
def test_random_every_schedule_and_same_bits_as_mk_layout(act, dtype):
    M, N, K = 304, 264, 136
    A = synth.random_bits((M, K), dtype, 1)
    B = synth.random_bits((K, N), dtype, 2, scale=0.25)
    bias = synth.random_bits((N,), dtype, 3)
    At = np.ascontiguousarray(A.T)
    W = np.ascontiguousarray(B.T)
    R, S = oracle.gemm_bias_act(At, B, bias, act, dtype, with_abs=True, transpose_a=True)
    for s in ta_schedules():
        say("tn random", act, dtype, sched_id(s))
        got = run(At, B, bias, act, dtype, sched=dict(s))
        rep = compare.check(oracle.decode(got, dtype), R, K=K, dtype=dtype,
                            act=oracle.ACTS[act], S=S)
        assert rep["ok"] and rep["strict_ok"], (sched_id(s), rep)
        mk = run(A, B, bias, act, dtype, sched=dict(s), transpose_a=False)
        assert np.array_equal(got, mk), sched_id(s)
        tt = run(At, W, bias, act, dtype, sched=dict(s), transpose_b=True)
        assert np.array_equal(got, tt), sched_id(s)


@pytest.mark.parametrize("name", ["c3_gelu", "c5_gelu"])
def test_full_size_sampled_rows(name):
    # the workload's A, stored transposed ([K, M])
    w = synth.WORKLOADS[name]
    A, B, bias = synth.make_inputs(w)
    At = np.ascontiguousarray(A.T)
    del A
    rows = synth.sample_rows(w.M, 64, seed=w.seed)
    say("tn full", name, gba.get_schedule(w.M, w.N, w.K, w.act, w.dtype, transpose_a=True))
    got = run(At, B, bias, w.act, w.dtype)
    R, S = oracle.gemm_bias_act(At, B, bias, w.act, w.dtype, rows=rows, with_abs=True,
                                transpose_a=True, nthreads=16)
    rep = compare.check(oracle.decode(got[rows], w.dtype), R, K=w.K, dtype=w.dtype,
                        act=oracle.ACTS[w.act], S=S)
    assert rep["ok"] and rep["strict_ok"], rep
    expmask = 0x7C00 if w.dtype == "f16" else 0x7F80
    assert not np.any((got & expmask) == expmask)


def test_reduced_c4_and_no_bias():
    w = synth.WORKLOADS["c4_relu"]
    A, B, bias = synth.make_inputs(w, M=1000, N=1280, K=1000)
    At = np.ascontiguousarray(A.T)
    say("tn c4 reduced")
    R, S = oracle.gemm_bias_act(At, B, bias, "relu", "f16", with_abs=True, transpose_a=True)
    rep = compare.check(oracle.decode(run(At, B, bias, "relu", "f16"), "f16"), R, K=1000,
                        dtype="f16", act=oracle.ACTS["relu"], S=S)
    assert rep["ok"] and rep["strict_ok"], rep
    for (M, N, K) in [(64, 64, 8), (72, 72, 40), (264, 264, 264)]:
        At = synth.random_bits((K, M), "f16", M)
        B = synth.random_bits((K, N), "f16", N)
        say("tn nobias", M, N, K)
        R, S = oracle.gemm_bias_act(At, B, None, "gelu", "f16", with_abs=True, transpose_a=True)
        rep = compare.check(oracle.decode(run(At, B, None, "gelu", "f16"), "f16"), R, K=K,
                            dtype="f16", act=oracle.ACTS["gelu"], S=S)
        assert rep["ok"] and rep["strict_ok"], rep


def test_short_k_runs_on_the_persistent_schedule():
    # K <= 64: one slice per tile, run by the non-persistent kernel with that tile
    At, B, bias = int_inputs(600, 520, 64, "f16", 5)
    want = oracle.encode(oracle.gemm_bias_act(At, B, bias, "none", "f16", transpose_a=True), "f16")
    say("tn persistent K=64")
    assert np.array_equal(run(At, B, bias, "none", "f16", sched=PERSISTENT), want)


@pytest.mark.parametrize("transpose_b", [False, True], ids=["kn", "nk"])
@pytest.mark.parametrize("shape", [(256, 256, 4096), (136, 264, 2056)],
                         ids=lambda s: "x".join(map(str, s)))
def test_split_k_bitwise_and_equal_to_one_kernel(shape, transpose_b):
    import torch
    M, N, K = shape
    At, B, bias = int_inputs(M, N, K, "bf16", M + N, transpose_b)
    nb = gba.workspace_size(M, N, K, "relu", "bf16", transpose_b=transpose_b, transpose_a=True)
    assert nb > 0, "this shape is expected to split"
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    want = oracle.encode(oracle.gemm_bias_act(At, B, bias, "relu", "bf16", transpose_a=True,
                                              transpose_b=transpose_b, nthreads=16), "bf16")
    say("tn splitk exact", shape, transpose_b, nb)
    got = run(At, B, bias, "relu", "bf16", transpose_b=transpose_b, ws=ws)
    assert np.array_equal(got, want)
    assert np.array_equal(got, run(At, B, bias, "relu", "bf16", transpose_b=transpose_b))
    # random inputs: the split's summation order is the [M, K] split's order at
    # the same schedule (the [M, K] layout's own choice may be another tile, as
    # the 64x64 one has no [K, M] form)
    At = synth.random_bits((K, M), "bf16", 7)
    Bb = synth.random_bits((N, K) if transpose_b else (K, N), "bf16", 8, scale=0.05)
    got = run(At, Bb, bias, "gelu", "bf16", transpose_b=transpose_b, ws=ws)
    A = np.ascontiguousarray(At.T)
    s = gba.get_schedule(M, N, K, "gelu", "bf16", transpose_b=transpose_b, transpose_a=True)
    assert np.array_equal(got, run(A, Bb, bias, "gelu", "bf16", sched=s, transpose_a=False,
                                   transpose_b=transpose_b, ws=ws))
    R, S = oracle.gemm_bias_act(At, Bb, bias, "gelu", "bf16", with_abs=True, transpose_a=True,
                                transpose_b=transpose_b, nthreads=16)
    rep = compare.check(oracle.decode(got, "bf16"), R, K=K, dtype="bf16",
                        act=oracle.ACTS["gelu"], S=S)
    assert rep["ok"] and rep["strict_ok"], rep


def test_gemm_and_degenerate_shapes():
    import torch
    At, B, _ = int_inputs(80, 96, 200, "f16", 8)
    a, b = to_dev(At, "f16"), to_dev(B, "f16")
    c = empty((80, 96), "f16", fill_bits=0x7E00)
    say("tn gemm")
    gba.gemm(a, b, c, transpose_a=True)
    torch.cuda.synchronize()
    want = oracle.encode(oracle.gemm_bias_act(At, B, None, "none", "f16", transpose_a=True), "f16")
    assert np.array_equal(to_bits(c), want)
    bias = synth.random_bits((16,), "f16", 5)
    for act in ACTS:
        say("tn k0", act)
        got = run(np.zeros((0, 8), np.uint16), np.zeros((0, 16), np.uint16), bias, act, "f16")
        want = oracle.encode(np.broadcast_to(oracle.act(oracle.decode(bias), act), (8, 16)), "f16")
        assert np.array_equal(got, want), act
    gba.gemm_bias_act(torch.zeros(8, 0, dtype=torch.float16, device="cuda"),
                      torch.zeros(8, 16, dtype=torch.float16, device="cuda"), None,
                      torch.zeros(0, 16, dtype=torch.float16, device="cuda"), "gelu",
                      transpose_a=True)


def test_schedule_without_the_path_is_refused():
    import torch
    a = torch.zeros(64, 64, dtype=torch.float16, device="cuda")
    c = torch.zeros(64, 64, dtype=torch.float16, device="cuda")
    for s0 in [s for s in gba.list_schedules() if s["kernel"] in (0, 1, 2)][:2]:
        gba.set_schedule(s0)
        try:
            with pytest.raises(gba.GbaError) as e:
                gba.gemm_bias_act(a, a, None, c, "none", transpose_a=True)
            assert e.value.status == 9
        finally:
            gba.set_schedule(None)
    with pytest.raises(gba.GbaError) as e:   # M not a multiple of 8
        gba.gemm_bias_act(torch.zeros(64, 60, dtype=torch.float16, device="cuda"), a, None,
                          torch.zeros(60, 64, dtype=torch.float16, device="cuda"), "none",
                          transpose_a=True)
    assert e.value.status == 5
    # the built-in choice for A stored (K,M) is the plain layout's when that has
    # the path (else the next larger tile: 1024^2 outputs take 64x64 tiles,
    # which have none)
    for (M, N, K) in [(4096, 4096, 4096), (3000 // 8 * 8, 5120, 1000), (1024, 1024, 1024)]:
        s = gba.get_schedule(M, N, K, "gelu", "f16", transpose_a=True)
        s0 = gba.get_schedule(M, N, K, "gelu", "f16")
        assert _has_ta(s) and (s == s0) == _has_ta(s0)


def test_autotune_transpose_a_is_cached_under_its_own_key(tmp_path, monkeypatch):
    import json
    import torch
    monkeypatch.setenv("GBA_CACHE_DIR", str(tmp_path))
    M, N, K = 512, 512, 256
    At = synth.random_bits((K, M), "bf16", 1)
    B = synth.random_bits((K, N), "bf16", 2)
    bias = synth.random_bits((N,), "bf16", 3)
    a, b, bb = to_dev(At, "bf16"), to_dev(B, "bf16"), to_dev(bias, "bf16")
    c = empty((M, N), "bf16")
    say("tn autotune")
    best, ms = gba.autotune(a, b, bb, c, "relu", transpose_a=True)
    torch.cuda.synchronize()
    assert ms > 0 and best["kernel"] in (3, 4) and _has_ta(best)
    R, S = oracle.gemm_bias_act(At, B, bias, "relu", "bf16", with_abs=True, transpose_a=True)
    rep = compare.check(oracle.decode(to_bits(c), "bf16"), R, K=K, dtype="bf16",
                        act=oracle.ACTS["relu"], S=S)
    assert rep["ok"] and rep["strict_ok"], rep
    keys = [e["key"] for e in json.load(open(tmp_path / "schedules.json"))["entries"]]
    assert any(k.endswith("|bf16|relu|tn|512|512|256") for k in keys)
    assert gba.get_schedule(M, N, K, "relu", "bf16", transpose_a=True) == best
