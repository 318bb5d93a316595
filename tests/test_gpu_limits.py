"""Entry points at the sizes the header gives as limits, through the C ABI.

K = 2^21 (every compiled-in schedule, both B layouts, A stored [K, M] too,
split-K, 8-bit inputs),
N = 2^23 (2^30 for bias_act), M = 2^31 - 1 (the largest tile offsets; the
last tile is ragged) and, with A stored [K, M], M = 2^23. Inputs are small integers, so every sum is exact in fp32
and the results must equal the fp64 oracle's bitwise (relu, or no activation).

At M = 2^31 - 1 and at N = 2^30 the inputs repeat with period P along the large
dimension, so the exact result does too: the oracle computes the first P rows
(columns), every later one must equal its copy P earlier, bit for bit, over
the whole output, and a guard region past the output must keep its fill.
"""
import numpy as np
import pytest

import oracle
import synth
import tiled_dense_gemm_bias_amd as gba
from tests.gpu_util import empty, say, to_bits, to_dev, torch_dtype

pytestmark = pytest.mark.gpu

KMAX, NMAX, MMAX = 1 << 21, 1 << 23, (1 << 31) - 1
NMAX_BIAS_ACT = 1 << 30
P = 4099            # prime period of the repeated inputs
SENT = 0x7E00       # output fill: no exact integer result has these bits
GUARD = 1 << 16     # elements past the output that must keep the fill


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    gba.set_schedule(None)
    torch.cuda.empty_cache()


def enc(v, dtype):
    """Small integers -> fp16 / bf16 bit patterns (exact)."""
    v = np.asarray(v)
    if dtype == "f16":
        return v.astype(np.float16).view(np.uint16)
    return synth.to_bits(v.astype(np.float32), "bf16")


def enc8(v, fmt):
    return synth.f32_to_fp8_bits(np.asarray(v, dtype=np.float32), fmt)


def dev8(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits)).to("cuda:0")


def sched_id(s):
    return "k%d_%dx%dx%d_s%d_l%d_p%d" % (s["kernel"], s["bm"], s["bn"], s["bk"], s["stages"],
                                         s["loaders"], s["spread"])


def first_mismatch(got, want):
    bad = np.argwhere(got != want)
    return "%d mismatches, first %s" % (len(bad), bad[:3].tolist())


def run_forced(sched, a, b, bias, c, act, transpose_b):
    """gemm_bias_act with schedule `sched` forced; False if that kernel has no
    path for this B layout (GBA_ERR_SCHEDULE)."""
    gba.set_schedule(sched)
    try:
        gba.gemm_bias_act(a, b, bias, c, act, transpose_b=transpose_b)
    except gba.GbaError as e:
        if transpose_b and e.status == 9:
            return False
        raise
    finally:
        gba.set_schedule(None)
    return True


# ------------------------------------------------------------- K = 2^21 ----

@pytest.fixture(scope="module")
def kmax():
    """37 x 136 x 2^21 in {-1, 0, 1}, bias in [-8, 8]: ragged M and N, sums |.| <= 2^21."""
    rng = np.random.default_rng(21)
    A = rng.integers(-1, 2, (37, KMAX), dtype=np.int8)
    W = rng.integers(-1, 2, (136, KMAX), dtype=np.int8)
    bias = rng.integers(-8, 9, 136, dtype=np.int8)
    return A, W, bias


_kmax_cache = {}


def kmax_case(kmax, dtype):
    """(device A, B [K,N], W [N,K], bias, oracle bits) for dtype, built once."""
    if dtype not in _kmax_cache:
        A, W, bias = kmax
        Ab, Wb, bb = enc(A, dtype), enc(W, dtype), enc(bias, dtype)
        want = oracle.encode(oracle.gemm_bias_act(Ab, Wb, bb, "relu", dtype, transpose_b=True,
                                                  nthreads=16), dtype)
        _kmax_cache[dtype] = (to_dev(Ab, dtype), to_dev(np.ascontiguousarray(Wb.T), dtype),
                              to_dev(Wb, dtype), to_dev(bb, dtype), want)
    return _kmax_cache[dtype]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_max_k_every_schedule_both_layouts(kmax, dtype):
    a, b, w, bias, want = kmax_case(kmax, dtype)
    M, N = want.shape
    ran = 0
    for s in gba.list_schedules():
        for tb in (False, True):
            c = empty((M, N), dtype, fill_bits=SENT)
            say("max K", dtype, sched_id(s), "NK" if tb else "KN")
            if not run_forced(s, a, w if tb else b, bias, c, "relu", tb):
                continue
            got = to_bits(c)
            assert np.array_equal(got, want), (sched_id(s), tb, first_mismatch(got, want))
            ran += 1
    assert ran >= len(gba.list_schedules()) + 2   # every kernel KN, kernels 3 and 4 NK too


@pytest.mark.parametrize("transpose_b", [False, True], ids=["kn", "nk"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_max_k_split(kmax, dtype, transpose_b):
    import torch
    a, b, w, bias, want = kmax_case(kmax, dtype)
    M, N = want.shape
    nb = gba.workspace_size(M, N, KMAX, "relu", dtype, transpose_b=transpose_b)
    assert nb > 0, "37 x 136 x 2^21 is expected to split"
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    c = empty((M, N), dtype, fill_bits=SENT)
    say("max K split", dtype, transpose_b, nb)
    gba.gemm_bias_act(a, w if transpose_b else b, bias, c, "relu", transpose_b=transpose_b,
                      workspace=ws)
    got = to_bits(c)
    assert np.array_equal(got, want), first_mismatch(got, want)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_max_k_transpose_a_every_schedule_and_split(kmax, dtype):
    # A stored [K, M] at K = 2^21, the largest slice count. M must be a multiple
    # of 8 in that layout, so A gets three more rows, copies of rows 0..2, and C's
    # rows 37..39 must equal rows 0..2.
    import torch
    a, b, w, bias, want37 = kmax_case(kmax, dtype)
    want = np.concatenate([want37, want37[:3]])
    M, N = want.shape
    at = torch.cat([a, a[:3]]).t().contiguous()
    ran = 0
    for s in gba.list_schedules():
        for tb in (False, True):
            c = empty((M, N), dtype, fill_bits=SENT)
            say("max K transpose_A", dtype, sched_id(s), "NK" if tb else "KN")
            gba.set_schedule(s)
            try:
                gba.gemm_bias_act(at, w if tb else b, bias, c, "relu", transpose_b=tb,
                                  transpose_a=True)
            except gba.GbaError as e:
                if e.status == 9:   # no transpose_A path in this kernel
                    continue
                raise
            finally:
                gba.set_schedule(None)
            got = to_bits(c)
            assert np.array_equal(got, want), (sched_id(s), tb, first_mismatch(got, want))
            ran += 1
    # kernel 4 and kernel 3 at 256x128, 128x256 and 128x128 s4, both B layouts
    assert ran >= 8
    for tb in (False, True):
        nb = gba.workspace_size(M, N, KMAX, "relu", dtype, transpose_b=tb, transpose_a=True)
        assert nb > 0, "40 x 136 x 2^21 is expected to split"
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        c = empty((M, N), dtype, fill_bits=SENT)
        say("max K transpose_A split", dtype, tb, nb)
        gba.gemm_bias_act(at, w if tb else b, bias, c, "relu", transpose_b=tb,
                          transpose_a=True, workspace=ws)
        got = to_bits(c)
        assert np.array_equal(got, want), (tb, first_mismatch(got, want))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_max_k_fp8_one_kernel_and_split(kmax, fmt):
    import torch
    A, W, bias = kmax
    A8, W8, bb = enc8(A, fmt), enc8(W, fmt), enc(bias, "bf16")
    want = oracle.encode(oracle.gemm_bias_act_fp8(A8, W8, bb, 0.5, "relu", fmt, "bf16",
                                                  nthreads=16), "bf16")
    M, N = want.shape
    a, w, bias_d = dev8(A8), dev8(W8), to_dev(bb, "bf16")
    nb = gba.workspace_size(M, N, KMAX, "relu", "bf16", fp8=True)
    assert nb > 0
    for ws in (None, torch.empty(nb, dtype=torch.uint8, device="cuda")):
        c = empty((M, N), "bf16", fill_bits=SENT)
        say("max K fp8", fmt, "split" if ws is not None else "one kernel")
        gba.gemm_bias_act_fp8(a, w, bias_d, c, 0.5, "relu", fmt, workspace=ws)
        got = to_bits(c)
        assert np.array_equal(got, want), (ws is not None, first_mismatch(got, want))


# ------------------------------------------------------------- N = 2^23 ----

def test_max_n_every_schedule_both_layouts():
    M, N, K = 3, NMAX, 72   # 32768 column tiles; K = 72: a 64-deep slice and a tail
    rng = np.random.default_rng(23)
    A = enc(rng.integers(-1, 2, (M, K), dtype=np.int8), "f16")
    W = enc(rng.integers(-1, 2, (N, K), dtype=np.int8), "f16")
    bias = enc(rng.integers(-8, 9, N, dtype=np.int8), "f16")
    want = oracle.encode(oracle.gemm_bias_act(A, W, bias, "relu", "f16", transpose_b=True,
                                              nthreads=16), "f16")
    a, w, bb = to_dev(A, "f16"), to_dev(W, "f16"), to_dev(bias, "f16")
    b = to_dev(np.ascontiguousarray(W.T), "f16")
    for s in [None] + gba.list_schedules():
        for tb in (False, True):
            c = empty((M, N), "f16", fill_bits=SENT)
            say("max N", "heuristic" if s is None else sched_id(s), "NK" if tb else "KN")
            if not run_forced(s, a, w if tb else b, bb, c, "relu", tb):
                continue
            got = to_bits(c)
            assert np.array_equal(got, want), (s, tb, first_mismatch(got, want))


def test_max_n_fp8():
    M, N, K = 3, NMAX, 144   # a 128-deep slice and a 16-deep tail
    rng = np.random.default_rng(24)
    A8 = enc8(rng.integers(-1, 2, (M, K), dtype=np.int8), "e4m3")
    W8 = enc8(rng.integers(-1, 2, (N, K), dtype=np.int8), "e4m3")
    bias = enc(rng.integers(-8, 9, N, dtype=np.int8), "f16")
    want = oracle.encode(oracle.gemm_bias_act_fp8(A8, W8, bias, 0.5, "relu", "e4m3", "f16",
                                                  nthreads=16), "f16")
    c = empty((M, N), "f16", fill_bits=SENT)
    say("max N fp8")
    gba.gemm_bias_act_fp8(dev8(A8), dev8(W8), to_dev(bias, "f16"), c, 0.5, "relu", "e4m3")
    got = to_bits(c)
    assert np.array_equal(got, want), first_mismatch(got, want)


# --------------------------------------------- repeated inputs, full check ----

def repeat_rows(t, M):
    """Rows of t (P of them) repeated to M rows, contiguous on the device."""
    reps = -(-M // t.shape[0])
    return t.repeat(reps, *([1] * (t.dim() - 1)))[:M].contiguous()


def refill(flat):
    import torch
    flat.view(torch.int16).fill_(int(np.uint16(SENT).view(np.int16)))


def guarded(M, N, dtype):
    """A fill-initialised flat buffer and its leading (M, N) view."""
    import torch
    flat = torch.empty(M * N + GUARD, dtype=torch_dtype(dtype), device="cuda")
    refill(flat)
    return flat, flat[: M * N].view(M, N)


def check_row_periodic(flat, C, want_head):
    """C's first P rows are want_head bitwise; row r equals row r - P for every
    later r; the guard past C keeps the fill."""
    import torch
    M, N = C.shape
    head = to_bits(C[:P])
    assert np.array_equal(head, want_head), first_mismatch(head, want_head)
    Ci = C.view(torch.int16)
    step = 1 << 24
    for r0 in range(P, M, step):
        r1 = min(M, r0 + step)
        same = torch.equal(Ci[r0:r1], Ci[r0 - P:r1 - P])
        if not same:
            rows = (Ci[r0:r1] != Ci[r0 - P:r1 - P]).any(dim=1).nonzero()
            raise AssertionError("row %d differs from row %d" % (r0 + int(rows[0]),
                                                                r0 + int(rows[0]) - P))
    g = flat.view(torch.int16)[M * N:]
    assert bool((g == int(np.uint16(SENT).view(np.int16))).all()), "write past the end of C"


@pytest.fixture
def _free():
    yield
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_max_m_every_schedule_both_layouts(_free):
    M, N, K = MMAX, 8, 8   # 32 GiB A, 32 GiB C; the last 256-row tile has 255 rows
    rng = np.random.default_rng(31)
    T = enc(rng.integers(-1, 2, (P, K), dtype=np.int8), "f16")
    W = enc(rng.integers(-1, 2, (N, K), dtype=np.int8), "f16")
    bias = enc(rng.integers(-8, 9, N, dtype=np.int8), "f16")
    want = oracle.encode(oracle.gemm_bias_act(T, W, bias, "relu", "f16", transpose_b=True),
                         "f16")
    say("max M: building A", M, K)
    a = repeat_rows(to_dev(T, "f16"), M)
    w, bb = to_dev(W, "f16"), to_dev(bias, "f16")
    b = to_dev(np.ascontiguousarray(W.T), "f16")
    flat, c = guarded(M, N, "f16")
    for s in [None] + gba.list_schedules():
        for tb in (False, True):
            refill(flat)
            say("max M", "heuristic" if s is None else sched_id(s), "NK" if tb else "KN")
            if not run_forced(s, a, w if tb else b, bb, c, "relu", tb):
                continue
            check_row_periodic(flat, c, want)


def test_max_m_fp8(_free):
    M, N, K = MMAX, 8, 16
    rng = np.random.default_rng(32)
    T8 = enc8(rng.integers(-1, 2, (P, K), dtype=np.int8), "e5m2")
    W8 = enc8(rng.integers(-1, 2, (N, K), dtype=np.int8), "e5m2")
    bias = enc(rng.integers(-8, 9, N, dtype=np.int8), "bf16")
    want = oracle.encode(oracle.gemm_bias_act_fp8(T8, W8, bias, 0.5, "relu", "e5m2", "bf16"),
                         "bf16")
    say("max M fp8: building A", M, K)
    a = repeat_rows(dev8(T8), M)
    flat, c = guarded(M, N, "bf16")
    say("max M fp8")
    gba.gemm_bias_act_fp8(a, dev8(W8), to_dev(bias, "bf16"), c, 0.5, "relu", "e5m2")
    check_row_periodic(flat, c, want)


def test_max_m_bias_act(_free):
    M, N = MMAX, 8
    rng = np.random.default_rng(33)
    T = enc(rng.integers(-64, 65, (P, N), dtype=np.int8), "bf16")
    bias = enc(rng.integers(-8, 9, N, dtype=np.int8), "bf16")
    want = oracle.encode(oracle.bias_act(T, bias, "relu", "bf16"), "bf16")
    say("max M bias_act: building X", M, N)
    x = repeat_rows(to_dev(T, "bf16"), M)
    flat, y = guarded(M, N, "bf16")
    say("max M bias_act")
    gba.bias_act(x, to_dev(bias, "bf16"), y, "relu")
    check_row_periodic(flat, y, want)


def test_max_n_bias_act(_free):
    import torch
    M, N = 2, NMAX_BIAS_ACT
    Q = 4096   # bias period; X repeats every P columns, so the result every P * Q
    rng = np.random.default_rng(34)
    xs = enc(rng.integers(-64, 65, P, dtype=np.int8), "f16")
    bs = enc(rng.integers(-8, 9, Q, dtype=np.int8), "f16")
    L = P * Q
    cols = np.arange(L)
    X_head = np.stack([xs[cols % P], xs[(cols + 7) % P]])   # row 1: X shifted by 7 columns
    want = oracle.encode(oracle.bias_act(X_head, bs[cols % Q], "relu", "f16"), "f16")
    say("max N bias_act: building X", M, N)
    xd = to_dev(xs, "f16")
    x = torch.stack([repeat_rows(xd, N), repeat_rows(torch.roll(xd, -7), N)])
    bias = repeat_rows(to_dev(bs, "f16"), N)
    flat, y = guarded(M, N, "f16")
    say("max N bias_act")
    gba.bias_act(x, bias, y, "relu")
    head = to_bits(y[:, :L])
    assert np.array_equal(head, want), first_mismatch(head, want)
    yi = y.view(torch.int16)
    step = 1 << 27
    for c0 in range(L, N, step):
        c1 = min(N, c0 + step)
        assert torch.equal(yi[:, c0:c1], yi[:, c0 - L:c1 - L]), "columns %d..%d" % (c0, c1)
    g = flat.view(torch.int16)[M * N:]
    assert bool((g == int(np.uint16(SENT).view(np.int16))).all()), "write past the end of Y"


def test_max_m_transpose_a_every_schedule_both_layouts(_free):
    # A stored [K, M]: M is then a row pitch, limited to 2^23 like N. At's columns
    # repeat with period P, so C's rows do; K = 72 is a 64-deep slice and a tail,
    # N = 24 a ragged column tile.
    import torch
    M, N, K = NMAX, 24, 72
    rng = np.random.default_rng(35)
    T = enc(rng.integers(-1, 2, (K, P), dtype=np.int8), "bf16")   # At's first P columns
    W = enc(rng.integers(-1, 2, (N, K), dtype=np.int8), "bf16")
    bias = enc(rng.integers(-8, 9, N, dtype=np.int8), "bf16")
    want = oracle.encode(oracle.gemm_bias_act(T, W, bias, "relu", "bf16", transpose_a=True,
                                              transpose_b=True), "bf16")
    say("max M transpose_A: building At", K, M)
    td = to_dev(T, "bf16")
    at = td.repeat(1, -(-M // P))[:, :M].contiguous()
    del td
    w, bb = to_dev(W, "bf16"), to_dev(bias, "bf16")
    b = to_dev(np.ascontiguousarray(W.T), "bf16")
    flat, c = guarded(M, N, "bf16")
    ran = 0
    for s in [None] + gba.list_schedules():
        for tb in (False, True):
            refill(flat)
            say("max M transpose_A", "heuristic" if s is None else sched_id(s),
                "NK" if tb else "KN")
            gba.set_schedule(s)
            try:
                gba.gemm_bias_act(at, w if tb else b, bb, c, "relu", transpose_b=tb,
                                  transpose_a=True)
            except gba.GbaError as e:
                if s is not None and e.status == 9:   # no transpose_A path in this kernel
                    continue
                raise
            finally:
                gba.set_schedule(None)
            torch.cuda.synchronize()
            check_row_periodic(flat, c, want)
            ran += 1
    # the heuristic, kernel 4 and kernel 3 at 256x128, 128x256, 128x128 s4; both B layouts
    assert ran >= 10
