"""Pins for the CPU oracle: facts that do not come from the oracle itself.

Each test checks one part of oracle/gemm_oracle.c against something fixed
independently of it: exact rational arithmetic on tiny inputs, closed forms
(identity, permutation, zero, rank-1, exact integers), numpy's float16 cast and
float64 matmul, mpmath's arbitrary-precision erf/exp, and tabulated values in
tests/golden/. They are chosen so that a dropped term, a wrong index, a
transposed operand, a wrong sign or a misplaced bias fails at least one of
them (test_oracle_mutants.py plants such mistakes and checks exactly that).
"""
from fractions import Fraction
import math
import os

import mpmath
import numpy as np
import pytest

import oracle
from oracle import compare
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
mpmath.mp.dps = 40


def f16(vals):
    return np.asarray(vals, dtype=np.float64).astype(np.float16).view(np.uint16)


# ---------------------------------------------------------------- decoders --

F16_KNOWN = {
    0x0000: 0.0, 0x3C00: 1.0, 0xBC00: -1.0, 0x4000: 2.0, 0xC000: -2.0,
    0x3800: 0.5, 0x3555: 0.333251953125, 0x7BFF: 65504.0, 0x0400: 2.0 ** -14,
    0x0001: 2.0 ** -24, 0x03FF: 1023 * 2.0 ** -24, 0x7C00: math.inf,
    0xFC00: -math.inf, 0x4248: 3.140625,
}
BF16_KNOWN = {
    0x0000: 0.0, 0x3F80: 1.0, 0xBF80: -1.0, 0x4000: 2.0, 0x4049: 3.140625,
    0x3EAB: 0.333984375, 0x7F7F: (2 - 2.0 ** -7) * 2.0 ** 127, 0x0080: 2.0 ** -126,
    0x0001: 2.0 ** -133, 0x7F80: math.inf, 0xFF80: -math.inf,
}


def test_decode_f16_known_bit_patterns(orc):
    bits = np.array(list(F16_KNOWN), dtype=np.uint16)
    got = orc.decode(bits, "f16")
    assert list(got) == list(F16_KNOWN.values())
    assert math.copysign(1.0, orc.decode(np.array([0x8000], np.uint16), "f16")[0]) == -1.0


def test_decode_bf16_known_bit_patterns(orc):
    bits = np.array(list(BF16_KNOWN), dtype=np.uint16)
    assert list(orc.decode(bits, "bf16")) == list(BF16_KNOWN.values())


def test_decode_f16_all_patterns_match_numpy(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.decode(bits, "f16")
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_decode_bf16_all_patterns_are_top_half_of_float32(orc):
    # bfloat16 is by definition the upper 16 bits of an IEEE binary32.
    bits = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        ref = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    got = orc.decode(bits.astype(np.uint16), "bf16")
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ---------------------------------------------------------------- encoders --

def test_encode_f16_matches_numpy_rne(orc):
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(200_000) * np.exp2(rng.integers(-30, 17, 200_000)),
        [0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e9, -1e9, 2.0 ** -25, 2.0 ** -25 * 1.0001,
         3 * 2.0 ** -26, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 2.0 ** -14 - 2.0 ** -25],
    ])
    got = orc.encode(x, "f16")
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)   # numpy: float64 -> half, RNE
    assert np.array_equal(got, ref)


def test_encode_f16_ties_go_to_even(orc):
    # 1 + 2^-11 is exactly half-way between 1 and 1 + 2^-10: even is 1.0.
    # 1 + 3*2^-11 is half-way between 1+2^-10 (odd) and 1+2^-9 (even).
    got = orc.encode([1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 2.0 ** -25, 3 * 2.0 ** -25], "f16")
    assert list(got) == [0x3C00, 0x3C02, 0x0000, 0x0002]


def _nearest_bf16_exact(x: float) -> int:
    """Brute force: the bf16 pattern nearest to x, ties to even, in exact rationals."""
    fx = Fraction(x)
    cand = []
    base = int((np.array([x], np.float32).view(np.uint32)[0] >> 16))
    for b in range(max(base - 2, 0), min(base + 3, 0x7F80)):
        v = Fraction((np.array([b << 16], np.uint32).view(np.float32)[0]).item())
        cand.append((abs(v - fx), b & 1, b))
    cand.sort()
    return cand[0][2]


def test_encode_bf16_against_exact_rational_nearest(orc):
    rng = np.random.default_rng(11)
    x = np.abs(rng.standard_normal(3000) * np.exp2(rng.integers(-40, 40, 3000)))
    # exact ties: midpoints between adjacent bf16 values
    lo = rng.integers(0x3000, 0x5000, 200).astype(np.uint32)
    mids = ((lo << 16).view(np.float32).astype(np.float64)
            + ((lo + 1) << 16).view(np.float32).astype(np.float64)) / 2
    x = np.concatenate([x, mids])
    got = orc.encode(x, "bf16")
    want = np.array([_nearest_bf16_exact(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, want)
    assert np.array_equal(orc.encode(-x, "bf16"), want | 0x8000)


def test_encode_decode_round_trip_every_finite_pattern(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for dt, expmask in (("f16", 0x7C00), ("bf16", 0x7F80)):
        finite = bits[(bits & expmask) != expmask]
        back = orc.encode(orc.decode(finite, dt), dt)
        assert np.array_equal(back, finite), dt


def test_encode_overflow_to_inf(orc):
    assert list(orc.encode([65520.0, -70000.0], "f16")) == [0x7C00, 0xFC00]
    big = (2 - 2.0 ** -8) * 2.0 ** 127      # half-way above bf16's max: rounds to inf
    assert list(orc.encode([big, -big], "bf16")) == [0x7F80, 0xFF80]


# ------------------------------------------------------------- epilogues --

def _golden_table():
    rows = []
    with open(os.path.join(GOLDEN, "erf_phi_table.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].split()
            if line:
                rows.append((line[0], float(line[1]), float(line[2])))
    return rows


def test_golden_table_is_consistent_with_mpmath():
    for kind, x, v in _golden_table():
        ref = mpmath.erf(x) if kind == "erf" else mpmath.ncdf(x)
        assert abs(float(ref) - v) < 2e-16 * max(1, abs(v)) * 4, (kind, x, v)


def test_gelu_matches_tabulated_phi(orc):
    for kind, x, v in _golden_table():
        if kind == "phi":
            got = orc.act([x, -x], "gelu")
            assert got[0] == pytest.approx(x * v, rel=1e-14, abs=0)
            assert got[1] == pytest.approx(-x * (1 - v), rel=1e-12, abs=0)
        else:
            # erf(x) = 2 Phi(x sqrt2) - 1 = 2 GELU(x sqrt2) / (x sqrt2) - 1
            z = x * math.sqrt(2)
            assert 2 * orc.act([z], "gelu")[0] / z - 1 == pytest.approx(v, rel=1e-14)


def test_gelu_closed_forms(orc):
    assert orc.act([0.0], "gelu")[0] == 0.0
    assert orc.act([1.0], "gelu")[0] == pytest.approx(0.8413447460685429, rel=1e-15)
    x = np.linspace(-12, 12, 2401)
    g = orc.act(x, "gelu")
    gm = orc.act(-x, "gelu")
    # Phi(-z) = 1 - Phi(z)  =>  GELU(-x) = GELU(x) - x
    assert np.all(np.abs(gm - (g - x)) <= 4e-15 * np.maximum(1, np.abs(x)))
    big = x >= 10
    np.testing.assert_array_equal(g[big], x[big])   # Phi(10) = 1 - 7.6e-24


def test_activations_at_non_finite_inputs(orc):
    """At +-inf each activation takes its limit (mpmath's limit of the formula
    at +-1e6 stands for it: every limit is reached there to double precision),
    and a NaN input gives NaN (ReLU: 0, max(NaN, 0) read as IEEE maxNum, the
    hardware max). GELU(-inf) and tanh-GELU(-inf) are 0, not the
    -inf * 0 = NaN that the formulas give when evaluated at the infinity."""
    lim = {"none": (math.inf, -math.inf), "relu": (math.inf, 0.0), "sigmoid": (1.0, 0.0),
           "gelu": (math.inf, 0.0), "softplus": (math.inf, 0.0), "gelu_tanh": (math.inf, 0.0)}
    big = mpmath.mpf(10) ** 6
    mp = {"sigmoid": lambda v: 1 / (1 + mpmath.exp(-v)), "gelu": lambda v: v * mpmath.ncdf(v),
          "softplus": lambda v: mpmath.log(1 + mpmath.exp(v)),
          "gelu_tanh": lambda v: v / 2 * (1 + mpmath.tanh(mpmath.sqrt(2 / mpmath.pi)
                                                        * (v + mpmath.mpf("0.044715") * v ** 3)))}
    for act, (hi, lo) in lim.items():
        got = orc.act([math.inf, -math.inf, math.nan], act)
        assert got[0] == hi and got[1] == lo, (act, got)
        if act == "relu":
            assert got[2] == 0.0   # max(z, 0) as IEEE maxNum: the number wins over NaN
        else:
            assert math.isnan(got[2]), act
        if act in mp:
            # the finite side of each limit, from the formula itself
            assert abs(float(mp[act](-big)) - lo) < 1e-300, act
            if math.isfinite(hi):
                assert abs(float(mp[act](big)) - hi) < 1e-15, act
            else:
                assert float(mp[act](big)) > 1e5, act


def test_gelu_dense_grid_against_mpmath(orc):
    x = np.concatenate([np.linspace(-40, 40, 4001), np.geomspace(1e-300, 1e3, 500)])
    x = np.concatenate([x, -x])
    got = orc.act(x, "gelu")
    ref = np.array([float(mpmath.mpf(v) * mpmath.ncdf(v)) for v in x])
    # Deep in the left tail Phi(z) ~ exp(-z^2/2): the rounding of z/sqrt(2) alone
    # is amplified by ~z^2, so the relative bound grows as (1 + z^2) * 1e-15.
    rel = np.abs(got - ref) / np.maximum(np.abs(ref), 1e-300)
    assert np.all(rel <= np.maximum(1e-13, (1 + x * x) * 1e-15))


def test_sigmoid_closed_forms_and_mpmath(orc):
    assert orc.act([0.0], "sigmoid")[0] == 0.5
    assert orc.act([math.log(3.0)], "sigmoid")[0] == pytest.approx(0.75, rel=1e-15)
    x = np.linspace(-700, 700, 7001)
    s = orc.act(x, "sigmoid")
    np.testing.assert_allclose(s + orc.act(-x, "sigmoid"), 1.0, rtol=0, atol=2.3e-16)
    ref = np.array([float(1 / (1 + mpmath.exp(-mpmath.mpf(v)))) for v in x])
    np.testing.assert_allclose(s, ref, rtol=1e-14, atol=0)


def test_relu_and_identity(orc):
    x = np.linspace(-5, 5, 1001)
    r = orc.act(x, "relu")
    np.testing.assert_array_equal(r - orc.act(-x, "relu"), x)
    np.testing.assert_array_equal(r, np.where(x > 0, x, 0.0))
    np.testing.assert_array_equal(orc.act(x, "none"), x)


def test_softplus_closed_forms_and_mpmath(orc):
    # the pages' elementwise template: log(1 + e^z)
    assert orc.act([0.0], "softplus")[0] == pytest.approx(math.log(2.0), rel=1e-16)
    assert orc.act([math.log(3.0)], "softplus")[0] == pytest.approx(2 * math.log(2.0), rel=1e-15)
    assert orc.act([math.log(math.e - 1)], "softplus")[0] == pytest.approx(1.0, rel=1e-15)
    x = np.concatenate([np.linspace(-60, 60, 2401), np.geomspace(1e-8, 700, 400)])
    x = np.concatenate([x, -x])
    sp = orc.act(x, "softplus")
    ref = np.array([float(mpmath.log1p(mpmath.exp(mpmath.mpf(v)))) for v in x])
    np.testing.assert_allclose(sp, ref, rtol=4e-16, atol=0)
    # log(1+e^z) - log(1+e^-z) = z
    np.testing.assert_allclose(sp - orc.act(-x, "softplus"), x, rtol=2e-16, atol=2e-16)


def test_gelu_tanh_against_torch_and_identities(orc):
    # the tanh form of GELU against an independent implementation (torch's CPU
    # float64 gelu with approximate="tanh")
    torch = pytest.importorskip("torch")
    x = np.concatenate([np.linspace(-12, 12, 4801), np.geomspace(1e-8, 1e4, 400)])
    x = np.concatenate([x, -x])
    g = orc.act(x, "gelu_tanh")
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    # torch forms 0.5 z (1 + tanh(y)) directly, which cancels for z << 0: its
    # absolute error there is up to |z| ulp(1)/2; the oracle avoids the cancellation.
    assert np.all(np.abs(g - ref) <= 1e-14 * np.abs(ref) + 2.3e-16 * np.abs(x))
    assert orc.act([0.0], "gelu_tanh")[0] == 0.0
    # tanh is odd, so g(z) - g(-z) = z
    np.testing.assert_allclose(g - orc.act(-x, "gelu_tanh"), x, rtol=1e-15, atol=1e-15)
    # an approximation of z * Phi(z): within 1e-3 of the erf form everywhere
    assert np.abs(g - orc.act(x, "gelu")).max() < 1e-3


# ------------------------------------------------------------ 8-bit inputs --

E4M3_KNOWN = {0x00: 0.0, 0x38: 1.0, 0xB8: -1.0, 0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9,
              0x07: 7 * 2.0 ** -9, 0x40: 2.0, 0x3C: 1.5, 0x77: 240.0}
E5M2_KNOWN = {0x00: 0.0, 0x3C: 1.0, 0xBC: -1.0, 0x7B: 57344.0, 0x04: 2.0 ** -14, 0x01: 2.0 ** -16,
              0x7C: math.inf, 0xFC: -math.inf, 0x3E: 1.5, 0x40: 2.0}


def test_fp8_decoders_known_values_and_every_pattern_against_torch(orc):
    torch = pytest.importorskip("torch")
    for fmt, known, tdt in (("e4m3", E4M3_KNOWN, torch.float8_e4m3fn),
                            ("e5m2", E5M2_KNOWN, torch.float8_e5m2)):
        bits = np.array(list(known), dtype=np.uint8)
        assert list(orc.decode_fp8(bits, fmt)) == list(known.values()), fmt
        allb = np.arange(256, dtype=np.uint16).astype(np.uint8)
        ref = torch.from_numpy(allb).view(tdt).to(torch.float64).numpy()
        got = orc.decode_fp8(allb, fmt)
        np.testing.assert_array_equal(got, ref)
    assert np.isnan(orc.decode_fp8(np.array([0x7F, 0xFF], np.uint8), "e4m3")).all()


def _fp8_bits(rng, shape, fmt):
    """Random finite 8-bit patterns of moderate magnitude."""
    b = rng.integers(0, 256, size=shape).astype(np.uint8)
    top = 0x70 if fmt == "e4m3" else 0x78      # cap the exponent: no NaN / inf
    return (b & np.uint8(0x80)) | np.minimum(b & np.uint8(0x7F), np.uint8(top - 1))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 5, 7), (4, 3, 33)])
def test_fp8_gemm_equals_exact_rational_sum(orc, fmt, shape):
    M, N, K = shape
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    A, W = _fp8_bits(rng, (M, K), fmt), _fp8_bits(rng, (N, K), fmt)
    bias = synth.random_bits((N,), "bf16", 7)
    scale = 0.375
    Av, Wv, bv = orc.decode_fp8(A, fmt), orc.decode_fp8(W, fmt), orc.decode(bias, "bf16")
    got, S = orc.gemm_bias_act_fp8(A, W, bias, scale, "none", fmt, "bf16", with_abs=True)
    for i in range(M):
        for j in range(N):
            s = sum((Fraction(Av[i, k]) * Fraction(Wv[j, k]) for k in range(K)), Fraction(0))
            exact = Fraction(scale) * s + Fraction(bv[j])
            bound = (K + 2) * 2.0 ** -53 * S[i, j]
            assert abs(Fraction(got[i, j]) - exact) <= Fraction(bound), (i, j)


def test_fp8_integer_matmul_scale_and_bias_order(orc):
    rng = np.random.default_rng(9)
    M, N, K = 21, 19, 150
    Ai, Wi = rng.integers(-4, 5, (M, K)), rng.integers(-4, 5, (N, K))
    torch = pytest.importorskip("torch")
    enc = lambda v: torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    A, W = enc(Ai), enc(Wi)
    bi = rng.integers(-8, 9, N)
    bias = f16(bi)
    for scale in (1.0, 0.125, -3.0):
        got = orc.gemm_bias_act_fp8(A, W, bias, scale, "none", "e4m3", "f16")
        np.testing.assert_array_equal(got, scale * (Ai @ Wi.T) + bi)
    relu = orc.gemm_bias_act_fp8(A, W, None, 0.5, "relu", "e4m3", "f16")
    np.testing.assert_array_equal(relu, np.maximum(0.5 * (Ai @ Wi.T), 0))


# ------------------------------------------------------------ GEMM core ----

def _hand_gemm():
    d = {}
    with open(os.path.join(GOLDEN, "hand_gemm.txt")) as f:
        for line in f:
            t = line.split("#", 1)[0].split()
            if t:
                d[t[0]] = [float(v) for v in t[1:]]
    A = np.array(d["A"][2:]).reshape(int(d["A"][0]), int(d["A"][1]))
    B = np.array(d["B"][2:]).reshape(int(d["B"][0]), int(d["B"][1]))
    return A, B, np.array(d["bias"]), d


def test_hand_worked_example(orc):
    A, B, bias, d = _hand_gemm()
    a, b, bb = f16(A), f16(B), f16(bias)
    np.testing.assert_array_equal(orc.gemm_bias_act(a, b, None, "none").ravel(), d["none"])
    np.testing.assert_array_equal(orc.gemm_bias_act(a, b, bb, "none").ravel(), d["zb"])
    np.testing.assert_array_equal(orc.gemm_bias_act(a, b, bb, "relu").ravel(), d["relu"])
    for act in ("sigmoid", "gelu"):
        np.testing.assert_allclose(orc.gemm_bias_act(a, b, bb, act).ravel(), d[act],
                                   rtol=1e-14, atol=1e-30)


def _fraction_gemm(Av, Bv, biasv):
    M, K = Av.shape
    N = Bv.shape[1]
    out = np.empty((M, N), dtype=object)
    for i in range(M):
        for j in range(N):
            s = sum((Fraction(Av[i, k]) * Fraction(Bv[k, j]) for k in range(K)), Fraction(0))
            if biasv is not None:
                s += Fraction(biasv[j])
            out[i, j] = s
    return out


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 5, 7), (7, 4, 9), (5, 6, 1), (4, 3, 33)])
def test_gemm_equals_exact_rational_sum(orc, dtype, shape):
    M, N, K = shape
    A = synth.random_bits((M, K), dtype, 100 + M)
    B = synth.random_bits((K, N), dtype, 200 + N)
    bias = synth.random_bits((N,), dtype, 300 + K)
    Av, Bv, bv = orc.decode(A, dtype), orc.decode(B, dtype), orc.decode(bias, dtype)
    exact = _fraction_gemm(Av, Bv, bv)
    got, S = orc.gemm_bias_act(A, B, bias, "none", dtype, with_abs=True)
    for i in range(M):
        for j in range(N):
            # fp64 summation error <= (K+1) * 2^-53 * sum|terms| (textbook bound)
            bound = (K + 1) * 2.0 ** -53 * S[i, j]
            assert abs(Fraction(got[i, j]) - exact[i, j]) <= Fraction(bound), (i, j)
            sabs = sum(abs(Fraction(Av[i, k]) * Fraction(Bv[k, j])) for k in range(K))
            assert S[i, j] == pytest.approx(float(sabs + abs(Fraction(bv[j]))), rel=1e-14)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 5, 7), (7, 4, 9), (4, 3, 33)])
def test_transpose_b_equals_exact_rational_sum(orc, dtype, shape):
    # transpose_B: the second operand is stored (N, K) and enters as its transpose
    M, N, K = shape
    A = synth.random_bits((M, K), dtype, 110 + M)
    W = synth.random_bits((N, K), dtype, 210 + N)
    bias = synth.random_bits((N,), dtype, 310 + K)
    Av, Wv, bv = orc.decode(A, dtype), orc.decode(W, dtype), orc.decode(bias, dtype)
    exact = _fraction_gemm(Av, Wv.T, bv)
    got, S = orc.gemm_bias_act(A, W, bias, "none", dtype, with_abs=True, transpose_b=True)
    for i in range(M):
        for j in range(N):
            bound = (K + 1) * 2.0 ** -53 * S[i, j]
            assert abs(Fraction(got[i, j]) - exact[i, j]) <= Fraction(bound), (i, j)


def test_transpose_b_identity_permutation_and_integers(orc):
    K = 40
    A = synth.random_bits((12, K), "f16", 14)
    eye = f16(np.eye(K))
    np.testing.assert_array_equal(orc.gemm_bias_act(A, eye, None, transpose_b=True), orc.decode(A))
    # W = P (rows permuted): column j of the result is column perm[j] of A
    perm = np.random.default_rng(5).permutation(K)
    P = f16(np.eye(K)[perm])
    np.testing.assert_array_equal(orc.gemm_bias_act(A, P, None, transpose_b=True),
                                  orc.decode(A)[:, perm])
    rng = np.random.default_rng(22)
    M, N, K = 23, 31, 77
    Ai, Wi, bi = rng.integers(-3, 4, (M, K)), rng.integers(-3, 4, (N, K)), rng.integers(-9, 10, N)
    for act in ("none", "relu"):
        got = orc.gemm_bias_act(f16(Ai), f16(Wi), f16(bi), act, transpose_b=True)
        want = Ai @ Wi.T + bi
        np.testing.assert_array_equal(got, np.maximum(want, 0) if act == "relu" else want)


@pytest.mark.parametrize("transpose_b", [False, True], ids=["kn", "nk"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 5, 7), (7, 4, 9), (4, 3, 33)])
def test_transpose_a_equals_exact_rational_sum(orc, dtype, shape, transpose_b):
    # transpose_A: the first operand is stored (K, M) and enters as its transpose
    M, N, K = shape
    At = synth.random_bits((K, M), dtype, 120 + M)
    B = synth.random_bits((N, K) if transpose_b else (K, N), dtype, 220 + N)
    bias = synth.random_bits((N,), dtype, 320 + K)
    Atv, Bv, bv = orc.decode(At, dtype), orc.decode(B, dtype), orc.decode(bias, dtype)
    exact = _fraction_gemm(Atv.T, Bv.T if transpose_b else Bv, bv)
    got, S = orc.gemm_bias_act(At, B, bias, "none", dtype, with_abs=True, transpose_a=True,
                               transpose_b=transpose_b)
    assert got.shape == (M, N)
    for i in range(M):
        for j in range(N):
            bound = (K + 1) * 2.0 ** -53 * S[i, j]
            assert abs(Fraction(got[i, j]) - exact[i, j]) <= Fraction(bound), (i, j)


def test_transpose_a_identity_permutation_and_integers(orc):
    K = 40
    B = synth.random_bits((K, 12), "f16", 15)
    np.testing.assert_array_equal(orc.gemm_bias_act(f16(np.eye(K)), B, None, transpose_a=True),
                                  orc.decode(B))
    # At = P (rows of I permuted, not symmetric): A = P^T, whose row i picks row
    # inv[i] of B, inv the inverse permutation
    perm = np.random.default_rng(6).permutation(K)
    P = f16(np.eye(K)[perm])
    np.testing.assert_array_equal(orc.gemm_bias_act(P, B, None, transpose_a=True),
                                  orc.decode(B)[np.argsort(perm)])
    rng = np.random.default_rng(23)
    M, N, K = 23, 31, 77   # M != K: a swapped leading dimension cannot hide
    Ati, Bi, bi = rng.integers(-3, 4, (K, M)), rng.integers(-3, 4, (K, N)), rng.integers(-9, 10, N)
    Wi = np.ascontiguousarray(Bi.T)
    for act in ("none", "relu"):
        want = Ati.T @ Bi + bi
        want = np.maximum(want, 0) if act == "relu" else want
        np.testing.assert_array_equal(
            orc.gemm_bias_act(f16(Ati), f16(Bi), f16(bi), act, transpose_a=True), want)
        np.testing.assert_array_equal(
            orc.gemm_bias_act(f16(Ati), f16(Wi), f16(bi), act, transpose_a=True, transpose_b=True),
            want)
    # sampled rows of the transposed-A product are the same rows of the full one
    rows = np.array([22, 0, 7])
    full = orc.gemm_bias_act(f16(Ati), f16(Bi), f16(bi), "none", transpose_a=True)
    np.testing.assert_array_equal(
        orc.gemm_bias_act(f16(Ati), f16(Bi), f16(bi), "none", transpose_a=True, rows=rows),
        full[rows])


def test_identity_and_permutation(orc):
    K, N = 48, 40
    B = synth.random_bits((K, N), "f16", 5)
    eye = f16(np.eye(K))
    np.testing.assert_array_equal(orc.gemm_bias_act(eye, B, None), orc.decode(B))
    perm = np.random.default_rng(3).permutation(K)
    P = f16(np.eye(K)[perm])
    np.testing.assert_array_equal(orc.gemm_bias_act(P, B, None), orc.decode(B)[perm])
    # right-multiplication by a permutation permutes columns
    A = synth.random_bits((12, K), "f16", 6)
    Q = f16(np.eye(K)[:, perm])
    np.testing.assert_array_equal(orc.gemm_bias_act(A, Q, None), orc.decode(A)[:, perm])


def test_zero_matrix_gives_activation_of_bias_per_column(orc):
    M, N, K = 5, 9, 16
    Z = f16(np.zeros((M, K)))
    B = synth.random_bits((K, N), "f16", 8)
    bias = synth.random_bits((N,), "f16", 9)
    bv = orc.decode(bias)
    for act in ("none", "relu", "sigmoid", "gelu", "softplus", "gelu_tanh"):
        got = orc.gemm_bias_act(Z, B, bias, act)
        want = np.broadcast_to(orc.act(bv, act), (M, N))
        np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(orc.gemm_bias_act(Z, B, None, "gelu"), 0.0)
    # K == 0: the empty sum
    got = orc.gemm_bias_act(np.zeros((M, 0), np.uint16), np.zeros((0, N), np.uint16), bias)
    np.testing.assert_array_equal(got, np.broadcast_to(bv, (M, N)))


def test_rank_one_closed_form(orc):
    M, N, K = 7, 11, 40
    a = np.arange(M) - 3.0
    b = np.arange(N) * 0.5 - 2.0
    A = f16(np.repeat(a[:, None], K, axis=1))
    B = f16(np.repeat(b[None, :], K, axis=0))
    np.testing.assert_array_equal(orc.gemm_bias_act(A, B, None), K * np.outer(a, b))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_exact_integers_match_integer_matmul(orc, dtype):
    rng = np.random.default_rng(21)
    M, N, K = 37, 29, 301
    Ai = rng.integers(-2, 3, (M, K))
    Bi = rng.integers(-2, 3, (K, N))
    biasi = rng.integers(-8, 9, N)
    to = (lambda v: f16(v)) if dtype == "f16" else (lambda v: synth.to_bits(v.astype(np.float32), "bf16"))
    got = orc.gemm_bias_act(to(Ai), to(Bi), to(biasi), "none", dtype)
    np.testing.assert_array_equal(got, (Ai @ Bi + biasi).astype(np.float64))
    relu = orc.gemm_bias_act(to(Ai), to(Bi), to(biasi), "relu", dtype)
    np.testing.assert_array_equal(relu, np.maximum(Ai @ Bi + biasi, 0).astype(np.float64))


def test_linearity_in_A(orc):
    rng = np.random.default_rng(4)
    A1 = rng.integers(-3, 4, (9, 20))
    A2 = rng.integers(-3, 4, (9, 20))
    B = f16(rng.integers(-3, 4, (20, 13)))
    np.testing.assert_array_equal(orc.gemm_bias_act(f16(A1 + A2), B, None),
                                  orc.gemm_bias_act(f16(A1), B, None)
                                  + orc.gemm_bias_act(f16(A2), B, None))


def test_transpose_identity(orc):
    A = synth.random_bits((19, 33), "f16", 12)
    B = synth.random_bits((33, 26), "f16", 13)
    C = orc.gemm_bias_act(A, B, None)
    Ct = orc.gemm_bias_act(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T), None)
    np.testing.assert_array_equal(C, Ct.T)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_mid_size_against_numpy_float64_matmul(orc, dtype):
    M, N, K = 96, 80, 130
    A = synth.random_bits((M, K), dtype, 31)
    B = synth.random_bits((K, N), dtype, 32)
    bias = synth.random_bits((N,), dtype, 33)
    Av, Bv, bv = orc.decode(A, dtype), orc.decode(B, dtype), orc.decode(bias, dtype)
    got, S = orc.gemm_bias_act(A, B, bias, "none", dtype, with_abs=True)
    ref = Av @ Bv + bv
    assert np.all(np.abs(got - ref) <= 2 * (K + 1) * 2.0 ** -53 * S)
    np.testing.assert_allclose(S, np.abs(Av) @ np.abs(Bv) + np.abs(bv), rtol=1e-13)
    # the epilogue is applied per element after the sum
    for act in ("relu", "sigmoid", "gelu", "softplus", "gelu_tanh"):
        np.testing.assert_array_equal(orc.gemm_bias_act(A, B, bias, act, dtype),
                                      orc.act(got, act))


def test_sampled_rows_equal_full_rows(orc):
    w = synth.WORKLOADS["c1_gelu"]
    A, B, bias = synth.make_inputs(w, M=300, N=64, K=96)
    full = orc.gemm_bias_act(A, B, bias, "gelu")
    rows = synth.sample_rows(300, 20, seed=1)
    np.testing.assert_array_equal(orc.gemm_bias_act(A, B, bias, "gelu", rows=rows), full[rows])


def test_thread_count_does_not_change_bits(orc):
    A = synth.random_bits((70, 64), "bf16", 41)
    B = synth.random_bits((64, 50), "bf16", 42)
    r1 = orc.gemm_bias_act(A, B, None, "gelu", "bf16", nthreads=1)
    r7 = orc.gemm_bias_act(A, B, None, "gelu", "bf16", nthreads=7)
    np.testing.assert_array_equal(r1, r7)


def test_oracle_rejects_bad_arguments(orc):
    A = np.zeros((4, 5), np.uint16)
    with pytest.raises(ValueError):
        orc.gemm_bias_act(A, np.zeros((6, 3), np.uint16), None)
    with pytest.raises(ValueError):
        orc.gemm_bias_act(A, np.zeros((5, 3), np.uint16), np.zeros(4, np.uint16))
    with pytest.raises(ValueError):
        orc.gemm_bias_act(A, np.zeros((5, 3), np.uint16), None, rows=[4])


# -------------------------------------------------------- unfused half --

def test_bias_act_oracle_elementwise(orc):
    X = synth.random_bits((33, 24), "f16", 51, scale=3.0)
    bias = synth.random_bits((24,), "f16", 52)
    xv, bv = orc.decode(X), orc.decode(bias)
    for act in ("none", "relu", "sigmoid", "gelu"):
        got = orc.bias_act(X, bias, act)
        z = xv + bv
        if act == "none":
            want = z
        elif act == "relu":
            want = np.maximum(z, 0)
        elif act == "sigmoid":
            want = np.array([float(1 / (1 + mpmath.exp(-mpmath.mpf(v)))) for v in z.ravel()])
        else:
            want = np.array([float(mpmath.mpf(v) * mpmath.ncdf(v)) for v in z.ravel()])
        np.testing.assert_allclose(got.ravel(), np.ravel(want), rtol=1e-14, atol=1e-300)
    np.testing.assert_array_equal(orc.bias_act(X, None, "none"), xv)


# ------------------------------------------------------ tolerance checker --

def test_ulp_out_values():
    np.testing.assert_array_equal(compare.ulp_out([1.0, 1.5, 2.0, 1000.0, 0.0, 2.0 ** -20], "f16"),
                                  [2.0 ** -10, 2.0 ** -10, 2.0 ** -9, 0.5, 2.0 ** -24, 2.0 ** -24])
    np.testing.assert_array_equal(compare.ulp_out([1.0, 3.0, 0.0], "bf16"),
                                  [2.0 ** -7, 2.0 ** -6, 2.0 ** -133])


def test_checker_flags_planted_errors():
    rng = np.random.default_rng(0)
    R = rng.standard_normal((64, 64)) * 8
    C = np.asarray(R).astype(np.float16).astype(np.float64)
    S = np.abs(R) + 1
    ok = compare.check(C, R, K=64, dtype="f16", act=0, S=S)
    assert ok["ok"] and ok["strict_ok"] and ok["max_ulp"] <= 0.5
    bad = C.copy()
    bad[3, 5] += 4 * compare.ulp_out(R[3, 5], "f16") + 0.01   # one element off
    rep = compare.check(bad, R, K=64, dtype="f16", act=0, S=S)
    assert not rep["strict_ok"] and rep["worst"]["index"] == [3, 5]
    swapped = C[:, ::-1]                                       # columns mixed up
    assert not compare.check(swapped, R, K=64, dtype="f16")["ok"]
    nan = C.copy()
    nan[0, 0] = np.nan
    assert not compare.check(nan, R, K=64, dtype="f16")["ok"]


def _f32_add_rz(a, b):
    """a + b rounded toward zero to float32 (a, b float32 whose exact sum fits
    a float64: true for the exponent ranges used here)."""
    s = float(a) + float(b)
    r = np.float32(s)
    if abs(float(r)) > abs(s):
        r = np.nextafter(r, np.float32(0.0))
    return np.float32(r)


def test_fp8_gate_bounds_fp32_summation_in_any_order():
    """compare.fp8_sum_rel models the 8-bit kernel's accumulation as fp32 sums
    of exact products, each addition faithfully rounded: any order within each
    128-term instruction, then in order across instructions. Brute force: sum
    exact E4M3 products of random data that way in float32, with adversarial
    inner orders (largest first, smallest first, sorted by sign, random) and
    both round-to-nearest and truncation, and check that the error per unit of
    sum |x| stays within the bound."""
    rng = np.random.default_rng(3)
    f32 = np.float32
    for K in (128, 512, 4096):
        worst = 0.0
        for trial in range(8):
            # E4M3 values (4-bit significands): products have <= 8 significant bits
            a = np.ldexp(rng.integers(8, 16, K) * rng.choice([-1, 1], K), rng.integers(-9, 1, K))
            w = np.ldexp(rng.integers(8, 16, K) * rng.choice([-1, 1], K), rng.integers(-9, 1, K))
            if trial >= 4:        # one sign throughout: the partial sums grow to S
                a, w = np.abs(a), np.abs(w)
            x = (a * w).astype(np.float64)
            assert np.array_equal(x.astype(f32).astype(np.float64), x)   # exact in fp32
            exact = math.fsum(x.tolist())
            for add in ((lambda p, v: f32(p + v)), _f32_add_rz):
                acc = f32(0.0)
                for i0 in range(0, K, 128):
                    blk = x[i0:i0 + 128]
                    order = [np.argsort(-np.abs(blk)), np.argsort(np.abs(blk)),
                             np.argsort(blk), rng.permutation(blk.size)][trial % 4]
                    part = f32(0.0)
                    for v in blk[order]:
                        part = add(part, f32(v))
                    acc = add(acc, part)
                worst = max(worst, abs(float(acc) - exact) / np.abs(x).sum())
        assert worst <= compare.fp8_sum_rel(K), (K, worst, compare.fp8_sum_rel(K))
    # and the coefficient grows with the number of instructions in the chain
    assert compare.fp8_sum_rel(4096) == (127 + 31 + 2) * 2.0 ** -23
    assert compare.fp8_sum_rel(128) < compare.fp8_sum_rel(4096) < compare.fp8_sum_rel(14336)


# ---------------------------------------------------------- generators --

def test_generators_are_deterministic_and_shaped():
    w = synth.WORKLOADS["c4_relu"]
    a1, b1, c1 = synth.make_inputs(w, M=64, N=72, K=40)
    a2, b2, c2 = synth.make_inputs(w, M=64, N=72, K=40)
    assert a1.shape == (64, 40) and b1.shape == (40, 72) and c1.shape == (72,)
    assert np.array_equal(a1, a2) and np.array_equal(b1, b2) and np.array_equal(c1, c2)
    v = a1.view(np.float16).astype(np.float64)
    assert v.min() >= -1 and v.max() <= 1


def test_generator_moments(orc):
    w = synth.WORKLOADS["c5_gelu"]
    A, B, bias = synth.make_inputs(w, M=256, N=512, K=4096)
    assert w.dtype == "bf16"
    b = orc.decode(B, "bf16")
    assert abs(b.std() - 1 / 64) < 2e-4 and abs(b.mean()) < 2e-4
    assert abs(orc.decode(bias, "bf16").std() - math.sqrt(0.02)) < 0.01
    a = orc.decode(A, "bf16")
    assert abs(a.std() - 1) < 0.01
    w3 = synth.WORKLOADS["c3_gelu"]
    A3, _, _ = synth.make_inputs(w3, M=128, N=8, K=1024)
    assert abs(orc.decode(A3).std() - 1 / math.sqrt(2)) < 0.01


def test_sample_rows():
    r = synth.sample_rows(16384, 64, seed=5)
    assert len(r) == 64 and len(set(r.tolist())) == 64
    assert r[0] == 0 and r[-1] == 16383 and np.all(np.diff(r) > 0)
    assert np.array_equal(synth.sample_rows(40, 64), np.arange(40))
