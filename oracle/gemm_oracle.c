/*
 * CPU oracle for the fused tiled GEMM C = act(A.B + bias).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path links, loads or calls
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do. It shares no code, header or table with the HIP library.
 *
 * What it computes, and where the pages define it:
 *   - "TileLang: Write, Autotune, and Ship Fused Tensor-Core Kernels from
 *     Python" (saipien.org), section "Why tile-level control matters": the
 *     GEMM's accumulator gets a bias add and an activation such as GELU before
 *     the single write of the result.
 *   - "writing-tilelang-kernels" (skillsmp.com), sections "Kernel Anatomy" and
 *     "Step-by-Step Workflow": A is (M,K), B is (K,N), C is (M,N), all
 *     row-major, fp16 inputs with a float accumulator, and the reference
 *     program is the plain product A @ B.
 *   - Same page, "Pre-flight Checklist" and "Key API Patterns": the fused
 *     epilogues are ReLU (max) and sigmoid.
 *   - Same page, "Quick Templates" (Elementwise 2D): softplus, log(1 + e^z),
 *     evaluated in the float accumulator type.
 *   - The tanh form of GELU, 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3)))
 *     (Hendrycks and Gimpel, "Gaussian Error Linear Units", 2016), as the
 *     second GELU variant next to the erf form the pages' GELU epilogue reads as.
 *   - 8-bit float inputs ("tilelang" (skillsmp.com), Documentation Structure:
 *     the type system lists float8_e4m3/e5m2 and the GEMM examples an FP8
 *     GEMM): A and the (N,K) operand W in one OCP 8-bit format, E4M3 or E5M2
 *     ("OCP 8-bit Floating Point Specification (OFP8)", 2023), with one fp32
 *     dequantization scale for the product: s = scale * sum_k A[i][k] * W[j][k];
 *     bias and result in fp16/bf16 (oracle_gemm_bias_act_fp8_nt).
 *   - Same page, "Key API Patterns": the tile GEMM takes a transpose_B flag.
 *     With it, the second operand is given as an (N,K) row-major array W and
 *     the product is A times its transpose: s[i][j] = sum_k A[i][k] * W[j][k]
 *     (oracle_gemm_bias_act_nt).
 *   - The same call takes a transpose_A flag: the first operand is then given
 *     as a (K,M) row-major array At, and A[i][k] = At[k][i]
 *     (oracle_gemm_bias_act_ex, which takes both flags).
 *
 * The oracle is the mathematical definition written out, in fp64:
 *     s[i][j] = sum_{k<K} A[i][k] * B[k][j]        (each product exact in fp64)
 *     z[i][j] = s[i][j] + bias[j]                  (bias[N], broadcast over rows)
 *     y[i][j] = act(z[i][j])
 * with act in { identity, max(z,0), 1/(1+exp(-z)), z*Phi(z) (erf form),
 * log(1+exp(z)), tanh-form GELU }.
 * The loop order is i, then k, then j; the sum over k for one (i,j) is formed
 * left to right in k. fp16/bf16 bit patterns are decoded by this file's own
 * decoders; the fp64 result can be rounded to fp16/bf16 by this file's own
 * round-to-nearest-even encoders.
 *
 * Readings where the pages are silent (each one is listed in the design notes):
 *   - bias has N entries and is added before the activation;
 *   - GELU is the erf form, z * 0.5 * erfc(-z / sqrt(2));
 *   - a NULL bias means "no bias"; K == 0 gives the empty sum 0.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

enum { OR_F16 = 0, OR_BF16 = 1 };
enum { OR_NONE = 0, OR_RELU = 1, OR_SIGMOID = 2, OR_GELU = 3, OR_SOFTPLUS = 4, OR_GELU_TANH = 5 };

/* ---- bit decoders (IEEE binary16 and bfloat16) ---------------------------- */

static double dec_f16(uint16_t h) {
    int sign = h >> 15, ex = (h >> 10) & 0x1f, fr = h & 0x3ff;
    double v;
    if (ex == 0)
        v = ldexp((double)fr, -24);                 /* subnormal: fr * 2^-24 */
    else if (ex == 31)
        v = fr ? NAN : INFINITY;
    else
        v = ldexp((double)(fr | 0x400), ex - 25);   /* (1024+fr) * 2^(ex-15-10) */
    return sign ? -v : v;
}

static double dec_bf16(uint16_t h) {
    int sign = h >> 15, ex = (h >> 7) & 0xff, fr = h & 0x7f;
    double v;
    if (ex == 0)
        v = ldexp((double)fr, -133);                /* subnormal: fr * 2^-133 */
    else if (ex == 255)
        v = fr ? NAN : INFINITY;
    else
        v = ldexp((double)(fr | 0x80), ex - 134);   /* (128+fr) * 2^(ex-127-7) */
    return sign ? -v : v;
}

static double dec(int dtype, uint16_t h) { return dtype == OR_F16 ? dec_f16(h) : dec_bf16(h); }

/* OCP E4M3: 1 sign, 4 exponent (bias 7), 3 fraction bits; no infinities,
 * S.1111.111 is NaN, largest finite 448. */
static double dec_e4m3(uint8_t x) {
    int sign = x >> 7, ex = (x >> 3) & 0xf, fr = x & 0x7;
    double v;
    if (ex == 0)
        v = ldexp((double)fr, -9);                  /* subnormal: fr * 2^-9 */
    else if (ex == 15 && fr == 7)
        v = NAN;
    else
        v = ldexp((double)(fr | 0x8), ex - 10);     /* (8+fr) * 2^(ex-7-3) */
    return sign ? -v : v;
}

/* OCP E5M2: 1 sign, 5 exponent (bias 15), 2 fraction bits; IEEE-style
 * infinities and NaNs at exponent 31, largest finite 57344. */
static double dec_e5m2(uint8_t x) {
    int sign = x >> 7, ex = (x >> 2) & 0x1f, fr = x & 0x3;
    double v;
    if (ex == 0)
        v = ldexp((double)fr, -16);                 /* subnormal: fr * 2^-16 */
    else if (ex == 31)
        v = fr ? NAN : INFINITY;
    else
        v = ldexp((double)(fr | 0x4), ex - 17);     /* (4+fr) * 2^(ex-15-2) */
    return sign ? -v : v;
}

/* Operand kinds: the two 16-bit types (their gba dtype codes) and the two
 * 8-bit formats. */
enum { OK_F16 = 0, OK_BF16 = 1, OK_E4M3 = 2, OK_E5M2 = 3 };

static double dec_op(int kind, const void *base, int64_t idx) {
    switch (kind) {
    case OK_E4M3: return dec_e4m3(((const uint8_t *)base)[idx]);
    case OK_E5M2: return dec_e5m2(((const uint8_t *)base)[idx]);
    default: return dec(kind, ((const uint16_t *)base)[idx]);
    }
}

/* ---- round-to-nearest-even encoders from fp64 ----------------------------- */
/* man_bits: stored fraction bits; emin: smallest normal exponent; emax: largest. */
static uint16_t enc_generic(double x, int man_bits, int emin, int emax, int exp_bias) {
    const uint16_t sign = signbit(x) ? 0x8000 : 0;
    const uint16_t exp_all_ones = (uint16_t)(((1 << (15 - man_bits)) - 1) << man_bits);
    if (isnan(x)) return (uint16_t)(exp_all_ones | (1 << (man_bits - 1)));
    double a = fabs(x);
    if (a == 0.0) return sign;
    if (isinf(a)) return sign | exp_all_ones;
    int e2;
    frexp(a, &e2);              /* a = m * 2^e2, m in [0.5, 1) */
    int E = e2 - 1;             /* a in [2^E, 2^(E+1)) */
    if (E < emin) E = emin;     /* subnormal range shares the quantum of emin */
    double q = ldexp(1.0, E - man_bits);
    double r = rint(a / q);     /* a / q is exact: q is a power of two */
    uint32_t ri = (uint32_t)r;
    const uint32_t hidden = 1u << man_bits;
    if (ri < hidden) return sign | (uint16_t)ri;          /* subnormal (E == emin) */
    if (ri == 2 * hidden) { ri = hidden; E += 1; }        /* rounding carried */
    if (E > emax) return sign | exp_all_ones;             /* overflow to inf */
    return sign | (uint16_t)(((uint32_t)(E + exp_bias) << man_bits) | (ri - hidden));
}

static uint16_t enc(int dtype, double x) {
    return dtype == OR_F16 ? enc_generic(x, 10, -14, 15, 15)
                           : enc_generic(x, 7, -126, 127, 127);
}

/* ---- activations ---------------------------------------------------------- */

static double act_apply(int act, double z) {
    switch (act) {
    case OR_RELU:
        return z > 0.0 ? z : 0.0;
    case OR_SIGMOID:
        if (z >= 0.0) return 1.0 / (1.0 + exp(-z));
        else { double e = exp(z); return e / (1.0 + e); }
    case OR_GELU:
        /* z * Phi(z); Phi(z) = 0.5 * (1 + erf(z/sqrt2)) = 0.5 * erfc(-z/sqrt2).
         * At z = -inf the product is -inf * 0: the value there is the limit, 0. */
        if (isinf(z) && z < 0.0) return 0.0;
        return 0.5 * z * erfc(-z / sqrt(2.0));
    case OR_SOFTPLUS:
        /* log(1 + e^z), written so that neither branch overflows or cancels:
         * z + log(1 + e^-z) = log(e^z (1 + e^-z)) for z > 0. */
        return z > 0.0 ? z + log1p(exp(-z)) : log1p(exp(z));
    case OR_GELU_TANH: {
        /* 0.5 z (1 + tanh(y)); for y < 0, 1 + tanh(y) = 2 e^(2y) / (1 + e^(2y))
         * (no cancellation). At z = -inf: the limit, 0. */
        if (isinf(z) && z < 0.0) return 0.0;
        const double y = sqrt(2.0 / 3.14159265358979323846) * (z + 0.044715 * z * z * z);
        if (y >= 0.0) return 0.5 * z * (1.0 + tanh(y));
        const double e = exp(2.0 * y);
        return z * e / (1.0 + e);
    }
    default:
        return z;
    }
}

/* ---- the fused GEMM ------------------------------------------------------- */

typedef struct {
    const void *A;         /* operand kind a_kind; (M,K), or (K,M) when a_km */
    const uint16_t *bias;  /* dtype */
    const double *Bd;      /* B decoded to fp64, K x N */
    double *out, *absout;
    const int64_t *rows;
    int64_t nrows, M, N, K;
    int act, dtype, a_kind, a_km;
    double scale;          /* multiplies the sum before the bias (1 for 16-bit inputs) */
    int64_t r0, r1;        /* this worker's slice of [0, nrows) */
} gemm_job;

static void *gemm_worker(void *p) {
    gemm_job *j = (gemm_job *)p;
    const int64_t N = j->N, K = j->K;
    double *acc = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    double *aacc = j->absout ? (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1)) : NULL;
    for (int64_t r = j->r0; r < j->r1; ++r) {
        const int64_t i = j->rows ? j->rows[r] : r;
        for (int64_t c = 0; c < N; ++c) acc[c] = 0.0;
        if (aacc) for (int64_t c = 0; c < N; ++c) aacc[c] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = dec_op(j->a_kind, j->A, j->a_km ? k * j->M + i : i * K + k);
            const double *brow = j->Bd + k * N;
            for (int64_t c = 0; c < N; ++c) acc[c] += a * brow[c];
            if (aacc) {
                const double aa = fabs(a);
                for (int64_t c = 0; c < N; ++c) aacc[c] += aa * fabs(brow[c]);
            }
        }
        double *o = j->out + r * N;
        for (int64_t c = 0; c < N; ++c) {
            double z = j->scale * acc[c];
            if (j->bias) z += dec(j->dtype, j->bias[c]);
            o[c] = act_apply(j->act, z);
        }
        if (aacc) {
            double *ao = j->absout + r * N;
            for (int64_t c = 0; c < N; ++c)
                ao[c] = fabs(j->scale) * aacc[c] + (j->bias ? fabs(dec(j->dtype, j->bias[c])) : 0.0);
        }
    }
    free(acc);
    free(aacc);
    return NULL;
}

typedef struct {
    const void *B;
    double *Bd;
    int64_t lo, hi, N, K;
    int b_kind, b_nk;
} dec_job;

/* Bd[k][j] = the (k, j) entry of the second operand: B[k][j] when B is stored
 * (K,N), W[j][k] when it is stored (N,K) (transpose_B). */
static void *dec_worker(void *p) {
    dec_job *d = (dec_job *)p;
    for (int64_t t = d->lo; t < d->hi; ++t) {
        const int64_t k = t / d->N, j = t % d->N;
        d->Bd[t] = dec_op(d->b_kind, d->B, d->b_nk ? j * d->K + k : t);
    }
    return NULL;
}

static int pick_threads(int nthreads, int64_t work_items) {
    int t = nthreads > 0 ? nthreads : (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (t < 1) t = 1;
    if (t > 256) t = 256;
    if (work_items < t) t = (int)(work_items > 0 ? work_items : 1);
    return t;
}

/*
 * out[r][c] = act(sum_k A[i][k]*B[k][c] + bias[c]) for i = rows[r] (or i = r when
 * rows == NULL, nrows == M). absout, when not NULL, receives sum_k |A[i][k]*B[k][c]|
 * + |bias[c]|, the magnitude that bounds any fp32 summation's rounding error.
 * Returns 0, or -1 on a bad argument.
 */
static int gemm_impl(const void *A, int a_km, const void *B, int op_kind, int b_nk, double scale,
                     const uint16_t *bias, double *out, double *absout, int64_t M, int64_t N,
                     int64_t K, int act, int dtype, const int64_t *rows, int64_t nrows,
                     int nthreads) {
    if (M < 0 || N < 0 || K < 0 || act < 0 || act > 5 || (dtype != OR_F16 && dtype != OR_BF16))
        return -1;
    if (op_kind < OK_F16 || op_kind > OK_E5M2 || !isfinite(scale)) return -1;
    if (!rows) nrows = M;
    if (nrows == 0 || N == 0) return 0;
    if (rows)
        for (int64_t r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= M) return -1;

    double *Bd = (double *)malloc(sizeof(double) * (size_t)(K * N > 0 ? K * N : 1));
    if (!Bd) return -1;
    {
        int T = pick_threads(nthreads, K * N);
        pthread_t th[256];
        dec_job dj[256];
        for (int t = 0; t < T; ++t) {
            dj[t].B = B; dj[t].Bd = Bd; dj[t].b_kind = op_kind; dj[t].b_nk = b_nk;
            dj[t].N = N; dj[t].K = K;
            dj[t].lo = (K * N) * t / T; dj[t].hi = (K * N) * (t + 1) / T;
            pthread_create(&th[t], NULL, dec_worker, &dj[t]);
        }
        for (int t = 0; t < T; ++t) pthread_join(th[t], NULL);
    }
    int T = pick_threads(nthreads, nrows);
    pthread_t th[256];
    gemm_job jb[256];
    for (int t = 0; t < T; ++t) {
        gemm_job g = {A, bias, Bd, out, absout, rows, nrows, M, N, K, act, dtype, op_kind,
                      a_km, scale, nrows * t / T, nrows * (t + 1) / T};
        jb[t] = g;
        pthread_create(&th[t], NULL, gemm_worker, &jb[t]);
    }
    for (int t = 0; t < T; ++t) pthread_join(th[t], NULL);
    free(Bd);
    return 0;
}

/* B stored (K,N): out = act(A.B + bias). */
int oracle_gemm_bias_act(const uint16_t *A, const uint16_t *B, const uint16_t *bias,
                         double *out, double *absout, int64_t M, int64_t N, int64_t K,
                         int act, int dtype, const int64_t *rows, int64_t nrows,
                         int nthreads) {
    return gemm_impl(A, 0, B, dtype, 0, 1.0, bias, out, absout, M, N, K, act, dtype, rows, nrows,
                     nthreads);
}

/* W stored (N,K) (transpose_B): out[r][c] = act(sum_k A[i][k]*W[c][k] + bias[c]). */
int oracle_gemm_bias_act_nt(const uint16_t *A, const uint16_t *W, const uint16_t *bias,
                            double *out, double *absout, int64_t M, int64_t N, int64_t K,
                            int act, int dtype, const int64_t *rows, int64_t nrows,
                            int nthreads) {
    return gemm_impl(A, 0, W, dtype, 1, 1.0, bias, out, absout, M, N, K, act, dtype, rows, nrows,
                     nthreads);
}

/* Either operand stored transposed: transpose_a: the first operand is At, stored
 * (K,M), with A[i][k] = At[k][i]; transpose_b: the second is W, stored (N,K).
 * out[r][c] = act(sum_k A[i][k]*B[k][c] + bias[c]) with B[k][c] = W[c][k]. */
int oracle_gemm_bias_act_ex(const uint16_t *A, const uint16_t *B, const uint16_t *bias,
                            double *out, double *absout, int64_t M, int64_t N, int64_t K,
                            int act, int dtype, int transpose_a, int transpose_b,
                            const int64_t *rows, int64_t nrows, int nthreads) {
    return gemm_impl(A, transpose_a != 0, B, dtype, transpose_b != 0, 1.0, bias, out, absout, M,
                     N, K, act, dtype, rows, nrows, nthreads);
}

/* 8-bit inputs, W stored (N,K): out[r][c] = act(scale * sum_k A[i][k]*W[c][k] + bias[c]),
 * A and W in format fmt (0 = E4M3, 1 = E5M2), bias in dtype (fp16/bf16). absout
 * receives |scale| sum_k |A[i][k]*W[c][k]| + |bias[c]|. */
int oracle_gemm_bias_act_fp8_nt(const uint8_t *A, const uint8_t *W, const uint16_t *bias,
                                double *out, double *absout, int64_t M, int64_t N, int64_t K,
                                double scale, int act, int fmt, int dtype,
                                const int64_t *rows, int64_t nrows, int nthreads) {
    if (fmt != 0 && fmt != 1) return -1;
    return gemm_impl(A, 0, W, fmt == 0 ? OK_E4M3 : OK_E5M2, 1, scale, bias, out, absout, M, N, K,
                     act, dtype, rows, nrows, nthreads);
}

/* out[i][j] = act(X[i][j] + bias[j]) in fp64: the elementwise second half of the
 * unfused pair, applied to the fp16/bf16 intermediate exactly as stored. */
int oracle_bias_act(const uint16_t *X, const uint16_t *bias, double *out, int64_t M,
                    int64_t N, int act, int dtype) {
    if (M < 0 || N < 0 || act < 0 || act > 5 || (dtype != OR_F16 && dtype != OR_BF16))
        return -1;
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) {
            double z = dec(dtype, X[i * N + j]);
            if (bias) z += dec(dtype, bias[j]);
            out[i * N + j] = act_apply(act, z);
        }
    return 0;
}

/* Elementwise helpers, exported so that the pins can reach every piece. */
void oracle_decode(int dtype, const uint16_t *bits, double *out, int64_t n) {
    for (int64_t t = 0; t < n; ++t) out[t] = dec(dtype, bits[t]);
}

void oracle_encode(int dtype, const double *x, uint16_t *bits, int64_t n) {
    for (int64_t t = 0; t < n; ++t) bits[t] = enc(dtype, x[t]);
}

void oracle_decode_fp8(int fmt, const uint8_t *bits, double *out, int64_t n) {
    for (int64_t t = 0; t < n; ++t) out[t] = fmt == 0 ? dec_e4m3(bits[t]) : dec_e5m2(bits[t]);
}

void oracle_act(int act, const double *z, double *out, int64_t n) {
    for (int64_t t = 0; t < n; ++t) out[t] = act_apply(act, z[t]);
}
