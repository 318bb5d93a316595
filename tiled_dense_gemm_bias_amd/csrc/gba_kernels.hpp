// gfx950 kernels of the fused tiled GEMM C = act(A.B + bias).
//
// The computation is the tiled GEMM of "writing-tilelang-kernels" (Kernel
// Anatomy): each workgroup owns one BM x BN tile of C, clears an fp32
// accumulator held in registers, walks K in BK-deep slices staged through
// on-chip memory, and writes its tile once. "TileLang: Write, Autotune, and Ship
// Fused Tensor-Core Kernels from Python" (Why tile-level control matters) adds
// the bias + activation epilogue applied to that register accumulator.
//
// CDNA4 mapping used here:
//  * MFMA v_mfma_f32_32x32x16_{f16,bf16}: a 64-lane wave multiplies a 32x16 by a
//    16x32 block into 16 fp32 accumulators per lane.
//  * The MFMA's first operand is fed from B (rows n of B^T) and its second from
//    A (columns m of A^T), so the 32x32 result block is C^T: lane l then holds
//    C[m = l%32][n = 8i + 4(l/32) + j] in accumulator 4i+j, i.e. four adjacent
//    columns of one row -- one 8-byte store per i.
//  * LDS holds each stage as A[BM][BK] and B^T[BN][BK], both K-contiguous, in
//    16-byte chunks; chunk c of row r sits at c ^ swz(r), which keeps both the
//    loader's writes and the MFMA operand reads free of bank conflicts.
//  * B is row-major [K,N] in HBM, so the loader transposes it on the way into
//    LDS: each thread reads an 8(k) x 8(n) block as eight 16-byte row pieces and
//    writes eight 16-byte column pieces, repacked with v_perm_b32.
//  * Two LDS stages: the global loads of slice k+1 are in flight while slice k
//    is multiplied; one barrier per slice.
//  * Workgroup ids are remapped so that each of the 8 XCDs runs a contiguous
//    block of tiles, walked in groups of group_m tile rows (L2 panel reuse).
#pragma once

#include <hip/hip_runtime.h>
#include <utility>
#include <stdint.h>

namespace gba {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
// Native 16-byte vector (HIP's u32x4 is a struct, whose copies defeat register promotion).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

enum { DT_F16 = 0, DT_BF16 = 1 };
enum { ACT_NONE = 0, ACT_RELU = 1, ACT_SIGMOID = 2, ACT_GELU = 3, ACT_SOFTPLUS = 4, ACT_GELU_TANH = 5 };
constexpr int kNumActs = 6;

constexpr int kNumXcd = 8;

// ceil(x / b) for x up to 2^31 - 1 (x + b - 1 would overflow int there).
__host__ __device__ constexpr int ceil_div(int x, int b) { return (int)(((long long)x + b - 1) / b); }

// Grids of tile workgroups. HIP caps a grid dimension's work-items (workgroups
// x threads) below 2^32, so more than 2^16 workgroups are launched as a 2-D grid
// 2^16 wide. The linear id y * gridDim.x + x is the dispatch order (and what
// xcd_remap assumes); ids past the last tile do nothing.
constexpr long long kGridX = 1LL << 16;
inline dim3 tile_grid(long long n) {
    return n <= kGridX ? dim3((unsigned)n) : dim3((unsigned)kGridX, (unsigned)((n + kGridX - 1) / kGridX));
}
__device__ __forceinline__ int linear_block() { return (int)(blockIdx.y * gridDim.x + blockIdx.x); }
__device__ __forceinline__ int linear_grid() { return (int)(gridDim.x * gridDim.y); }

// Compute units of the current device for the persistent launchers' grids,
// queried from the runtime once per device (a launch then costs no query).
inline hipError_t current_cus(int *cus) {
    static int cached[64];   // 0: not queried yet
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    int c = __atomic_load_n(&cached[dev], __ATOMIC_RELAXED);
    if (c <= 0) {
        e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        if (c <= 0) return hipErrorInvalidDevice;
        __atomic_store_n(&cached[dev], c, __ATOMIC_RELAXED);
    }
    *cus = c;
    return hipSuccess;
}

// f(std::integral_constant<int, I>{}) for I = 0 .. N-1, unrolled at compile time.
template <class F, int... I>
__device__ __forceinline__ void static_for_seq(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_seq(f, std::make_integer_sequence<int, N>{});
}

// ---------------------------------------------------------------- scalars --

template <int DT>
__device__ __forceinline__ float to_f32(uint32_t h) {
    if constexpr (DT == DT_F16) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
    } else {
        return __uint_as_float(h << 16);
    }
}

// fp32 pair -> storage type, round to nearest even, in one v_cvt_pk_f16_f32 /
// v_cvt_pk_bf16_f32 (gfx950); lo lands in the low half.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    if constexpr (DT == DT_F16)
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
    else
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Activation on the fp32 accumulator.
//  RELU:    max(z, 0).
//  SIGMOID: 1 / (1 + 2^(-z log2 e)) with the hardware exp2 and reciprocal.
//  GELU:    z * Phi(z), written as max(z, 0) - |z| Phi(-|z|) (Phi(z) = 1 - Phi(-z)),
//           with Phi(-x) = 2^Q(x): Q is a degree-7 polynomial fitted to
//           log2 Phi(-x) on [0, 6] (tiled_dense_gemm_bias_amd/gelu_fit.py), with
//           fractional error below 8e-6 there. Its leading coefficient is
//           negative, so past 6 the correction term |z| 2^Q(|z|) falls below
//           6e-9 and keeps falling. Seven fma and one exp2, no division.
//  SOFTPLUS: log(1 + e^z) = max(z, 0) + log1p(t), t = e^-|z| in (0, 1]; log1p(t)
//           as ln(u) * t / (u - 1) with u = 1 + t rounded (Kahan's correction:
//           the rounding of u cancels to first order), t itself when u == 1.
//  GELU_TANH: 0.5 z (1 + tanh(y)), y = sqrt(2/pi) (z + 0.044715 z^3), written as
//           z / (1 + e^(-2y)) (1 + tanh(y) = 2 / (1 + e^(-2y))): one exp2 and one
//           reciprocal. For z << 0, e^(-2y) overflows to +inf and the result is
//           -0 (the true value is below 1e-30 in magnitude there).
//  Non-finite z (an fp32 accumulator can overflow with bf16 operands): every
//  activation gives its limit at z = +-inf (GELU and GELU_TANH: +inf and 0,
//  the latter instead of inf * 0) and NaN for NaN.
template <int ACT>
__device__ __forceinline__ float act_fn(float z) {
    if constexpr (ACT == ACT_RELU) {
        return fmaxf(z, 0.0f);
    } else if constexpr (ACT == ACT_SIGMOID) {
        const float e = __builtin_amdgcn_exp2f(-z * 1.4426950408889634f);
        return __builtin_amdgcn_rcpf(1.0f + e);
    } else if constexpr (ACT == ACT_GELU) {
        const float az = fabsf(z);
        float q = fmaf(az, -1.8348076764596044e-06f, 6.15982135059312e-05f);
        q = fmaf(az, q, -0.0009305241401307285f);
        q = fmaf(az, q, 0.008507887832820415f);
        q = fmaf(az, q, -0.05396006256341934f);
        q = fmaf(az, q, -0.4584644138813019f);
        q = fmaf(az, q, -1.1512510776519775f);
        q = fmaf(az, q, -0.9999952912330627f);
        // The multiplier is clamped below +inf so that z = +-inf gives
        // max(z, 0) - 3e38 * 0 (the limits +inf and 0) rather than inf * 0; a NaN z
        // still reaches the result through q.
        return fmaf(-fminf(az, 3.0e38f), __builtin_amdgcn_exp2f(q), fmaxf(z, 0.0f));
    } else if constexpr (ACT == ACT_SOFTPLUS) {
        const float t = __builtin_amdgcn_exp2f(-fabsf(z) * 1.4426950408889634f);
        const float u = 1.0f + t;
        const float d = u - 1.0f;
        const float lu = __builtin_amdgcn_logf(u) * 0.6931471824645996f;   // ln(u)
        const float lp = d == 0.0f ? t : lu * (t * __builtin_amdgcn_rcpf(d));
        return fmaxf(z, 0.0f) + lp;
    } else if constexpr (ACT == ACT_GELU_TANH) {
        // -2 y log2(e) = -z (c1 + c3 z^2), c1 = 2 sqrt(2/pi) log2(e), c3 = 0.044715 c1
        const float a = -z * fmaf(z * z, 0.10294324159622192f, 2.302208185195923f);
        // z clamped above -inf: at z = -inf the reciprocal is 0 and the result the
        // limit 0 rather than -inf * 0 (a NaN z still propagates through a).
        return fmaxf(z, -3.0e38f) * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(a));
    } else {
        return z;
    }
}

template <int DT>
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (DT == DT_F16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
}

// Component d of a u32x4; d is a compile-time constant after unrolling.
__device__ __forceinline__ uint32_t dword(const u32x4 &v, int d) {
    return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
}

// ------------------------------------------------------------- tile order --

// Bijection on [0, n): workgroup w runs on XCD w % 8 (round-robin dispatch);
// return an index such that the workgroups of XCD x get one contiguous range.
__device__ __forceinline__ int xcd_remap(int w, int n) {
    const int q = n / kNumXcd, r = n % kNumXcd;
    const int x = w % kNumXcd, i = w / kNumXcd;
    return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// Logical tile index -> (tile_m, tile_n), walking group_m tile rows at a time.
__device__ __forceinline__ void grouped_tile(int t, int tiles_m, int tiles_n, int group_m,
                                             int &tm, int &tn) {
    const int group_size = group_m * tiles_n;
    const int g = t / group_size;
    const int first_m = g * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int in_group = t - g * group_size;
    tm = first_m + in_group % gm;
    tn = in_group / gm;
}

// ----------------------------------------------------------------- GEMM ----

// Physical 16-byte chunk of logical chunk c in LDS row r. CH chunks per row;
// rows that share a 128-byte bank window, and rows 8 apart, land on different
// chunk slots, so 8 consecutive lanes never collide.
template <int CH>
__device__ __forceinline__ int swz(int r, int c) {
    constexpr int RPW = 8 / CH;   // rows per 128-byte window
    return c ^ (((r / RPW) ^ (r >> 3)) & (CH - 1));
}

template <int BM, int BN, int BK, int WM, int WN, int DT, int ACT>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_bias_act_kernel(const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
                     const uint16_t *__restrict__ bias, uint16_t *__restrict__ C, int M, int N,
                     int K, int tiles_m, int tiles_n, int raster, int group_m) {
    constexpr int NT = WM * WN * 64;
    constexpr int CH = BK / 8;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int A_CHUNKS = BM * CH;
    constexpr int A_PER_T = A_CHUNKS / NT;
    constexpr int B_SUB = (BK / 8) * (BN / 8);
    constexpr int B_PER_T = (B_SUB + NT - 1) / NT;
    static_assert(BK == 32 || BK == 64, "BK must be 32 or 64");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert(A_CHUNKS % NT == 0, "A slice must split evenly over the threads");
    constexpr int STAGE = (BM + BN) * CH;   // u32x4 per stage
    static_assert(2 * STAGE * 16 <= 160 * 1024, "LDS ring exceeds 160 KiB");

    __shared__ u32x4 lds[2 * STAGE];

    int tm, tn;
    {
        int t = linear_block();
        if (raster) t = xcd_remap(t, linear_grid());
        if (t >= tiles_m * tiles_n) return;   // padding of a 2-D grid
        if (raster) {
            grouped_tile(t, tiles_m, tiles_n, group_m, tm, tn);
        } else {
            tm = t / tiles_n;
            tn = t % tiles_n;
        }
    }
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wid = tid >> 6;
    const int wm = wid / WN, wn = wid % WN;
    const int lrow = lane & 31, lhalf = lane >> 5;

    const u32x4 zero4 = {0u, 0u, 0u, 0u};
    u32x4 ra[A_PER_T];
    u32x4 rb[B_PER_T][8];

    auto load_slice = [&](int kt) {
        const int k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i) {
            const int s = tid + i * NT;
            const int r = s / CH, c = s % CH;
            const int gm = m0 + r, gk = k0 + c * 8;
            ra[i] = (gm < M && gk < K)
                        ? *reinterpret_cast<const u32x4 *>(A + (size_t)gm * K + gk)
                        : zero4;
        }
#pragma unroll
        for (int i = 0; i < B_PER_T; ++i) {
            const int s = tid + i * NT;
            if (B_SUB % NT == 0 || s < B_SUB) {
                const int kb = s / (BN / 8), nb = s % (BN / 8);
                const int gn = n0 + nb * 8;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int gk = k0 + kb * 8 + e;
                    rb[i][e] = (gk < K && gn < N)
                                   ? *reinterpret_cast<const u32x4 *>(B + (size_t)gk * N + gn)
                                   : zero4;
                }
            }
        }
    };

    auto store_slice = [&](int st) {
        u32x4 *As = lds + st * STAGE;
        u32x4 *Bs = As + BM * CH;
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i) {
            const int s = tid + i * NT;
            const int r = s / CH, c = s % CH;
            As[r * CH + swz<CH>(r, c)] = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_PER_T; ++i) {
            const int s = tid + i * NT;
            if (B_SUB % NT == 0 || s < B_SUB) {
                const int kb = s / (BN / 8), nb = s % (BN / 8);
                // rb[i][e] holds B[k = kb*8+e][n = nb*8 .. nb*8+7]; column j of the
                // 8x8 block becomes row n = nb*8+j of B^T, eight k values.
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
                    const int d = j >> 1;
                    u32x4 t;
                    t.x = __builtin_amdgcn_perm(dword(rb[i][1], d), dword(rb[i][0], d), sel);
                    t.y = __builtin_amdgcn_perm(dword(rb[i][3], d), dword(rb[i][2], d), sel);
                    t.z = __builtin_amdgcn_perm(dword(rb[i][5], d), dword(rb[i][4], d), sel);
                    t.w = __builtin_amdgcn_perm(dword(rb[i][7], d), dword(rb[i][6], d), sel);
                    const int n = nb * 8 + j;
                    Bs[n * CH + swz<CH>(n, kb)] = t;
                }
            }
        }
    };

    f32x16 acc[FN][FM];
#pragma unroll
    for (int a = 0; a < FN; ++a)
#pragma unroll
        for (int b = 0; b < FM; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

    auto compute_slice = [&](int st) {
        const u32x4 *As = lds + st * STAGE;
        const u32x4 *Bs = As + BM * CH;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int c = 2 * kk + lhalf;
            u32x4 af[FM], bf[FN];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int r = wm * WTM + fm * 32 + lrow;
                af[fm] = As[r * CH + swz<CH>(r, c)];
            }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int n = wn * WTN + fn * 32 + lrow;
                bf[fn] = Bs[n * CH + swz<CH>(n, c)];
            }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
                    acc[fn][fm] = mfma32x32x16<DT>(bf[fn], af[fm], acc[fn][fm]);
        }
    };

    const int nk = (K + BK - 1) / BK;
    if (nk > 0) {
        load_slice(0);
        store_slice(0);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int st = kt & 1;
        if (kt + 1 < nk) load_slice(kt + 1);
        compute_slice(st);
        if (kt + 1 < nk) store_slice(st ^ 1);
        __syncthreads();
    }

    // Epilogue: + bias[n], activation, round once, masked 8-byte stores.
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = n0 + wn * WTN + fn * 32 + i * 8 + lhalf * 4;
            if (n >= N) continue;
            float b0 = 0.f, b1 = 0.f, b2 = 0.f, b3 = 0.f;
            if (bias) {
                const u32x2 bb = *reinterpret_cast<const u32x2 *>(bias + n);
                b0 = to_f32<DT>(bb.x & 0xffffu);
                b1 = to_f32<DT>(bb.x >> 16);
                b2 = to_f32<DT>(bb.y & 0xffffu);
                b3 = to_f32<DT>(bb.y >> 16);
            }
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int m = m0 + wm * WTM + fm * 32 + lrow;
                if (m >= M) continue;
                const f32x16 &a = acc[fn][fm];
                u32x2 o;
                o.x = pack2<DT>(act_fn<ACT>(a[4 * i + 0] + b0), act_fn<ACT>(a[4 * i + 1] + b1));
                o.y = pack2<DT>(act_fn<ACT>(a[4 * i + 2] + b2), act_fn<ACT>(a[4 * i + 3] + b3));
                *reinterpret_cast<u32x2 *>(C + (size_t)m * N + n) = o;
            }
        }
    }
}

template <int BM, int BN, int BK, int WM, int WN, int DT, int ACT>
hipError_t launch_gemm(const void *A, const void *B, const void *bias, void *C, int M, int N,
                       int K, int raster, int group_m, hipStream_t stream) {
    const int tiles_m = ceil_div(M, BM), tiles_n = ceil_div(N, BN);
    const long long grid = (long long)tiles_m * tiles_n;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL - kGridX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_bias_act_kernel<BM, BN, BK, WM, WN, DT, ACT>), tile_grid(grid),
                       dim3(WM * WN * 64), 0, stream, (const uint16_t *)A, (const uint16_t *)B,
                       (const uint16_t *)bias, (uint16_t *)C, M, N, K, tiles_m, tiles_n, raster,
                       group_m < 1 ? 1 : group_m);
    return hipGetLastError();
}

// ------------------------------------------------------------- bias_act ----

// Y[r][c] = act(X[r][c] + bias[c]). Each thread owns one 8-column chunk of a
// row (its bias chunk is loaded once) and strides down the rows; a wave's
// 16-byte accesses are contiguous within a row. X and Y are streamed with
// non-temporal loads and stores (each byte is touched once): 5.7 TB/s at
// 4096x4096 against 5.4 with ordinary ones.
template <int DT, int ACT>
__global__ void __launch_bounds__(256)
bias_act_kernel(const uint16_t *X, const uint16_t *__restrict__ bias, uint16_t *Y, int M,
                int N) {
    const int cpr = N / 8;
    const int chunk = blockIdx.x * 256 + threadIdx.x;
    if (chunk >= cpr) return;
    float bv[8];
    if (bias) {
        const u32x4 b = *reinterpret_cast<const u32x4 *>(bias + chunk * 8);
        const uint32_t w[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            bv[2 * e] = to_f32<DT>(w[e] & 0xffffu);
            bv[2 * e + 1] = to_f32<DT>(w[e] >> 16);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) bv[e] = 0.0f;
    }
    constexpr int U = 4;
    // 64-bit row index: r0 + gridDim.y * U may pass 2^31 - 1 on the last step.
    for (long long r0 = (long long)blockIdx.y * U; r0 < M; r0 += (long long)gridDim.y * U) {
        u32x4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (r0 + u < M)
                x[u] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4 *>(X + (size_t)(r0 + u) * N + chunk * 8));
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (r0 + u >= M) continue;
            const uint32_t w[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o[e] = pack2<DT>(act_fn<ACT>(to_f32<DT>(w[e] & 0xffffu) + bv[2 * e]),
                                 act_fn<ACT>(to_f32<DT>(w[e] >> 16) + bv[2 * e + 1]));
            u32x4 y = {o[0], o[1], o[2], o[3]};
            __builtin_nontemporal_store(y, reinterpret_cast<u32x4 *>(Y + (size_t)(r0 + u) * N + chunk * 8));
        }
    }
}

// Split-K second pass: C[r][c] = act(sum_{s<S} P[s][r][c] + bias[c]), with P
// the fp32 partial sums [S][M][N] of disjoint K ranges, added in s order (the
// result does not depend on which partial was written first), then one
// rounding. Thread layout as bias_act_kernel: one 8-column chunk per thread,
// striding down the rows.
template <int DT, int ACT>
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const float *__restrict__ P, int S, const uint16_t *__restrict__ bias,
                     uint16_t *__restrict__ C, int M, int N) {
    const int cpr = N / 8;
    const int chunk = blockIdx.x * 256 + threadIdx.x;
    if (chunk >= cpr) return;
    float bv[8];
    if (bias) {
        const u32x4 b = *reinterpret_cast<const u32x4 *>(bias + chunk * 8);
        const uint32_t w[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            bv[2 * e] = to_f32<DT>(w[e] & 0xffffu);
            bv[2 * e + 1] = to_f32<DT>(w[e] >> 16);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) bv[e] = 0.0f;
    }
    const size_t plane = (size_t)M * N;
    for (long long r = blockIdx.y; r < M; r += gridDim.y) {   // 64-bit: see bias_act_kernel
        const float *p = P + (size_t)r * N + chunk * 8;
        f32x4 lo = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
        f32x4 hi = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p + 4));
        for (int s = 1; s < S; ++s) {
            lo += __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p + s * plane));
            hi += __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p + s * plane + 4));
        }
        u32x4 y;
        y.x = pack2<DT>(act_fn<ACT>(lo[0] + bv[0]), act_fn<ACT>(lo[1] + bv[1]));
        y.y = pack2<DT>(act_fn<ACT>(lo[2] + bv[2]), act_fn<ACT>(lo[3] + bv[3]));
        y.z = pack2<DT>(act_fn<ACT>(hi[0] + bv[4]), act_fn<ACT>(hi[1] + bv[5]));
        y.w = pack2<DT>(act_fn<ACT>(hi[2] + bv[6]), act_fn<ACT>(hi[3] + bv[7]));
        *reinterpret_cast<u32x4 *>(C + (size_t)r * N + chunk * 8) = y;
    }
}

template <int ACT>
__global__ void __launch_bounds__(256) epilogue_probe_kernel(const float *z, float *y, long long n) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i < n) y[i] = act_fn<ACT>(z[i]);
}

}  // namespace gba
