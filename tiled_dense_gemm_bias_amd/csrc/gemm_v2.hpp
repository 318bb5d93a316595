// Direct-to-LDS pipelined GEMM kernel for gfx950 (the library's main kernel).
//
// Same computation and epilogue as the register-staged kernel in
// gba_kernels.hpp; what changes is how tiles reach the matrix cores:
//  * Global -> LDS: buffer_load_dwordx4 ... lds. Each lane's 16 bytes go straight
//    into LDS at (wave base + 16 * lane); no VGPRs hold the tile, and the buffer
//    descriptor's range check writes zeros for rows, columns or K past the edge
//    (the masking of edge tiles and of the K tail).
//  * STAGES-deep LDS ring: slice t+STAGES is requested as soon as every wave has
//    finished reading slice t, so STAGES-1 slices of global latency are covered.
//  * A stays K-contiguous in LDS ([BM][BK], 16-byte chunks XOR-swizzled by row);
//    B stays N-contiguous ([BK][BN], chunks swizzled by k row) and the MFMA's
//    K-contiguous B^T operand is read with ds_read_b64_tr_b16: in each group of
//    16 lanes, lanes 4r..4r+3 name four 8-byte pieces of k row r and lane i
//    receives column i of that 4 x 16 block.
//  * Fragments for the next 16-deep K step are read while the current step's
//    MFMAs run; the barrier that publishes slice t+1 sits before the last step
//    of slice t, so its first fragments are also prefetched.
//  * One barrier per slice, with explicit vmcnt waits: the loads of later slices
//    stay in flight across it.
#pragma once

#include "gba_kernels.hpp"

namespace gba {

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define GBA_LDS __attribute__((address_space(3)))

// s_waitcnt with only vmcnt limited (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// vmcnt limited to N and lgkmcnt to 0: this wave's loads of the slice being
// published have landed and its own LDS reads have all returned.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

__device__ __forceinline__ void block_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Raw buffer resource over [base, base + bytes); reads past it return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

constexpr uint32_t kOobOffset = 0x80000000u;   // beyond every descriptor's range

// buffer_load_dwordx4 ... lds: lane l's 16 bytes land at LDS byte address
// lds_base + 16 l (lds_base wave-uniform, in M0). Issued as inline assembly so
// that the compiler neither counts it nor guards later LDS reads with vmcnt(0):
// the kernel waits for these loads itself, with explicit vmcnt limits. (Waits
// the compiler places for its own loads only ever over-wait because of them.)
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voffset,
                                                  uint32_t lds_base) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %0, %1, 0 offen lds"
        :
        : "v"(voffset), "s"(rsrc), "s"(lds_base)
        : "memory", "m0");
}

template <int BM, int BN, int BK, int WM, int WN, int STAGES, int DT, int ACT>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_v2_kernel(const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
               const uint16_t *__restrict__ bias, uint16_t *__restrict__ C, int M, int N, int K,
               int tiles_m, int tiles_n, int raster, int group_m) {
    constexpr int NT = WM * WN * 64;
    constexpr int CHA = BK / 8;          // 16-byte chunks per A row in LDS
    constexpr int CHB = BN / 8;          // 16-byte chunks per B row in LDS
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int KK = BK / 16;          // MFMA K steps per slice
    constexpr int A_BYTES = BM * BK * 2, B_BYTES = BK * BN * 2;
    constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    constexpr int A_LD = BM * CHA / NT;  // buffer loads per thread per slice
    constexpr int B_LD = BK * CHB / NT;
    constexpr int LD = A_LD + B_LD;
    static_assert(BK == 32 || BK == 64, "BK must be 32 or 64");
    static_assert(BN >= 128, "B swizzle needs at least 16 chunks per row");
    static_assert((BM * CHA) % NT == 0 && (BK * CHB) % NT == 0, "slices split evenly");
    static_assert(STAGES >= 2 && STAGES * STAGE_BYTES <= 160 * 1024, "LDS ring too large");
    static_assert((STAGES - 1) * LD < 64, "vmcnt range");

    __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE_BYTES];

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
    const int nk = (K + BK - 1) / BK;

    const int rows_a = min(M - m0, BM);
    const uint32_t smem_lds = (uint32_t)(uintptr_t)(GBA_LDS void *)smem;
    const int wid_s = __builtin_amdgcn_readfirstlane(wid);

    // Per-thread load offsets within a slice (bytes), fixed for the whole K loop:
    // the per-slice K (A) and k-row (B) advance goes into the descriptor base.
    uint32_t a_off[A_LD];
    int a_k[A_LD];
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
        const int s = i * NT + tid;
        const int r = s / CHA, p = s % CHA;
        const int c = swz<CHA>(r, p);                 // XOR swizzle is an involution
        a_k[i] = c * 8;
        a_off[i] = (uint32_t)r * (uint32_t)K * 2u + (uint32_t)c * 16u;
    }
    uint32_t b_off[B_LD];
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
        const int s = i * NT + tid;
        const int r = s / CHB, p = s % CHB;
        const int c = p ^ (((r & 3) * 2 + ((r >> 3) & 1) * 8) & (CHB - 1));
        const bool ok = n0 + c * 8 < N;
        b_off[i] = ok ? (uint32_t)r * (uint32_t)N * 2u + (uint32_t)c * 16u : kOobOffset;
    }

    auto issue_slice = [&](int kt) {
        const int stage = kt % STAGES;
        const uint32_t la = smem_lds + (uint32_t)(stage * STAGE_BYTES + wid_s * 64 * 16);
        const uint32_t lb = la + A_BYTES;
        const int k0 = kt * BK;
        // A: rows [m0, m0+rows_a) from column k0 on; rows past M read zero.
        const __amdgpu_buffer_rsrc_t rsrc_a =
            make_rsrc(A + (size_t)m0 * K + k0, (uint32_t)rows_a * (uint32_t)K * 2u - (uint32_t)k0 * 2u);
        if (k0 + BK <= K) {
#pragma unroll
            for (int i = 0; i < A_LD; ++i) buffer_load_lds16(rsrc_a, a_off[i], la + i * NT * 16);
        } else {
            // K tail: chunks past K would wrap into the next row; send them out of range.
#pragma unroll
            for (int i = 0; i < A_LD; ++i)
                buffer_load_lds16(rsrc_a, k0 + a_k[i] < K ? a_off[i] : kOobOffset,
                                  la + i * NT * 16);
        }
        // B: k rows [k0, min(K, k0+BK)) of columns from n0; rows past K read zero.
        const int rows_b = min(K - k0, BK);
        const __amdgpu_buffer_rsrc_t rsrc_b =
            make_rsrc(B + (size_t)k0 * N + n0, (uint32_t)rows_b * (uint32_t)N * 2u);
#pragma unroll
        for (int i = 0; i < B_LD; ++i) buffer_load_lds16(rsrc_b, b_off[i], lb + i * NT * 16);
    };

    // Fragment addresses (bytes within a stage) for MFMA step kk.
    const int lrow = lane & 31, lhalf = lane >> 5;
    const int tg = lane >> 4, tj = lane & 15;
    auto a_addr = [&](int fm, int kk) -> int {
        const int r = wm * WTM + fm * 32 + lrow;
        return r * (BK * 2) + swz<CHA>(r, 2 * kk + lhalf) * 16;
    };
    auto b_addr = [&](int fn, int kk, int h) -> int {
        const int k = kk * 16 + 8 * (tg >> 1) + 4 * h + (tj >> 2);
        const int n = wn * WTN + fn * 32 + 16 * (tg & 1) + 4 * (tj & 3);
        const int c = (n >> 3) ^ (((k & 3) * 2 + ((k >> 3) & 1) * 8) & (CHB - 1));
        return A_BYTES + k * (BN * 2) + c * 16 + (n & 4) * 2;
    };

    f32x16 acc[FN][FM];
#pragma unroll
    for (int a = 0; a < FN; ++a)
#pragma unroll
        for (int b = 0; b < FM; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

    u32x4 fa[2][FM], fb[2][FN];
    auto load_frags = [&](int buf, int stage, int kk) {
        const char *base = smem + stage * STAGE_BYTES;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            fa[buf][fm] = *reinterpret_cast<const u32x4 *>(base + a_addr(fm, kk));
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (GBA_LDS i16x4 *)(base + b_addr(fn, kk, 0)));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (GBA_LDS i16x4 *)(base + b_addr(fn, kk, 1)));
            fb[buf][fn] = __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    };

    // Prologue: request slices 0 .. STAGES-1, wait for slice 0.
#pragma unroll
    for (int s = 0; s < STAGES; ++s)
        if (s < nk) issue_slice(s);
    if (nk > 0) {
        // slices 1..STAGES-1 may stay in flight
        if (nk >= STAGES)
            wait_vmcnt<(STAGES - 1) * LD>();
        else
            wait_vmcnt<0>();
        block_barrier();
        load_frags(0, 0, 0);
    }

    for (int kt = 0; kt < nk; ++kt) {
        const int stage = kt % STAGES;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const int cur = kk & 1;
            if (kk + 1 < KK) {
                load_frags(cur ^ 1, stage, kk + 1);
            } else if (kt + 1 < nk) {
                // Publish slice kt+1: own loads landed and own reads of slice kt
                // returned, then the same for every wave.
                const int later = nk - 1 - (kt + 1);   // slices issued after kt+1
                if (later >= STAGES - 2)
                    wait_vmcnt_lgkm0<(STAGES - 2) * LD>();
                else if (STAGES >= 4 && later == 2)
                    wait_vmcnt_lgkm0<2 * LD>();
                else if (STAGES >= 3 && later == 1)
                    wait_vmcnt_lgkm0<LD>();
                else
                    wait_vmcnt_lgkm0<0>();
                block_barrier();
                // Every wave is done reading slice kt's LDS (its last fragments were
                // read before the barrier): reuse that stage for slice kt+STAGES.
                if (kt + STAGES < nk) issue_slice(kt + STAGES);
                load_frags(cur ^ 1, (kt + 1) % STAGES, 0);
            }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
                    acc[fn][fm] = mfma32x32x16<DT>(fb[cur][fn], fa[cur][fm], acc[fn][fm]);
        }
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

template <int BM, int BN, int BK, int WM, int WN, int STAGES, int DT, int ACT>
hipError_t launch_gemm_v2(const void *A, const void *B, const void *bias, void *C, int M, int N,
                          int K, int raster, int group_m, hipStream_t stream) {
    const int tiles_m = ceil_div(M, BM), tiles_n = ceil_div(N, BN);
    const long long grid = (long long)tiles_m * tiles_n;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL - kGridX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_v2_kernel<BM, BN, BK, WM, WN, STAGES, DT, ACT>), tile_grid(grid),
                       dim3(WM * WN * 64), 0, stream, (const uint16_t *)A, (const uint16_t *)B,
                       (const uint16_t *)bias, (uint16_t *)C, M, N, K, tiles_m, tiles_n, raster,
                       group_m < 1 ? 1 : group_m);
    return hipGetLastError();
}

}  // namespace gba
