// Persistent GEMM with 8-bit float inputs: C = act(scale * A.W^T + bias), A
// [M,K] and W [N,K] (the transpose_B layout) in OCP E4M3 or E5M2, bias and C
// in fp16/bf16, fp32 accumulation, on gfx950's v_mfma_f32_16x16x128_f8f6f4.
//
// The tiles have the shape of the 16-bit transpose_B kernel's (gemm_v5.hpp): a
// 256x256 output tile per workgroup, K slices of 128 bytes (here 128 values),
// A's and W's tiles 256 rows of 8 16-byte chunks, loaded straight into a
// two-stage LDS ring with buffer range checks zero-filling the edges. One MFMA
// consumes a whole slice: lane l of a 16-row block holds row r = l % 16 and the
// 32 bytes of logical chunks 2g, 2g+1 (g = l / 16), i.e. k = 32g .. 32g+31. The
// matrix instruction pairs lane i + 16g of one operand with lane j + 16g of the
// other, so every row must hand over its 32 bytes in the same order: the
// swizzle moves whole 32-byte pairs, logical chunk c of row r at physical chunk
// c ^ 2((r / 2) % 4). A lane's fragment is then one contiguous, aligned 32-byte
// read from pair g ^ ((r / 2) % 4), and the 8 rows one read serves per cycle
// hit 8 distinct bank groups.
//
// Each wave owns a 128x128 block: 8 x 8 MFMAs of 16x16 per slice, issued in two
// steps by row-block halves:
//   step 0: rows 0..3 x columns 0..7, reading this slice's A fragments 4..7;
//   barrier (the next slice has landed; every wave is done with this one);
//   step 1: rows 4..7 x columns 0..7, reading the next slice's A fragments
//           0..3 and each W fragment right after its last use, and issuing
//           the global->LDS loads two slices ahead into the stage just freed.
// The slice stream runs across a workgroup's tiles as in gemm_v5.hpp: the next
// tile's first two slices load during the current tile's last steps.
//
// PARTIAL (split-K first pass): the work units are (tile, split) pairs; unit
// (t, s) runs K slices [s nk / S, (s+1) nk / S) of tile t and stores scale * its
// fp32 sums to part[s][M][N]; splitk_reduce_kernel adds them, then bias, act.
#pragma once

#include "gemm_v5.hpp"

namespace gba {

enum { FP8_E4M3 = 0, FP8_E5M2 = 1 };
typedef int i32x8 __attribute__((ext_vector_type(8)));

// acc += A.B on 16x16x128 8-bit blocks (cbsz/blgp 0: E4M3, 1: E5M2, for the
// first and second operand). Issued as inline assembly with the accumulator
// tied to the destination: the compiler's own form of this instruction does not
// tie them, so each MFMA wrote a fresh register and the 64 accumulators of a
// wave were copied around (and spilled) every slice. The compiler therefore
// sees neither this instruction's latency nor its register hazards; the kernel
// covers them itself (see hazard_gap below). The operands come from LDS reads,
// whose waits the compiler places from the asm operands.
// FIRST: the accumulator input is the constant 0 (the tile's first slice), so
// every definition of an accumulator is one of these instructions and the
// accumulators stay in AGPRs throughout.
template <int FMT, bool FIRST>
__device__ __forceinline__ void mfma16x16x128_f8(f32x4 &acc, const i32x8 &a, const i32x8 &b) {
    if constexpr (FIRST) {
        if constexpr (FMT == FP8_E4M3)
            asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
        else
            asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, 0 cbsz:1 blgp:1"
                         : "=a"(acc)
                         : "v"(a), "v"(b));
    } else {
        if constexpr (FMT == FP8_E4M3)
            asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
        else
            asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0 cbsz:1 blgp:1"
                         : "+a"(acc)
                         : "v"(a), "v"(b));
    }
}

// An accumulator as a VGPR value (the compiler copies it out of its AGPRs).
__device__ __forceinline__ f32x4 acc_value(const f32x4 &acc) {
    f32x4 v;
    asm volatile("" : "=v"(v) : "0"(acc));
    return v;
}

// 32 wait states: more than any matrix instruction needs between writing an
// accumulator and a vector instruction reading it (at most 19, for 16 passes).
__device__ __forceinline__ void hazard_gap() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

template <int FMT, int DT, int ACT, bool PARTIAL = false>
__global__ void __launch_bounds__(256)
gemm_f8_kernel(const uint8_t *__restrict__ A, const uint8_t *__restrict__ W,
               const uint16_t *__restrict__ bias, uint16_t *__restrict__ C, int M, int N, int K,
               float scale, int tiles_m, int tiles_n, int raster, int group_m, int splits,
               float *__restrict__ part) {
    constexpr int BM = 256, BN = 256, BK = 128;   // BK in values = bytes
    constexpr int NT = 256, BD = 16;
    constexpr int WTM = 128, WTN = 128, FM = 8, FN = 8, HM = FM / 2;
    constexpr int A_BYTES = BM * BK, STAGE_BYTES = 2 * A_BYTES;
    constexpr int A_LD = BM * 8 / NT, LD = 2 * A_LD;   // 16-byte loads per thread and slice

    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE_BYTES];
    // A tile's bias, staged in LDS with the tile's first slice (as in the 16-bit
    // persistent kernel): one 1 KiB slot per wave and per tile parity.
    __shared__ __attribute__((aligned(1024))) char bias_smem[2 * 4 * 1024];
    // Epilogue staging: two buffers of 16 rows x 64 columns of C per wave.
    constexpr int STG_BYTES = 16 * 64 * 2;
    __shared__ __attribute__((aligned(1024))) char stage_smem[PARTIAL ? 16 : 4 * 2 * STG_BYTES];
    static_assert(2 * STAGE_BYTES + 2 * 4 * 1024 + 4 * 2 * STG_BYTES <= 160 * 1024,
                  "LDS ring + bias slots + staging too large");

    const int tid = threadIdx.x;
    const int lane = tid & 63, wid = tid >> 6;
    const int wm = wid >> 1, wn = wid & 1;
    const int nk_all = (K + BK - 1) / BK;
    const int tiles = tiles_m * tiles_n;
    const int T = PARTIAL ? tiles * splits : tiles;   // work units
    const int G = gridDim.x;
    const int wid_s = __builtin_amdgcn_readfirstlane(wid);
    const uint32_t smem_lds = (uint32_t)(uintptr_t)(GBA_LDS void *)smem;
    const int slot = raster ? xcd_remap(blockIdx.x, G) : (int)blockIdx.x;

    // A work unit: its tile, split, and K slices [kt0, kt0 + nkl). It streams
    // nk = max(nkl, 2) slices (the stream below assumes two); the extra one,
    // for a single-slice unit, is all zeros.
    struct Tile {
        int m0, n0, kt0, nkl, nk, split;
    };
    auto tile_of = [&](int r, Tile &t) -> bool {
        int idx = r * G + slot;
        if (idx >= T) return false;
        t.split = 0;
        if constexpr (PARTIAL) {
            t.split = idx / tiles;
            idx -= t.split * tiles;
        }
        t.kt0 = PARTIAL ? (int)((long long)t.split * nk_all / splits) : 0;
        t.nkl = PARTIAL ? (int)((long long)(t.split + 1) * nk_all / splits) - t.kt0 : nk_all;
        t.nk = max(t.nkl, 2);
        int tm, tn;
        if (raster) {
            grouped_tile(idx, tiles_m, tiles_n, group_m, tm, tn);
        } else {
            tm = idx / tiles_n;
            tn = idx % tiles_n;
        }
        t.m0 = tm * BM;
        t.n0 = tn * BN;
        return true;
    };

    // Load i of a thread fills row 32 i + tid/8 of A's (i < 8) or W's tile at
    // physical chunk tid % 8, i.e. logical chunk (tid%8) ^ 2((row/2)%4), where
    // (row/2) % 4 = (tid/16) % 4 for every i.
    const int c_a = (tid & 7) ^ (2 * ((tid >> 4) & 3));
    const uint32_t ld_base = (uint32_t)(tid >> 3) * (uint32_t)K + (uint32_t)c_a * 16u;
    struct SliceDma {
        __amdgpu_buffer_rsrc_t ra, rw;
        uint32_t la;
        int k0;
    };
    // Slice kt of tile t into stage `stage`; slices past K (or of no tile) read
    // nothing: every lane is out of range and lands zeros, which keeps the wait
    // counts uniform.
    // (Selects, not conditional code: in the main loop this is formed in the
    // MFMA stream, where a taken branch stalls the wave.)
    // In the main loop the pieces are formed one per MFMA gap (dma_part), each
    // pinned where it is formed, with selects rather than conditional code: a
    // burst of scalar work or a taken branch between two MFMAs stalls the wave.
    auto dma_part = [&](SliceDma &d, int part, const Tile &t, bool live, int kt, int stage)
        __attribute__((always_inline)) {
        const bool any = live & (kt < t.nkl);
        const int k0 = (t.kt0 + kt) * BK;
        if (part == 0) {
            d.la = __builtin_amdgcn_readfirstlane(smem_lds + (uint32_t)(stage * STAGE_BYTES + wid_s * 64 * 16));
            d.k0 = any ? k0 : K;
            asm volatile("" : "+s"(d.la), "+s"(d.k0));
        } else if (part == 1) {
            const uint32_t rows_a = (uint32_t)min(M - t.m0, BM);
            const size_t oa = (size_t)t.m0 * K + k0;
            d.ra = make_rsrc(A + (any ? oa : 0), any ? rows_a * (uint32_t)K - (uint32_t)k0 : 0u);
            asm volatile("" : "+s"(d.ra));
        } else {
            const uint32_t rows_w = (uint32_t)min(N - t.n0, BN);
            const size_t ow = (size_t)t.n0 * K + k0;
            d.rw = make_rsrc(W + (any ? ow : 0), any ? rows_w * (uint32_t)K - (uint32_t)k0 : 0u);
            asm volatile("" : "+s"(d.rw));
        }
    };
    auto slice_dma = [&](const Tile &t, bool live, int kt, int stage) __attribute__((always_inline)) {
        SliceDma d;
        dma_part(d, 0, t, live, kt, stage);
        dma_part(d, 1, t, live, kt, stage);
        dma_part(d, 2, t, live, kt, stage);
        return d;
    };
    // Load j of a thread reads row 32 j + tid/8 of its tile's slice: offset lo[j]
    // from the slice corner, held for the whole stream; eo[j] is the offset the
    // next slice's loads use, lo[j] or (chunks past K) out of range, formed in
    // step 0's shadow so that no address arithmetic sits between step 1's loads.
    uint32_t lo[A_LD], eo[A_LD];
#pragma unroll
    for (int j = 0; j < A_LD; ++j) lo[j] = ld_base + (uint32_t)(j * 32) * (uint32_t)K;
    auto dma_one = [&](const SliceDma &d, int i) __attribute__((always_inline)) {
        const int j = i & (A_LD - 1);
        if (i < A_LD)
            buffer_load_lds16(d.ra, eo[j], d.la + j * NT * 16);
        else
            buffer_load_lds16(d.rw, eo[j], d.la + A_BYTES + j * NT * 16);
    };
    auto set_eo = [&](int k0, int j) __attribute__((always_inline)) {
        eo[j] = k0 + c_a * 16 < K ? lo[j] : kOobOffset;
        asm volatile("" : "+v"(eo[j]));
    };

    // Bias of tile t into this wave's slot of parity p: lanes 0..31 load 16 bytes
    // each (columns past N read zeros), the rest land zeros; counted in vmcnt.
    const uint32_t bias_lds = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(GBA_LDS void *)bias_smem + (uint32_t)(wid_s * 1024));
    auto bias_dma = [&](const Tile &t, int p) {
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(bias + t.n0, (uint32_t)min(N - t.n0, BN) * 2u);
        buffer_load_lds16(rb, lane < BN / 8 ? (uint32_t)lane * 16u : kOobOffset,
                          bias_lds + (uint32_t)(p * 4 * 1024));
    };

    // Fragment bases: lane l of block f reads row 16 f + l%16 of the wave's
    // rows ((row/2) % 4 = (l/2) % 4), 32-byte pair (l/16) ^ ((l/2) % 4).
    const int tg = lane >> 4, tj = lane & 15;
    const uint32_t pair = (uint32_t)((tg ^ ((tj >> 1) & 3)) * 32);
    const uint32_t ra_row = (uint32_t)(wm * WTM + tj) * BK + pair;
    const uint32_t rw_row = (uint32_t)(A_BYTES + (wn * WTN + tj) * BK) + pair;
    auto read_frag = [&](const char *base, uint32_t row0, int f) -> i32x8 {
        return *reinterpret_cast<const i32x8 *>(base + row0 + f * BD * BK);
    };

    f32x4 acc[FN][FM];
    i32x8 fa[2][HM];   // A fragments: [0] rows 0..3, [1] rows 4..7
    i32x8 fw[FN];      // W fragments of the slice being multiplied

    Tile cur_t;
    if (!tile_of(0, cur_t)) return;

    {
        const SliceDma d0 = slice_dma(cur_t, true, 0, 0), d1 = slice_dma(cur_t, true, 1, 1);
        if (bias) bias_dma(cur_t, 0);   // lands with slice 0 (waited for below)
#pragma unroll
        for (int j = 0; j < A_LD; ++j) set_eo(d0.k0, j);
#pragma unroll
        for (int i = 0; i < LD; ++i) dma_one(d0, i);
#pragma unroll
        for (int j = 0; j < A_LD; ++j) set_eo(d1.k0, j);
#pragma unroll
        for (int i = 0; i < LD; ++i) dma_one(d1, i);
    }
    wait_vmcnt<LD>();
    block_barrier();
#pragma unroll
    for (int f = 0; f < HM; ++f) fa[0][f] = read_frag(smem, ra_row, f);
#pragma unroll
    for (int f = 0; f < FN; ++f) fw[f] = read_frag(smem, rw_row, f);

    const int mrow = wm * WTM + tj;
    int stage0 = 0;
    for (int r = 0;; ++r) {
        Tile nxt_t;
        const bool nxt_live = tile_of(r + 1, nxt_t);
        if (!nxt_live) nxt_t = cur_t;

        // Slice kt of this tile (FIRST: kt == 0, whose MFMAs start from zero).
        auto slice = [&](int kt, auto first) {
            constexpr bool F = decltype(first)::value;
            const int sc = (stage0 + kt) & 1;
            const char *cur_base = smem + sc * STAGE_BYTES;
            const char *nxt_base = smem + (sc ^ 1) * STAGE_BYTES;
            // step 0: rows 0..3; this slice's A fragments 4..7 are read meanwhile,
            // and (in the MFMA stream's shadow, not after the barrier where they
            // would delay step 1's first MFMA) the descriptors of the loads two
            // slices ahead
            const bool here = kt + 2 < cur_t.nk;
            SliceDma dn;
            bool bias_next = false;
#pragma unroll
            for (int q = 0; q < FN * HM; ++q) {
                const int fn = q / HM, fm = q % HM;
                mfma16x16x128_f8<FMT, F>(acc[fn][fm], fw[fn], fa[0][fm]);
                if (q % 8 == 0) fa[1][q / 8] = read_frag(cur_base, ra_row, HM + q / 8);
                if (q >= 12 && q <= 16 && q % 2 == 0)
                    dma_part(dn, (q - 12) / 2, here ? cur_t : nxt_t, here | nxt_live,
                             here ? kt + 2 : kt + 2 - cur_t.nk, sc);
                // with the next tile's slice 0, its bias into the other parity's slot
                if (q == 17) bias_next = (bias != nullptr) & (!here) & (kt + 2 == cur_t.nk) & nxt_live;
                if (q >= 18 && q < 18 + A_LD) set_eo(dn.k0, q - 18);
                __builtin_amdgcn_sched_barrier(0);
            }
            wait_vmcnt_lgkm0<0>();
            block_barrier();
            if (__builtin_expect(bias_next, 0)) bias_dma(nxt_t, (r + 1) & 1);
            // step 1: rows 4..7; the next slice's A fragments 0..3, each W
            // fragment after its last MFMA here, and the loads two slices ahead
#pragma unroll
            for (int q = 0; q < FN * HM; ++q) {
                const int fn = q / HM, fm = q % HM;
                mfma16x16x128_f8<FMT, F>(acc[fn][HM + fm], fw[fn], fa[1][fm]);
                if (q % 2 == 0) dma_one(dn, q / 2);
                if (fm == HM - 1) fw[fn] = read_frag(nxt_base, rw_row, fn);
                if (q % 8 == 1) fa[0][q / 8] = read_frag(nxt_base, ra_row, q / 8);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        slice(0, std::true_type{});
        for (int kt = 1; kt < cur_t.nk; ++kt) slice(kt, std::false_type{});

        // Epilogue while the next tile's first slices land: z = scale * acc + bias.
        hazard_gap();   // the last MFMAs' results are complete before they are read
        asm volatile("" ::: "memory");
        if constexpr (PARTIAL) {
            // scale * raw sums, 4 adjacent n of one row per lane, masked at the edges
            float *const Pt = part + (size_t)cur_t.split * M * N + (size_t)cur_t.m0 * N + cur_t.n0;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int cn = wn * WTN + 4 * tg + fn * BD;
                if (cur_t.n0 + cn >= N) continue;
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    const int rr = mrow + fm * BD;
                    if (cur_t.m0 + rr >= M) continue;
                    *reinterpret_cast<f32x4 *>(Pt + (size_t)rr * N + cn) = acc_value(acc[fn][fm]) * scale;
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            // As in the 16-bit persistent kernel: the wave's 128 x 128 block leaves
            // through two alternating 16 x 64 staging buffers of its own in LDS,
            // so that each 16-byte (non-temporal) store instruction writes 8 whole
            // 128-byte row segments; the bias is converted to fp32 once per tile (upper half of
            // the wave's slot) and read into registers once per column half.
            int ln;
            asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
            const int wn_s = wid_s & 1, wm_s = wid_s >> 1;
            char *const bias_mine = bias_smem + ((r & 1) * 4 + wid_s) * 1024;
            if (bias) {
                const uint32_t bb =
                    *reinterpret_cast<const uint32_t *>(bias_mine + wn_s * (WTN * 2) + 4 * ln);
                *reinterpret_cast<f32x2 *>(bias_mine + 512 + 8 * ln) =
                    f32x2{to_f32<DT>(bb & 0xffffu), to_f32<DT>(bb >> 16)};
            }
            char *const stg = stage_smem + wid_s * 2 * STG_BYTES;
            const int wr = ln & 15, wg = ln >> 4;   // write side: row, 4-column group
            const int rr = ln >> 3, rc = ln & 7;    // read side: row (of 8), 16-byte chunk
            char *const Cw = reinterpret_cast<char *>(C + (size_t)cur_t.m0 * N + cur_t.n0) +
                             ((size_t)wm_s * WTM * N + (size_t)wn_s * WTN) * 2;
            uint32_t st_off = (uint32_t)rr * (uint32_t)N * 2u + (uint32_t)rc * 16u;
            uint32_t pitch8 = (uint32_t)N * 16u;   // bytes between read rows rr and rr + 8
            asm volatile("" : "+v"(st_off), "+s"(pitch8));
            const int rows_left = M - cur_t.m0 - wm_s * WTM, cols_left = N - cur_t.n0 - wn_s * WTN;
            const bool full = rows_left >= WTM && cols_left >= WTN;   // no m0 + BM: overflows near 2^31
            constexpr int NG = 2 * FM;
            auto store_all = [&](auto masked) {
                f32x4 bq[4];
#pragma unroll
                for (int g = 0; g <= NG; ++g) {
                    u32x4 v[2];
                    if (g > 0) {
                        const char *const sb = stg + ((g - 1) & 1) * STG_BYTES;
#pragma unroll
                        for (int j = 0; j < 2; ++j)
                            v[j] = *reinterpret_cast<const u32x4 *>(sb + (8 * j + rr) * 128 +
                                                                    ((rc ^ (rr & 7)) * 16));
                    }
                    if (g < NG) {
                        const int fh = g / FM, fm = g % FM;
                        char *const sb = stg + (g & 1) * STG_BYTES;
                        if (g % FM == 0) {
#pragma unroll
                            for (int f = 0; f < 4; ++f)
                                bq[f] = bias ? *reinterpret_cast<const f32x4 *>(
                                                   bias_mine + 512 + (16 * (4 * fh + f) + 4 * wg) * 4)
                                             : f32x4{0.f, 0.f, 0.f, 0.f};
                        }
#pragma unroll
                        for (int f = 0; f < 4; ++f) {
                            const f32x4 a = acc_value(acc[4 * fh + f][fm]);
                            u32x2 o;
                            o.x = pack2<DT>(act_fn<ACT>(fmaf(a[0], scale, bq[f][0])),
                                            act_fn<ACT>(fmaf(a[1], scale, bq[f][1])));
                            o.y = pack2<DT>(act_fn<ACT>(fmaf(a[2], scale, bq[f][2])),
                                            act_fn<ACT>(fmaf(a[3], scale, bq[f][3])));
                            const int chunk = 2 * f + (wg >> 1);
                            *reinterpret_cast<u32x2 *>(sb + wr * 128 + ((chunk ^ (wr & 7)) * 16) +
                                                       (wg & 1) * 8) = o;
                        }
                    }
                    if (g > 0) {
                        const int fh = (g - 1) / FM, fm = (g - 1) % FM;
#pragma unroll
                        for (int j = 0; j < 2; ++j) {
                            if (masked && (fm * BD + 8 * j + rr >= rows_left || fh * 64 + rc * 8 >= cols_left))
                                continue;
                            const uint32_t offs = st_off + (uint32_t)(2 * fm + j) * pitch8 +
                                                  (uint32_t)(fh * 128);
                            __builtin_nontemporal_store(v[j], reinterpret_cast<u32x4 *>(Cw + offs));
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
            if (full)
                store_all(std::false_type{});
            else
                store_all(std::true_type{});
        }

        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        stage0 = (stage0 + cur_t.nk) & 1;
        if (!nxt_live) break;
        cur_t = nxt_t;
    }
    wait_vmcnt<0>();
}

// Grid: one workgroup per CU, or fewer when there are fewer tiles.
template <int FMT, int DT, int ACT>
hipError_t launch_gemm_f8(const void *A, const void *W, const void *bias, void *C, int M, int N,
                          int K, float scale, int raster, int group_m, hipStream_t stream) {
    const int tiles_m = ceil_div(M, 256), tiles_n = ceil_div(N, 256);
    const long long tiles = (long long)tiles_m * tiles_n;
    if (tiles <= 0) return hipSuccess;
    // Tile indices r * G + slot run up to tiles + G - 1: keep them in int.
    if (tiles > 0x7fffffffLL - 0x10000) return hipErrorInvalidValue;
    int cus = 0;
    const hipError_t e = current_cus(&cus);
    if (e != hipSuccess) return e;
    const int grid = (int)(tiles < cus ? tiles : cus);
    hipLaunchKernelGGL((gemm_f8_kernel<FMT, DT, ACT>), dim3((unsigned)grid), dim3(256), 0, stream,
                       (const uint8_t *)A, (const uint8_t *)W, (const uint16_t *)bias,
                       (uint16_t *)C, M, N, K, scale, tiles_m, tiles_n, raster,
                       group_m < 1 ? 1 : group_m, 1, (float *)nullptr);
    return hipGetLastError();
}

// Split-K first pass: tiles x splits work units, one workgroup per CU (or per
// unit when there are fewer), scale * partial sums into part ([splits][M][N]).
template <int FMT>
hipError_t launch_gemm_f8_partial(const void *A, const void *W, float *part, int M, int N, int K,
                                  float scale, int splits, int raster, int group_m,
                                  hipStream_t stream) {
    const int tiles_m = ceil_div(M, 256), tiles_n = ceil_div(N, 256);
    const long long units = (long long)tiles_m * tiles_n * splits;
    if (units <= 0) return hipSuccess;
    if (units > 0x7fffffffLL - 0x10000 || splits < 1) return hipErrorInvalidValue;
    int cus = 0;
    const hipError_t e = current_cus(&cus);
    if (e != hipSuccess) return e;
    const int grid = (int)(units < cus ? units : cus);
    hipLaunchKernelGGL((gemm_f8_kernel<FMT, 0, ACT_NONE, true>), dim3((unsigned)grid), dim3(256), 0,
                       stream, (const uint8_t *)A, (const uint8_t *)W, (const uint16_t *)nullptr,
                       (uint16_t *)nullptr, M, N, K, scale, tiles_m, tiles_n, raster,
                       group_m < 1 ? 1 : group_m, splits, part);
    return hipGetLastError();
}

}  // namespace gba
