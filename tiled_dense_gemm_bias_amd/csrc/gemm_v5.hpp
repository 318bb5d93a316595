// Persistent GEMM kernel (kernel 4): the interleaved 16x16x32 main loop of
// gemm_v3.hpp, run by one workgroup per CU over all of its tiles.
//
// One workgroup per CU walks its tiles (t = w, w + G, w + 2G, ... in raster
// order, G = grid size) as one stream of 64-deep K slices through a two-stage
// LDS ring. The loads of stream position p + 2 are issued in the last MFMA step
// of position p; positions past a tile's last slice are the next tile's first
// slices. So when a tile's main loop ends, the next tile's slice 0 is already in
// LDS (published by the last barrier) and its slice 1 is in flight; both land
// while the epilogue (bias, activation, rounding, stores) runs, and the next
// main loop starts without the pipeline fill of a fresh workgroup.
//
// The main loop is written so that a wave issues almost nothing but MFMAs, LDS
// reads and direct-to-LDS loads (vector ALU work between MFMAs that also carry
// memory instructions costs the matrix core issue time; address arithmetic is
// kept out of the stream):
//  * LDS ring layout [A stage 0 | A stage 1 | B stage 0 | B stage 1] (32 KiB
//    each). Every fragment read is a per-thread base register, which names the
//    stage being read, plus a compile-time offset (the ds_read offset field).
//    Once per slice each base moves to the other stage (one add, issued among
//    MFMAs that carry no memory instructions).
//  * Each thread's load offsets (one per load of a slice) are held in
//    registers for the whole stream; a slice's K position moves the buffer
//    descriptor's base, not the offsets. They are re-masked (out-of-range
//    offset) only where the load stream enters a tile (N or M edge) or the
//    last, partial K slice (chunks past K), a few times per tile.
//  * The LDS destination of each load is one scalar add into M0 from a scalar
//    stage base.
//
// Tiles, LDS swizzles, fragments, MFMA order and epilogue are gemm_v3's, so
// results are bit-identical to it. TB (transpose_B, B given as an (N,K) array
// W) and TA (transpose_A, A given as a (K,M) array At) are gemm_v3's layouts.
#pragma once

#include "gemm_v3.hpp"

#include <type_traits>
#include <utility>

namespace gba {


// This lane's index in its wave, read afresh (volatile: not merged with earlier
// reads, so no register has to hold it across the loops).
__device__ __forceinline__ int lane_now() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// buffer_load_dwordx4 ... lds into LDS byte address lds_base + IMM (+ 16 per lane).
template <uint32_t IMM>
__device__ __forceinline__ void buffer_load_lds16_at(__amdgpu_buffer_rsrc_t rsrc, uint32_t voffset,
                                                     uint32_t lds_base) {
    asm volatile(
        "s_add_u32 m0, %2, %3\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %0, %1, 0 offen lds"
        :
        : "v"(voffset), "s"(rsrc), "s"(lds_base), "n"(IMM)
        : "memory", "m0", "scc");
}

template <int BM, int BN, int WM, int WN, int DT, int ACT, bool TB = false, bool TA = false>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_v5_kernel(const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
               const uint16_t *__restrict__ bias, uint16_t *__restrict__ C, int M, int N, int K,
               int tiles_m, int tiles_n, int raster, int group_m) {
    constexpr int BK = 64, MS = 16, BD = 16, KS = 32, KK = BK / KS;
    constexpr int NW = WM * WN, NT = NW * 64;
    constexpr int CHA = BK / 8, CHB = BN / 8;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / BD, FN = WTN / BD;
    constexpr int NFA = (TA ? 2 : 1) * FM;
    constexpr int NMF = FM * FN, NPF = NFA + (TB ? 1 : 2) * FN;
    constexpr int A_BYTES = BM * BK * 2, B_BYTES = BK * BN * 2;
    constexpr uint32_t B_REGION = 2 * A_BYTES;   // B's stages follow A's
    constexpr int A_LD = BM * CHA / NT, B_LD = (TB ? BN * CHA : BK * CHB) / NT, LD = A_LD + B_LD;
    constexpr int EVERY = NMF / LD;
    static_assert(KK == 2, "two MFMA steps per slice");
    static_assert(WTM % BD == 0 && WTN % BD == 0, "wave tile must be whole MFMA blocks");
    static_assert(BN >= 128, "B swizzle needs at least 16 chunks per row");
    static_assert(!TA || BM == BN, "At's tile is loaded with B's per-thread mapping");
    static_assert((BM * CHA) % NT == 0 && B_LD * NT == (TB ? BN * CHA : BK * CHB),
                  "slices split evenly");
    static_assert(A_BYTES == 32768 && B_BYTES == 32768,
                  "fragment offsets (stage + block) must fit the 16-bit ds_read offset");
    static_assert(2 * LD < 64 && NMF % LD == 0 && NPF <= NMF, "step layout");
    static_assert(A_LD == 8 && B_LD == 8, "one register of load offsets per load");
    // Needs at least two K slices (K > 64): the library sends K <= 64 elsewhere.

    __shared__ __attribute__((aligned(1024))) char smem[2 * (A_BYTES + B_BYTES)];
    // The bias of a tile, staged in LDS with the tile's first slice so that the
    // epilogue reads it with ds_read instead of waiting on global loads (which
    // would also wait for the next tile's slices in flight). One 1 KiB slot per
    // wave (its own copy: no barrier needed) and per tile parity.
    __shared__ __attribute__((aligned(1024))) char bias_smem[2 * NW * 1024];
    static_assert(BN * 2 <= 1024 && BN / 8 <= 64, "a tile's bias fits one load per wave");
    // Epilogue staging: two buffers of 16 rows x 64 columns of C per wave (see
    // the epilogue).
    constexpr int STG_BYTES = 16 * 64 * 2;
    __shared__ __attribute__((aligned(1024))) char stage_smem[NW * 2 * STG_BYTES];
    static_assert(WTN == 128 && BD == 16, "the epilogue stages 16 x 64 halves of 128-column wave blocks");
    static_assert(2 * (A_BYTES + B_BYTES) + 2 * NW * 1024 + NW * 2 * STG_BYTES <= 160 * 1024,
                  "LDS ring + bias slots + staging too large");

    const int tid = threadIdx.x;
    const int wid = tid >> 6;
    const int nk = (K + BK - 1) / BK;
    // Index of every tile's partial last slice (K % 64 != 0), or -1 (kept as an
    // int: a uniform bool can end up materialised in a vector register).
    const int tail_k = (K % BK) != 0 ? nk - 1 : -1;
    const int T = tiles_m * tiles_n;
    const int G = gridDim.x;
    const int wid_s = __builtin_amdgcn_readfirstlane(wid);
    const uint32_t smem_lds = (uint32_t)(uintptr_t)(GBA_LDS void *)smem;
    // Position of this workgroup inside every round of G tiles.
    const int slot = raster ? xcd_remap(blockIdx.x, G) : (int)blockIdx.x;

    // Tile of round r: index r*G + slot in raster order (-1 past the last tile).
    struct Tile {
        int m0, n0, rows;   // rows: of A's tile (M edge)
    };
    auto tile_of = [&](int r, Tile &t) -> bool {
        const int idx = r * G + slot;
        if (idx >= T) return false;
        int tm, tn;
        if (raster) {
            grouped_tile(idx, tiles_m, tiles_n, group_m, tm, tn);
        } else {
            tm = idx / tiles_n;
            tn = idx % tiles_n;
        }
        t.m0 = tm * BM;
        t.n0 = tn * BN;
        t.rows = min(M - t.m0, BM);
        return true;
    };

    // ---- loads ----
    // A-like tiles (A [M,K]; W [N,K] with TB): load i of a thread fills LDS chunk
    // i*NT + tid of the stage: row 32i + tid/8, logical chunk c_a = (tid%8) ^
    // (row%8), the same for every i. B-like tiles (B [K,N]; At [K,M] with TA):
    // k row 8j + tid/32, logical chunk c_b(j) = c_b0 ^ 8(j%4) (the B swizzle's
    // row/8 term). The offsets below are relative to the slice's corner, which
    // the buffer descriptor carries.
    static_assert(NT == 256 && CHA == 8 && CHB == 32, "loader mapping written for 256 threads, BK 64, BN 256");
    // av: A-like offsets (rows 32i); chunks past K of the last slice masked when
    // `tail`. bv: B [K,N] offsets (k rows 8j) of a tile at column n0, chunks
    // past N masked. tv: At [K,M] offsets of a tile at row m0, chunks past M
    // masked. The row and column masks of the descriptor's range cover the
    // other edges (rows of A/W past M/N, k rows past K).
    // The thread index is rebuilt in each call (lane_now), so that the offsets
    // are formed where they are set rather than hoisted out of the loops and
    // held, with the index, across them (which would spill).
    uint32_t av[8], bv[8], tv[8];
    auto set_av = [&](bool tail) __attribute__((always_inline)) {
        const int t = wid_s * 64 + lane_now();
        const int ca = (t & 7) ^ ((t >> 3) & 7);
        const bool ok = !tail || (nk - 1) * BK + ca * 8 < K;
        const uint32_t base = (uint32_t)(t >> 3) * (uint32_t)K * 2u + (uint32_t)ca * 16u;
#pragma unroll
        for (int i = 0; i < 8; ++i) av[i] = ok ? base + (uint32_t)(i * 64) * (uint32_t)K : kOobOffset;
    };
    auto set_bv = [&](int n0) __attribute__((always_inline)) {
        const int t = wid_s * 64 + lane_now();
        const int cb0 = (t & 31) ^ bswz<CHB>(t >> 5);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int c = cb0 ^ (8 * (j & 3));
            bv[j] = n0 + c * 8 < N ? (uint32_t)((t >> 5) + 8 * j) * (uint32_t)N * 2u + (uint32_t)c * 16u
                                   : kOobOffset;
        }
    };
    auto set_tv = [&](int m0) __attribute__((always_inline)) {
        const int t = wid_s * 64 + lane_now();
        const int cb0 = (t & 31) ^ bswz<CHB>(t >> 5);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int c = cb0 ^ (8 * (j & 3));
            tv[j] = m0 + c * 8 < M ? (uint32_t)((t >> 5) + 8 * j) * (uint32_t)M * 2u + (uint32_t)c * 16u
                                   : kOobOffset;
        }
    };
    // Descriptors of stream position (tile t, slice kt); a dead position (past the
    // last tile) has empty ranges: every lane reads zeros and no memory, which
    // keeps the wait counts uniform.
    struct SliceDma {
        __amdgpu_buffer_rsrc_t ra, rb;
    };
    // A position's slice corners and byte ranges, from which its descriptors are
    // made. From one slice to the next of a tile (other than into the partial
    // last slice) they change by constants: the A-like corner moves 64 elements
    // along K (its range shrinks by 128 bytes), the B-like corner 64 rows (its
    // range is one slice); so only the first slice of a tile, the last one and
    // dead positions are formed from scratch.
    struct DmaPos {
        const uint16_t *pa, *pb;
        uint32_t na, nb;
    };
    auto pos_full = [&](const Tile &t, bool live, int kt) __attribute__((always_inline)) {
        const int k0 = kt * BK;
        const uint32_t kin = (uint32_t)min(K - k0, BK);
        DmaPos p;
        if constexpr (TA) {
            p.pa = A + (live ? (size_t)k0 * M + t.m0 : 0);
            p.na = live ? kin * (uint32_t)M * 2u : 0u;
        } else {
            p.pa = A + (live ? (size_t)t.m0 * K + k0 : 0);
            p.na = live ? (uint32_t)t.rows * (uint32_t)K * 2u - (uint32_t)k0 * 2u : 0u;
        }
        if constexpr (TB) {
            p.pb = B + (live ? (size_t)t.n0 * K + k0 : 0);
            p.nb = live ? (uint32_t)min(N - t.n0, BN) * (uint32_t)K * 2u - (uint32_t)k0 * 2u : 0u;
        } else {
            p.pb = B + (live ? (size_t)k0 * N + t.n0 : 0);
            p.nb = live ? kin * (uint32_t)N * 2u : 0u;
        }
        return p;
    };
    auto pos_next = [&](DmaPos &p) __attribute__((always_inline)) {
        if constexpr (TA) {
            p.pa += (size_t)BK * M;
        } else {
            p.pa += BK;
            p.na -= 2u * BK;
        }
        if constexpr (TB) {
            p.pb += BK;
            p.nb -= 2u * BK;
        } else {
            p.pb += (size_t)BK * N;
        }
    };
    auto make_dma = [](const DmaPos &p) __attribute__((always_inline)) {
        SliceDma d;
        d.ra = make_rsrc(p.pa, p.na);
        d.rb = make_rsrc(p.pb, p.nb);
        return d;
    };
    // This wave's LDS load base in stage 0; load i of a slice lands at + region
    // + stage * 32 KiB + i * NT * 16 (the stage term comes with `lds_stage`).
    const uint32_t ld_wave = __builtin_amdgcn_readfirstlane(smem_lds + (uint32_t)(wid_s * 64 * 16));
    auto dma_one = [&](uint32_t lds_stage, const SliceDma &d, auto i_c) __attribute__((always_inline)) {
        constexpr int i = decltype(i_c)::value;
        if constexpr (i < A_LD) {
            constexpr uint32_t off = (uint32_t)(i * NT * 16);
            buffer_load_lds16_at<off>(d.ra, TA ? tv[i] : av[i], lds_stage);
        } else {
            constexpr int j = i - A_LD;
            constexpr uint32_t off = B_REGION + (uint32_t)(j * NT * 16);
            buffer_load_lds16_at<off>(d.rb, TB ? av[j] : bv[j], lds_stage);
        }
    };
    // Bias of tile t into this wave's slot of parity p: lanes 0 .. BN/8-1 load 16
    // bytes each (columns past N read zeros), the other lanes land zeros. Counted
    // in vmcnt with the slice loads around it.
    const uint32_t bias_lds = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(GBA_LDS void *)bias_smem + (uint32_t)(wid_s * 1024));
    auto bias_dma = [&](const Tile &t, int p) {
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(bias + t.n0, (uint32_t)min(N - t.n0, BN) * 2u);
        const int l = lane_now();   // formed here, not held across the loops
        buffer_load_lds16(rb, l < BN / 8 ? (uint32_t)l * 16u : kOobOffset,
                          bias_lds + (uint32_t)(p * NW * 1024));
    };

    // ---- fragments ----
    // (As gemm_v3 with 16x16x32 MFMAs.) A block fm, step kk: lane l reads row
    // wm*WTM + 16 fm + l%16, logical chunk 4 kk + l/16, stored at chunk ^ (row %
    // 8); row % 8 = l % 8, so the address is a per-kk lane base plus 16 fm rows.
    // B^T block fn, step kk, half h: k row 32 kk + 8 (l/16) + 4 h + (l%16)/4 and
    // columns n = wn*WTN + 16 fn + 4 (l%4); its swizzle term depends only on the
    // lane, so the address is a per-fn lane base plus the k-row offset of kk and
    // h. All bases are LDS addresses in the stage being read (stage 0 at the
    // start); the block and k-row terms are compile-time offsets.
    // The bases are formed by set_bases for the stage at byte offset `st` from
    // stage 0: at the start, and again after each epilogue (from the lane id
    // read afresh), so that they are not held across the epilogue.
    constexpr int NFB = TB ? KK : FN;
    uint32_t fa_base[KK];
    uint32_t fb_base[NFB];
    uint32_t ft_base[TA ? FM : 1];
    auto set_bases = [&](uint32_t st) __attribute__((always_inline)) {
        const int l = lane_now();
        const int tg = l >> 4, tj = l & 15;
        const int wm_s = wid_s / WN, wn_s = wid_s % WN;
        const uint32_t s0 = smem_lds + st;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const int r = wm_s * WTM + tj;
            fa_base[kk] = s0 + (uint32_t)(r * (BK * 2) + aswz<MS, CHA>(r, (KS / 8) * kk + tg) * 16);
        }
        // TB: W^T block fn, step kk: lane l reads row wn*WTN + 16 fn + l%16 of
        // W's tile like A's (a per-kk lane base plus 16 fn rows).
#pragma unroll
        for (int f = 0; f < NFB; ++f) {
            if constexpr (TB) {
                const int r = wn_s * WTN + tj;
                fb_base[f] = s0 + B_REGION + (uint32_t)(r * (BK * 2) + aswz<MS, CHA>(r, (KS / 8) * f + tg) * 16);
            } else {
                const int k = 8 * tg + (tj >> 2);
                const int n = wn_s * WTN + f * 16 + 4 * (tj & 3);
                const int c = (n >> 3) ^ bswz<CHB>(k);
                fb_base[f] = s0 + B_REGION + (uint32_t)(k * (BN * 2) + c * 16 + (n & 4) * 2);
            }
        }
        // TA: A block fm, step kk, half h gathered from At's tile like B^T's
        // from B's. Lane l asks for k row 32 kk + 8 (l/16) + 4 h + (l%16)/4 and
        // m = wm*WTM + 16 fm + 4 (l%4); 16 fm rows flip only chunk bits 1..3
        // (byte address bits 5..7) of the fm = 0 address: one base per block fm.
        if constexpr (TA) {
            const int k = 8 * tg + (tj >> 2);
            const int m = wm_s * WTM + 4 * (tj & 3);
            const int c = (m >> 3) ^ bswz<CHB>(k);
            const uint32_t b0 = (uint32_t)(k * (BM * 2) + c * 16 + (m & 4) * 2);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) ft_base[fm] = s0 + (b0 ^ (uint32_t)(fm << 5));
        }
    };
    set_bases(0u);

    f32x4 acc[FN][FM];
    u32x4 fa[2][FM];
    i16x4 fal[2][FM], fah[2][FM];
    i16x4 fbl[2][FN], fbh[2][FN];
    u32x4 fw[2][FN];
    // Fragment r of step kk of the slice in the bases' stage into buffer buf.
    auto read_one = [&](int buf, int kk, int r) __attribute__((always_inline)) {
        if (r < NFA) {
            if constexpr (TA) {
                const int fm = r >> 1, h = r & 1;
                const uint32_t o = (uint32_t)((32 * kk + 4 * h) * (BM * 2));
                const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GBA_LDS i16x4 *)(ft_base[fm] + o));
                if (h)
                    fah[buf][fm] = v;
                else
                    fal[buf][fm] = v;
            } else {
                const uint32_t o = (uint32_t)(r * BD * (BK * 2));
                fa[buf][r] = *(GBA_LDS const u32x4 *)(fa_base[kk] + o);
            }
        } else if constexpr (TB) {
            const int fn = r - NFA;
            const uint32_t o = (uint32_t)(fn * BD * (BK * 2));
            fw[buf][fn] = *(GBA_LDS const u32x4 *)(fb_base[kk] + o);
        } else {
            const int fn = (r - NFA) >> 1, h = (r - NFA) & 1;
            const uint32_t o = (uint32_t)((32 * kk + 4 * h) * (BN * 2));
            const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GBA_LDS i16x4 *)(fb_base[fn] + o));
            if (h)
                fbh[buf][fn] = v;
            else
                fbl[buf][fn] = v;
        }
    };
    // Moves base b (A bases, then B's, then At's) to the other stage.
    constexpr int NBA = TA ? FM : KK, NBB = NFB, NBASE = NBA + NBB;
    static_assert(NPF + NBASE <= NMF, "base moves after the step's reads");
    // (An asm statement: a plain add is sunk by the compiler to the first use,
    // past the barrier, where it delays the next step's first MFMA.)
    auto add_to = [](uint32_t &x, int delta) __attribute__((always_inline)) {
        asm volatile("v_add_u32 %0, %1, %0" : "+v"(x) : "s"(delta));
    };
    auto move_base = [&](int b, int delta) __attribute__((always_inline)) {
        if (b < NBA) {
            if constexpr (TA)
                add_to(ft_base[b], delta);
            else
                add_to(fa_base[b], delta);
        } else {
            add_to(fb_base[b - NBA], delta);
        }
    };
    // One MFMA step on buffer `cur`: with READS, reads the next step's fragments
    // (step pf_kk of the slice in the bases' stage); with MOVE, then moves every base to the
    // other stage (by `delta`); with DMA, issues the LD loads of slice d into the
    // stage at `lds_stage`, one per EVERY MFMAs.
    // payload(q) runs after MFMA q: per-slice scalar work placed in pieces
    // into the MFMA stream's shadow (a wave issues only a few instructions
    // between two MFMAs without delaying the second).
    constexpr int PQ = NPF + NBASE + 2;
    static_assert(PQ + 8 < NMF, "payload slots inside the step");
    auto step = [&](int cur, auto reads_c, int pf_kk, auto move_c, int delta, auto dma_c,
                    uint32_t lds_stage, const SliceDma &d, auto &&payload) __attribute__((always_inline)) {
        constexpr bool READS = decltype(reads_c)::value;
        constexpr bool MOVE = decltype(move_c)::value, DMA = decltype(dma_c)::value;
        static_for<NMF>([&](auto q_c) __attribute__((always_inline)) {
            constexpr int q = decltype(q_c)::value;
            // Column block outer, row blocks in alternating direction, so that
            // consecutive MFMAs share an operand across the column-block change
            // as well (0.3-0.8 % faster than restarting each column at row 0,
            // same results: every accumulator still gets one MFMA per step).
            constexpr int fn = q / FM, fm = (fn & 1) ? FM - 1 - q % FM : q % FM;
            u32x4 bop;
            if constexpr (TB)
                bop = fw[cur][fn];
            else
                bop = __builtin_bit_cast(u32x4, __builtin_shufflevector(fbl[cur][fn], fbh[cur][fn],
                                                                        0, 1, 2, 3, 4, 5, 6, 7));
            u32x4 aop;
            if constexpr (TA)
                aop = __builtin_bit_cast(u32x4, __builtin_shufflevector(fal[cur][fm], fah[cur][fm],
                                                                        0, 1, 2, 3, 4, 5, 6, 7));
            else
                aop = fa[cur][fm];
            acc[fn][fm] = mfma16x16x32<DT>(bop, aop, acc[fn][fm]);
            if constexpr (READS && q < NPF) read_one(cur ^ 1, pf_kk, q);
            if constexpr (MOVE && q >= NPF && q < NPF + NBASE) move_base(q - NPF, delta);
            if constexpr (DMA && q % EVERY == 0)
                dma_one(lds_stage, d, std::integral_constant<int, q / EVERY>{});
            payload(q_c);
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    auto no_payload = [](auto) __attribute__((always_inline)) {};

    Tile cur_t;
    if (!tile_of(0, cur_t)) return;   // more workgroups than tiles: nothing to do

    // av is always masked for the slice the last load went to (tail_k or not),
    // so a slice re-masks it only when the slice it loads differs in that.
    // Offsets for a tile whose slice k was loaded last.
    auto set_offsets = [&](const Tile &t, int k) __attribute__((always_inline)) {
        set_av(k == tail_k);
        if constexpr (!TB) set_bv(t.n0);
        if constexpr (TA) set_tv(t.m0);
    };

    // Prologue: slices 0 and 1 of the first tile; slice 0 waited for and
    // published, and its first fragments read. pos: the position loaded last.
    DmaPos pos;
    {
        set_offsets(cur_t, 0);
        if (bias) bias_dma(cur_t, 0);   // lands with slice 0 (waited for below)
        const SliceDma d0 = make_dma(pos_full(cur_t, true, 0));
        static_for<LD>([&](auto i_c) { dma_one(ld_wave, d0, i_c); });
        if (tail_k == 1) set_av(true);
        pos = pos_full(cur_t, true, 1);
        const SliceDma d1 = make_dma(pos);
        static_for<LD>([&](auto i_c) { dma_one(ld_wave + (uint32_t)A_BYTES, d1, i_c); });
    }
    wait_vmcnt<LD>();
    block_barrier();
#pragma unroll
    for (int q = 0; q < NPF; ++q) read_one(0, 0, q);

    // Stream state: the stage of the slice being computed (its LDS load base),
    // and the add that moves a fragment base from that stage to the other.
    uint32_t lds_cur = ld_wave;
    int delta = A_BYTES;
    for (int r = 0;; ++r) {
#pragma unroll
        for (int a = 0; a < FN; ++a)
#pragma unroll
            for (int b = 0; b < FM; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
        Tile nxt_t;
        const bool nxt_live = tile_of(r + 1, nxt_t);
        if (!nxt_live) nxt_t = cur_t;
        // Offsets for this tile's loads from slice 2 on, as after loading slice 1
        // (recomputed here so that they are dead across the previous epilogue).
        if (r > 0) set_offsets(cur_t, 1);

        // Slice kt: step 0 reads its kk=1 fragments, moves the bases to the other
        // stage and, in its shadow, prepares the loads of stream position kt+2
        // (offsets at a tile edge or K tail, descriptors); the barrier publishes
        // position kt+1 (the next tile's slice 0 after the last slice) and frees
        // this slice's stage; step 1 loads position kt+2 into it and reads position
        // kt+1's kk=0 fragments, except in a tile's last slice: the next tile's
        // first fragments are read after the epilogue, which then has their
        // registers. Nothing but the wait and the barrier sits between the steps.
        auto slice = [&](int kt, auto reads_c) __attribute__((always_inline)) {
            const bool here = kt + 2 < nk;
            const int k2 = here ? kt + 2 : kt + 2 - nk;
            const int k1 = kt + 1 < nk ? kt + 1 : kt + 1 - nk;   // the slice loaded last
            SliceDma dn;
            bool bias_next = false;
            auto prep = [&](auto q_c) __attribute__((always_inline)) {
                constexpr int q = decltype(q_c)::value;
                if constexpr (q == PQ) {
                    // One step on along K: all a tile's slices but its last
                    // three load the next slice of the same tile, full.
                    pos_next(pos);
                    asm volatile("" : "+s"(pos.pa), "+s"(pos.pb), "+s"(pos.na), "+s"(pos.nb));
                } else if constexpr (q == PQ + 4) {
                    // Near a tile's end (position kt+2 is the tile's partial last
                    // slice, the next tile's first, or past the last tile): the
                    // tile edges, the K-tail mask and the position from scratch,
                    // in one rarely taken block.
                    if (__builtin_expect(kt + 3 >= nk, 0)) {
                        if ((!here) & (k2 == 0) & nxt_live) {
                            if constexpr (!TB) set_bv(nxt_t.n0);
                            if constexpr (TA) set_tv(nxt_t.m0);
                        }
                        if ((k2 == tail_k) != (k1 == tail_k)) set_av(k2 == tail_k);
                        if ((k2 == 0) | (k2 == tail_k) | !(here | nxt_live))
                            pos = pos_full(here ? cur_t : nxt_t, here | nxt_live, k2);
                        bias_next = (bias != nullptr) & (!here) & (k2 == 0) & nxt_live;
                    }
                    asm volatile("" : "+s"(pos.pa), "+s"(pos.pb), "+s"(pos.na), "+s"(pos.nb));
                } else if constexpr (q == PQ + 8) {
                    dn = make_dma(pos);
                    // Formed here, in the MFMA shadow, not at their first use
                    // after the barrier.
                    asm volatile("" : "+s"(dn.ra), "+s"(dn.rb));
                }
            };
            step(0, std::true_type{}, 1, std::true_type{}, delta, std::false_type{}, 0u, SliceDma{}, prep);
            wait_vmcnt_lgkm0<0>();
            block_barrier();
            // With the next tile's slice 0: its bias, into the other parity's slot
            // (this tile's epilogue still reads its own). Landed by the next
            // slice's vmcnt(0) wait, long before that tile's epilogue.
            if (__builtin_expect(bias_next, 0)) bias_dma(nxt_t, (r + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
            step(1, reads_c, 0, std::false_type{}, 0, std::true_type{}, lds_cur, dn, no_payload);
            lds_cur += (uint32_t)delta;   // the next slice's stage
            delta = -delta;
        };
        // The last slice also reads the next position's first fragments (they
        // are read again after the epilogue, which needs their registers): so it
        // runs the loop's own code, not a copy that starts cold in the
        // instruction cache (about 1000 cycles a tile). With W [N,K] and A
        // [M,K] that leaves the register allocator shuffling accumulators in
        // the loop; there the last slice keeps its own copy.
        if constexpr (TB && !TA) {
            for (int kt = 0; kt + 1 < nk; ++kt) slice(kt, std::true_type{});
            slice(nk - 1, std::false_type{});
        } else {
            for (int kt = 0; kt < nk; ++kt) slice(kt, std::true_type{});
        }

        // Epilogue of this tile while the next tile's first slices land. The
        // scheduling fences keep the next tile's fragment reads and the epilogue
        // apart (mixing them would hold both register sets live at once).
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        {
            // Lane id from a volatile mbcnt (not merged with the copies from before
            // the K loop) and the scalar wave id: no vector register is held across
            // the loop for the epilogue's rows and columns.
            int ln;
            asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
            const int wn_s = wid_s % WN, wm_s = wid_s / WN;
            char *const bias_mine = bias_smem + ((r & 1) * NW + wid_s) * 1024;
            // This wave's 128 bias values as fp32, once per tile, into the upper
            // half of its own slot (the lower half holds the tile's raw values).
            if (bias) {
                const uint32_t bb =
                    *reinterpret_cast<const uint32_t *>(bias_mine + wn_s * (WTN * 2) + 4 * ln);
                *reinterpret_cast<f32x2 *>(bias_mine + 512 + 8 * ln) =
                    f32x2{to_f32<DT>(bb & 0xffffu), to_f32<DT>(bb >> 16)};
            }
            // The wave's 128 x 128 block of C leaves through 16 x 64 staging
            // areas of its own: each group of four MFMA blocks (row block fm,
            // column half fh) is written there in the MFMA layout (lane: one row,
            // four adjacent columns) and read back by rows, so that one 16-byte
            // store instruction writes 8 whole 128-byte row segments instead of
            // 16 pieces of 32 bytes. Chunk c of staging row w sits at c ^ (w % 8).
            // The stores are non-temporal: C is not read again by this kernel
            // (1-4 % faster than cached stores on every shape measured).
            char *const stg = stage_smem + wid_s * 2 * STG_BYTES;
            const int wr = ln & 15, wg = ln >> 4;   // write side: row, 4-column group
            const int rr = ln >> 3, rc = ln & 7;    // read side: row (of 8), 16-byte chunk
            char *const Cw = reinterpret_cast<char *>(C + (size_t)cur_t.m0 * N + cur_t.n0) +
                             ((size_t)wm_s * WTM * N + (size_t)wn_s * WTN) * 2;
            // Byte offset of this lane's store in row block 0, column half 0 (32
            // bits: 127 rows of at most 2^24 bytes); opaque to the optimiser, so
            // the per-store offsets are not hoisted and held across the K loop.
            uint32_t st_off = (uint32_t)rr * (uint32_t)N * 2u + (uint32_t)rc * 16u;
            uint32_t pitch8 = __builtin_amdgcn_readfirstlane((uint32_t)N * 16u);   // bytes between read rows rr and rr + 8
            asm volatile("" : "+v"(st_off), "+s"(pitch8));
            // Rows and columns left in this wave's block (edge tiles; no m0 + BM:
            // it overflows near 2^31).
            const int rows_left = M - cur_t.m0 - wm_s * WTM, cols_left = N - cur_t.n0 - wn_s * WTN;
            const bool full = rows_left >= WTM && cols_left >= WTN;
            // Group g = (column half g / FM, row block g % FM) alternates between
            // two staging buffers: while group g is computed and written, group
            // g - 1 (written one group earlier) is read back and stored, so the LDS
            // round trip stays off the critical path. The bias of a column half is
            // read once, into registers, before its first group.
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
                            const int fn = 4 * fh + f;
                            const f32x4 &a = acc[fn][fm];
                            u32x2 o;
                            o.x = pack2<DT>(act_fn<ACT>(a[0] + bq[f][0]), act_fn<ACT>(a[1] + bq[f][1]));
                            o.y = pack2<DT>(act_fn<ACT>(a[2] + bq[f][2]), act_fn<ACT>(a[3] + bq[f][3]));
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
                    // One group at a time: the next tile's first fragments are
                    // live here, so the scheduler may not interleave the whole
                    // tile's epilogue.
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
        if (!nxt_live) break;
        cur_t = nxt_t;
        // The next tile's slice 0 was published by the last barrier, in the
        // stage lds_cur names; its first fragments.
        set_bases(lds_cur - ld_wave);
#pragma unroll
        for (int q = 0; q < NPF; ++q) read_one(0, 0, q);
    }
    // No direct-to-LDS write may outlive the workgroup's LDS.
    wait_vmcnt<0>();
}

// Grid: one workgroup per CU (two 64 KiB stages fill the LDS), or fewer when
// there are fewer tiles. K must exceed 64 (at least two K slices per tile): the
// library sends K <= 64 to kernel 3.
template <int BM, int BN, int WM, int WN, int DT, int ACT, bool TB = false, bool TA = false>
hipError_t launch_gemm_v5(const void *A, const void *B, const void *bias, void *C, int M, int N,
                          int K, int raster, int group_m, hipStream_t stream) {
    const int tiles_m = ceil_div(M, BM), tiles_n = ceil_div(N, BN);
    const long long tiles = (long long)tiles_m * tiles_n;
    if (tiles <= 0) return hipSuccess;
    // Tile indices r * G + slot run up to tiles + G - 1: keep them in int.
    if (tiles > 0x7fffffffLL - 0x10000) return hipErrorInvalidValue;
    if (K <= 64) return hipErrorInvalidValue;   // needs two K slices; see the note above
    int cus = 0;
    const hipError_t e = current_cus(&cus);
    if (e != hipSuccess) return e;
    const int grid = (int)(tiles < cus ? tiles : cus);
    hipLaunchKernelGGL((gemm_v5_kernel<BM, BN, WM, WN, DT, ACT, TB, TA>), dim3((unsigned)grid),
                       dim3(WM * WN * 64), 0, stream, (const uint16_t *)A, (const uint16_t *)B,
                       (const uint16_t *)bias, (uint16_t *)C, M, N, K, tiles_m, tiles_n, raster,
                       group_m < 1 ? 1 : group_m);
    return hipGetLastError();
}

}  // namespace gba
