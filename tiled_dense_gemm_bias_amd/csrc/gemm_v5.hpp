// Persistent variant of the interleaved 16x16x32 GEMM kernel (gemm_v3.hpp).
//
// One workgroup per CU walks its tiles (t = w, w + G, w + 2G, ... in raster
// order, G = grid size) as one stream of 64-deep K slices through the same
// two-stage LDS ring. The loads of stream position p + 2 are issued in the
// last MFMA step of position p, exactly as in gemm_v3, except that positions
// past a tile's last slice are the next tile's first slices. So when a tile's
// main loop ends, the next tile's slice 0 is already in LDS (published by the
// last barrier) and its slice 1 is in flight; both land while the epilogue
// (bias, activation, rounding, stores) runs, and the next main loop starts
// without the pipeline fill of a fresh workgroup. Tiles, LDS layouts,
// fragments, MFMA order and epilogue are gemm_v3's (results are bit-identical).
// TB (transpose_B, B given as an (N,K) array W) is gemm_v3's TB layout, and TA
// (transpose_A, A given as a (K,M) array At) gemm_v3's TA layout.
#pragma once

#include "gemm_v3.hpp"

namespace gba {

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
    constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    constexpr int A_LD = BM * CHA / NT, B_LD = (TB ? BN * CHA : BK * CHB) / NT, LD = A_LD + B_LD;
    constexpr int EVERY = NMF / LD;
    static_assert(KK == 2, "two MFMA steps per slice");
    static_assert(WTM % BD == 0 && WTN % BD == 0, "wave tile must be whole MFMA blocks");
    static_assert(BN >= 128, "B swizzle needs at least 16 chunks per row");
    static_assert(!TA || BM == BN, "At's tile is loaded with B's per-thread mapping");
    static_assert((BM * CHA) % NT == 0 && B_LD * NT == (TB ? BN * CHA : BK * CHB),
                  "slices split evenly");
    static_assert(2 * STAGE_BYTES <= 160 * 1024, "LDS ring too large");
    static_assert(2 * LD < 64 && NMF % LD == 0 && NPF <= NMF, "step layout");
    // Needs at least two K slices (K > 64): the launcher uses gemm_v3 below that.

    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE_BYTES];
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
    static_assert(2 * STAGE_BYTES + 2 * NW * 1024 + NW * 2 * STG_BYTES <= 160 * 1024,
                  "LDS ring + bias slots + staging too large");

    const int tid = threadIdx.x;
    const int lane = tid & 63, wid = tid >> 6;
    const int wm = wid / WN, wn = wid % WN;
    const int nk = (K + BK - 1) / BK;
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

    // Loader offsets within a slice (independent of the tile). Load i of a
    // thread fills LDS chunk s = i*NT + tid of the A (B) part. For A that is row
    // 32i + tid/8, logical chunk c_a = (tid%8) ^ (row%8), the same for every i;
    // for B, k row 8i + tid/32 and logical chunk c_b(i) = c_b(0) ^ 8(i%4)
    // (the B swizzle's row/8 term). So a handful of registers describe them all.
    static_assert(NT == 256 && CHA == 8 && CHB == 32, "loader mapping written for 256 threads, BK 64, BN 256");
    // TB: W's tile is loaded like A's (BN = 256 rows of 64 k), with the same
    // per-thread base.
    const int c_a = (tid & 7) ^ ((tid >> 3) & 7);
    const uint32_t a_base = (uint32_t)(tid >> 3) * (uint32_t)K * 2u + (uint32_t)c_a * 16u;
    const int c_b0 = (tid & 31) ^ bswz<CHB>(tid >> 5);
    const uint32_t b_row = (uint32_t)(tid >> 5) * (uint32_t)N * 2u;
    // TA: At's tile (64 k rows of BM = BN values) is loaded like B's.
    const uint32_t t_row = (uint32_t)(tid >> 5) * (uint32_t)M * 2u;
    // Loads of slice kt of tile t (live) into stage `stage`; a dead slice reads
    // nothing (every lane out of range) but keeps the wait counts uniform.
    struct SliceDma {
        __amdgpu_buffer_rsrc_t ra, rb;
        uint32_t la, lb;
        int k0, n0, m0;
    };
    auto slice_dma = [&](const Tile &t, bool live, int kt, int stage) {
        SliceDma d;
        d.la = __builtin_amdgcn_readfirstlane(smem_lds + (uint32_t)(stage * STAGE_BYTES + wid_s * 64 * 16));
        d.lb = d.la + A_BYTES;
        d.k0 = live ? kt * BK : K;
        d.n0 = live ? t.n0 : N;
        d.m0 = live ? t.m0 : M;
        if constexpr (TA)
            d.ra = make_rsrc(A + (live ? (size_t)d.k0 * M + t.m0 : 0),
                             live ? (uint32_t)min(K - d.k0, BK) * (uint32_t)M * 2u : 0u);
        else
            d.ra = make_rsrc(A + (live ? (size_t)t.m0 * K + d.k0 : 0),
                             live ? (uint32_t)t.rows * (uint32_t)K * 2u - (uint32_t)d.k0 * 2u : 0u);
        if constexpr (TB)
            d.rb = make_rsrc(B + (live ? (size_t)t.n0 * K + d.k0 : 0),
                             live ? (uint32_t)min(N - t.n0, BN) * (uint32_t)K * 2u - (uint32_t)d.k0 * 2u
                                  : 0u);
        else
            d.rb = make_rsrc(B + (live ? (size_t)d.k0 * N + t.n0 : 0),
                             live ? (uint32_t)min(K - d.k0, BK) * (uint32_t)N * 2u : 0u);
        return d;
    };
    // Bias of tile t into this wave's slot of parity p: lanes 0 .. BN/8-1 load 16
    // bytes each (columns past N read zeros), the other lanes land zeros. Counted
    // in vmcnt with the slice loads around it.
    const uint32_t bias_lds = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(GBA_LDS void *)bias_smem + (uint32_t)(wid_s * 1024));
    auto bias_dma = [&](const Tile &t, int p) {
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(bias + t.n0, (uint32_t)min(N - t.n0, BN) * 2u);
        buffer_load_lds16(rb, lane < BN / 8 ? (uint32_t)lane * 16u : kOobOffset,
                          bias_lds + (uint32_t)(p * NW * 1024));
    };
    // `kx`, `nx`: K and N re-read opaquely in each slice, so that the per-load
    // row offsets (multiples of 64 K and 16 N bytes) are recomputed where used
    // rather than held in scalar registers for the whole loop.
    auto dma_one = [&](const SliceDma &d, int i, uint32_t kx, uint32_t nx, uint32_t mx) {
        if (i < A_LD) {
            if constexpr (TA) {
                const int c = c_b0 ^ (8 * (i & 3));
                const uint32_t o = d.m0 + c * 8 < M
                                       ? t_row + (uint32_t)(i * 16) * mx + (uint32_t)c * 16u
                                       : kOobOffset;
                buffer_load_lds16(d.ra, o, d.la + i * NT * 16);
            } else {
                const uint32_t o = d.k0 + c_a * 8 < K ? a_base + (uint32_t)(i * 64) * kx : kOobOffset;
                buffer_load_lds16(d.ra, o, d.la + i * NT * 16);
            }
        } else if constexpr (TB) {
            const int j = i - A_LD;
            const uint32_t o = d.k0 + c_a * 8 < K ? a_base + (uint32_t)(j * 64) * kx : kOobOffset;
            buffer_load_lds16(d.rb, o, d.lb + j * NT * 16);
        } else {
            const int j = i - A_LD;
            const int c = c_b0 ^ (8 * (j & 3));
            const uint32_t o = d.n0 + c * 8 < N
                                   ? b_row + (uint32_t)(j * 16) * nx + (uint32_t)c * 16u
                                   : kOobOffset;
            buffer_load_lds16(d.rb, o, d.lb + j * NT * 16);
        }
    };

    // Fragments (as gemm_v3 with 16x16x32 MFMAs). A block fm, step kk: lane l
    // reads row wm*WTM + 16 fm + l%16, logical chunk 4 kk + l/16, stored at
    // chunk ^ (row % 8); row % 8 = l % 8, so the address is a per-kk lane base
    // plus 16 fm rows (the ds_read offset field). B^T block fn, step kk, half
    // h: k row 32 kk + 8 (l/16) + 4 h + (l%16)/4 and columns n = wn*WTN + 16 fn
    // + 4 (l%4); its swizzle term depends only on the lane, and 16 fn columns
    // only flip chunk bits 1..3, so the address is a per-fn lane base plus the
    // k-row offset of kk and h.
    const int tg = lane >> 4, tj = lane & 15;
    uint32_t fa_base[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        const int r = wm * WTM + tj;
        fa_base[kk] = (uint32_t)(r * (BK * 2) + aswz<MS, CHA>(r, (KS / 8) * kk + tg) * 16);
    }
    // TB: W^T block fn, step kk: lane l reads row wn*WTN + 16 fn + l%16 of W's
    // tile like A's (a per-kk lane base plus 16 fn rows).
    constexpr int NFB = TB ? KK : FN;
    uint32_t fb_base[NFB];
#pragma unroll
    for (int f = 0; f < NFB; ++f) {
        if constexpr (TB) {
            const int r = wn * WTN + tj;
            fb_base[f] = (uint32_t)(A_BYTES + r * (BK * 2) + aswz<MS, CHA>(r, (KS / 8) * f + tg) * 16);
        } else {
            const int k = 8 * tg + (tj >> 2);
            const int n = wn * WTN + f * 16 + 4 * (tj & 3);
            const int c = (n >> 3) ^ bswz<CHB>(k);
            fb_base[f] = (uint32_t)(A_BYTES + k * (BN * 2) + c * 16 + (n & 4) * 2);
        }
    }
    auto a_addr = [&](int fm, int kk) -> uint32_t { return fa_base[kk] + fm * BD * (BK * 2); };
    // TA: A block fm, step kk, half h gathered from At's tile like B^T's from
    // B's. Lane l asks for k row 32 kk + 8 (l/16) + 4 h + (l%16)/4 and m =
    // wm*WTM + 16 fm + 4 (l%4); 16 fm rows flip only chunk bits 1..3 (byte
    // address bits 5..7) of the fm = 0 address, so one base serves every block.
    uint32_t ft_base;
    {
        const int k = 8 * tg + (tj >> 2);
        const int m = wm * WTM + 4 * (tj & 3);
        const int c = (m >> 3) ^ bswz<CHB>(k);
        ft_base = (uint32_t)(k * (BM * 2) + c * 16 + (m & 4) * 2);
    }
    auto t_addr = [&](int fm, int kk, int h) -> uint32_t {
        return (ft_base ^ (uint32_t)(fm << 5)) + (32 * kk + 4 * h) * (BM * 2);
    };
    auto b_addr = [&](int fn, int kk, int h) -> uint32_t {
        if constexpr (TB)
            return fb_base[kk] + fn * BD * (BK * 2);
        else
            return fb_base[fn] + (32 * kk + 4 * h) * (BN * 2);
    };

    f32x4 acc[FN][FM];
    u32x4 fa[2][FM];
    i16x4 fal[2][FM], fah[2][FM];
    i16x4 fbl[2][FN], fbh[2][FN];
    u32x4 fw[2][FN];
    auto read_one = [&](int buf, const char *base, int kk, int r) {
        if (r < NFA) {
            if constexpr (TA) {
                const int fm = r >> 1, h = r & 1;
                const i16x4 v =
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16((GBA_LDS i16x4 *)(base + t_addr(fm, kk, h)));
                if (h)
                    fah[buf][fm] = v;
                else
                    fal[buf][fm] = v;
            } else {
                fa[buf][r] = *reinterpret_cast<const u32x4 *>(base + a_addr(r, kk));
            }
        } else if constexpr (TB) {
            fw[buf][r - NFA] = *reinterpret_cast<const u32x4 *>(base + b_addr(r - NFA, kk, 0));
        } else {
            const int fn = (r - NFA) >> 1, h = (r - NFA) & 1;
            const i16x4 v =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((GBA_LDS i16x4 *)(base + b_addr(fn, kk, h)));
            if (h)
                fbh[buf][fn] = v;
            else
                fbl[buf][fn] = v;
        }
    };
    // One MFMA step on buffer `cur`; `reads`: the next step's fragments (from
    // `pf_base` step pf_kk); `dma`: all LD loads of slice d, one per EVERY MFMAs.
    auto step = [&](int cur, bool reads, const char *pf_base, int pf_kk, bool dma,
                    const SliceDma &d, uint32_t kx, uint32_t nx, uint32_t mx) {
#pragma unroll
        for (int q = 0; q < NMF; ++q) {
            const int fn = q / FM, fm = q % FM;
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
            if (reads && q < NPF) read_one(cur ^ 1, pf_base, pf_kk, q);
            if (dma && q % EVERY == 0) dma_one(d, q / EVERY, kx, nx, mx);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    Tile cur_t;
    if (!tile_of(0, cur_t)) return;   // more workgroups than tiles: nothing to do

    // Prologue: slices 0 and 1 of the first tile; slice 0 waited for and
    // published, and its first fragments read.
    {
        const SliceDma d0 = slice_dma(cur_t, true, 0, 0), d1 = slice_dma(cur_t, true, 1, 1);
        if (bias) bias_dma(cur_t, 0);   // lands with slice 0 (waited for below)
#pragma unroll
        for (int i = 0; i < LD; ++i) dma_one(d0, i, (uint32_t)K, (uint32_t)N, (uint32_t)M);
#pragma unroll
        for (int i = 0; i < LD; ++i) dma_one(d1, i, (uint32_t)K, (uint32_t)N, (uint32_t)M);
    }
    wait_vmcnt<LD>();
    block_barrier();
#pragma unroll
    for (int q = 0; q < NPF; ++q) read_one(0, smem, 0, q);

    int stage0 = 0;   // stage of the current tile's slice 0
    for (int r = 0;; ++r) {
#pragma unroll
        for (int a = 0; a < FN; ++a)
#pragma unroll
            for (int b = 0; b < FM; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
        Tile nxt_t;
        const bool nxt_live = tile_of(r + 1, nxt_t);
        if (!nxt_live) nxt_t = cur_t;

        // Slice kt: step 0 reads its kk=1 fragments; the barrier publishes stream
        // position kt+1 (the next tile's slice 0 after the last slice) and frees
        // kt's stage; step 1 loads position kt+2 into it and reads position
        // kt+1's kk=0 fragments.
        for (int kt = 0; kt < nk; ++kt) {
            const int sc = (stage0 + kt) & 1;
            const char *cur_base = smem + sc * STAGE_BYTES;
            const char *nxt_base = smem + (sc ^ 1) * STAGE_BYTES;
            uint32_t kx = (uint32_t)K, nx = (uint32_t)N, mx = (uint32_t)M;
            asm volatile("" : "+s"(kx), "+s"(nx), "+s"(mx));
            step(0, true, cur_base, 1, false, SliceDma{}, kx, nx, mx);
            wait_vmcnt_lgkm0<0>();
            block_barrier();
            const bool here = kt + 2 < nk;
            const SliceDma dn = slice_dma(here ? cur_t : nxt_t, here || nxt_live,
                                          here ? kt + 2 : kt + 2 - nk, sc);
            // With the next tile's slice 0: its bias, into the other parity's slot
            // (this tile's epilogue still reads its own). Landed by the next
            // slice's vmcnt(0) wait, long before that tile's epilogue.
            if (bias && !here && kt + 2 == nk && nxt_live) bias_dma(nxt_t, (r + 1) & 1);
            step(1, true, nxt_base, 0, true, dn, kx, nx, mx);
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
            char *const stg = stage_smem + wid_s * 2 * STG_BYTES;
            const int wr = ln & 15, wg = ln >> 4;   // write side: row, 4-column group
            const int rr = ln >> 3, rc = ln & 7;    // read side: row (of 8), 16-byte chunk
            char *const Cw = reinterpret_cast<char *>(C + (size_t)cur_t.m0 * N + cur_t.n0) +
                             ((size_t)wm_s * WTM * N + (size_t)wn_s * WTN) * 2;
            // Byte offset of this lane's store in row block 0, column half 0 (32
            // bits: 127 rows of at most 2^24 bytes); opaque to the optimiser, so
            // the per-store offsets are not hoisted and held across the K loop.
            uint32_t st_off = (uint32_t)rr * (uint32_t)N * 2u + (uint32_t)rc * 16u;
            uint32_t pitch8 = (uint32_t)N * 16u;   // bytes between read rows rr and rr + 8
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
                            *reinterpret_cast<u32x4 *>(Cw + offs) = v[j];
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
        stage0 = (stage0 + nk) & 1;
        if (!nxt_live) break;
        cur_t = nxt_t;
    }
    // No direct-to-LDS write may outlive the workgroup's LDS.
    wait_vmcnt<0>();
}

// Grid: one workgroup per CU (two 64 KiB stages fill the LDS), or fewer when
// there are fewer tiles. K must exceed 64 (at least two K slices per tile): the
// library sends K <= 64 to gemm_v3 with the same tile.
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
