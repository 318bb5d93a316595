// Interleaved direct-to-LDS GEMM kernel for gfx950.
//
// Each workgroup owns one BM x BN tile of C and walks K in BK-deep slices
// through a STAGES-deep LDS ring filled by direct-to-LDS loads (gba_dma.hpp).
// A stays K-contiguous in LDS ([BM][BK], 16-byte chunks XOR-swizzled by row) and
// is read with ds_read_b128; B stays N-contiguous ([BK][BN], chunks swizzled by
// k row) and the MFMA's K-contiguous B^T operand is gathered with
// ds_read_b64_tr_b16. The epilogue stores whole row segments through LDS (see
// there). What matters most is the order in which a wave issues its
// instructions. Moving a slice from HBM/L2 into
// LDS takes the CU's address path about as long as half of the slice's MFMA
// work, and a wave that issues all its direct-to-LDS loads back to back stalls
// in issue for that whole time. Here every MFMA step is written out
// as a fixed sequence: one MFMA, then the next step's fragment reads and this
// slice's share of global->LDS loads, then the next MFMA, ... so the matrix core
// keeps running while the loads drain.
//
//  * The loads of slice t+STAGES are issued in the MFMA step right after the
//    barrier that frees their stage (SPREAD = 1), before the next barrier, so
//    every wait is "all but the (STAGES-2) newest slices". Their descriptors
//    and K-masked offsets are formed in the step before the barrier, a few
//    instructions per MFMA gap: a burst of scalar or address work between two
//    MFMAs, or a taken branch, delays the second.
//  * Only the first LDW waves issue global->LDS loads; with LDW < waves, the
//    other waves on the same SIMDs keep issuing MFMAs while the loaders wait
//    on the address path.
//  * Slices past the end of K are still "loaded" with every lane out of range
//    (zeros, no memory access), which keeps the wait counts uniform.
//
// TB (transpose_B): B is given as an (N,K) row-major array W and the product is
// A.W^T. W's tile then has A's shape and layout (BN rows of BK K-contiguous
// values, the same chunk XOR), is loaded like A, and its MFMA operand is read
// like A's with ds_read_b128 -- no transposing reads. 16x16x32 MFMAs only.
//
// TA (transpose_A): A is given as a (K,M) row-major array At and the product is
// At^T.B. At's tile then has B's shape and layout (BK k rows of BM M-contiguous
// values, B's chunk XOR), is loaded like B (M edge masked per 16-byte chunk, K
// edge by the descriptor range), and its MFMA operand is gathered like B's by
// two transposing reads of four k rows each. 16x16x32 MFMAs only.
//
// PARTIAL (split-K, first pass): the grid holds `splits` work units per tile;
// unit s covers K slices [s nk / splits, (s+1) nk / splits) and writes its raw
// fp32 sums to part[s][M][N] instead of running the epilogue. The second pass
// (splitk_reduce_kernel) adds the partials in s order, then bias, act, rounding.
#pragma once

#include "gba_dma.hpp"

#include <type_traits>

namespace gba {

template <int MS> struct Acc;
template <> struct Acc<16> { typedef f32x4 type; static constexpr int n = 4; };

// v_mfma_f32_16x16x32_{f16,bf16}: lane l holds row/column l % 16 and K chunk
// l / 16 of the operands; the 16x16 result gives lane l column l % 16, rows
// 4 (l / 16) .. +3 -- with B^T as the first operand, four adjacent n of row m.
template <int DT>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (DT == DT_F16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
}

// Physical 16-byte chunk of logical chunk c in row r of an A stage. With the
// 16x16x32 operand pattern (lane l reads row l % 16 of a block, chunk l / 16)
// a plain XOR with r mod 8 keeps ds_read_b128 free of bank conflicts on gfx950
// (measured with SQ_LDS_BANK_CONFLICT); the 32x32x16 pattern keeps swz<>.
template <int MS, int CHA>
__device__ __forceinline__ int aswz(int r, int c) {
    if constexpr (MS == 16)
        return c ^ (r & (CHA - 1));
    else
        return swz<CHA>(r, c);
}

// XOR (in 16-byte chunks) of k row r of a B stage. The transposing reads of one
// instruction touch k rows r0 + {0..3} + 8 {0..3} at one 32-byte column pair;
// the even XOR moves each of those rows to its own pair slot. A 128-byte row
// (8 chunks, 64 columns) has only 4 pair slots: rows r and r + 2 share a bank
// half and take different slots by bit 1 of r, rows r and r + 8 by bit 3, so
// each half-wave's 8 rows (r0 + {0..3} + 8 {0, 1}) fall on distinct banks.
template <int CHB>
__device__ __forceinline__ int bswz(int r) {
    if constexpr (CHB == 8)
        return 4 * ((r >> 1) & 1) + 2 * ((r >> 3) & 1);
    else
        return (2 * (r & 3) + 8 * ((r >> 3) & 3)) & (CHB - 1);
}

template <int BM, int BN, int BK, int WM, int WN, int STAGES, int LDW, int SPREAD, int MS, int DT,
          int ACT, bool TB = false, bool PARTIAL = false, bool TA = false>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_v3_kernel(const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
               const uint16_t *__restrict__ bias, uint16_t *__restrict__ C, int M, int N, int K,
               int tiles_m, int tiles_n, int raster, int group_m, int splits,
               float *__restrict__ part) {
    constexpr int NW = WM * WN;
    constexpr int NTL = LDW * 64;         // loader threads
    constexpr int CHA = BK / 8;
    constexpr int CHB = BN / 8;
    constexpr int CHT = BM / 8;           // chunks per k row of At's tile (TA)
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int BD = MS;                // MFMA output block: BD x BD
    constexpr int KS = 32;                // K depth of one MFMA
    constexpr int FM = WTM / BD, FN = WTN / BD;
    constexpr int NMF = FM * FN;          // MFMAs per step
    constexpr int NFA = (TA ? 2 : 1) * FM;        // A fragment reads per step
    constexpr int NPF = NFA + (TB ? 1 : 2) * FN;  // fragment reads per step
    constexpr int KK = BK / KS;           // steps per slice
    constexpr int A_BYTES = BM * BK * 2, B_BYTES = BK * BN * 2;
    constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    constexpr int A_LD = BM * CHA / NTL;
    constexpr int B_LD = TB ? BN * CHA / NTL : BK * CHB / NTL;
    constexpr int LD = A_LD + B_LD;       // loads per loader thread per slice
    constexpr int LD_STEP = (LD + SPREAD - 1) / SPREAD;
    static_assert(MS == 16, "16x16x32 MFMAs");
    static_assert(BK == 32 || BK == 64, "BK must be 32 or 64");
    static_assert(KK % 2 == 0, "fragment buffers alternate within a slice");
    static_assert(WTM % BD == 0 && WTN % BD == 0, "wave tile must be whole MFMA blocks");
    static_assert(TB || BN >= 64, "B swizzle needs at least 8 chunks per row");
    static_assert(!TB || MS == 16, "transpose_B is written for 16x16x32 MFMAs");
    static_assert(!TA || (MS == 16 && BM >= 128), "transpose_A: 16x16x32 MFMAs, at least 16 chunks per k row");
    static_assert(!TA || (BK * CHT) % NTL == 0, "At slices split evenly");
    static_assert(LDW >= 1 && LDW <= NW && NW % LDW == 0, "loader waves");
    static_assert((BM * CHA) % NTL == 0 && (B_LD * NTL == (TB ? BN * CHA : BK * CHB)),
                  "slices split evenly");
    static_assert(STAGES >= 2 && STAGES * STAGE_BYTES <= 160 * 1024, "LDS ring too large");
    static_assert(STAGES * LD < 64, "vmcnt range");
    static_assert(SPREAD == 1, "a slice's loads are issued in the step after the barrier");
    static_assert(LD_STEP <= NMF, "at most one load per MFMA");

    __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE_BYTES];
    // Epilogue staging (16x16x32 MFMAs): two buffers of 16 rows x 64 columns of C
    // per wave, as in the persistent kernel.
    constexpr bool STAGED = MS == 16 && !PARTIAL;
    constexpr int STG_BYTES = 16 * 64 * 2;
    __shared__ __attribute__((aligned(1024))) char stage_smem[STAGED ? NW * 2 * STG_BYTES : 16];
    static_assert(!STAGED || (WTN % 64 == 0 && STAGES * STAGE_BYTES + NW * 2 * STG_BYTES <= 160 * 1024),
                  "staged epilogue: 64-column halves, LDS ring + staging within 160 KiB");

    static_assert(!PARTIAL || MS == 16, "split-K is written for 16x16x32 MFMAs");
    int tm, tn, split = 0;
    {
        int t = linear_block();
        if (raster) t = xcd_remap(t, linear_grid());
        if (t >= tiles_m * tiles_n * splits) return;   // padding of a 2-D grid
        if constexpr (PARTIAL) {
            // units of one split are contiguous, so each XCD walks whole tiles' panels
            split = t / (tiles_m * tiles_n);
            t -= split * (tiles_m * tiles_n);
        }
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
    // This unit's K slices: [kt0, kt0 + nk).
    const int nk_all = (K + BK - 1) / BK;
    const int kt0 = PARTIAL ? (int)((long long)split * nk_all / splits) : 0;
    const int nk = PARTIAL ? (int)((long long)(split + 1) * nk_all / splits) - kt0 : nk_all;
    const int wid_s = __builtin_amdgcn_readfirstlane(wid);
    const bool loader = (LDW == NW) || wid_s < LDW;
    const int rows_a = min(M - m0, BM);
    const int rows_b = min(N - n0, BN);   // rows of W's tile (TB)
    const uint32_t smem_lds = (uint32_t)(uintptr_t)(GBA_LDS void *)smem;

    // Loader lanes' byte offsets within a slice (row r, logical chunk c), fixed
    // for the whole K loop; the slice's K offset goes into the descriptor base.
    // K-contiguous tiles (A, and W when TB) also keep each load's first k.
    // With TA, At's loads are row-major like B's: k row r, chunk c, masked at
    // the M edge (no per-load k: the descriptor range ends at K).
    uint32_t off[LD];
    int a_k[LD];
#pragma unroll
    for (int i = 0; i < LD; ++i) {
        a_k[i] = 0;
        if (TA && i < A_LD) {
            const int s = i * NTL + tid;
            const int r = s / CHT, p = s % CHT;
            const int c = p ^ bswz<CHT>(r);
            off[i] = m0 + c * 8 < M ? (uint32_t)r * (uint32_t)M * 2u + (uint32_t)c * 16u
                                    : kOobOffset;
        } else if (i < A_LD || TB) {
            const int s = (i < A_LD ? i : i - A_LD) * NTL + tid;
            const int r = s / CHA, p = s % CHA;
            const int c = aswz<MS, CHA>(r, p);
            a_k[i] = c * 8;
            off[i] = (uint32_t)r * (uint32_t)K * 2u + (uint32_t)c * 16u;
        }
    }
    if constexpr (!TB) {
#pragma unroll
        for (int i = 0; i < B_LD; ++i) {
            const int s = i * NTL + tid;
            const int r = s / CHB, p = s % CHB;
            const int c = p ^ bswz<CHB>(r);
            off[A_LD + i] = n0 + c * 8 < N ? (uint32_t)r * (uint32_t)N * 2u + (uint32_t)c * 16u
                                           : kOobOffset;
        }
    }

    // Descriptors and LDS targets of one slice (slices at or past nk read nothing).
    // In the main loop they are formed in pieces (dma_part), one per MFMA gap of
    // the step before the barrier, each pinned where it is formed and written
    // with selects: a burst of scalar work, or a taken branch, between two MFMAs
    // delays the second.
    struct SliceDma {
        __amdgpu_buffer_rsrc_t ra, rb;
        uint32_t la, lb;
        int k0;
    };
    auto dma_part = [&](SliceDma &d, int part, int kt) __attribute__((always_inline)) {
        const int k0 = (kt0 + kt) * BK;
        const bool live = PARTIAL ? kt < nk : k0 < K;
        if (part == 0) {
            const int stage = kt % STAGES;
            d.la = __builtin_amdgcn_readfirstlane(smem_lds + (uint32_t)(stage * STAGE_BYTES + wid_s * 64 * 16));
            d.lb = d.la + A_BYTES;
            d.k0 = k0;
            asm volatile("" : "+s"(d.la), "+s"(d.lb), "+s"(d.k0));
        } else if (part == 1) {
            if constexpr (TA) {
                const uint32_t bytes_a = live ? (uint32_t)min(K - k0, BK) * (uint32_t)M * 2u : 0u;
                d.ra = make_rsrc(A + (size_t)(live ? k0 : 0) * M + m0, bytes_a);
            } else {
                const uint32_t bytes_a =
                    live ? (uint32_t)rows_a * (uint32_t)K * 2u - (uint32_t)k0 * 2u : 0u;
                d.ra = make_rsrc(A + (size_t)m0 * K + (live ? k0 : 0), bytes_a);
            }
            asm volatile("" : "+s"(d.ra));
        } else {
            if constexpr (TB) {
                const uint32_t bytes_b =
                    live ? (uint32_t)rows_b * (uint32_t)K * 2u - (uint32_t)k0 * 2u : 0u;
                d.rb = make_rsrc(B + (size_t)n0 * K + (live ? k0 : 0), bytes_b);
            } else {
                const uint32_t bytes_b = live ? (uint32_t)min(K - k0, BK) * (uint32_t)N * 2u : 0u;
                d.rb = make_rsrc(B + (size_t)(live ? k0 : 0) * N + n0, bytes_b);
            }
            asm volatile("" : "+s"(d.rb));
        }
    };
    auto slice_dma = [&](int kt) __attribute__((always_inline)) {
        SliceDma d;
        dma_part(d, 0, kt);
        dma_part(d, 1, kt);
        dma_part(d, 2, kt);
        return d;
    };
    // K-contiguous loads (A, and W with TB) of the slice being loaded take eo[i]:
    // off[i], or out of range for chunks past K; formed with the descriptors, so
    // that no address arithmetic sits between the loads.
    uint32_t eo[LD];
    auto masked = [](int i) { return i < A_LD ? !TA : TB; };
    auto set_eo = [&](const SliceDma &d, int i) __attribute__((always_inline)) {
        if (masked(i)) {
            eo[i] = d.k0 + a_k[i] < K ? off[i] : kOobOffset;
            asm volatile("" : "+v"(eo[i]));
        }
    };
    auto dma_one = [&](const SliceDma &d, int i) __attribute__((always_inline)) {
        const uint32_t o = masked(i) ? eo[i] : off[i];
        if (i < A_LD)
            buffer_load_lds16(d.ra, o, d.la + i * NTL * 16);
        else
            buffer_load_lds16(d.rb, o, d.lb + (i - A_LD) * NTL * 16);
    };

    // In the main loop of the [M,K]-A, one-pass instances a slice's corners and
    // ranges are carried from the slice loaded before it (DmaPos): from one full
    // slice to the next they move by a constant along K, so only the last slice,
    // and slices past the last, are formed from scratch (with the K-tail
    // offsets).
    struct DmaPos {
        const uint16_t *pa, *pb;
        uint32_t na, nb;
    };
    auto pos_full = [&](int kt) __attribute__((always_inline)) {
        const int k0 = (kt0 + kt) * BK;
        const bool live = PARTIAL ? kt < nk : k0 < K;
        DmaPos p;
        if constexpr (TA) {
            p.na = live ? (uint32_t)min(K - k0, BK) * (uint32_t)M * 2u : 0u;
            p.pa = A + (size_t)(live ? k0 : 0) * M + m0;
        } else {
            p.na = live ? (uint32_t)rows_a * (uint32_t)K * 2u - (uint32_t)k0 * 2u : 0u;
            p.pa = A + (size_t)m0 * K + (live ? k0 : 0);
        }
        if constexpr (TB) {
            p.nb = live ? (uint32_t)rows_b * (uint32_t)K * 2u - (uint32_t)k0 * 2u : 0u;
            p.pb = B + (size_t)n0 * K + (live ? k0 : 0);
        } else {
            p.nb = live ? (uint32_t)min(K - k0, BK) * (uint32_t)N * 2u : 0u;
            p.pb = B + (size_t)(live ? k0 : 0) * N + n0;
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

    // Fragment reads for MFMA step kk of a stage.
    const int lhalf = lane >> 5;
    const int tg = lane >> 4, tj = lane & 15;
    // A operand of block fm: lane l holds row (l % BD) of the block, K chunk
    // (KS/8) kk + l / BD. B^T operand of block fn: lane l holds column (l % BD),
    // the same K chunk, gathered by two transposing reads of four k rows each.
    const int lrow_b = lane % BD, lchunk = lane / BD;
    auto a_addr = [&](int fm, int kk) -> int {
        const int r = wm * WTM + fm * BD + lrow_b;
        return r * (BK * 2) + aswz<MS, CHA>(r, (KS / 8) * kk + lchunk) * 16;
    };
    auto b_addr = [&](int fn, int kk, int h) -> int {
        const int k = kk * 32 + 8 * tg + 4 * h + (tj >> 2);
        const int n = wn * WTN + fn * 16 + 4 * (tj & 3);
        const int c = (n >> 3) ^ bswz<CHB>(k);
        return A_BYTES + k * (BN * 2) + c * 16 + (n & 4) * 2;
    };
    // TA: A operand of block fm gathered from At's tile like B^T's from B's.
    auto t_addr = [&](int fm, int kk, int h) -> int {
        const int k = kk * 32 + 8 * tg + 4 * h + (tj >> 2);
        const int m = wm * WTM + fm * 16 + 4 * (tj & 3);
        const int c = (m >> 3) ^ bswz<CHT>(k);
        return k * (BM * 2) + c * 16 + (m & 4) * 2;
    };
    // TB: W^T operand of block fn read like A's (row n of W's tile, K chunk).
    auto w_addr = [&](int fn, int kk) -> int {
        const int r = wn * WTN + fn * BD + lrow_b;
        return A_BYTES + r * (BK * 2) + aswz<MS, CHA>(r, (KS / 8) * kk + lchunk) * 16;
    };

    using AccT = typename Acc<MS>::type;
    AccT acc[FN][FM];
#pragma unroll
    for (int a = 0; a < FN; ++a)
#pragma unroll
        for (int b = 0; b < FM; ++b)
#pragma unroll
            for (int e = 0; e < Acc<MS>::n; ++e) acc[a][b][e] = 0.0f;

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
            fw[buf][r - NFA] = *reinterpret_cast<const u32x4 *>(base + w_addr(r - NFA, kk));
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

    // One MFMA step: NMF MFMAs on buffer `cur`, with the next step's fragment
    // reads (into cur^1, from `pf_base` step pf_kk) and, when `dma` is set, `nd`
    // loads of slice `d` starting at load index `d0` woven in between.
    auto step = [&](int cur, const char *pf_base, int pf_kk, bool dma, const SliceDma &d, int d0,
                    int nd, auto &&payload) {
        constexpr int every = NMF / (LD_STEP > 0 ? LD_STEP : 1);
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
            if (q < NPF) read_one(cur ^ 1, pf_base, pf_kk, q);
            if (dma && q % every == 0 && q / every < nd) dma_one(d, d0 + q / every);
            payload(q);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int r = NMF; r < NPF; ++r) read_one(cur ^ 1, pf_base, pf_kk, r);
    };

    // Prologue: slices 0 .. STAGES-1 requested; slice 0 waited for.
    auto no_payload = [](int) {};
    if (loader) {
#pragma unroll
        for (int s = 0; s < STAGES; ++s) {
            const SliceDma d = slice_dma(s);
#pragma unroll
            for (int i = 0; i < LD; ++i) set_eo(d, i);
#pragma unroll
            for (int i = 0; i < LD; ++i) dma_one(d, i);
        }
    }
    DmaPos pos = pos_full(STAGES - 1);   // the slice loaded last (CARRY)
    wait_vmcnt<(STAGES - 1) * LD>();
    block_barrier();
#pragma unroll
    for (int r = 0; r < NPF; ++r) read_one(0, smem, 0, r);

    // The step before the barrier forms the descriptors and offsets of slice
    // kt+STAGES in its shadow, from MFMA PQ on (after its fragment reads where
    // the step has room). With CARRY: three pieces, the position one slice on;
    // near the end (slice kt+STAGES is the last or past it) the position from
    // scratch and the K-tail offsets, in one rarely taken block; the
    // descriptors. Otherwise three descriptor pieces from scratch, then the
    // NMASK offsets that carry the K mask (the k-th is load MI(k)). (Carrying
    // the position measured 2-6 % faster for the [M,K]-A one-pass instances
    // and 2-3 % slower for the split-K pass and the [K,M]-A instances.)
    constexpr bool CARRY = !TA && !PARTIAL;
    constexpr int NMASK = (TA ? 0 : A_LD) + (TB ? B_LD : 0);
    constexpr int NITEM = CARRY ? 3 : 3 + NMASK;
    constexpr int PQ = NPF < NMF - NITEM ? NPF : (NMF - NITEM > 0 ? NMF - NITEM : 0);
    // Gap of payload item i (in a step shorter than the payload, several share one).
    auto item_q = [](int i) { return PQ + NITEM <= NMF ? PQ + i : i * NMF / NITEM; };
    auto MI = [](int k) { return TA ? A_LD + k : k; };
    // Slice kt in stage S = kt % STAGES, a compile-time constant in each of the
    // STAGES copies of the slice below: the fragment reads then address their
    // stage with constant offsets, not with per-slice address arithmetic.
    auto slice = [&](int kt, auto s_c) __attribute__((always_inline)) {
        constexpr int S = decltype(s_c)::value;
        const char *cur_base = smem + S * STAGE_BYTES;
        const char *nxt_base = smem + ((S + 1) % STAGES) * STAGE_BYTES;
        SliceDma dnew;
        auto prep = [&](int q) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < NITEM; ++i) {
                if (item_q(i) != q) continue;
                if constexpr (!CARRY) {
                    if (i < 3)
                        dma_part(dnew, i, kt + STAGES);
                    else
                        set_eo(dnew, MI(i - 3));
                } else if (i == 0) {
                    pos_next(pos);
                    asm volatile("" : "+s"(pos.pa), "+s"(pos.pb), "+s"(pos.na), "+s"(pos.nb));
                } else if (i == 1) {
                    if (__builtin_expect(kt + STAGES + 1 >= nk, 0)) {
                        const int kn = kt + STAGES;
                        pos = pos_full(kn);
                        const int k0n = (kt0 + kn) * BK;
#pragma unroll
                        for (int j = 0; j < LD; ++j)
                            if (masked(j)) eo[j] = k0n + a_k[j] < K ? off[j] : kOobOffset;
                    }
                    asm volatile("" : "+s"(pos.pa), "+s"(pos.pb), "+s"(pos.na), "+s"(pos.nb));
#pragma unroll
                    for (int j = 0; j < LD; ++j)
                        if (masked(j)) asm volatile("" : "+v"(eo[j]));
                } else {
                    dnew.la = __builtin_amdgcn_readfirstlane(
                        smem_lds + (uint32_t)(S * STAGE_BYTES + wid_s * 64 * 16));
                    dnew.lb = dnew.la + A_BYTES;
                    dnew.ra = make_rsrc(pos.pa, pos.na);
                    dnew.rb = make_rsrc(pos.pb, pos.nb);
                    asm volatile("" : "+s"(dnew.ra), "+s"(dnew.rb), "+s"(dnew.la), "+s"(dnew.lb));
                }
            }
        };
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const int cur = kk & 1;
            if (kk + 1 < KK) {
                if (kk + 2 == KK)
                    step(cur, cur_base, kk + 1, false, dnew, 0, 0, prep);
                else
                    step(cur, cur_base, kk + 1, false, dnew, 0, 0, no_payload);
            } else {
                // Publish slice kt+1 (own loads landed, own reads of slice kt
                // returned; then the same for all waves) and recycle slice kt's
                // stage for slice kt+STAGES.
                wait_vmcnt_lgkm0<(STAGES - 2) * LD>();
                block_barrier();
                if (loader)
                    step(cur, nxt_base, 0, true, dnew, 0, LD, no_payload);
                else
                    step(cur, nxt_base, 0, false, dnew, 0, 0, no_payload);
            }
        }
    };
    for (int kb = 0; kb < nk; kb += STAGES) {
        static_for<STAGES>([&](auto s_c) __attribute__((always_inline)) {
            constexpr int S = decltype(s_c)::value;
            if (S == 0 || kb + S < nk) slice(kb + S, s_c);
        });
    }
    // No direct-to-LDS write may outlive the workgroup's LDS.
    wait_vmcnt<0>();

    if constexpr (PARTIAL) {
        // Raw fp32 sums of this unit: lane l holds 4 adjacent n of one row m per
        // block; 16-byte stores into part[split], masked at the M / N edges.
        float *const Pt = part + (size_t)split * M * N + (size_t)m0 * N + n0;
        const int prow = wm * WTM + (lane & 15);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int cn = wn * WTN + fn * BD + 4 * (lane >> 4);
            if (n0 + cn >= N) continue;
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int r = prow + fm * BD;
                if (m0 + r >= M) continue;
                // Through a vector-register copy, as the fused epilogue reads
                // them: stored straight from the accumulators, the register
                // allocator moved accumulators between register files in every
                // slice of the main loop (96 moves per slice at 128x128).
                f32x4 v = acc[fn][fm];
                asm volatile("" : "+v"(v));
                *reinterpret_cast<f32x4 *>(Pt + (size_t)r * N + cn) = v;
            }
        }
        return;
    }

    {
        // + bias[n], activation, round once; each group of four 16x16 blocks (one
        // row block fm, one 64-column half fh) goes through the wave's staging
        // buffers and leaves as 16-byte stores of whole 128-byte row segments (8
        // rows per store instruction, non-temporal as in the persistent kernel).
        // Two buffers alternate so the LDS round trip
        // of group g - 1 overlaps the arithmetic of group g. Lane l holds row l % 16
        // and columns 16 fn + 4 (l / 16) .. +3 of the MFMA blocks.
        const int wid_u = __builtin_amdgcn_readfirstlane(wid);
        char *const stg = stage_smem + wid_u * 2 * STG_BYTES;
        const int wr = lane & 15, wg = lane >> 4;   // write side: row, 4-column group
        const int rr = lane >> 3, rc = lane & 7;    // read side: row (of 8), 16-byte chunk
        char *const Cw = reinterpret_cast<char *>(C + (size_t)m0 * N + n0) +
                         ((size_t)wm * WTM * N + (size_t)wn * WTN) * 2;
        const uint32_t st_off = (uint32_t)rr * (uint32_t)N * 2u + (uint32_t)rc * 16u;
        const uint32_t pitch8 = (uint32_t)N * 16u;   // bytes between read rows rr and rr + 8
        const int rows_left = M - m0 - wm * WTM, cols_left = N - n0 - wn * WTN;
        const bool full = rows_left >= WTM && cols_left >= WTN;   // no m0 + BM: overflows near 2^31
        // bias of the lane's columns, columns past N as zero
        u32x2 bvals[FN];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int cn = wn * WTN + fn * BD + 4 * wg;
            bvals[fn] = bias && n0 + cn < N ? *reinterpret_cast<const u32x2 *>(bias + n0 + cn)
                                            : u32x2{0u, 0u};
        }
        constexpr int NH = WTN / 64, NG = NH * FM;
        auto store_all = [&](auto masked) {
            float bq[4][4];
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
                        for (int f = 0; f < 4; ++f) {
                            const u32x2 bb = bvals[4 * fh + f];
                            bq[f][0] = to_f32<DT>(bb.x & 0xffffu);
                            bq[f][1] = to_f32<DT>(bb.x >> 16);
                            bq[f][2] = to_f32<DT>(bb.y & 0xffffu);
                            bq[f][3] = to_f32<DT>(bb.y >> 16);
                        }
                    }
#pragma unroll
                    for (int f = 0; f < 4; ++f) {
                        const AccT &a = acc[4 * fh + f][fm];
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
                        const uint32_t offs = st_off + (uint32_t)(2 * fm + j) * pitch8 + (uint32_t)(fh * 128);
                        __builtin_nontemporal_store(v[j], reinterpret_cast<u32x4 *>(Cw + offs));
                    }
                }
            }
        };
        if (full)
            store_all(std::false_type{});
        else
            store_all(std::true_type{});
        return;
    }
}

template <int BM, int BN, int BK, int WM, int WN, int STAGES, int LDW, int SPREAD, int MS, int DT,
          int ACT, bool TB = false, bool TA = false>
hipError_t launch_gemm_v3(const void *A, const void *B, const void *bias, void *C, int M, int N,
                          int K, int raster, int group_m, hipStream_t stream) {
    const int tiles_m = ceil_div(M, BM), tiles_n = ceil_div(N, BN);
    const long long grid = (long long)tiles_m * tiles_n;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL - kGridX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_v3_kernel<BM, BN, BK, WM, WN, STAGES, LDW, SPREAD, MS, DT, ACT, TB, false, TA>),
                       tile_grid(grid), dim3(WM * WN * 64), 0, stream, (const uint16_t *)A,
                       (const uint16_t *)B, (const uint16_t *)bias, (uint16_t *)C, M, N, K, tiles_m,
                       tiles_n, raster, group_m < 1 ? 1 : group_m, 1, (float *)nullptr);
    return hipGetLastError();
}

// Split-K first pass: `splits` units per tile write fp32 partials to part
// ([splits][M][N]); the epilogue runs in splitk_reduce_kernel.
template <int BM, int BN, int BK, int WM, int WN, int STAGES, int LDW, int SPREAD, int DT, bool TB,
          bool TA = false>
hipError_t launch_gemm_v3_partial(const void *A, const void *B, float *part, int M, int N, int K,
                                  int splits, int raster, int group_m, hipStream_t stream) {
    const int tiles_m = ceil_div(M, BM), tiles_n = ceil_div(N, BN);
    const long long grid = (long long)tiles_m * tiles_n * splits;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL - kGridX || splits < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(
        (gemm_v3_kernel<BM, BN, BK, WM, WN, STAGES, LDW, SPREAD, 16, DT, ACT_NONE, TB, true, TA>),
        tile_grid(grid), dim3(WM * WN * 64), 0, stream, (const uint16_t *)A, (const uint16_t *)B,
        (const uint16_t *)nullptr, (uint16_t *)nullptr, M, N, K, tiles_m, tiles_n, raster,
        group_m < 1 ? 1 : group_m, splits, part);
    return hipGetLastError();
}

}  // namespace gba
