// Table entry for one compiled-in GEMM schedule: its shape and the launchers of
// its (dtype x activation) kernel instances, for B stored (K,N) and, where the
// kernel has that path, for B stored (N,K) (transpose_B), and for A stored
// (K,M) (transpose_A) with either B layout.
#pragma once

#include "gba.h"
#include "gba_kernels.hpp"
#include "gba_dma.hpp"
#include "gemm_v3.hpp"
#include "gemm_v5.hpp"
#include "gemm_f8.hpp"

namespace gba {

using GemmLaunchFn = hipError_t (*)(const void *, const void *, const void *, void *, int, int,
                                    int, int, int, hipStream_t);
// Split-K first pass: (A, B, part, M, N, K, splits, raster, group_m, stream).
using PartialLaunchFn = hipError_t (*)(const void *, const void *, float *, int, int, int, int,
                                       int, int, hipStream_t);

struct ScheduleEntry {
    gba_schedule sched;      // raster / group_m hold the defaults
    GemmLaunchFn fn[2][kNumActs];   // [dtype][act], B stored (K,N)
    GemmLaunchFn tb[2][kNumActs];   // [dtype][act], B stored (N,K); null without that path
    PartialLaunchFn part[2][2];     // split-K first pass [dtype][B stored (N,K)]; null if none
    GemmLaunchFn ta[2][2][kNumActs];  // A stored (K,M): [B stored (N,K)][dtype][act]; null if none
    PartialLaunchFn part_ta[2][2];  // split-K first pass with A stored (K,M) [dtype][B (N,K)]
};

}  // namespace gba

#define GBA_KERNEL_INST_(BM, BN, BK, WM, WN, DT, ACT)                                       \
    template __global__ void gba::gemm_bias_act_kernel<BM, BN, BK, WM, WN, DT, ACT>(          \
        const uint16_t *__restrict__, const uint16_t *__restrict__, const uint16_t *__restrict__, \
        uint16_t *__restrict__, int, int, int, int, int, int, int);

#define GBA_KERNEL_INSTS_(BM, BN, BK, WM, WN)                                                  \
    GBA_KERNEL_INST_(BM, BN, BK, WM, WN, 0, 0)                                                 \
    GBA_KERNEL_INST_(BM, BN, BK, WM, WN, 0, 1)                                                 \
    GBA_KERNEL_INST_(BM, BN, BK, WM, WN, 0, 2)                                                 \
    GBA_KERNEL_INST_(BM, BN, BK, WM, WN, 0, 3)                                                 \
    GBA_KERNEL_INST_(BM, BN, BK, WM, WN, 0, 4) \
    GBA_KERNEL_INST_(BM, BN, BK, WM, WN, 0, 5) \
    GBA_KERNEL_INST_(BM, BN, BK, WM, WN, 1, 0)                                                 \
    GBA_KERNEL_INST_(BM, BN, BK, WM, WN, 1, 1)                                                 \
    GBA_KERNEL_INST_(BM, BN, BK, WM, WN, 1, 2)                                                 \
    GBA_KERNEL_INST_(BM, BN, BK, WM, WN, 1, 3)    \
    GBA_KERNEL_INST_(BM, BN, BK, WM, WN, 1, 4) \
    GBA_KERNEL_INST_(BM, BN, BK, WM, WN, 1, 5)

#define GBA_LAUNCHERS_(BM, BN, BK, WM, WN, DT)                                              \
    {gba::launch_gemm<BM, BN, BK, WM, WN, DT, 0>, gba::launch_gemm<BM, BN, BK, WM, WN, DT, 1>, \
     gba::launch_gemm<BM, BN, BK, WM, WN, DT, 2>, gba::launch_gemm<BM, BN, BK, WM, WN, DT, 3>, \
     gba::launch_gemm<BM, BN, BK, WM, WN, DT, 4>, gba::launch_gemm<BM, BN, BK, WM, WN, DT, 5>}

// Instantiates the twelve kernels (2 dtypes x 6 activations; device and host
// passes) and, in the host pass only, defines gba::NAME with external linkage
// for the host registry. The other families below follow the same pattern.
#ifdef __HIP_DEVICE_COMPILE__
#define GBA_SCHEDULE_ENTRY(NAME, BM, BN, BK, WM, WN, GROUP_M) GBA_KERNEL_INSTS_(BM, BN, BK, WM, WN)
#else
#define GBA_SCHEDULE_ENTRY(NAME, BM, BN, BK, WM, WN, GROUP_M)                               \
    GBA_KERNEL_INSTS_(BM, BN, BK, WM, WN)                                                   \
    namespace gba {                                                                         \
    extern const ScheduleEntry NAME;                                                        \
    const ScheduleEntry NAME = {{BM, BN, BK, WM, WN, 2, 1, GROUP_M, 0, 0, 0},                     \
                                {GBA_LAUNCHERS_(BM, BN, BK, WM, WN, 0),                     \
                                 GBA_LAUNCHERS_(BM, BN, BK, WM, WN, 1)}};                   \
    }
#endif

// ---- interleaved direct-to-LDS kernel (gemm_v3.hpp) ----
#define GBA_V3_INST_(BM, BN, BK, WM, WN, S, L, SP, MS, DT, ACT)                               \
    template __global__ void gba::gemm_v3_kernel<BM, BN, BK, WM, WN, S, L, SP, MS, DT, ACT>(  \
        const uint16_t *__restrict__, const uint16_t *__restrict__, const uint16_t *__restrict__, \
        uint16_t *__restrict__, int, int, int, int, int, int, int, int, float *__restrict__);

#define GBA_V3_INSTS_(BM, BN, BK, WM, WN, S, L, SP, MS)                                        \
    GBA_V3_INST_(BM, BN, BK, WM, WN, S, L, SP, MS, 0, 0)                                       \
    GBA_V3_INST_(BM, BN, BK, WM, WN, S, L, SP, MS, 0, 1)                                       \
    GBA_V3_INST_(BM, BN, BK, WM, WN, S, L, SP, MS, 0, 2)                                       \
    GBA_V3_INST_(BM, BN, BK, WM, WN, S, L, SP, MS, 0, 3)                                       \
    GBA_V3_INST_(BM, BN, BK, WM, WN, S, L, SP, MS, 0, 4) \
    GBA_V3_INST_(BM, BN, BK, WM, WN, S, L, SP, MS, 0, 5) \
    GBA_V3_INST_(BM, BN, BK, WM, WN, S, L, SP, MS, 1, 0)                                       \
    GBA_V3_INST_(BM, BN, BK, WM, WN, S, L, SP, MS, 1, 1)                                       \
    GBA_V3_INST_(BM, BN, BK, WM, WN, S, L, SP, MS, 1, 2)                                       \
    GBA_V3_INST_(BM, BN, BK, WM, WN, S, L, SP, MS, 1, 3)    \
    GBA_V3_INST_(BM, BN, BK, WM, WN, S, L, SP, MS, 1, 4) \
    GBA_V3_INST_(BM, BN, BK, WM, WN, S, L, SP, MS, 1, 5)

#define GBA_V3_LAUNCHERS_(BM, BN, BK, WM, WN, S, L, SP, MS, DT)                                \
    {gba::launch_gemm_v3<BM, BN, BK, WM, WN, S, L, SP, MS, DT, 0>,                             \
     gba::launch_gemm_v3<BM, BN, BK, WM, WN, S, L, SP, MS, DT, 1>,                             \
     gba::launch_gemm_v3<BM, BN, BK, WM, WN, S, L, SP, MS, DT, 2>,                             \
     gba::launch_gemm_v3<BM, BN, BK, WM, WN, S, L, SP, MS, DT, 3>, \
     gba::launch_gemm_v3<BM, BN, BK, WM, WN, S, L, SP, MS, DT, 4>, gba::launch_gemm_v3<BM, BN, BK, WM, WN, S, L, SP, MS, DT, 5>}

// transpose_B instances (16x16x32 MFMAs only)
#define GBA_V3T_INST_(BM, BN, BK, WM, WN, S, L, SP, DT, ACT)                                  \
    template __global__ void gba::gemm_v3_kernel<BM, BN, BK, WM, WN, S, L, SP, 16, DT, ACT, true>( \
        const uint16_t *__restrict__, const uint16_t *__restrict__, const uint16_t *__restrict__, \
        uint16_t *__restrict__, int, int, int, int, int, int, int, int, float *__restrict__);

// split-K first-pass instances: [dtype][B stored (N,K)]
#define GBA_V3P_INST_(BM, BN, BK, WM, WN, S, L, SP, DT, TB)                                    \
    template __global__ void                                                                  \
    gba::gemm_v3_kernel<BM, BN, BK, WM, WN, S, L, SP, 16, DT, 0, TB, true>(                   \
        const uint16_t *__restrict__, const uint16_t *__restrict__, const uint16_t *__restrict__, \
        uint16_t *__restrict__, int, int, int, int, int, int, int, int, float *__restrict__);

#define GBA_V3P_INSTS_(BM, BN, BK, WM, WN, S, L, SP)                                           \
    GBA_V3P_INST_(BM, BN, BK, WM, WN, S, L, SP, 0, false)                                      \
    GBA_V3P_INST_(BM, BN, BK, WM, WN, S, L, SP, 0, true)                                       \
    GBA_V3P_INST_(BM, BN, BK, WM, WN, S, L, SP, 1, false)                                      \
    GBA_V3P_INST_(BM, BN, BK, WM, WN, S, L, SP, 1, true)

#define GBA_V3P_LAUNCHERS_(BM, BN, BK, WM, WN, S, L, SP)                                       \
    {{gba::launch_gemm_v3_partial<BM, BN, BK, WM, WN, S, L, SP, 0, false>,                      \
      gba::launch_gemm_v3_partial<BM, BN, BK, WM, WN, S, L, SP, 0, true>},                      \
     {gba::launch_gemm_v3_partial<BM, BN, BK, WM, WN, S, L, SP, 1, false>,                      \
      gba::launch_gemm_v3_partial<BM, BN, BK, WM, WN, S, L, SP, 1, true>}}

#define GBA_V3T_INSTS_(BM, BN, BK, WM, WN, S, L, SP)                                           \
    GBA_V3T_INST_(BM, BN, BK, WM, WN, S, L, SP, 0, 0)                                          \
    GBA_V3T_INST_(BM, BN, BK, WM, WN, S, L, SP, 0, 1)                                          \
    GBA_V3T_INST_(BM, BN, BK, WM, WN, S, L, SP, 0, 2)                                          \
    GBA_V3T_INST_(BM, BN, BK, WM, WN, S, L, SP, 0, 3)                                          \
    GBA_V3T_INST_(BM, BN, BK, WM, WN, S, L, SP, 0, 4) \
    GBA_V3T_INST_(BM, BN, BK, WM, WN, S, L, SP, 0, 5) \
    GBA_V3T_INST_(BM, BN, BK, WM, WN, S, L, SP, 1, 0)                                          \
    GBA_V3T_INST_(BM, BN, BK, WM, WN, S, L, SP, 1, 1)                                          \
    GBA_V3T_INST_(BM, BN, BK, WM, WN, S, L, SP, 1, 2)                                          \
    GBA_V3T_INST_(BM, BN, BK, WM, WN, S, L, SP, 1, 3)    \
    GBA_V3T_INST_(BM, BN, BK, WM, WN, S, L, SP, 1, 4) \
    GBA_V3T_INST_(BM, BN, BK, WM, WN, S, L, SP, 1, 5)

#define GBA_V3T_LAUNCHERS_(BM, BN, BK, WM, WN, S, L, SP, DT)                                   \
    {gba::launch_gemm_v3<BM, BN, BK, WM, WN, S, L, SP, 16, DT, 0, true>,                        \
     gba::launch_gemm_v3<BM, BN, BK, WM, WN, S, L, SP, 16, DT, 1, true>,                        \
     gba::launch_gemm_v3<BM, BN, BK, WM, WN, S, L, SP, 16, DT, 2, true>,                        \
     gba::launch_gemm_v3<BM, BN, BK, WM, WN, S, L, SP, 16, DT, 3, true>, \
     gba::launch_gemm_v3<BM, BN, BK, WM, WN, S, L, SP, 16, DT, 4, true>, gba::launch_gemm_v3<BM, BN, BK, WM, WN, S, L, SP, 16, DT, 5, true>}

// transpose_A instances (16x16x32 MFMAs only), for B stored (K,N) and (N,K)
#define GBA_V3A_INST_(BM, BN, BK, WM, WN, S, L, SP, DT, ACT, TB)                              \
    template __global__ void                                                                  \
    gba::gemm_v3_kernel<BM, BN, BK, WM, WN, S, L, SP, 16, DT, ACT, TB, false, true>(          \
        const uint16_t *__restrict__, const uint16_t *__restrict__, const uint16_t *__restrict__, \
        uint16_t *__restrict__, int, int, int, int, int, int, int, int, float *__restrict__);

#define GBA_V3A_INSTS1_(BM, BN, BK, WM, WN, S, L, SP, TB)                                      \
    GBA_V3A_INST_(BM, BN, BK, WM, WN, S, L, SP, 0, 0, TB)                                      \
    GBA_V3A_INST_(BM, BN, BK, WM, WN, S, L, SP, 0, 1, TB)                                      \
    GBA_V3A_INST_(BM, BN, BK, WM, WN, S, L, SP, 0, 2, TB)                                      \
    GBA_V3A_INST_(BM, BN, BK, WM, WN, S, L, SP, 0, 3, TB)                                      \
    GBA_V3A_INST_(BM, BN, BK, WM, WN, S, L, SP, 0, 4, TB)                                      \
    GBA_V3A_INST_(BM, BN, BK, WM, WN, S, L, SP, 0, 5, TB)                                      \
    GBA_V3A_INST_(BM, BN, BK, WM, WN, S, L, SP, 1, 0, TB)                                      \
    GBA_V3A_INST_(BM, BN, BK, WM, WN, S, L, SP, 1, 1, TB)                                      \
    GBA_V3A_INST_(BM, BN, BK, WM, WN, S, L, SP, 1, 2, TB)                                      \
    GBA_V3A_INST_(BM, BN, BK, WM, WN, S, L, SP, 1, 3, TB)                                      \
    GBA_V3A_INST_(BM, BN, BK, WM, WN, S, L, SP, 1, 4, TB)                                      \
    GBA_V3A_INST_(BM, BN, BK, WM, WN, S, L, SP, 1, 5, TB)

#define GBA_V3A_INSTS_(BM, BN, BK, WM, WN, S, L, SP)                                           \
    GBA_V3A_INSTS1_(BM, BN, BK, WM, WN, S, L, SP, false)                                       \
    GBA_V3A_INSTS1_(BM, BN, BK, WM, WN, S, L, SP, true)

#define GBA_V3A_LAUNCHERS1_(BM, BN, BK, WM, WN, S, L, SP, DT, TB)                              \
    {gba::launch_gemm_v3<BM, BN, BK, WM, WN, S, L, SP, 16, DT, 0, TB, true>,                    \
     gba::launch_gemm_v3<BM, BN, BK, WM, WN, S, L, SP, 16, DT, 1, TB, true>,                    \
     gba::launch_gemm_v3<BM, BN, BK, WM, WN, S, L, SP, 16, DT, 2, TB, true>,                    \
     gba::launch_gemm_v3<BM, BN, BK, WM, WN, S, L, SP, 16, DT, 3, TB, true>,                    \
     gba::launch_gemm_v3<BM, BN, BK, WM, WN, S, L, SP, 16, DT, 4, TB, true>,                    \
     gba::launch_gemm_v3<BM, BN, BK, WM, WN, S, L, SP, 16, DT, 5, TB, true>}

// [B stored (N,K)][dtype][act]
#define GBA_V3A_LAUNCHERS_(BM, BN, BK, WM, WN, S, L, SP)                                       \
    {{GBA_V3A_LAUNCHERS1_(BM, BN, BK, WM, WN, S, L, SP, 0, false),                             \
      GBA_V3A_LAUNCHERS1_(BM, BN, BK, WM, WN, S, L, SP, 1, false)},                            \
     {GBA_V3A_LAUNCHERS1_(BM, BN, BK, WM, WN, S, L, SP, 0, true),                              \
      GBA_V3A_LAUNCHERS1_(BM, BN, BK, WM, WN, S, L, SP, 1, true)}}

// split-K first pass with A stored (K,M): [dtype][B stored (N,K)]
#define GBA_V3PA_INST_(BM, BN, BK, WM, WN, S, L, SP, DT, TB)                                   \
    template __global__ void                                                                  \
    gba::gemm_v3_kernel<BM, BN, BK, WM, WN, S, L, SP, 16, DT, 0, TB, true, true>(             \
        const uint16_t *__restrict__, const uint16_t *__restrict__, const uint16_t *__restrict__, \
        uint16_t *__restrict__, int, int, int, int, int, int, int, int, float *__restrict__);

#define GBA_V3PA_INSTS_(BM, BN, BK, WM, WN, S, L, SP)                                          \
    GBA_V3PA_INST_(BM, BN, BK, WM, WN, S, L, SP, 0, false)                                     \
    GBA_V3PA_INST_(BM, BN, BK, WM, WN, S, L, SP, 0, true)                                      \
    GBA_V3PA_INST_(BM, BN, BK, WM, WN, S, L, SP, 1, false)                                     \
    GBA_V3PA_INST_(BM, BN, BK, WM, WN, S, L, SP, 1, true)

#define GBA_V3PA_LAUNCHERS_(BM, BN, BK, WM, WN, S, L, SP)                                      \
    {{gba::launch_gemm_v3_partial<BM, BN, BK, WM, WN, S, L, SP, 0, false, true>,                \
      gba::launch_gemm_v3_partial<BM, BN, BK, WM, WN, S, L, SP, 0, true, true>},                \
     {gba::launch_gemm_v3_partial<BM, BN, BK, WM, WN, S, L, SP, 1, false, true>,                \
      gba::launch_gemm_v3_partial<BM, BN, BK, WM, WN, S, L, SP, 1, true, true>}}

// kernel id 2: 32x32x16 MFMAs (B stored (K,N) only); kernel id 3: 16x16x32
// MFMAs, both B layouts (GBA_V3_SCHEDULE_ENTRY_TB).
#ifdef __HIP_DEVICE_COMPILE__
#define GBA_V3_SCHEDULE_ENTRY(NAME, BM, BN, BK, WM, WN, S, L, SP, MS, GROUP_M)               \
    GBA_V3_INSTS_(BM, BN, BK, WM, WN, S, L, SP, MS)
#else
#define GBA_V3_SCHEDULE_ENTRY(NAME, BM, BN, BK, WM, WN, S, L, SP, MS, GROUP_M)               \
    GBA_V3_INSTS_(BM, BN, BK, WM, WN, S, L, SP, MS)                                          \
    namespace gba {                                                                          \
    extern const ScheduleEntry NAME;                                                         \
    const ScheduleEntry NAME = {{BM, BN, BK, WM, WN, S, 1, GROUP_M, MS == 32 ? 2 : 3, L, SP}, \
                                {GBA_V3_LAUNCHERS_(BM, BN, BK, WM, WN, S, L, SP, MS, 0),     \
                                 GBA_V3_LAUNCHERS_(BM, BN, BK, WM, WN, S, L, SP, MS, 1)}};   \
    }
#endif

// Both B layouts and the split-K first pass.
#ifdef __HIP_DEVICE_COMPILE__
#define GBA_V3_SCHEDULE_ENTRY_TBP(NAME, BM, BN, BK, WM, WN, S, L, SP, GROUP_M)                \
    GBA_V3_INSTS_(BM, BN, BK, WM, WN, S, L, SP, 16)                                          \
    GBA_V3T_INSTS_(BM, BN, BK, WM, WN, S, L, SP)                                             \
    GBA_V3P_INSTS_(BM, BN, BK, WM, WN, S, L, SP)
#else
#define GBA_V3_SCHEDULE_ENTRY_TBP(NAME, BM, BN, BK, WM, WN, S, L, SP, GROUP_M)                \
    GBA_V3_INSTS_(BM, BN, BK, WM, WN, S, L, SP, 16)                                          \
    GBA_V3T_INSTS_(BM, BN, BK, WM, WN, S, L, SP)                                             \
    GBA_V3P_INSTS_(BM, BN, BK, WM, WN, S, L, SP)                                             \
    namespace gba {                                                                          \
    extern const ScheduleEntry NAME;                                                         \
    const ScheduleEntry NAME = {{BM, BN, BK, WM, WN, S, 1, GROUP_M, 3, L, SP},                \
                                {GBA_V3_LAUNCHERS_(BM, BN, BK, WM, WN, S, L, SP, 16, 0),     \
                                 GBA_V3_LAUNCHERS_(BM, BN, BK, WM, WN, S, L, SP, 16, 1)},    \
                                {GBA_V3T_LAUNCHERS_(BM, BN, BK, WM, WN, S, L, SP, 0),        \
                                 GBA_V3T_LAUNCHERS_(BM, BN, BK, WM, WN, S, L, SP, 1)},       \
                                GBA_V3P_LAUNCHERS_(BM, BN, BK, WM, WN, S, L, SP)};           \
    }
#endif

#ifdef __HIP_DEVICE_COMPILE__
#define GBA_V3_SCHEDULE_ENTRY_TB(NAME, BM, BN, BK, WM, WN, S, L, SP, GROUP_M)                 \
    GBA_V3_INSTS_(BM, BN, BK, WM, WN, S, L, SP, 16)                                          \
    GBA_V3T_INSTS_(BM, BN, BK, WM, WN, S, L, SP)
#else
#define GBA_V3_SCHEDULE_ENTRY_TB(NAME, BM, BN, BK, WM, WN, S, L, SP, GROUP_M)                 \
    GBA_V3_INSTS_(BM, BN, BK, WM, WN, S, L, SP, 16)                                          \
    GBA_V3T_INSTS_(BM, BN, BK, WM, WN, S, L, SP)                                             \
    namespace gba {                                                                          \
    extern const ScheduleEntry NAME;                                                         \
    const ScheduleEntry NAME = {{BM, BN, BK, WM, WN, S, 1, GROUP_M, 3, L, SP},                \
                                {GBA_V3_LAUNCHERS_(BM, BN, BK, WM, WN, S, L, SP, 16, 0),     \
                                 GBA_V3_LAUNCHERS_(BM, BN, BK, WM, WN, S, L, SP, 16, 1)},    \
                                {GBA_V3T_LAUNCHERS_(BM, BN, BK, WM, WN, S, L, SP, 0),        \
                                 GBA_V3T_LAUNCHERS_(BM, BN, BK, WM, WN, S, L, SP, 1)}};      \
    }
#endif

// Both B layouts, both A layouts, and the split-K first pass of all four.
#ifdef __HIP_DEVICE_COMPILE__
#define GBA_V3_SCHEDULE_ENTRY_TBPA(NAME, BM, BN, BK, WM, WN, S, L, SP, GROUP_M)               \
    GBA_V3_INSTS_(BM, BN, BK, WM, WN, S, L, SP, 16)                                          \
    GBA_V3T_INSTS_(BM, BN, BK, WM, WN, S, L, SP)                                             \
    GBA_V3P_INSTS_(BM, BN, BK, WM, WN, S, L, SP)                                             \
    GBA_V3A_INSTS_(BM, BN, BK, WM, WN, S, L, SP)                                             \
    GBA_V3PA_INSTS_(BM, BN, BK, WM, WN, S, L, SP)
#else
#define GBA_V3_SCHEDULE_ENTRY_TBPA(NAME, BM, BN, BK, WM, WN, S, L, SP, GROUP_M)               \
    GBA_V3_INSTS_(BM, BN, BK, WM, WN, S, L, SP, 16)                                          \
    GBA_V3T_INSTS_(BM, BN, BK, WM, WN, S, L, SP)                                             \
    GBA_V3P_INSTS_(BM, BN, BK, WM, WN, S, L, SP)                                             \
    GBA_V3A_INSTS_(BM, BN, BK, WM, WN, S, L, SP)                                             \
    GBA_V3PA_INSTS_(BM, BN, BK, WM, WN, S, L, SP)                                            \
    namespace gba {                                                                          \
    extern const ScheduleEntry NAME;                                                         \
    const ScheduleEntry NAME = {{BM, BN, BK, WM, WN, S, 1, GROUP_M, 3, L, SP},                \
                                {GBA_V3_LAUNCHERS_(BM, BN, BK, WM, WN, S, L, SP, 16, 0),     \
                                 GBA_V3_LAUNCHERS_(BM, BN, BK, WM, WN, S, L, SP, 16, 1)},    \
                                {GBA_V3T_LAUNCHERS_(BM, BN, BK, WM, WN, S, L, SP, 0),        \
                                 GBA_V3T_LAUNCHERS_(BM, BN, BK, WM, WN, S, L, SP, 1)},       \
                                GBA_V3P_LAUNCHERS_(BM, BN, BK, WM, WN, S, L, SP),            \
                                GBA_V3A_LAUNCHERS_(BM, BN, BK, WM, WN, S, L, SP),            \
                                GBA_V3PA_LAUNCHERS_(BM, BN, BK, WM, WN, S, L, SP)};          \
    }
#endif

// Both B layouts and both A layouts (no split-K pass).
#ifdef __HIP_DEVICE_COMPILE__
#define GBA_V3_SCHEDULE_ENTRY_TBA(NAME, BM, BN, BK, WM, WN, S, L, SP, GROUP_M)                \
    GBA_V3_INSTS_(BM, BN, BK, WM, WN, S, L, SP, 16)                                          \
    GBA_V3T_INSTS_(BM, BN, BK, WM, WN, S, L, SP)                                             \
    GBA_V3A_INSTS_(BM, BN, BK, WM, WN, S, L, SP)
#else
#define GBA_V3_SCHEDULE_ENTRY_TBA(NAME, BM, BN, BK, WM, WN, S, L, SP, GROUP_M)                \
    GBA_V3_INSTS_(BM, BN, BK, WM, WN, S, L, SP, 16)                                          \
    GBA_V3T_INSTS_(BM, BN, BK, WM, WN, S, L, SP)                                             \
    GBA_V3A_INSTS_(BM, BN, BK, WM, WN, S, L, SP)                                             \
    namespace gba {                                                                          \
    extern const ScheduleEntry NAME;                                                         \
    const ScheduleEntry NAME = {{BM, BN, BK, WM, WN, S, 1, GROUP_M, 3, L, SP},                \
                                {GBA_V3_LAUNCHERS_(BM, BN, BK, WM, WN, S, L, SP, 16, 0),     \
                                 GBA_V3_LAUNCHERS_(BM, BN, BK, WM, WN, S, L, SP, 16, 1)},    \
                                {GBA_V3T_LAUNCHERS_(BM, BN, BK, WM, WN, S, L, SP, 0),        \
                                 GBA_V3T_LAUNCHERS_(BM, BN, BK, WM, WN, S, L, SP, 1)},       \
                                {},                                                          \
                                GBA_V3A_LAUNCHERS_(BM, BN, BK, WM, WN, S, L, SP)};           \
    }
#endif

// ---- persistent interleaved kernel (gemm_v5.hpp), kernel id 4 ----
#define GBA_V5_INST_(BM, BN, WM, WN, DT, ACT, TB, TA)                                         \
    template __global__ void gba::gemm_v5_kernel<BM, BN, WM, WN, DT, ACT, TB, TA>(            \
        const uint16_t *__restrict__, const uint16_t *__restrict__, const uint16_t *__restrict__, \
        uint16_t *__restrict__, int, int, int, int, int, int, int);

#define GBA_V5_INSTS1_(BM, BN, WM, WN, TB, TA)                                                     \
    GBA_V5_INST_(BM, BN, WM, WN, 0, 0, TB, TA)                                                     \
    GBA_V5_INST_(BM, BN, WM, WN, 0, 1, TB, TA)                                                     \
    GBA_V5_INST_(BM, BN, WM, WN, 0, 2, TB, TA)                                                     \
    GBA_V5_INST_(BM, BN, WM, WN, 0, 3, TB, TA)                                                     \
    GBA_V5_INST_(BM, BN, WM, WN, 0, 4, TB, TA) \
    GBA_V5_INST_(BM, BN, WM, WN, 0, 5, TB, TA) \
    GBA_V5_INST_(BM, BN, WM, WN, 1, 0, TB, TA)                                                     \
    GBA_V5_INST_(BM, BN, WM, WN, 1, 1, TB, TA)                                                     \
    GBA_V5_INST_(BM, BN, WM, WN, 1, 2, TB, TA)                                                     \
    GBA_V5_INST_(BM, BN, WM, WN, 1, 3, TB, TA)    \
    GBA_V5_INST_(BM, BN, WM, WN, 1, 4, TB, TA) \
    GBA_V5_INST_(BM, BN, WM, WN, 1, 5, TB, TA)

#define GBA_V5_INSTS_(BM, BN, WM, WN)                                                          \
    GBA_V5_INSTS1_(BM, BN, WM, WN, false, false) GBA_V5_INSTS1_(BM, BN, WM, WN, true, false)   \
    GBA_V5_INSTS1_(BM, BN, WM, WN, false, true) GBA_V5_INSTS1_(BM, BN, WM, WN, true, true)

#define GBA_V5_LAUNCHERS_(BM, BN, WM, WN, DT, TB)  GBA_V5_LAUNCHERS2_(BM, BN, WM, WN, DT, TB, false)
#define GBA_V5_LAUNCHERS2_(BM, BN, WM, WN, DT, TB, TA)                                         \
    {gba::launch_gemm_v5<BM, BN, WM, WN, DT, 0, TB, TA>,                                       \
     gba::launch_gemm_v5<BM, BN, WM, WN, DT, 1, TB, TA>,                                       \
     gba::launch_gemm_v5<BM, BN, WM, WN, DT, 2, TB, TA>,                                       \
     gba::launch_gemm_v5<BM, BN, WM, WN, DT, 3, TB, TA>,                                       \
     gba::launch_gemm_v5<BM, BN, WM, WN, DT, 4, TB, TA>,                                       \
     gba::launch_gemm_v5<BM, BN, WM, WN, DT, 5, TB, TA>}

#ifdef __HIP_DEVICE_COMPILE__
#define GBA_V5_SCHEDULE_ENTRY(NAME, BM, BN, WM, WN, GROUP_M) GBA_V5_INSTS_(BM, BN, WM, WN)
#else
#define GBA_V5_SCHEDULE_ENTRY(NAME, BM, BN, WM, WN, GROUP_M)                                   \
    GBA_V5_INSTS_(BM, BN, WM, WN)                                                              \
    namespace gba {                                                                            \
    extern const ScheduleEntry NAME;                                                           \
    const ScheduleEntry NAME = {{BM, BN, 64, WM, WN, 2, 1, GROUP_M, 4, WM * WN, 1},            \
                                {GBA_V5_LAUNCHERS_(BM, BN, WM, WN, 0, false),                  \
                                 GBA_V5_LAUNCHERS_(BM, BN, WM, WN, 1, false)},                 \
                                {GBA_V5_LAUNCHERS_(BM, BN, WM, WN, 0, true),                   \
                                 GBA_V5_LAUNCHERS_(BM, BN, WM, WN, 1, true)},                  \
                                {},                                                            \
                                {{GBA_V5_LAUNCHERS2_(BM, BN, WM, WN, 0, false, true),          \
                                  GBA_V5_LAUNCHERS2_(BM, BN, WM, WN, 1, false, true)},         \
                                 {GBA_V5_LAUNCHERS2_(BM, BN, WM, WN, 0, true, true),           \
                                  GBA_V5_LAUNCHERS2_(BM, BN, WM, WN, 1, true, true)}}};        \
    }
#endif

// ---- 8-bit-input persistent kernel (gemm_f8.hpp) ----
namespace gba {
using F8LaunchFn = hipError_t (*)(const void *, const void *, const void *, void *, int, int, int,
                                  float, int, int, hipStream_t);
// Split-K first pass: (A, W, part, M, N, K, scale, splits, raster, group_m, stream).
using F8PartialLaunchFn = hipError_t (*)(const void *, const void *, float *, int, int, int, float,
                                         int, int, int, hipStream_t);
}  // namespace gba

#define GBA_F8_INST_(FMT, DT, ACT)                                                             \
    template __global__ void gba::gemm_f8_kernel<FMT, DT, ACT>(                                \
        const uint8_t *__restrict__, const uint8_t *__restrict__, const uint16_t *__restrict__, \
        uint16_t *__restrict__, int, int, int, float, int, int, int, int, int, float *__restrict__);
#define GBA_F8P_INST_(FMT)                                                                     \
    template __global__ void gba::gemm_f8_kernel<FMT, 0, 0, true>(                             \
        const uint8_t *__restrict__, const uint8_t *__restrict__, const uint16_t *__restrict__, \
        uint16_t *__restrict__, int, int, int, float, int, int, int, int, int, float *__restrict__);

#define GBA_F8_INSTS_(FMT)                                                                     \
    GBA_F8_INST_(FMT, 0, 0) GBA_F8_INST_(FMT, 0, 1) GBA_F8_INST_(FMT, 0, 2)                    \
    GBA_F8_INST_(FMT, 0, 3) GBA_F8_INST_(FMT, 0, 4) GBA_F8_INST_(FMT, 0, 5)                    \
    GBA_F8_INST_(FMT, 1, 0) GBA_F8_INST_(FMT, 1, 1) GBA_F8_INST_(FMT, 1, 2)                    \
    GBA_F8_INST_(FMT, 1, 3) GBA_F8_INST_(FMT, 1, 4) GBA_F8_INST_(FMT, 1, 5)

#define GBA_F8_LAUNCHERS_(FMT, DT)                                                             \
    {gba::launch_gemm_f8<FMT, DT, 0>, gba::launch_gemm_f8<FMT, DT, 1>,                         \
     gba::launch_gemm_f8<FMT, DT, 2>, gba::launch_gemm_f8<FMT, DT, 3>,                         \
     gba::launch_gemm_f8<FMT, DT, 4>, gba::launch_gemm_f8<FMT, DT, 5>}

// Defines gba::NAME[dtype][act] and gba::NAME_part (host pass) for 8-bit format FMT.
#ifdef __HIP_DEVICE_COMPILE__
#define GBA_F8_ENTRY(NAME, FMT) GBA_F8_INSTS_(FMT) GBA_F8P_INST_(FMT)
#else
#define GBA_F8_ENTRY(NAME, FMT)                                                                \
    GBA_F8_INSTS_(FMT)                                                                         \
    GBA_F8P_INST_(FMT)                                                                         \
    namespace gba {                                                                            \
    extern const F8LaunchFn NAME[2][kNumActs];                                                 \
    const F8LaunchFn NAME[2][kNumActs] = {GBA_F8_LAUNCHERS_(FMT, 0), GBA_F8_LAUNCHERS_(FMT, 1)}; \
    extern const F8PartialLaunchFn NAME##_part;                                                \
    const F8PartialLaunchFn NAME##_part = gba::launch_gemm_f8_partial<FMT>;                    \
    }
#endif
