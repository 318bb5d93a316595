// Direct-to-LDS building blocks for gfx950 shared by the GEMM kernels.
//
//  * Global -> LDS: buffer_load_dwordx4 ... lds. Each lane's 16 bytes go straight
//    into LDS at (wave base + 16 * lane); no VGPRs hold the tile, and the buffer
//    descriptor's range check writes zeros for rows, columns or K past the edge
//    (the masking of edge tiles and of the K tail).
//  * The kernels wait for these loads themselves, with explicit vmcnt limits, so
//    that later slices stay in flight across the barrier that publishes a slice.
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

}  // namespace gba
