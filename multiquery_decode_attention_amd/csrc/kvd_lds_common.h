// kvd_lds_common.h -- device helpers of the LDS-staged partial kernels:
// workgroup-wide waits on the direct global->LDS loads of a ring stage.
#pragma once

#include "kvd_mfma_common.h"

namespace kvd {
namespace lds {

typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt vmcnt(N) lgkmcnt(0), then s_barrier; a compiler memory barrier
// so no LDS access moves across it.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// s_waitcnt vmcnt(N) lgkmcnt(0) without a barrier: a wave waiting for its
// own direct loads, whose LDS bytes it then reads (and whose earlier LDS
// reads have then returned, so their slots may be refilled).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
}

// Wait until at most `stages_after` stages of this wave's own loads (PERW
// each) are still in flight; no barrier.
template <int PERW, int MAXA>
__device__ __forceinline__ void wait_own_stage(int stages_after) {
    static_assert(MAXA >= 0 && MAXA <= 4, "ring depth");
    switch (stages_after) {
        case 0: wait_vm<0>(); break;
        case 1: wait_vm<(MAXA >= 1) * PERW>(); break;
        case 2: wait_vm<(MAXA >= 2) * 2 * PERW>(); break;
        case 3: wait_vm<(MAXA >= 3) * 3 * PERW>(); break;
        default: wait_vm<(MAXA >= 4) * 4 * PERW>(); break;
    }
}

// Index of the calling wave in its workgroup, as a wave-uniform value.
__device__ __forceinline__ int wave_index() {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// Maximum of x over lanes i, i^16, i^32, i^48 with gfx950's lane swaps (no
// LDS round trip): given the same value twice, the 16-lane swap returns the
// values of rows (0, 1) and (2, 3) in its two results, and the 32-lane swap
// those of the two halves.
__device__ __forceinline__ float max_over_row_groups(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const uint32_t w = __float_as_uint(x);
    const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// True when the predicate holds in any active lane of the wave.
__device__ __forceinline__ bool wave_any(bool p) { return __any(p); }

// Wait until at most `stages_after` stages of this wave's loads (PERW
// each) are still in flight, then meet the workgroup at the barrier.
template <int PERW, int MAXA>
__device__ __forceinline__ void wait_stage(int stages_after) {
    static_assert(MAXA >= 0 && MAXA <= 6, "ring depth");
    switch (stages_after) {
        case 0: wait_vm_barrier<0>(); break;
        case 1: wait_vm_barrier<(MAXA >= 1) * PERW>(); break;
        case 2: wait_vm_barrier<(MAXA >= 2) * 2 * PERW>(); break;
        case 3: wait_vm_barrier<(MAXA >= 3) * 3 * PERW>(); break;
        case 4: wait_vm_barrier<(MAXA >= 4) * 4 * PERW>(); break;
        case 5: wait_vm_barrier<(MAXA >= 5) * 5 * PERW>(); break;
        default: wait_vm_barrier<(MAXA >= 6) * 6 * PERW>(); break;
    }
}

}  // namespace lds
}  // namespace kvd
