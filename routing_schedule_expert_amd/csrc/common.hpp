// Internal device/host helpers of the HIP library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Round-to-nearest-even float -> bf16 bits (v_cvt_pk_bf16_f32; NaN stays NaN).
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
    return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }
// popcount of mask bits below this lane
__device__ __forceinline__ int lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}
__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0)); }

// Mask of the lanes holding the same value v (0 <= v < 2^nbits); inactive
// lanes must not call.  Built from one ballot per bit.
__device__ __forceinline__ uint64_t match_lanes(uint32_t v, int nbits) {
    uint64_t peers = __ballot(1);
    for (int b = 0; b < nbits; ++b) {
        uint64_t m = __ballot((v >> b) & 1u);
        peers &= ((v >> b) & 1u) ? m : ~m;
    }
    return peers;
}

// Device-wide barrier for a cooperative (all workgroups resident) launch.
// `bar` points at zero-initialised uint32 words: [0] arrival count, [1]
// generation, [2] set to 1 if a wait ever gave up.  Every workgroup calls it
// the same number of times.  The wait is bounded (about a second of polling):
// if the grid were not co-resident the kernel finishes with undefined
// results and bar[2] = 1 instead of hanging the device.
__device__ __forceinline__ void grid_barrier(uint32_t *bar, uint32_t nblocks) {
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();
        uint32_t gen = __hip_atomic_load(bar + 1, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
        uint32_t arrived = __hip_atomic_fetch_add(bar, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (arrived == nblocks - 1) {
            __hip_atomic_store(bar, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(bar + 1, gen + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            for (uint32_t spins = 0;
                 __hip_atomic_load(bar + 1, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) == gen; ++spins) {
                if (spins > (1u << 24)) {
                    __hip_atomic_store(bar + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
        }
        __threadfence();
    }
    __syncthreads();
}

}  // namespace moe

// Host-side helpers.
#define MOE_HIP_TRY(expr)                                  \
    do {                                                   \
        hipError_t _e = (expr);                            \
        if (_e != hipSuccess) return MOE_EHIP;             \
    } while (0)
