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
// lanes must not call.  Built from one ballot per bit: a lane keeps the
// ballot of its bit value (the ballot, or its complement where its bit is 0).
__device__ __forceinline__ uint64_t match_lanes(uint32_t v, int nbits) {
    uint64_t peers = __ballot(1);
    for (int b = 0; b < nbits; ++b) {
        const uint64_t flip = (uint64_t)((v >> b) & 1u) - 1ull;  // 0 where the bit is 1, all ones where 0
        peers &= __ballot((v >> b) & 1u) ^ flip;
    }
    return peers;
}

// The same with the bit count fixed at compile time (the loop unrolled);
// bits of v at or above NB must be zero.
template <int NB>
__device__ __forceinline__ uint64_t match_lanes_n(uint32_t v) {
    uint64_t peers = __ballot(1);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const uint64_t flip = (uint64_t)((v >> b) & 1u) - 1ull;
        peers &= __ballot((v >> b) & 1u) ^ flip;
    }
    return peers;
}

// Device-wide barrier for a cooperative (all workgroups resident) launch.
//
// Memory on this part is cached per XCD (each XCD has its own L2), so data
// written before a barrier by one XCD must be written back from its L2 and
// the readers' L2 must be invalidated.  Doing that from every workgroup
// (one agent-scope fence each) costs tens of microseconds per barrier; here one
// elected workgroup per XCD does it for all workgroups of its XCD:
//   1. every wave waits for its own stores (s_waitcnt), then the workgroup
//      arrives at its XCD's counter;
//   2. the last arrival of an XCD writes back that XCD's L2 (release fence)
//      and arrives at the device counter; the last XCD publishes the epoch;
//   3. each XCD's elected workgroup then invalidates its L2 (acquire fence)
//      and releases its XCD; the other workgroups take an acquire fence too,
//      which drops their L1 (the shared L2 holds no stale lines by then).
// Every workgroup counts the barriers it has passed (`epoch`), so all waits are
// for an exact value and no counter is ever reset: after barrier e the XCD
// counter of x holds e * (workgroups on x), the device counter e * (XCDs in
// use), the device epoch and the release word of every XCD hold e.
// Words of `bar` (zero on entry, 64 words): [0] device arrivals, [1] device
// epoch, [2] set if a wait gave up, [4] census arrivals, [8+x] arrivals of XCD
// x, [16+x] release epoch of XCD x, [24+x] workgroups on XCD x, [32] XCDs in
// use.  Every wait is bounded (about a second): if the grid were not
// co-resident the kernel finishes with undefined results and bar[2] = 1
// instead of hanging (bar[2] is the caller-visible MOE_WS_BARRIER_STATUS
// word).  Only thread 0 of a workgroup holds meaningful fields.

__device__ __forceinline__ uint32_t xcc_id() {
    uint32_t v;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
    return v & 7u;
}

__device__ __forceinline__ uint32_t ld_agent(uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void spin_until_equal(uint32_t *p, uint32_t want, uint32_t *flag) {
    for (uint32_t spins = 0; ld_agent(p) != want; ++spins) {
        if (spins > (1u << 22)) {
            __hip_atomic_store(flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        __builtin_amdgcn_s_sleep(2);
    }
}

struct GridBarrier {
    uint32_t *bar;
    uint32_t xcc, here, nxcc, epoch;

    // Registers this workgroup's XCD; one fenced barrier publishes the census.
    __device__ __forceinline__ explicit GridBarrier(uint32_t *b) : bar(b), xcc(0), here(0), nxcc(0), epoch(0) {
        if (threadIdx.x == 0) {
            xcc = xcc_id();
            if (__hip_atomic_fetch_add(bar + 24 + xcc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0)
                __hip_atomic_fetch_add(bar + 32, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __threadfence();
            __hip_atomic_fetch_add(bar + 4, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
            spin_until_equal(bar + 4, gridDim.x, bar + 2);
            __threadfence();
            here = ld_agent(bar + 24 + xcc);
            nxcc = ld_agent(bar + 32);
        }
        __syncthreads();
    }

    __device__ __forceinline__ void sync() {
        __builtin_amdgcn_s_waitcnt(0);  // every wave's stores have reached its XCD's L2
        __syncthreads();
        if (threadIdx.x == 0) {
            const uint32_t e = ++epoch;
            const uint32_t n = __hip_atomic_fetch_add(bar + 8 + xcc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (n == e * here - 1) {
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // write back this XCD's L2
                const uint32_t m = __hip_atomic_fetch_add(bar, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
                if (m == e * nxcc - 1)
                    __hip_atomic_store(bar + 1, e, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
                else
                    spin_until_equal(bar + 1, e, bar + 2);
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // invalidate this XCD's L2
                __hip_atomic_store(bar + 16 + xcc, e, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            } else {
                spin_until_equal(bar + 16 + xcc, e, bar + 2);
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // invalidate this CU's L1
            }
        }
        __syncthreads();
    }
};

}  // namespace moe

// Host-side helpers.
#define MOE_HIP_TRY(expr)                                  \
    do {                                                   \
        hipError_t _e = (expr);                            \
        if (_e != hipSuccess) return MOE_EHIP;             \
    } while (0)
