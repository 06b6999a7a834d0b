// Wide-tile grouped bf16 GEMM for the down projection of the expert FFN
// (gfx950).
//
// Same product as the 256 x 256 tile of gemm.hpp (the down projection of the
// Mixture-of-Kittens notes, section 3, over 256-row tiles of the expert
// segments), with a tile of 256 x 384 outputs.
//
// Why: in the 256 x 256 K loop every CU must bring 32 bytes of operands per
// clock from L2 to keep its matrix units busy, and the counters show the
// vector-memory path delivering about 20 bytes per clock: the L1 waits on
// pending L2 data about 40% of the cycles, and the requests it has in flight
// at the L2's read latency, not the L2 or LDS bandwidth, set the pace.
// Operand bytes per flop fall with the tile's area over its perimeter, and
// the accumulators bound the area: 256 x 384 outputs on 8 waves is 192 fp32
// accumulators per lane, which the compiler keeps in VGPRs beside the
// fragments and the DMA offsets (248 of a wave's 256 registers at two waves
// per SIMD); (256 + 384) / (256 * 384) operand rows per output against
// (256 + 256) / (256 * 256) is 17% fewer bytes per flop (the down launch:
// 1.67 -> 1.49 ms at the Kimi-shaped share, 8% fewer L2 read requests).
//
// Layout: 8 waves (two per SIMD, 4 x 2 grid), each 64 x 192 outputs = 2 x 6
// blocks of v_mfma_f32_32x32x16_bf16.  K steps of 64, so every operand row of
// a stage is one whole 128-byte line (with 64-byte rows each line is
// requested twice, once per half, and the requests double); two LDS stages of
// (256 + 384) x 64 bf16 (80 KiB each, all 160 KiB of the CU's LDS) filled by
// buffer_load ... lds in the window swizzle of gemm.hpp, the next stage's DMAs
// each issued ahead of one MFMA of the first sub-step as in the 256 x 256
// loop.  Buffer loads take a 32-bit offset per DMA instead of a 64-bit
// pointer, which is what keeps the registers inside the budget.  Each
// accumulator takes the same MFMAs in the same ascending K order as the
// 256 x 256 tile, so both give bitwise the same Y.  Output columns past the
// last whole wide tile use BN = 256 with the same code.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "gemm.hpp"

namespace moe {

constexpr int kWideThreads = 512;  // 8 waves
constexpr int kWBK = 64;           // K per step
constexpr int kWideBN = 384;
constexpr int kWideLds = 2 * (256 + kWideBN) * kWBK * 2;  // 160 KiB

// Raw buffer over [base, base + 1 GiB); word 3 as for every raw buffer on
// gfx9 parts.  The host keeps every offset, plus a row's length, inside it.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wide_rsrc(const void *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, 1 << 30, 0x00020000);
}

// 16 bytes per lane from a raw buffer into LDS (buffer_load_dwordx4 ... lds).
// Only the device pass sees the builtin: the host pass, which never runs
// device code, rejects its 16-byte size (it checks against the host's target).
__device__ __forceinline__ void wide_buffer_lds(const void *base, lds_void_t *dst, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(wide_rsrc(base), dst, 16, voff, soff, 0, 0);
#else
    (void)base, (void)dst, (void)voff, (void)soff;
#endif
}

// (row, 16-byte chunk) of this lane's part of the wave's j-th 1 KiB DMA
// block of a tile whose blocks are dealt to the waves in runs of `per`.
__device__ __forceinline__ void wide_dma_slot(int per, int j, int t, int &row, int &kc) {
    tile_slot_owner<kWBK, 3>(((t >> 6) * per + j) * 1024 + (t & 63) * 16, row, kc);
}

template <int BN>
using AccWide = f32x16[2][BN / 64];

// The K loop of a 256 x BN tile: A rows a + r * lda (r < 256), B rows
// b + r * ldb (r < BN), both K-contiguous; nk steps of 64; acc is zeroed
// first.  Each step starts with a barrier after this wave's DMAs of the
// step's stage have landed (the other stage is then free: every wave has
// finished the previous step).  On return every DMA has landed and the
// workgroup has met (LDS free for the epilogue).
template <int BN>
__device__ __forceinline__ void wide_mainloop(const uint16_t *a, int64_t lda, const uint16_t *b, int64_t ldb, int nk,
                                              char *lds, AccWide<BN> &acc) {
    constexpr int NI = BN / 64, A_BYTES = 256 * kWBK * 2, B_BYTES = BN * kWBK * 2, STAGE = A_BYTES + B_BYTES;
    constexpr int AJ = A_BYTES / 1024 / 8, BJ = B_BYTES / 1024 / 8, NDMA = AJ + BJ;
    static_assert(AJ * 8 * 1024 == A_BYTES && BJ * 8 * 1024 == B_BYTES, "whole DMA blocks per wave");
    static_assert(NDMA <= 2 * NI, "one DMA ahead of each of the first sub-step's MFMAs at most");
    // the thread index through an empty asm: per-lane values are then
    // recomputed for each tile instead of being hoisted out of the tile loop
    // into registers held across it
    const int t = opaque_tid(), wave = t >> 6, lane = t & 63, wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[mi][ni][e] = 0.f;
    if (nk <= 0) return;
    // Fragment addresses: with 128-byte rows, row 32 q + l % 32 at 16-byte
    // chunk 2 s + l / 32 sits at 4096 q + (off(l % 32, l / 32) ^ 32 s).
    const uint32_t lo0 = tile_off_t<kWBK, 3>(lane & 31, lane >> 5);
    // DMA byte offsets of this lane's rows and chunks
    uint32_t ao[AJ], bo[BJ];
#pragma unroll
    for (int j = 0; j < AJ; ++j) {
        int row, kc;
        wide_dma_slot(AJ, j, t, row, kc);
        ao[j] = (uint32_t)(row * lda * 2 + kc * 16);
    }
#pragma unroll
    for (int j = 0; j < BJ; ++j) {
        int row, kc;
        wide_dma_slot(BJ, j, t, row, kc);
        bo[j] = (uint32_t)(row * ldb * 2 + kc * 16);
    }
    // DMA j of this wave for the step at K offset k0 (elements) into `stage`
    auto dma = [&](int j, int k0, char *stage) {
        if (j < AJ)
            wide_buffer_lds(a, (lds_void_t *)(stage + (wave * AJ + j) * 1024), ao[j], k0 * 2);
        else
            wide_buffer_lds(b, (lds_void_t *)(stage + A_BYTES + (wave * BJ + j - AJ) * 1024), bo[j - AJ], k0 * 2);
    };
    // one K step on `stage`; FILL: the next stage's DMAs, each issued ahead of
    // one MFMA of the first sub-step (a template flag, so no branch splits
    // the interleave)
    auto step = [&](auto fill_tag, const char *stage, char *next, int k0n) {
        constexpr bool FILL = decltype(fill_tag)::value;
        uint32_t lo = lo0;
        asm volatile("" : "+v"(lo));  // recomputed per step, not held in registers
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8 fa[2], fb[NI];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
                fa[mi] = *reinterpret_cast<const bf16x8 *>(stage + (2 * wm + mi) * 4096 + (lo ^ (s << 5)));
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
                fb[ni] = *reinterpret_cast<const bf16x8 *>(stage + A_BYTES + (wn * NI + ni) * 4096 +
                                                           (lo ^ (s << 5)));
#pragma unroll
            for (int q = 0; q < 2 * NI; ++q) {
                if constexpr (FILL) {
                    if (s == 0 && q < NDMA) dma(q, k0n, next);
                }
                acc[q % 2][q / 2] =
                    __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[q % 2], fb[q / 2], acc[q % 2][q / 2], 0, 0, 0);
            }
            if constexpr (FILL) {
                if (s == 0) {
#pragma unroll
                    for (int q = 0; q < NDMA; ++q) {
                        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one VMEM read (the DMA)
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                    }
                }
            }
        }
    };
    __syncthreads();  // the previous tile's epilogue may still read LDS
#pragma unroll
    for (int j = 0; j < NDMA; ++j) dma(j, 0, lds);
    int slot = 0;
    for (int kt = 0; kt + 1 < nk; ++kt) {
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        step(std::true_type{}, lds + slot * STAGE, lds + (slot ^ 1) * STAGE, (kt + 1) * kWBK);
        slot ^= 1;
    }
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    step(std::false_type{}, lds + slot * STAGE, nullptr, 0);
    __syncthreads();
}


// ---------------------------------------------------------------------------
// Epilogues: the tile is staged in LDS as bf16 and written with 16-byte
// stores.  Wave (wm, wn) holds rows wm*64 + [0, 64) and, per block ni, 32
// columns; element e of lane l of a block is row 8(e/4) + 4(l/32) + e%4,
// column l%32.
// ---------------------------------------------------------------------------

// Copy `rows` staged rows of NC bf16 (row stride NC) to dst (row stride ld).
// With ig, a row whose ig[row] >= 0 goes to out[ig[row]] (columns n0 ...,
// row stride ld) times iw[row] instead (RowCombine).
template <int NC>
__device__ __forceinline__ void wide_copy_out(const char *st, int rows, uint16_t *dst, int64_t ld,
                                              const int *ig = nullptr, const float *iw = nullptr,
                                              uint16_t *out = nullptr, int n0 = 0) {
    constexpr int CPR = NC / 8;
    const int total = rows * CPR;
    for (int c0 = opaque_tid(); c0 < total; c0 += 4 * kWideThreads) {
        u32x4 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = c0 + i * kWideThreads;
            if (c < total) v[i] = *reinterpret_cast<const u32x4 *>(st + (c / CPR) * (NC * 2) + (c % CPR) * 16);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = c0 + i * kWideThreads;
            if (c >= total) continue;
            const int g = ig ? ig[c / CPR] : -1;
            if (g < 0)
                *reinterpret_cast<u32x4 *>(dst + (int64_t)(c / CPR) * ld + (c % CPR) * 8) = v[i];
            else
                *reinterpret_cast<u32x4 *>(out + (int64_t)g * ld + n0 + (c % CPR) * 8) =
                    scale_bf16x8(v[i], iw[c / CPR]);
        }
    }
}

// Plain bf16 store of the 256 x BN tile, in two passes of 128 rows.  With
// rc.out, the rows whose tokens have one local route (rows m0 ..., columns
// n0 ...) go to those tokens' outputs instead (times the router weight), and
// their rows of dst are not written: nothing else reads them.  Each row's
// token and weight are loaded before the first pass is staged and kept past
// the staged rows in LDS.
template <int BN>
__device__ __forceinline__ void wide_epilogue_store(AccWide<BN> &acc, char *lds, uint16_t *dst, int64_t ld,
                                                    const RowCombine &rc, int64_t m0, int n0) {
    constexpr int NI = BN / 64;
    const int t = opaque_tid(), wave = t >> 6, lane = t & 63, wm = wave >> 1, wn = wave & 1;
    uint16_t *st = reinterpret_cast<uint16_t *>(lds);  // [128][BN]
    int *ig = reinterpret_cast<int *>(lds + 128 * BN * 2);
    float *iw = reinterpret_cast<float *>(ig + 256);
    const int r0 = (wm & 1) * 64 + 4 * (lane >> 5), c0 = wn * (NI * 32) + (lane & 31);
    const bool comb = rc.out != nullptr;
    RowCombineRow rr;
    if (comb && t < 256) rr.load(rc, m0 + t);
    for (int pass = 0; pass < 2; ++pass) {
        if (pass) __syncthreads();
        if ((wm >> 1) == pass) {  // rows [128 pass, 128 pass + 128)
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
                for (int ni = 0; ni < NI; ++ni)
#pragma unroll
                    for (int q = 0; q < 16; ++q)
                        st[(r0 + mi * 32 + 8 * (q >> 2) + (q & 3)) * BN + c0 + ni * 32] = f2bf(acc[mi][ni][q]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (comb && pass == 0 && t < 256) rr.publish(ig, iw, t);
        __syncthreads();
        uint16_t *d = dst + (int64_t)pass * 128 * ld;
        if (comb)
            wide_copy_out<BN>(lds, 128, d, ld, ig + 128 * pass, iw + 128 * pass, rc.out, n0);
        else
            wide_copy_out<BN>(lds, 128, d, ld);
    }
}

// ---------------------------------------------------------------------------
// N tiling: wide tiles of WC output columns, then narrow ones of NCN columns
// for the rest (n a multiple of NCN).  Returns the counts; tile j covers
// columns [col(j), col(j) + width(j)).
// ---------------------------------------------------------------------------
struct WideSplit {
    int nw, nn, wc, ncn;  // wide tiles, narrow tiles, their widths
    __device__ __forceinline__ int col(int j) const { return j < nw ? j * wc : nw * wc + (j - nw) * ncn; }
};

__device__ __forceinline__ WideSplit wide_split(int n, int wc, int ncn) {
    WideSplit s;
    s.wc = wc;
    s.ncn = ncn;
    s.nw = n / wc;
    int rem = n - s.nw * wc;
    while (rem % ncn) {  // give back wide tiles until the rest is whole narrow tiles
        --s.nw;
        rem += wc;
    }
    s.nn = rem / ncn;
    return s;
}

}  // namespace moe
