// Grouped bf16 GEMM core for the expert FFN and its backward (gfx950).
//
// The expert FFN of the Mixture-of-Kittens notes (section 3: gate/up
// projections in parallel, then the down projection, over expert-grouped
// rows; section 5: SwiGLU fused into the grouped GEMMs) is a set of GEMMs, one
// per expert segment.  Every 256-row M tile lies inside one segment because
// segments are padded to multiples of 256 rows, so a tile needs no masking.
//
// Tile: 256 x 256 outputs, K step 64, one workgroup of 4 waves (2 x 2), each
// wave 128 x 128 outputs = 4 x 4 blocks of v_mfma_f32_32x32x16_bf16 with fp32
// accumulators (256 per lane).  Operand tiles [256][64] bf16 are staged in LDS,
// double buffered (2 x 64 KiB), with the 16-byte chunk index XOR-ed by the
// row so that the 8 lanes of a ds_read_b128 phase hit distinct banks.  Global
// loads of step k+1 are issued before the MFMAs of step k.
//
// Operands come K-contiguous ([mn][k], loaded with 16-byte vectors straight
// into the LDS layout) or MN-contiguous ([k][mn], loaded as 8 x 8 bf16 blocks
// and transposed in registers), which covers the forward (Xd W^T), the data
// gradients (dO W) and the weight gradients (dO^T A).  No float atomics: each
// output element is reduced over K inside one workgroup in ascending K.
#pragma once

#include "common.hpp"

namespace moe {

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kGemmThreads = 256;
constexpr int kOpTileBytes = 256 * kBK * 2;    // 32 KiB
constexpr int kStageBytes = 2 * kOpTileBytes;  // A + B
constexpr int kGemmLds = 2 * kStageBytes;      // 128 KiB

__device__ __forceinline__ uint32_t tile_off(int row, int kc) {
    return (uint32_t)(row * 128 + ((kc ^ (row & 7)) << 4));
}

// A K-contiguous operand window: row `i` of the tile starts at
// (i < 128 ? lo : hi) + (i & 127) * ld (elements), at the current k offset.
// Every row of a K-contiguous window is valid (tiles never straddle a
// segment, and N is a multiple of the tile).
struct KOp {
    const uint16_t *lo, *hi;
    int64_t ld;
};

// An MN-contiguous operand window: element (mn, k) at base[k * ld + mn];
// columns mn >= mn_valid read as zero.
struct MNOp {
    const uint16_t *base;
    int64_t ld;
    int mn_valid;
    const float *kscale;  // optional per-k scale (nullptr = none)
};

typedef __attribute__((address_space(3))) void lds_void_t;

// K-contiguous tile -> LDS by direct DMA (global_load_lds_dwordx4): wave w's
// i-th load fills LDS bytes [(8w+i) KiB, +1 KiB) of the tile, i.e. rows
// 8(8w+i) .. +7, lane L landing at row 8(8w+i) + L/8, physical chunk L%8.
// The lane therefore fetches logical chunk (L%8) ^ (row%8), which realises
// the XOR swizzle of tile_off() without passing through registers.
__device__ __forceinline__ void dma_k(const KOp &op, int k0, char *tile) {
    const int t = threadIdx.x, w = t >> 6, L = t & 63;
    const int kc = (L & 7) ^ ((L >> 3) & 7);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = 8 * (8 * w + i) + (L >> 3);
        const uint16_t *p = (row < 128 ? op.lo : op.hi) + (int64_t)(row & 127) * op.ld + k0 + kc * 8;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(p),
                                         (lds_void_t *)(tile + (8 * w + i) * 1024), 16, 0, 0);
    }
}

__device__ __forceinline__ uint32_t scale_pair(uint32_t v, float s) {
    return pack_bf2(__uint_as_float(v << 16) * s, __uint_as_float(v & 0xffff0000u) * s);
}

__device__ __forceinline__ void load_mn(const MNOp &op, int k0, u32x4 (&r)[8]) {
    const int t = threadIdx.x, mn = 8 * (t & 31), kb = t >> 5;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int k = k0 + 8 * kb + i;
        u32x4 v = u32x4{0, 0, 0, 0};
        if (mn < op.mn_valid) v = *reinterpret_cast<const u32x4 *>(op.base + (int64_t)k * op.ld + mn);
        if (op.kscale) {
            const float s = op.kscale[k];
#pragma unroll
            for (int d = 0; d < 4; ++d) v[d] = scale_pair(v[d], s);
        }
        r[i] = v;
    }
}

// 8 (k) x 8 (mn) block transpose: LDS row mn = 8*(t&31) + j receives the 8 k
// values of column j, as chunk kb.
__device__ __forceinline__ void store_mn(char *tile, const u32x4 (&r)[8]) {
    const int t = threadIdx.x, mn0 = 8 * (t & 31), kb = t >> 5;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        u32x4 o;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t a = r[2 * d][j >> 1], b = r[2 * d + 1][j >> 1];
            o[d] = (j & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
        }
        *reinterpret_cast<u32x4 *>(tile + tile_off(mn0 + j, kb)) = o;
    }
}

// B-tile row of block ni for this wave: plain layout {wn*128 + 32 ni}; the
// SwiGLU layout puts gate columns in rows [0,128) and up columns in
// [128,256), and gives each wave 64 gate + the matching 64 up columns.
__device__ __forceinline__ int b_block_row(bool swiglu, int wn, int ni) {
    return swiglu ? ((ni & 2) << 6) + wn * 64 + (ni & 1) * 32 : wn * 128 + ni * 32;
}

// acc[mi][ni][e] holds tile element (row, col) with
//   row = wm*128 + mi*32 + 8*(e/4) + 4*(lane/32) + e%4,  col = b_block_row + lane%32.
__device__ __forceinline__ int acc_row(int wm, int mi, int e, int lane) {
    return wm * 128 + mi * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
}

__device__ __forceinline__ void load_frags(const char *stage, int s, int arow, const int (&brow)[4], int lane,
                                           bf16x8 (&fa)[4], bf16x8 (&fb)[4]) {
    const int kc = 2 * s + (lane >> 5);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
        fa[mi] = *reinterpret_cast<const bf16x8 *>(stage + tile_off(arow + mi * 32, kc));
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
        fb[ni] = *reinterpret_cast<const bf16x8 *>(stage + kOpTileBytes + tile_off(brow[ni], kc));
}

__device__ __forceinline__ void mfma_block(const bf16x8 (&fa)[4], const bf16x8 (&fb)[4], f32x16 (&acc)[4][4]) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fb[ni], acc[mi][ni], 0, 0, 0);
}

// 64-deep slice of the tile from one stage; the fragments of sub-step s+1 are
// read while the MFMAs of sub-step s run.
__device__ __forceinline__ void compute_stage(const char *stage, int arow, const int (&brow)[4], int lane,
                                              f32x16 (&acc)[4][4]) {
    bf16x8 fa0[4], fb0[4], fa1[4], fb1[4];
    load_frags(stage, 0, arow, brow, lane, fa0, fb0);
    load_frags(stage, 1, arow, brow, lane, fa1, fb1);
    mfma_block(fa0, fb0, acc);
    load_frags(stage, 2, arow, brow, lane, fa0, fb0);
    mfma_block(fa1, fb1, acc);
    load_frags(stage, 3, arow, brow, lane, fa1, fb1);
    mfma_block(fa0, fb0, acc);
    mfma_block(fa1, fb1, acc);
}

template <bool AK, bool BK>
struct Pipe {
    const KOp &ak;
    const MNOp &amn;
    const KOp &bk;
    const MNOp &bmn;
    u32x4 ra[8], rb[8];
    __device__ __forceinline__ void issue(int k0) {  // global -> (LDS | registers)
        if (!AK) load_mn(amn, k0, ra);
        if (!BK) load_mn(bmn, k0, rb);
    }
    __device__ __forceinline__ void dma(int k0, char *stage) {
        if (AK) dma_k(ak, k0, stage);
        if (BK) dma_k(bk, k0, stage + kOpTileBytes);
    }
    __device__ __forceinline__ void commit(char *stage) {  // registers -> LDS
        if (!AK) store_mn(stage, ra);
        if (!BK) store_mn(stage + kOpTileBytes, rb);
    }
};

// LDS: two stages of [A tile 32 KiB | B tile 32 KiB] in one 128 KiB array.
// Step kt computes stage kt&1 while the DMA (or the register loads) of step
// kt+1 fill the other stage; one barrier per 64-deep step, whose vmcnt(0)
// wait is also what makes this wave's DMA for the step complete.
template <bool AK, bool BK>
__device__ __forceinline__ void gemm_mainloop(const KOp &ak, const MNOp &amn, const KOp &bk, const MNOp &bmn, int nk,
                                              bool swiglu, char *lds, f32x16 (&acc)[4][4]) {
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[mi][ni][e] = 0.f;
    if (nk <= 0) return;
    int brow[4];
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) brow[ni] = b_block_row(swiglu, wn, ni) + (lane & 31);
    const int arow = wm * 128 + (lane & 31);
    Pipe<AK, BK> pp{ak, amn, bk, bmn};
    pp.issue(0);
    __syncthreads();  // the previous tile's epilogue may still read LDS
    pp.dma(0, lds);
    pp.commit(lds);
    for (int kt = 0; kt < nk; ++kt) {
        __syncthreads();
        char *cur = lds + (kt & 1) * kStageBytes;
        char *nxt = lds + ((kt + 1) & 1) * kStageBytes;
        const bool more = kt + 1 < nk;
        if (more) {
            pp.dma((kt + 1) * kBK, nxt);
            pp.issue((kt + 1) * kBK);
        }
        compute_stage(cur, arow, brow, lane, acc);
        if (more) pp.commit(nxt);
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Deep pipeline for the forward (both operands K-contiguous): NST stages of
// BKT-deep [256][BKT] A and B tiles, DMA issued NST-1 steps ahead.  Each step
// waits only for its own stage (s_waitcnt vmcnt(G*(NST-2)), G = DMA
// instructions per wave per stage; vector memory operations complete in
// order) and then meets the other waves at a plain s_barrier, so the loads of
// the next NST-2 stages stay in flight across the barrier.
// ---------------------------------------------------------------------------

// Byte offset of 16-byte chunk kc (of BKT/8) of row `row` in a [256][BKT]
// tile.  SW selects the swizzle:
//   SW = 0   XOR the chunk with a function of the row inside its own row
//            (row%8 for BKT=64, (row/2)%4 for BKT=32);
//   SW = 3   "window" swizzle: the rows sharing one 256-byte span (2 rows of
//            128 B or 4 rows of 64 B) form 16 slots of 16 bytes, and the slot
//            index is XOR-ed with the span index.  A ds_read_b128 phase of 16
//            lanes (16 consecutive rows, one chunk) then hits 16 distinct
//            slots of the 256-byte bank window.
template <int BKT, int SW>
__device__ __forceinline__ uint32_t tile_off_t(int row, int kc) {
    constexpr int cpr = BKT / 8;          // chunks per row
    constexpr int rps = 16 / cpr;         // rows per 256-byte span
    if constexpr (SW == 3) {
        const int span = row / rps;
        const int slot = (((row % rps) * cpr) | kc) ^ (span & 15);
        return (uint32_t)(span * 256 + slot * 16);
    } else if constexpr (BKT == 64) {
        return (uint32_t)(row * 128 + ((kc ^ (row & 7)) << 4));
    } else {
        const int x = SW == 0 ? ((row >> 1) & 3) : SW == 1 ? ((row >> 2) & 3) : (row & 3);
        return (uint32_t)(row * 64 + ((kc ^ x) << 4));
    }
}

// Inverse of tile_off_t for a physical 16-byte slot: the (row, chunk) whose
// data belongs at physical byte offset `off` of the tile.
template <int BKT, int SW>
__device__ __forceinline__ void tile_slot_owner(int off, int &row, int &kc) {
    constexpr int cpr = BKT / 8;
    constexpr int rps = 16 / cpr;
    if constexpr (SW == 3) {
        const int span = off >> 8;
        const int logical = ((off >> 4) & 15) ^ (span & 15);
        row = span * rps + logical / cpr;
        kc = logical % cpr;
    } else {
        row = off / (BKT * 2);
        const int pc = (off >> 4) % cpr;
        if constexpr (BKT == 64) {
            kc = pc ^ (row & 7);
        } else {
            const int x = SW == 0 ? ((row >> 1) & 3) : SW == 1 ? ((row >> 2) & 3) : (row & 3);
            kc = pc ^ x;
        }
    }
}

// One K-contiguous [256][BKT] tile by DMA: each wave's i-th instruction fills
// a contiguous 1 KiB block, lane L writing physical bytes [16L, 16L+16); the
// lane fetches the (row, chunk) the swizzle places there.
template <int BKT, int SW>
__device__ __forceinline__ void dma_k_t(const KOp &op, int k0, char *tile) {
    constexpr int blks_per_wave = 256 * BKT * 2 / 1024 / 4;
    const int t = threadIdx.x, w = t >> 6, L = t & 63;
#pragma unroll
    for (int i = 0; i < blks_per_wave; ++i) {
        const int blk = w * blks_per_wave + i;
        int row, kc;
        tile_slot_owner<BKT, SW>(blk * 1024 + L * 16, row, kc);
        const uint16_t *p = (row < 128 ? op.lo : op.hi) + (int64_t)(row & 127) * op.ld + k0 + kc * 8;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(p), (lds_void_t *)(tile + blk * 1024), 16, 0,
                                         0);
    }
}

template <int BKT, int SW>
__device__ __forceinline__ void load_frags_t(const char *stage, int s, int arow, const int (&brow)[4], int lane,
                                             bf16x8 (&fa)[4], bf16x8 (&fb)[4]) {
    constexpr int tile_bytes = 256 * BKT * 2;
    const int kc = 2 * s + (lane >> 5);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
        fa[mi] = *reinterpret_cast<const bf16x8 *>(stage + tile_off_t<BKT, SW>(arow + mi * 32, kc));
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
        fb[ni] = *reinterpret_cast<const bf16x8 *>(stage + tile_bytes + tile_off_t<BKT, SW>(brow[ni], kc));
}

// One stage of BKT/16 sub-steps.  IL = 1 software-pipelines the fragment
// reads: the 8 ds_reads of sub-step s+1 are interleaved one-for-one with the
// first 8 of the 16 MFMAs of sub-step s (sched_group_barrier).
template <int BKT, int SW, int IL>
__device__ __forceinline__ void compute_stage_t(const char *stage, int arow, const int (&brow)[4], int lane,
                                                f32x16 (&acc)[4][4]) {
    constexpr int S = BKT / 16;
    if constexpr (IL == 0) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            bf16x8 fa[4], fb[4];
            load_frags_t<BKT, SW>(stage, s, arow, brow, lane, fa, fb);
            mfma_block(fa, fb, acc);
        }
    } else {
        bf16x8 fa[2][4], fb[2][4];
        load_frags_t<BKT, SW>(stage, 0, arow, brow, lane, fa[0], fb[0]);
#pragma unroll
        for (int s = 0; s < S; ++s) {
            if (s + 1 < S) load_frags_t<BKT, SW>(stage, s + 1, arow, brow, lane, fa[(s + 1) & 1], fb[(s + 1) & 1]);
            mfma_block(fa[s & 1], fb[s & 1], acc);
            if (s + 1 < S) {
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 DS read
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
            }
        }
    }
}

template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int BKT, int NST, int SW, int IL = 0>
__device__ __forceinline__ void gemm_mainloop_deep(const KOp &ak, const KOp &bk, int nk, bool swiglu, char *lds,
                                                   f32x16 (&acc)[4][4]) {
    constexpr int tile_bytes = 256 * BKT * 2;
    constexpr int stage_bytes = 2 * tile_bytes;
    constexpr int G = 2 * (256 * BKT * 2 / 1024) / 4;  // DMA instructions per wave per stage
    static_assert(NST >= 2 && NST * stage_bytes <= kGemmLds, "LDS budget");
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[mi][ni][e] = 0.f;
    if (nk <= 0) return;
    int brow[4];
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) brow[ni] = b_block_row(swiglu, wn, ni) + (lane & 31);
    const int arow = wm * 128 + (lane & 31);
    __syncthreads();  // the previous tile's epilogue may still read LDS
#pragma unroll
    for (int s = 0; s < NST - 1; ++s)
        if (s < nk) {
            dma_k_t<BKT, SW>(ak, s * BKT, lds + s * stage_bytes);
            dma_k_t<BKT, SW>(bk, s * BKT, lds + s * stage_bytes + tile_bytes);
        }
    int slot = 0;
    for (int kt = 0; kt < nk; ++kt) {
        if (kt + NST - 2 < nk) wait_vm_barrier<G * (NST - 2)>();
        else wait_vm_barrier<0>();
        const int ahead = kt + NST - 1;
        if (ahead < nk) {
            int as = slot + NST - 1;
            if (as >= NST) as -= NST;
            dma_k_t<BKT, SW>(ak, ahead * BKT, lds + as * stage_bytes);
            dma_k_t<BKT, SW>(bk, ahead * BKT, lds + as * stage_bytes + tile_bytes);
        }
        compute_stage_t<BKT, SW, IL>(lds + slot * stage_bytes, arow, brow, lane, acc);
        if (++slot == NST) slot = 0;
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Wave-grid generalisation: a 256 x 256 tile computed by WM x WN waves, each
// owning (256/WM) x (256/WN) outputs = MI x NI blocks of 32 x 32.  With 8
// waves (two per SIMD) one wave's MFMAs cover the other's LDS waits.
// ---------------------------------------------------------------------------
template <int WM, int WN>
struct WaveGrid {
    static constexpr int NW = WM * WN;
    static constexpr int THREADS = 64 * NW;
    static constexpr int MI = 256 / WM / 32;
    static constexpr int NI = 256 / WN / 32;
    // B-tile row of block ni for wave column wn.  SwiGLU: rows [0,128) hold
    // gate columns and [128,256) the matching up columns; each wave takes
    // NI/2 gate blocks and the same NI/2 up blocks.
    static __device__ __forceinline__ int brow(bool swiglu, int wn, int ni) {
        if (swiglu) {
            constexpr int half = NI / 2;
            return (ni / half) * 128 + wn * (half * 32) + (ni % half) * 32;
        }
        return wn * (NI * 32) + ni * 32;
    }
    static __device__ __forceinline__ int row(int wm, int mi, int e, int lane) {
        return wm * (MI * 32) + mi * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
    }
};

template <int WM, int WN>
using AccW = f32x16[WaveGrid<WM, WN>::MI][WaveGrid<WM, WN>::NI];

template <int BKT, int SW, int NW>
__device__ __forceinline__ void dma_k_w(const KOp &op, int k0, char *tile) {
    constexpr int blks_per_wave = 256 * BKT * 2 / 1024 / NW;
    const int t = threadIdx.x, w = t >> 6, L = t & 63;
#pragma unroll
    for (int i = 0; i < blks_per_wave; ++i) {
        const int blk = w * blks_per_wave + i;
        int row, kc;
        tile_slot_owner<BKT, SW>(blk * 1024 + L * 16, row, kc);
        const uint16_t *p = (row < 128 ? op.lo : op.hi) + (int64_t)(row & 127) * op.ld + k0 + kc * 8;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(p), (lds_void_t *)(tile + blk * 1024), 16, 0,
                                         0);
    }
}

// The i-th of this wave's DMA instructions for one K-contiguous [256][BKT]
// tile (the same 1 KiB blocks dma_k_w fills, one at a time).
template <int BKT, int SW, int NW>
__device__ __forceinline__ void dma_blk_w(const KOp &op, int k0, char *tile, int i) {
    constexpr int blks_per_wave = 256 * BKT * 2 / 1024 / NW;
    const int t = threadIdx.x, w = t >> 6, L = t & 63;
    const int blk = w * blks_per_wave + i;
    int row, kc;
    tile_slot_owner<BKT, SW>(blk * 1024 + L * 16, row, kc);
    const uint16_t *p = (row < 128 ? op.lo : op.hi) + (int64_t)(row & 127) * op.ld + k0 + kc * 8;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(p), (lds_void_t *)(tile + blk * 1024), 16, 0, 0);
}

// Main loop with NST stages of BKT.  The DMA instructions that fill stage
// kt+NST-1 are not issued in one burst after the barrier: they are spread
// over the first SPREAD sub-steps of stage kt, one after every few MFMAs
// (pinned there with sched_group_barrier), so a wave blocked on a full
// vector-memory queue still has MFMAs of its own in flight and the two waves
// of a SIMD keep the matrix unit busy.  Measured at the gate/up shape: about
// 10% faster than the burst.
template <int WM, int WN, int BKT, int NST, int SW, int LDS_BYTES = kGemmLds, int SPREAD = 2>
__device__ __forceinline__ void gemm_mainloop_w(const KOp &ak, const KOp &bk, int nk, bool swiglu, char *lds,
                                                AccW<WM, WN> &acc) {
    using WG = WaveGrid<WM, WN>;
    constexpr int MI = WG::MI, NI = WG::NI, NW = WG::NW;
    constexpr int tile_bytes = 256 * BKT * 2;
    constexpr int stage_bytes = 2 * tile_bytes;
    constexpr int GH = tile_bytes / 1024 / NW;  // DMA instructions per wave per operand per stage
    constexpr int G = 2 * GH;
    constexpr int S = BKT / 16;                 // MFMA sub-steps per stage
    static_assert(SPREAD >= 1 && SPREAD <= S && G % SPREAD == 0, "DMA spread");
    constexpr int D = G / SPREAD;               // DMA instructions per sub-step
    static_assert((MI * NI) % D == 0, "DMA slots");
    constexpr int EVERY = MI * NI / D;          // MFMAs between two DMA instructions
    static_assert(NST >= 2 && NST * stage_bytes <= LDS_BYTES, "LDS budget");
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
    const int wm = wave / WN, wn = wave % WN;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[mi][ni][e] = 0.f;
    if (nk <= 0) return;
    int brow[NI];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) brow[ni] = WG::brow(swiglu, wn, ni) + (lane & 31);
    const int arow = wm * (MI * 32) + (lane & 31);
    __syncthreads();  // the previous tile's epilogue may still read LDS
#pragma unroll
    for (int s = 0; s < NST - 1; ++s)
        if (s < nk) {
            dma_k_w<BKT, SW, NW>(ak, s * BKT, lds + s * stage_bytes);
            dma_k_w<BKT, SW, NW>(bk, s * BKT, lds + s * stage_bytes + tile_bytes);
        }
    int slot = 0;
    for (int kt = 0; kt < nk; ++kt) {
        if (kt + NST - 2 < nk) wait_vm_barrier<G * (NST - 2)>();
        else wait_vm_barrier<0>();
        const int ahead = kt + NST - 1;
        const bool fill = ahead < nk;
        int as = slot + NST - 1;
        if (as >= NST) as -= NST;
        char *dst = lds + as * stage_bytes;
        const char *stage = lds + slot * stage_bytes;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int kc = 2 * s + (lane >> 5);
            bf16x8 fa[MI], fb[NI];
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
                fa[mi] = *reinterpret_cast<const bf16x8 *>(stage + tile_off_t<BKT, SW>(arow + mi * 32, kc));
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
                fb[ni] = *reinterpret_cast<const bf16x8 *>(stage + tile_bytes + tile_off_t<BKT, SW>(brow[ni], kc));
#pragma unroll
            for (int q = 0; q < MI * NI; ++q) {
                acc[q / NI][q % NI] =
                    __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[q / NI], fb[q % NI], acc[q / NI][q % NI], 0, 0, 0);
                if (s < SPREAD && (q + 1) % EVERY == 0 && fill) {
                    const int g = s * D + (q + 1) / EVERY - 1;
                    if (g < GH) dma_blk_w<BKT, SW, NW>(ak, ahead * BKT, dst, g);
                    else dma_blk_w<BKT, SW, NW>(bk, ahead * BKT, dst + tile_bytes, g - GH);
                }
            }
            if (s < SPREAD) {
#pragma unroll
                for (int j = 0; j < D; ++j) {
                    __builtin_amdgcn_sched_group_barrier(0x008, EVERY, 0);  // EVERY MFMAs
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);      // then one VMEM read (the DMA)
                }
            }
        }
        if (++slot == NST) slot = 0;
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Tile ordering.
// ---------------------------------------------------------------------------

// Round-robin XCD placement: in each round of G = gridDim.x concurrent tiles,
// XCD x%8 gets a contiguous run of G/8 logical tiles, so tiles that share
// operands (same M tile, neighbouring N tiles) meet in one L2.
__device__ __forceinline__ int64_t logical_tile(int64_t it) {
    const int64_t G = gridDim.x;
    const int64_t round = it / G, x = it % G;
    return round * G + (x & 7) * (G >> 3) + (x >> 3);
}

// Grouped order inside a (mtiles x ntiles) grid: GM M tiles sweep all N tiles.
__device__ __forceinline__ void grouped_mn(int64_t lid, int mtiles, int ntiles, int GM, int &m, int &n) {
    const int64_t per = (int64_t)GM * ntiles;
    const int g = (int)(lid / per);
    const int first = g * GM;
    const int gm = min(GM, mtiles - first);
    const int in = (int)(lid % per);
    m = first + in % gm;
    n = in / gm;
}

__device__ __forceinline__ int expert_of(const int32_t *seg_off, int L, int row) {
    int lo = 0, hi = L;  // largest l with seg_off[l] <= row
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (seg_off[mid] <= row) lo = mid; else hi = mid;
    }
    return lo;
}

// ---------------------------------------------------------------------------
// Epilogues.
// ---------------------------------------------------------------------------

// A 256 x NC bf16 staging tile (NC = 128 or 256) in LDS: rows [0,128) in
// stage 0, rows [128,256) in stage 1, at byte offset `off` of the stage.  Wave
// (wm, wn) only ever writes rows of half wm, so each lane keeps one base
// address and every element it writes sits at a compile-time offset from it.
template <int NC>
struct LaneStage {
    char *base;
    __device__ __forceinline__ LaneStage(char *lds, int off, int wm, int lane, int col0) {
        base = lds + wm * kStageBytes + off + ((4 * (lane >> 5)) * NC + col0 + (lane & 31)) * 2;
    }
    // element (mi, e) of block column offset c (multiple of 32)
    __device__ __forceinline__ void put(int mi, int e, int c, float v) const {
        *reinterpret_cast<uint16_t *>(base + ((mi * 32 + 8 * (e >> 2) + (e & 3)) * NC + c) * 2) = f2bf(v);
    }
};

// Write a staged 256 x NC tile with 16-byte row-contiguous stores: dst row i
// at dst + i*ld, columns valid < nvalid.
template <int NC>
__device__ __forceinline__ void flush_tile(const char *lds, int off, uint16_t *dst, int64_t ld, int nvalid) {
    constexpr int per_row = NC / 8;
    for (int c = threadIdx.x; c < 256 * per_row; c += kGemmThreads) {
        const int row = c / per_row, cc = (c % per_row) * 8;
        const char *src = lds + (row >> 7) * kStageBytes + off + ((row & 127) * NC + cc) * 2;
        if (cc < nvalid)
            *reinterpret_cast<u32x4 *>(dst + (int64_t)row * ld + cc) = *reinterpret_cast<const u32x4 *>(src);
    }
}

__device__ __forceinline__ float silu_f(float h) { return h * __builtin_amdgcn_rcpf(1.0f + __expf(-h)); }

// Gate/up tile -> A = silu(gate) * up (256 x 128), optional HU (gate and up).
__device__ __forceinline__ void epilogue_swiglu(f32x16 (&acc)[4][4], char *lds, uint16_t *Aout, int64_t ldA,
                                                uint16_t *HUg, uint16_t *HUu, int64_t ldHU) {
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63, wm = wave >> 1, wn = wave & 1;
    const LaneStage<128> sa(lds, 0, wm, lane, wn * 64), sg(lds, 32768, wm, lane, wn * 64);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float h = acc[mi][ni][e], u = acc[mi][ni + 2][e];
                sa.put(mi, e, ni * 32, silu_f(h) * u);
                if (HUg) sg.put(mi, e, ni * 32, h);
            }
        __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    flush_tile<128>(lds, 0, Aout, ldA, 128);
    if (HUg) {
        flush_tile<128>(lds, 32768, HUg, ldHU, 128);
        __syncthreads();
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                for (int e = 0; e < 16; ++e) sa.put(mi, e, ni * 32, acc[mi][ni + 2][e]);
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
        flush_tile<128>(lds, 0, HUu, ldHU, 128);
    }
}

// Plain bf16 store of a 256 x 256 tile, columns valid < nvalid.
__device__ __forceinline__ void epilogue_store_bf16(f32x16 (&acc)[4][4], char *lds, uint16_t *dst, int64_t ld,
                                                    int nvalid) {
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63, wm = wave >> 1, wn = wave & 1;
    const LaneStage<256> sg(lds, 0, wm, lane, wn * 128);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e) sg.put(mi, e, ni * 32, acc[mi][ni][e]);
        __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    flush_tile<256>(lds, 0, dst, ld, nvalid);
}

// Staging for a WM x WN wave grid: wave (wm, wn) writes rows
// [wm*256/WM, (wm+1)*256/WM), all inside one 128-row half of the staging tile.
template <int NC, int WM>
struct LaneStageW {
    char *base;
    __device__ __forceinline__ LaneStageW(char *lds, int off, int wm, int lane, int col0) {
        constexpr int rows_per_wave = 256 / WM;
        const int r0 = wm * rows_per_wave;
        base = lds + (r0 >> 7) * kStageBytes + off + (((r0 & 127) + 4 * (lane >> 5)) * NC + col0 + (lane & 31)) * 2;
    }
    __device__ __forceinline__ void put(int mi, int e, int c, float v) const {
        *reinterpret_cast<uint16_t *>(base + ((mi * 32 + 8 * (e >> 2) + (e & 3)) * NC + c) * 2) = f2bf(v);
    }
};

template <int WM, int WN>
__device__ __forceinline__ void epilogue_swiglu_w(AccW<WM, WN> &acc, char *lds, uint16_t *Aout, int64_t ldA, uint16_t *HUg, uint16_t *HUu,
                                                  int64_t ldHU) {
    using WG = WaveGrid<WM, WN>;
    constexpr int MI = WG::MI, half = WG::NI / 2;
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63, wm = wave / WN, wn = wave % WN;
    const LaneStageW<128, WM> sa(lds, 0, wm, lane, wn * half * 32), sg(lds, 32768, wm, lane, wn * half * 32);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
        for (int ni = 0; ni < half; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float h = acc[mi][ni][e], u = acc[mi][ni + half][e];
                sa.put(mi, e, ni * 32, silu_f(h) * u);
                if (HUg) sg.put(mi, e, ni * 32, h);
            }
        __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    for (int c = threadIdx.x; c < 256 * 16; c += WG::THREADS) {
        const int row = c >> 4, cc = (c & 15) * 8;
        const char *src = lds + (row >> 7) * kStageBytes + ((row & 127) * 128 + cc) * 2;
        *reinterpret_cast<u32x4 *>(Aout + (int64_t)row * ldA + cc) = *reinterpret_cast<const u32x4 *>(src);
        if (HUg)
            *reinterpret_cast<u32x4 *>(HUg + (int64_t)row * ldHU + cc) =
                *reinterpret_cast<const u32x4 *>(src + 32768);
    }
    if (HUg) {
        __syncthreads();
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
            for (int ni = 0; ni < half; ++ni)
#pragma unroll
                for (int e = 0; e < 16; ++e) sa.put(mi, e, ni * 32, acc[mi][ni + half][e]);
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
        for (int c = threadIdx.x; c < 256 * 16; c += WG::THREADS) {
            const int row = c >> 4, cc = (c & 15) * 8;
            const char *src = lds + (row >> 7) * kStageBytes + ((row & 127) * 128 + cc) * 2;
            *reinterpret_cast<u32x4 *>(HUu + (int64_t)row * ldHU + cc) = *reinterpret_cast<const u32x4 *>(src);
        }
    }
}

template <int WM, int WN>
__device__ __forceinline__ void epilogue_store_bf16_w(AccW<WM, WN> &acc, char *lds, uint16_t *dst, int64_t ld, int nvalid) {
    using WG = WaveGrid<WM, WN>;
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63, wm = wave / WN, wn = wave % WN;
    const LaneStageW<256, WM> sg(lds, 0, wm, lane, wn * WG::NI * 32);
#pragma unroll
    for (int mi = 0; mi < WG::MI; ++mi) {
#pragma unroll
        for (int ni = 0; ni < WG::NI; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e) sg.put(mi, e, ni * 32, acc[mi][ni][e]);
        __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    for (int c = threadIdx.x; c < 256 * 32; c += WG::THREADS) {
        const int row = c >> 5, cc = (c & 31) * 8;
        const char *src = lds + (row >> 7) * kStageBytes + ((row & 127) * 256 + cc) * 2;
        if (cc < nvalid)
            *reinterpret_cast<u32x4 *>(dst + (int64_t)row * ld + cc) = *reinterpret_cast<const u32x4 *>(src);
    }
}

template <int WM, int WN>
__device__ __forceinline__ void epilogue_store_f32_w(AccW<WM, WN> &acc, float *dst, int64_t ld, int mvalid, int nvalid) {
    using WG = WaveGrid<WM, WN>;
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63, wm = wave / WN, wn = wave % WN;
    float *base = dst + (int64_t)WG::row(wm, 0, 0, lane) * ld + wn * (WG::NI * 32) + (lane & 31);
    const int row0 = WG::row(wm, 0, 0, lane), col0 = wn * (WG::NI * 32) + (lane & 31);
#pragma unroll
    for (int mi = 0; mi < WG::MI; ++mi) {
#pragma unroll
        for (int ni = 0; ni < WG::NI; ++ni) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int dr = mi * 32 + 8 * (e >> 2) + (e & 3);
                if (row0 + dr < mvalid && col0 + ni * 32 < nvalid) base[(int64_t)dr * ld + ni * 32] = acc[mi][ni][e];
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// Down-projection dgrad tile dA' (256 rows x 256 columns of I, columns from
// n0) -> SwiGLU backward and the router-weight partial sums:
//   dA = w dA'; dh = dA * u * silu'(h); du = dA * silu(h)  -> dHU (bf16)
//   part[row][(n0 / 256) * WN + wn] = sum over the wave's columns of dA' * a
// A, HU, wrow, dHU, part are already offset to the tile's first row.
template <int WM, int WN>
__device__ __forceinline__ void epilogue_swiglu_bwd_w(AccW<WM, WN> &acc, const uint16_t *A, const uint16_t *HU,
                                                      const float *wrow, uint16_t *dHU, float *part, int nparts, int I,
                                                      int n0) {
    using WG = WaveGrid<WM, WN>;
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63, wm = wave / WN, wn = wave % WN;
#pragma unroll
    for (int mi = 0; mi < WG::MI; ++mi) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int row = WG::row(wm, mi, e, lane);
            const float wr = wrow[row];
            float dot = 0.f;
#pragma unroll
            for (int ni = 0; ni < WG::NI; ++ni) {
                const int col = n0 + wn * (WG::NI * 32) + ni * 32 + (lane & 31);
                if (col < I) {
                    const float dap = acc[mi][ni][e];
                    const float a = bf2f(A[(int64_t)row * I + col]);
                    const float h = bf2f(HU[(int64_t)row * 2 * I + col]);
                    const float u = bf2f(HU[(int64_t)row * 2 * I + I + col]);
                    const float dA = wr * dap;
                    const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-h));
                    dHU[(int64_t)row * 2 * I + col] = f2bf(dA * u * sg * (1.0f + h * (1.0f - sg)));
                    dHU[(int64_t)row * 2 * I + I + col] = f2bf(dA * h * sg);
                    dot = fmaf(dap, a, dot);
                }
            }
            // fixed-order butterfly over the 32 lanes that share this row
#pragma unroll
            for (int off = 16; off >= 1; off >>= 1) dot += __shfl_xor(dot, off, 64);
            if ((lane & 31) == 0) part[(int64_t)row * nparts + (n0 / 256) * WN + wn] = dot;
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// fp32 store of a 256 x 256 tile (rows < mvalid, columns < nvalid).
__device__ __forceinline__ void epilogue_store_f32(f32x16 (&acc)[4][4], float *dst, int64_t ld, int mvalid, int nvalid) {
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63, wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = acc_row(wm, mi, e, lane), col = wn * 128 + ni * 32 + (lane & 31);
                if (row < mvalid && col < nvalid) dst[(int64_t)row * ld + col] = acc[mi][ni][e];
            }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Down-projection dgrad tile dA' (256 rows x 256 columns of I) -> SwiGLU
// backward and the router-weight partial sums:
//   dA = w dA'; dh = dA * u * silu'(h); du = dA * silu(h)  -> dHU (bf16)
//   part[row][2*nt + wn] = sum over the wave's 128 columns of dA' * a
__device__ __forceinline__ void epilogue_swiglu_bwd(f32x16 (&acc)[4][4], const uint16_t *A, const uint16_t *HU, const float *wrow,
                                    uint16_t *dHU, float *part, int nparts, int I, int n0, int nt) {
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63, wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int row = acc_row(wm, mi, e, lane);
            const float wr = wrow[row];
            float dot = 0.f;
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
                const int col = n0 + wn * 128 + ni * 32 + (lane & 31);
                if (col < I) {
                    const float dap = acc[mi][ni][e];
                    const float a = bf2f(A[(int64_t)row * I + col]);
                    const float h = bf2f(HU[(int64_t)row * 2 * I + col]);
                    const float u = bf2f(HU[(int64_t)row * 2 * I + I + col]);
                    const float dA = wr * dap;
                    const float s = 1.0f / (1.0f + __expf(-h));
                    dHU[(int64_t)row * 2 * I + col] = f2bf(dA * u * s * (1.0f + h * (1.0f - s)));
                    dHU[(int64_t)row * 2 * I + I + col] = f2bf(dA * h * s);
                    dot = fmaf(dap, a, dot);
                }
            }
            // fixed-order butterfly over the 32 lanes that share this row
#pragma unroll
            for (int off = 16; off >= 1; off >>= 1) dot += __shfl_xor(dot, off, 64);
            if ((lane & 31) == 0) part[(int64_t)row * nparts + 2 * nt + wn] = dot;
        }
}

}  // namespace moe
