// Grouped bf16 GEMM core for the expert FFN and its backward (gfx950).
//
// The expert FFN of the Mixture-of-Kittens notes (section 3: gate/up
// projections in parallel, then the down projection, over expert-grouped
// rows; section 5: SwiGLU fused into the grouped GEMMs) is a set of GEMMs, one
// per expert segment.  Every 256-row M tile lies inside one segment because
// segments are padded to multiples of 256 rows, so a tile needs no masking.
//
// Tile: 256 x 256 outputs, K step 64, one workgroup of 8 waves (a 4 x 2 wave
// grid, two waves per SIMD), each wave 64 x 128 outputs = 2 x 4 blocks of
// v_mfma_f32_32x32x16_bf16 with fp32 accumulators.  Both operands are
// K-contiguous ([mn][k]); their [256][64] bf16 tiles go global -> LDS by
// direct DMA (global_load_lds_dwordx4), double buffered (2 x 64 KiB), with a
// 256-byte window XOR swizzle that keeps the 16-lane phases of ds_read_b128
// conflict-free.  The backward's operands that lie MN-contiguous (the weights
// along their rows, the activations over their rows) use the same loop with
// transposing LDS reads (gemm_mainloop_x).  No float atomics: each output
// element is reduced over K inside one workgroup in ascending K.
#pragma once

#include "common.hpp"

namespace moe {

constexpr int kBM = 256;                      // rows per M tile (= segment padding)
constexpr int kOpTileBytes = 256 * 64 * 2;    // one [256][64] bf16 operand tile, 32 KiB
constexpr int kStageBytes = 2 * kOpTileBytes;  // A + B
constexpr int kGemmLds = 2 * kStageBytes;      // 128 KiB

// A K-contiguous operand window of 256 rows.  Contiguous form (rows ==
// nullptr): row i starts at (i < 128 ? lo : hi) + (i & 127) * ld.  Gathered
// form: row i is source row rows[i] = (part, tok) of src, i.e. src + (part * np
// + tok) * ld, and a row with part < 0 (segment padding) reads zeros.  Every
// row of a window is valid (tiles never straddle a segment, and N is a
// multiple of the tile).
struct KOp {
    const uint16_t *lo, *hi;
    int64_t ld;
    const moe_src *rows;
    const uint16_t *src;
    int32_t np;
};

// Source of the padding rows of a gathered operand: never written, so it
// stays zero (device globals are zero-initialised when the code object is
// loaded).  Gathered operands need K <= kZeroRowElems.
constexpr int kZeroRowElems = 32768;
__device__ uint16_t g_zero_row[kZeroRowElems];

typedef __attribute__((address_space(3))) void lds_void_t;

// Byte offset of 16-byte chunk kc (of BKT/8) of row `row` in a [256][BKT]
// tile, "window" swizzle (SW = 3): the rows sharing one 256-byte span (2 rows
// of 128 B or 4 rows of 64 B) form 16 slots of 16 bytes, and the slot index is
// XOR-ed with the span index.  A ds_read_b128 phase of 16 lanes (16
// consecutive rows, one chunk) then hits 16 distinct slots of the 256-byte
// bank window.
template <int BKT, int SW>
__device__ __forceinline__ uint32_t tile_off_t(int row, int kc) {
    static_assert(SW == 3, "only the window swizzle is implemented");
    constexpr int cpr = BKT / 8;          // chunks per row
    constexpr int rps = 16 / cpr;         // rows per 256-byte span
    const int span = row / rps;
    const int slot = (((row % rps) * cpr) | kc) ^ (span & 15);
    return (uint32_t)(span * 256 + slot * 16);
}

// Inverse of tile_off_t for a physical 16-byte slot: the (row, chunk) whose
// data belongs at physical byte offset `off` of the tile.
template <int BKT, int SW>
__device__ __forceinline__ void tile_slot_owner(int off, int &row, int &kc) {
    static_assert(SW == 3, "only the window swizzle is implemented");
    constexpr int cpr = BKT / 8;
    constexpr int rps = 16 / cpr;
    const int span = off >> 8;
    const int logical = ((off >> 4) & 15) ^ (span & 15);
    row = span * rps + logical / cpr;
    kc = logical % cpr;
}

// Wait for this wave's outstanding vector-memory operations down to N, then
// meet the other waves (vector memory operations complete in order).
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
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

// Source address (at k = 0) of this lane's 16 bytes in its i-th DMA block of
// one [256][BKT] operand tile: each wave's i-th instruction fills a
// contiguous 1 KiB block of the tile, lane L writing physical bytes
// [16L, 16L+16), and the lane fetches the (row, chunk) the swizzle places
// there.  Computed once per tile; a K step only adds k0.
template <int BKT, int SW, int NW>
__device__ __forceinline__ const uint16_t *dma_src_w(const KOp &op, int i) {
    constexpr int blks_per_wave = 256 * BKT * 2 / 1024 / NW;
    const int t = threadIdx.x, w = t >> 6, L = t & 63;
    const int blk = w * blks_per_wave + i;
    int row, kc;
    tile_slot_owner<BKT, SW>(blk * 1024 + L * 16, row, kc);
    const uint16_t *base;
    if (op.rows) {
        const uint2 s = reinterpret_cast<const uint2 *>(op.rows)[row];
        base = (int32_t)s.x >= 0 ? op.src + ((int64_t)(int32_t)s.x * op.np + (int32_t)s.y) * op.ld : g_zero_row;
    } else {
        base = (row < 128 ? op.lo : op.hi) + (int64_t)(row & 127) * op.ld;
    }
    return base + kc * 8;
}

template <int BKT, int NW>
__device__ __forceinline__ void dma_blk_w(const uint16_t *src, int k0, char *tile, int i) {
    constexpr int blks_per_wave = 256 * BKT * 2 / 1024 / NW;
    const int blk = (threadIdx.x >> 6) * blks_per_wave + i;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(src + k0), (lds_void_t *)(tile + blk * 1024), 16,
                                     0, 0);
}

// ---------------------------------------------------------------------------
// Operands stored MN-contiguous ([k][mn]): the backward's products need
// W2[l] and W13[l] along their rows, and the weight gradients reduce over the
// rows of the activations; instead of transposed copies in HBM, such an
// operand's [64][256] tile is moved to LDS as it lies (512-byte k rows) and
// its MFMA fragments are built with the transposing LDS read
// (ds_read_b64_tr_b16): within each 16-lane group, lane 4j + c points at 4
// consecutive mn values of k row j, and lane i receives, from the lanes
// 4j + i/4 (j = 0..3), their (i%4)-th values, i.e. the 4 k values of column
// i.  Two such reads give a lane its 8 k values of one column.
//
// T tile layout: k row r at r * 512 bytes; its 16-byte chunk c at physical
// chunk c ^ (4 * (r & 3)), so the 4 rows a 16-lane group reads fall in 4
// different 64-byte quarters of the 256-byte bank window.
// ---------------------------------------------------------------------------

// An MN-contiguous operand window: element (k, mn) at base + k * ld + mn, for
// mn < valid (128 or 256); columns past `valid` repeat the first ones (their
// results are masked by the caller).
struct TOp {
    const uint16_t *base;
    int64_t ld;
    int valid;
};

__device__ __forceinline__ uint32_t ttile_off(int r, int c) { return (uint32_t)(r * 512 + ((c ^ (4 * (r & 3))) << 4)); }

// Source (at k = 0) of this lane's 16 bytes in its i-th DMA block of a T
// tile: block b covers k rows 2b, 2b+1; lane L writes physical chunk L % 32 of
// row 2b + L / 32 and fetches the logical chunk the swizzle puts there.
template <int NW>
__device__ __forceinline__ const uint16_t *dma_src_t(const TOp &op, int i) {
    constexpr int blks_per_wave = 32 / NW;
    const int t = threadIdx.x, w = t >> 6, L = t & 63;
    const int r = 2 * (w * blks_per_wave + i) + (L >> 5);
    int c = (L & 31) ^ (4 * (r & 3));
    if (c * 8 >= op.valid) c -= op.valid / 8;
    return op.base + (int64_t)r * op.ld + c * 8;
}

// This wave's i-th 1 KiB DMA block of a [256][64]-sized operand tile, from a
// per-lane source already advanced to the K step.
template <int NW>
__device__ __forceinline__ void dma_blk_x(const uint16_t *src, char *tile, int i) {
    const int blk = (threadIdx.x >> 6) * (32 / NW) + i;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(src), (lds_void_t *)(tile + blk * 1024), 16, 0, 0);
}

// LDS byte address of a generic pointer into this workgroup's LDS.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)(const char *)p;
}

// The two transposing-read addresses of a T-operand fragment for MFMA block
// base `mnb` (a multiple of 32) and sub-step s: this lane's column
// mnb + lane % 32, k rows 16 s + 8 (lane / 32) + 0..3 and + 4..7.
__device__ __forceinline__ void t_frag_addr(const char *tile, int mnb, int s, int lane, uint32_t &a0, uint32_t &a1) {
    const int h2 = lane >> 5, g = (lane >> 4) & 1, q = lane & 15, j = q >> 2, cq = q & 3;
    const int c = (mnb >> 3) + 2 * g + (cq >> 1);
    a0 = lds_addr(tile + ttile_off(16 * s + 8 * h2 + j, c) + (cq & 1) * 8);
    a1 = lds_addr(tile + ttile_off(16 * s + 8 * h2 + 4 + j, c) + (cq & 1) * 8);
}

// N transposing LDS reads (ds_read_b64_tr_b16) and a wait for them, in one
// asm block, so the results are complete when it ends.  Issued as compiler
// builtins, each such read made the compiler wait for every outstanding DMA
// into LDS first (it cannot tell that they target the other stage), which
// serialised the next stage's loads with this one's MFMAs.
template <int N>
__device__ __forceinline__ void tr_reads(const uint32_t (&ad)[N], uint64_t (&o)[N]);
template <>
__device__ __forceinline__ void tr_reads<4>(const uint32_t (&ad)[4], uint64_t (&o)[4]) {
    asm volatile("ds_read_b64_tr_b16 %0, %4\n\t"
                 "ds_read_b64_tr_b16 %1, %5\n\t"
                 "ds_read_b64_tr_b16 %2, %6\n\t"
                 "ds_read_b64_tr_b16 %3, %7\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
                 : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]));
}

template <>
__device__ __forceinline__ void tr_reads<8>(const uint32_t (&ad)[8], uint64_t (&o)[8]) {
    asm volatile("ds_read_b64_tr_b16 %0, %8\n\t"
                 "ds_read_b64_tr_b16 %1, %9\n\t"
                 "ds_read_b64_tr_b16 %2, %10\n\t"
                 "ds_read_b64_tr_b16 %3, %11\n\t"
                 "ds_read_b64_tr_b16 %4, %12\n\t"
                 "ds_read_b64_tr_b16 %5, %13\n\t"
                 "ds_read_b64_tr_b16 %6, %14\n\t"
                 "ds_read_b64_tr_b16 %7, %15\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
                 : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7]));
}

template <>
__device__ __forceinline__ void tr_reads<12>(const uint32_t (&ad)[12], uint64_t (&o)[12]) {
    asm volatile("ds_read_b64_tr_b16 %0, %12\n\t"
                 "ds_read_b64_tr_b16 %1, %13\n\t"
                 "ds_read_b64_tr_b16 %2, %14\n\t"
                 "ds_read_b64_tr_b16 %3, %15\n\t"
                 "ds_read_b64_tr_b16 %4, %16\n\t"
                 "ds_read_b64_tr_b16 %5, %17\n\t"
                 "ds_read_b64_tr_b16 %6, %18\n\t"
                 "ds_read_b64_tr_b16 %7, %19\n\t"
                 "ds_read_b64_tr_b16 %8, %20\n\t"
                 "ds_read_b64_tr_b16 %9, %21\n\t"
                 "ds_read_b64_tr_b16 %10, %22\n\t"
                 "ds_read_b64_tr_b16 %11, %23\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7]), "=&v"(o[8]), "=&v"(o[9]), "=&v"(o[10]), "=&v"(o[11])
                 : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7]), "v"(ad[8]), "v"(ad[9]), "v"(ad[10]), "v"(ad[11]));
}

// Fragment from two transposing reads: 4 k values each, low then high.
__device__ __forceinline__ bf16x8 tr_frag(uint64_t lo, uint64_t hi) {
    typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
    const u64x2 v = {lo, hi};
    return __builtin_bit_cast(bf16x8, v);
}

// An operand of the general main loop: K-contiguous (KOp) or MN-contiguous (TOp).
template <bool T>
struct OpOf {
    using type = KOp;
};
template <>
struct OpOf<true> {
    using type = TOp;
};

// One K step of gemm_mainloop_x on stage `slot`; with FILL the next stage's
// DMA (sources already advanced by the caller) is spread over the first two
// sub-steps.  FILL is a template flag so no branch splits the pinned
// MFMA / DMA interleave.
template <int WM, int WN, bool AT, bool BT, bool FILL, int GH>
__device__ __forceinline__ void x_step(char *lds, int slot, int lane, int arow, const int (&brow)[WaveGrid<WM, WN>::NI],
                                       const uint16_t *const (&asrc)[GH], const uint16_t *const (&bsrc)[GH],
                                       int64_t ao, int64_t bo, AccW<WM, WN> &acc) {
    using WG = WaveGrid<WM, WN>;
    constexpr int MI = WG::MI, NI = WG::NI, NW = WG::NW;
    // DMAs after the MFMAs of the first sub-step; over two sub-steps when both
    // operands are MN-contiguous (the weight gradients' short K loops)
    constexpr int BKT = 64, SW = 3, SPREAD = (AT && BT) ? 2 : 1;
    constexpr int tile_bytes = 256 * BKT * 2, stage_bytes = 2 * tile_bytes;
    constexpr int G = 2 * GH, S = BKT / 16, D = G / SPREAD;
    static_assert((MI * NI) % D == 0, "DMA slots");
    constexpr int EVERY = MI * NI / D;
    wait_vm_barrier<0>();
    char *dst = lds + (slot ^ 1) * stage_bytes;
    const char *stage = lds + slot * stage_bytes;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int kc = 2 * s + (lane >> 5);
        bf16x8 fa[MI], fb[NI];
        if constexpr (!AT) {
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
                fa[mi] = *reinterpret_cast<const bf16x8 *>(stage + tile_off_t<BKT, SW>(arow + mi * 32, kc));
        }
        if constexpr (!BT) {
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
                fb[ni] = *reinterpret_cast<const bf16x8 *>(stage + tile_bytes + tile_off_t<BKT, SW>(brow[ni], kc));
        }
        if constexpr (AT || BT) {  // every transposing read of the sub-step in one batch
            constexpr int NA = AT ? 2 * MI : 0, NB = BT ? 2 * NI : 0;
            uint32_t ad[NA + NB];
            uint64_t o[NA + NB];
            if constexpr (AT) {
#pragma unroll
                for (int mi = 0; mi < MI; ++mi) t_frag_addr(stage, arow + mi * 32, s, lane, ad[2 * mi], ad[2 * mi + 1]);
            }
            if constexpr (BT) {
#pragma unroll
                for (int ni = 0; ni < NI; ++ni)
                    t_frag_addr(stage + tile_bytes, brow[ni], s, lane, ad[NA + 2 * ni], ad[NA + 2 * ni + 1]);
            }
            tr_reads<NA + NB>(ad, o);
            if constexpr (AT) {
#pragma unroll
                for (int mi = 0; mi < MI; ++mi) fa[mi] = tr_frag(o[2 * mi], o[2 * mi + 1]);
            }
            if constexpr (BT) {
#pragma unroll
                for (int ni = 0; ni < NI; ++ni) fb[ni] = tr_frag(o[NA + 2 * ni], o[NA + 2 * ni + 1]);
            }
        }
#pragma unroll
        for (int q = 0; q < MI * NI; ++q) {
            acc[q / NI][q % NI] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[q / NI], fb[q % NI], acc[q / NI][q % NI], 0, 0, 0);
            if constexpr (FILL) {
                if (s < SPREAD && (q + 1) % EVERY == 0) {
                    const int g = s * D + (q + 1) / EVERY - 1;
                    if (g < GH) dma_blk_x<NW>(asrc[g] + ao, dst, g);
                    else dma_blk_x<NW>(bsrc[g - GH] + bo, dst + tile_bytes, g - GH);
                }
            }
        }
        if constexpr (FILL) {
            if (s < SPREAD) {
#pragma unroll
                for (int j = 0; j < D; ++j) {
                    if constexpr (!AT && !BT) {  // each DMA ahead of its MFMA: the first right after the barrier
                        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x008, EVERY, 0);
                    } else {
                        __builtin_amdgcn_sched_group_barrier(0x008, EVERY, 0);
                        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                    }
                }
            }
        }
    }
}

// The bf16 main loop: K steps of 64, two stages double buffered in 128 KiB,
// the window swizzle for K-contiguous operands.  The DMA instructions that
// fill the next stage are not issued in one burst after the barrier: each
// follows one MFMA of the first of the four 16-deep sub-steps (pinned with
// sched_group_barrier), so a wave blocked on a full vector-memory queue still
// has MFMAs of its own in flight and the two waves of a SIMD keep the matrix
// unit busy.  At the gate/up shape this is about 10% faster than the burst
// and 3.5% faster than spreading the DMAs over two sub-steps (over all four:
// 10% slower), the stage's loads then start as early as the barrier allows.
// With both operands MN-contiguous the two-sub-step spread stays 2% faster.
// With both operands K-contiguous (the forward GEMMs) each DMA goes ahead of
// its MFMA, the first one right after the barrier (gate/up 0.7-1.5% faster;
// the down dgrad, one MN-contiguous operand, 2.8% slower that way).  Either operand may be MN-contiguous (AT / BT select TOp):
// a K-contiguous operand's DMA moves 64 elements along its rows per step, an
// MN-contiguous one's 64 rows; the MFMA inputs, and so the results, are those
// of the same product with transposed copies.
// With zero == false the products are added to what acc holds (a K loop
// continued over another range of rows).
template <int WM, int WN, bool AT, bool BT>
__device__ __forceinline__ void gemm_mainloop_x(const typename OpOf<AT>::type &ak, const typename OpOf<BT>::type &bk,
                                                int nk, bool swiglu, char *lds, AccW<WM, WN> &acc, bool zero = true) {
    using WG = WaveGrid<WM, WN>;
    constexpr int MI = WG::MI, NI = WG::NI, NW = WG::NW;
    constexpr int BKT = 64, SW = 3;
    constexpr int tile_bytes = 256 * BKT * 2;
    constexpr int GH = tile_bytes / 1024 / NW;
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
    const int wm = wave / WN, wn = wave % WN;
    if (zero) {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[mi][ni][e] = 0.f;
    }
    if (nk <= 0) return;
    int brow[NI];  // block base (T) or this lane's row (K-contiguous) of each B block
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) brow[ni] = WG::brow(swiglu, wn, ni) + (BT ? 0 : (lane & 31));
    const int arow = wm * (MI * 32) + (AT ? 0 : (lane & 31));
    const uint16_t *asrc[GH], *bsrc[GH];
#pragma unroll
    for (int i = 0; i < GH; ++i) {
        if constexpr (AT) asrc[i] = dma_src_t<NW>(ak, i);
        else asrc[i] = dma_src_w<BKT, SW, NW>(ak, i);
        if constexpr (BT) bsrc[i] = dma_src_t<NW>(bk, i);
        else bsrc[i] = dma_src_w<BKT, SW, NW>(bk, i);
    }
    int64_t astep, bstep;  // elements per K step
    if constexpr (AT) astep = BKT * ak.ld;
    else astep = BKT;
    if constexpr (BT) bstep = BKT * bk.ld;
    else bstep = BKT;
    __syncthreads();  // the previous tile's epilogue may still read LDS
#pragma unroll
    for (int i = 0; i < GH; ++i) {
        dma_blk_x<NW>(asrc[i], lds, i);
        dma_blk_x<NW>(bsrc[i], lds + tile_bytes, i);
    }
    int slot = 0;
    for (int kt = 0; kt + 1 < nk; ++kt) {
        x_step<WM, WN, AT, BT, true, GH>(lds, slot, lane, arow, brow, asrc, bsrc, (int64_t)(kt + 1) * astep,
                                         (int64_t)(kt + 1) * bstep, acc);
        slot ^= 1;
    }
    x_step<WM, WN, AT, BT, false, GH>(lds, slot, lane, arow, brow, asrc, bsrc, 0, 0, acc);
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Tile ordering.
// ---------------------------------------------------------------------------

// Tile numbers fit in 32 bits (the host rejects larger shapes), so the
// divisions below are 32-bit ones: a 64-bit division is a long software
// sequence paid between every two tiles.

// Round-robin XCD placement: in each round of G = gridDim.x concurrent tiles,
// XCD x%8 gets a contiguous run of G/8 logical tiles, so tiles that share
// operands (same M tile, neighbouring N tiles) meet in one L2.
__device__ __forceinline__ int64_t logical_tile(int64_t it64) {
    const uint32_t it = (uint32_t)it64, G = gridDim.x;
    const uint32_t round = it / G, x = it - round * G;
    return (int64_t)(round * G + (x & 7) * (G >> 3) + (x >> 3));
}

// Grouped order inside a (mtiles x ntiles) grid: GM M tiles sweep all N tiles.
template <int GM>
__device__ __forceinline__ void grouped_mn(int64_t lid64, int mtiles, int ntiles, int &m, int &n) {
    const uint32_t lid = (uint32_t)lid64, per = (uint32_t)(GM * ntiles);
    const uint32_t g = lid / per, in = lid - g * per;
    const int first = (int)g * GM;
    const int gm = min(GM, mtiles - first);
    if (gm == GM) {  // a full group: constant divisor
        m = first + (int)(in % GM);
        n = (int)(in / GM);
    } else {
        m = first + (int)(in % (uint32_t)gm);
        n = (int)(in / (uint32_t)gm);
    }
}

__device__ __forceinline__ int expert_of(const int32_t *seg_off, int L, int row) {
    int lo = 0, hi = L;  // largest l with seg_off[l] <= row
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (seg_off[mid] <= row) lo = mid; else hi = mid;
    }
    return lo;
}

// Expert-aligned order over the 256-row M tiles of a whole table: tile lid
// falls in expert l's range [m0 * ntiles, (m0 + ml) * ntiles) as in the plain
// row-major order, and inside it the expert's M tiles sweep the N tiles as one
// group when there are at most 8 of them (else in groups of 4, the last one
// short).  The concurrent tiles of an XCD then read one expert's weight
// strips: a group never mixes two experts' B operands.  Used by the gate/up
// products (K = H), where it cuts the modelled L2 fetch of a balanced Kimi
// share by a fifth and measured 1% (bf16) and 4% (MXFP8) faster; the
// down-shaped products (K = I or 2I) measured 1-6% slower with it and keep
// grouped_mn<4>.
__device__ __forceinline__ void expert_mn(int64_t lid64, const int32_t *seg_off, int L, int ntiles, int &m, int &n) {
    const uint32_t lid = (uint32_t)lid64, nt = (uint32_t)ntiles;
    const int l = expert_of(seg_off, L, (int)(lid / nt) * 256);
    const int m0 = seg_off[l] / 256, ml = (seg_off[l + 1] - seg_off[l]) / 256;
    uint32_t i = lid - (uint32_t)m0 * nt;
    int g0 = 0, gm = ml;
    if (ml > 8) {
        const uint32_t g = i / (4u * nt);
        g0 = 4 * (int)g;
        gm = min(4, ml - g0);
        i -= g * 4u * nt;
    }
    m = m0 + g0 + (int)(i % (uint32_t)gm);
    n = (int)(i / (uint32_t)gm);
}

// ---------------------------------------------------------------------------
// Epilogues.
// ---------------------------------------------------------------------------

__device__ __forceinline__ float silu_f(float h) { return h * __builtin_amdgcn_rcpf(1.0f + __expf(-h)); }

// One 16-bit LDS write per value, chunks in place (read with SWZ = false).
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

// Staging of bf16 values for a WM x WN wave grid: wave (wm, wn) writes rows
// [wm*256/WM, (wm+1)*256/WM), all inside one 128-row half (one 64 KiB stage)
// of the 256-row staging tile.  Lanes 2k and 2k+1 hold adjacent columns; for
// two consecutive rows e, e+1 of an accumulator block they trade one value
// (one DPP exchange), so the even lane writes both columns of row e and the
// odd lane both columns of row e+1 as one dword: half the LDS writes of one
// 16-bit write per value, and no two lanes share a dword.  The 16-byte chunks of a staged row are permuted by XOR with
// 4 * stage_swz(row): the four rows one write instruction touches (r, r+1,
// r+4, r+5) then sit in four different 64-byte bank groups.  Readers find
// column chunk q of row r at chunk q ^ (4 * stage_swz(r)).
__device__ __forceinline__ int stage_swz(int row) { return (row & 1) | ((row >> 1) & 2); }

__device__ __forceinline__ float dpp_swap_pair(float v) {  // value of lane ^ 1
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}

template <int NC, int WM>
struct PairStageW {
    char *rowbase;
    int col0, sw, odd;
    __device__ __forceinline__ PairStageW(char *lds, int off, int wm, int lane, int col0_) {
        constexpr int rows_per_wave = 256 / WM;
        static_assert(rows_per_wave % 32 == 0, "row blocks of 32");
        const int r0 = wm * rows_per_wave, hi = lane >> 5;
        odd = lane & 1;
        rowbase = lds + (r0 >> 7) * kStageBytes + off + ((r0 & 127) + 4 * hi + odd) * NC * 2;
        col0 = col0_ + (lane & 30);
        sw = 4 * (odd | (hi << 1));
    }
    // v0, v1: this lane's values of rows e and e+1 (e even) of block (mi, c)
    __device__ __forceinline__ void put2(int mi, int e, int c, float v0, float v1) const {
        const float recv = dpp_swap_pair(odd ? v0 : v1);
        const uint32_t w = odd ? pack_bf2(recv, v1) : pack_bf2(v0, recv);
        const int col = col0 + c;
        *reinterpret_cast<uint32_t *>(rowbase + (mi * 32 + 8 * (e >> 2) + (e & 3)) * NC * 2 +
                                      (((col >> 3) ^ sw) << 4) + (col & 7) * 2) = w;
    }
};

// The combine of the tokens that have exactly one local route, done where
// their one output row is written: out[g] = bf16(w * Y[row]) for the route of
// token g placed at the row.  That is the same single fp32 product and
// rounding as the combine's one-term sum (combine_body starts from 0 and adds
// w Y with one fma), so out is bitwise what the combine would write.
// out == nullptr: none.
struct RowCombine {
    uint16_t *out;    // [tokens][ld]
    const int2 *tab;  // row -> (token, bits of its weight) if the token has one local route, else (-1, 0)
};

// One tile row's entry, loaded by thread t < 256 of the epilogue for row
// m0 + t before the tile is staged and put in LDS (ig, iw) after.
struct RowCombineRow {
    int2 e = make_int2(-1, 0);
    __device__ __forceinline__ void load(const RowCombine &rc, int64_t row) { e = rc.tab[row]; }
    __device__ __forceinline__ void publish(int *ig, float *iw, int t) const {
        ig[t] = e.x;
        iw[t] = __int_as_float(e.y);
    }
};

// 8 bf16 values times wv, each product rounded once to bf16.
__device__ __forceinline__ u32x4 scale_bf16x8(u32x4 v, float wv) {
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        o[e] = pack_bf2(fmaf(wv, __uint_as_float(v[e] << 16), 0.f), fmaf(wv, __uint_as_float(v[e] & 0xffff0000u), 0.f));
    return o;
}

// Copy of a staged 256 x NC bf16 area (chunks placed as PairStageW writes
// them, or in place with SWZ = false) to rows of dst; columns from ncols on
// (a multiple of 8) are not written.  With ig, a row whose ig[row] >= 0 goes
// to out[ig[row]] (columns n0 ..., row stride ld) times iw[row] instead
// (RowCombine).  A thread keeps one 16-byte column chunk
// for all its rows and issues a batch of LDS reads before the batch's stores
// (one LDS round trip per batch, not per chunk).  tt is the thread index
// passed through an empty asm by the caller: the addresses, the same for
// every tile, are then not hoisted out of the tile loop to stay live (and
// spill) across the next tile's K loop.
template <int NC, int THREADS, bool SWZ = true>
__device__ __forceinline__ void copy_staged(const char *area, uint16_t *dst, int64_t ld, int ncols, int tt,
                                            const int *ig = nullptr, const float *iw = nullptr,
                                            uint16_t *out = nullptr, int n0 = 0) {
    constexpr int CPR = NC / 8, RSTEP = THREADS / CPR, kIt = 256 / RSTEP, kBatch = 8;
    static_assert(kIt % kBatch == 0, "whole batches");
    const int q = tt % CPR, r0 = tt / CPR;
#pragma unroll
    for (int b = 0; b < kIt; b += kBatch) {
        u32x4 v[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const int row = r0 + (b + i) * RSTEP;
            v[i] = *reinterpret_cast<const u32x4 *>(area + (row >> 7) * kStageBytes + (row & 127) * (NC * 2) +
                                                    ((SWZ ? q ^ (4 * stage_swz(row)) : q) << 4));
        }
        if (q * 8 < ncols) {
#pragma unroll
            for (int i = 0; i < kBatch; ++i) {
                const int row = r0 + (b + i) * RSTEP;
                const int g = ig ? ig[row] : -1;
                if (g < 0)
                    *reinterpret_cast<u32x4 *>(dst + (int64_t)row * ld + q * 8) = v[i];
                else
                    *reinterpret_cast<u32x4 *>(out + (int64_t)g * ld + n0 + q * 8) = scale_bf16x8(v[i], iw[row]);
            }
        }
    }
}

__device__ __forceinline__ int opaque_tid() {
    int tt = threadIdx.x;
    asm volatile("" : "+v"(tt));
    return tt;
}

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
    const int tt = opaque_tid();
    copy_staged<128, WG::THREADS, false>(lds, Aout, ldA, 128, tt);
    if (HUg) {
        copy_staged<128, WG::THREADS, false>(lds + 32768, HUg, ldHU, 128, tt);
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
        copy_staged<128, WG::THREADS, false>(lds, HUu, ldHU, 128, tt);
    }
}

template <int WM, int WN>
__device__ __forceinline__ void epilogue_store_bf16_w(AccW<WM, WN> &acc, char *lds, uint16_t *dst, int64_t ld, int nvalid) {
    using WG = WaveGrid<WM, WN>;
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63, wm = wave / WN, wn = wave % WN;
    const PairStageW<256, WM> sg(lds, 0, wm, lane, wn * WG::NI * 32);
#pragma unroll
    for (int mi = 0; mi < WG::MI; ++mi) {
#pragma unroll
        for (int ni = 0; ni < WG::NI; ++ni)
#pragma unroll
            for (int e = 0; e < 16; e += 2) sg.put2(mi, e, ni * 32, acc[mi][ni][e], acc[mi][ni][e + 1]);
        __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    copy_staged<256, WG::THREADS>(lds, dst, ld, nvalid, opaque_tid());
}

// epilogue_store_bf16_w of a whole 256 x 256 tile at rows m0 ..., columns
// n0 ... of the row buffer, except that the rows of single-route tokens go to
// those tokens' outputs (RowCombine) instead of dst; tab: 2 KiB of LDS past
// the staged tile for their tokens and weights.
template <int WM, int WN>
__device__ __forceinline__ void epilogue_store_bf16_comb(AccW<WM, WN> &acc, char *lds, uint16_t *dst, int64_t ld,
                                                         const RowCombine &rc, int64_t m0, int n0, char *tab) {
    using WG = WaveGrid<WM, WN>;
    static_assert(WG::THREADS >= 256, "one thread per tile row");
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63, wm = wave / WN, wn = wave % WN;
    const bool comb = rc.out != nullptr;
    RowCombineRow rr;
    if (comb && t < 256) rr.load(rc, m0 + t);
    const PairStageW<256, WM> sg(lds, 0, wm, lane, wn * WG::NI * 32);
#pragma unroll
    for (int mi = 0; mi < WG::MI; ++mi) {
#pragma unroll
        for (int ni = 0; ni < WG::NI; ++ni)
#pragma unroll
            for (int e = 0; e < 16; e += 2) sg.put2(mi, e, ni * 32, acc[mi][ni][e], acc[mi][ni][e + 1]);
        __builtin_amdgcn_sched_barrier(0);
    }
    int *ig = reinterpret_cast<int *>(tab);
    float *iw = reinterpret_cast<float *>(tab + 1024);
    if (comb && t < 256) rr.publish(ig, iw, t);
    __syncthreads();
    if (comb)
        copy_staged<256, WG::THREADS>(lds, dst, ld, 256, opaque_tid(), ig, iw, rc.out, n0);
    else
        copy_staged<256, WG::THREADS>(lds, dst, ld, 256, opaque_tid());
}

// fp32 tile store of the rows < mvalid and columns < nvalid; with accumulate
// each element is added to what dst holds (one fp32 add per call, so a
// sequence of calls sums in call order).  The old values of one mi block are
// all loaded before any of its stores: interleaved load / store pairs through
// one pointer cannot be reordered by the compiler and would wait out a full
// memory latency per element.
template <int WM, int WN>
__device__ __forceinline__ void epilogue_store_f32_w(AccW<WM, WN> &acc, float *dst, int64_t ld, int mvalid, int nvalid,
                                                     bool accumulate = false) {
    using WG = WaveGrid<WM, WN>;
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63, wm = wave / WN, wn = wave % WN;
    float *base = dst + (int64_t)WG::row(wm, 0, 0, lane) * ld + wn * (WG::NI * 32) + (lane & 31);
    const int row0 = WG::row(wm, 0, 0, lane), col0 = wn * (WG::NI * 32) + (lane & 31);
#pragma unroll
    for (int mi = 0; mi < WG::MI; ++mi) {
        if (accumulate) {
            float old[WG::NI][16];
#pragma unroll
            for (int ni = 0; ni < WG::NI; ++ni)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int dr = mi * 32 + 8 * (e >> 2) + (e & 3);
                    const bool ok = row0 + dr < mvalid && col0 + ni * 32 < nvalid;
                    old[ni][e] = ok ? base[(int64_t)dr * ld + ni * 32] : 0.f;
                }
#pragma unroll
            for (int ni = 0; ni < WG::NI; ++ni)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[mi][ni][e] = old[ni][e] + acc[mi][ni][e];
        }
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

// The activation a as the down-dgrad epilogue reads it: load() fetches 8
// consecutive columns of one row (col a multiple of 8), at() unpacks value i
// of them where it is used.  Bf16 rows [rows][ld].
struct ARowsBf16 {
    const uint16_t *p;
    int64_t ld;
    using Raw = u32x4;
    __device__ __forceinline__ Raw load(int row, int col) const {
        return *reinterpret_cast<const u32x4 *>(p + (int64_t)row * ld + col);
    }
    __device__ __forceinline__ static float at(const Raw &v, int i) {
        return __uint_as_float((i & 1) ? (v[i >> 1] & 0xffff0000u) : (v[i >> 1] << 16));
    }
};

// Down-dgrad tile -> SwiGLU backward.  acc holds dA' = dO_d W2 for 256 rows
// and the 256 columns [n0, n0+256) of the I activations; with w the row's
// router weight, h, u the saved gate/up pre-activations and a the activation:
//   dA = w dA',  dh = dA u s (1 + h (1 - s)),  du = dA h s  (s = sigmoid(h)),
//   part[row][n0/256] = sum over the tile's columns of dA' a  (the router-
//   weight gradient's partial dot product, SonicMoE form).
// The fp32 tile goes through LDS in two 128-row halves (128 KiB each); then
// every thread takes 8 contiguous columns of one row, so A, h, u are read and
// dh, du written with 16-byte accesses, and the 32 threads of a row add their
// partial dots in a fixed butterfly (ascending columns inside a thread).
template <int WM, int WN, class ARows>
__device__ __forceinline__ void epilogue_swiglu_bwd_w(AccW<WM, WN> &acc, char *lds, const ARows &A,
                                                      const uint16_t *HU, const float *wrow, uint16_t *dHU,
                                                      float *part, int nparts, int I, int n0) {
    using WG = WaveGrid<WM, WN>;
    constexpr int NT = WG::THREADS;
    static_assert((128 * 32) % NT == 0, "every thread runs the same number of chunks");
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63, wm = wave / WN, wn = wave % WN;
    float *st = reinterpret_cast<float *>(lds);  // [128][256]
    const int ncols = min(256, I - n0);          // a multiple of 128
    const int64_t ld2 = 2ll * I;
    // this wave's rows all lie in one half; each lane writes at compile-time
    // offsets (< 64 KiB) from one base
    constexpr int rows_per_wave = 256 / WM;
    static_assert(rows_per_wave <= 128 && 128 % rows_per_wave == 0, "a wave's rows stay in one half");
    const int my_half = (wm * rows_per_wave) / 128;
    float *base = st + ((wm * rows_per_wave) % 128 + 4 * (lane >> 5)) * 256 + wn * (WG::NI * 32) + (lane & 31);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        __syncthreads();  // the main loop or the previous half is done with LDS
        if (my_half == half) {
#pragma unroll
            for (int mi = 0; mi < WG::MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < WG::NI; ++ni)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        base[(mi * 32 + 8 * (e >> 2) + (e & 3)) * 256 + ni * 32] = acc[mi][ni][e];
        }
        __syncthreads();
        for (int c = t; c < 128 * 32; c += NT) {
            const int rl = c >> 5, cc = (c & 31) * 8;
            const int row = 128 * half + rl;
            float dot = 0.f;
            if (cc < ncols) {
                const float wr = wrow[row];
                const float4 d0 = *reinterpret_cast<const float4 *>(st + rl * 256 + cc);
                const float4 d1 = *reinterpret_cast<const float4 *>(st + rl * 256 + cc + 4);
                const float dap[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
                const typename ARows::Raw av = A.load(row, n0 + cc);
                const u32x4 hv = *reinterpret_cast<const u32x4 *>(HU + (int64_t)row * ld2 + n0 + cc);
                const u32x4 uv = *reinterpret_cast<const u32x4 *>(HU + (int64_t)row * ld2 + I + n0 + cc);
                u32x4 dh, du;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    float rh[2], ru[2];
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const float a = ARows::at(av, 2 * k + j);
                        const float h = __uint_as_float(j ? (hv[k] & 0xffff0000u) : (hv[k] << 16));
                        const float u = __uint_as_float(j ? (uv[k] & 0xffff0000u) : (uv[k] << 16));
                        const float d = dap[2 * k + j];
                        const float dA = wr * d;
                        const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-h));
                        rh[j] = dA * u * sg * (1.0f + h * (1.0f - sg));
                        ru[j] = dA * h * sg;
                        dot = fmaf(d, a, dot);
                    }
                    dh[k] = pack_bf2(rh[0], rh[1]);
                    du[k] = pack_bf2(ru[0], ru[1]);
                }
                *reinterpret_cast<u32x4 *>(dHU + (int64_t)row * ld2 + n0 + cc) = dh;
                *reinterpret_cast<u32x4 *>(dHU + (int64_t)row * ld2 + I + n0 + cc) = du;
            }
#pragma unroll
            for (int off = 16; off >= 1; off >>= 1) dot += __shfl_xor(dot, off, 64);
            if ((c & 31) == 0) part[(int64_t)row * nparts + n0 / 256] = dot;
        }
    }
}

}  // namespace moe
