// MXFP8 routed experts ("Mixture-of-Kittens: A MoE Megakernel for GB300
// NVL72", section 5, mixed precision: the routed experts run in MXFP8 with
// the activation quantization fused into the dispatch loads, the grouped GEMMs
// and SwiGLU).
//
// Format (OCP Microscaling, the reading of "MXFP8"): blocks of 32 consecutive
// elements along the reduction dimension share an E8M0 scale
// 2^(floor(log2 amax) - 8), stored as a byte (exponent + 127, clamped to
// [-127, 127]; an all-zero block gets 0); each element is x / scale rounded to
// FP8 E4M3 (bias 7, subnormals, no infinities) to nearest, ties to even,
// saturating at +-448.  Codes are stored row-major [rows][K] and scale bytes
// [rows][K/32].
//
// GEMM: gfx950's v_mfma_scale_f32_32x32x64_f8f6f4 multiplies 32 x 64 blocks of
// E4M3 codes with one scale per lane.  Lane l holds row l % 32; its bytes
// 0-15 are 16 elements of the first 32-element K block of the instruction and
// bytes 16-31 16 elements of the second, the two lane halves splitting each
// block; lane l supplies the scale of block l / 32 of its row in the byte the
// op_sel immediate names (checked on the hardware with controlled inputs).
// A 256 x 256 tile with 128-deep K steps therefore moves exactly the bytes of
// the bf16 tile with 64-deep steps (the same DMA and LDS swizzle) for twice
// the flops.
#pragma once

#include "common.hpp"
#include "gemm.hpp"

namespace moe {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// E4M3 codes of four finite floats, packed in order into one word: nearest
// with ties to even, saturating at +-448.  gfx950 converts to the OCP E4M3
// format in hardware (round to nearest even, with subnormals); a value past
// 448 is clamped to 448 first, which is where saturating rounding takes it.
__device__ __forceinline__ float e4m3_clamp(float y) { return fminf(fmaxf(y, -448.0f), 448.0f); }

__device__ __forceinline__ uint32_t e4m3_encode4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(c), e4m3_clamp(d), w, true);
    return (uint32_t)w;
}

// Block exponent: floor(log2 amax) - 8 clamped to [-127, 127]; -127 for 0.
__device__ __forceinline__ int mx_block_exp(float amax) {
    if (!(amax > 0.0f)) return -127;
    const uint32_t b = __float_as_uint(amax);
    int e = (int)(b >> 23) - 127;
    if ((b >> 23) == 0) e = -127 - (__builtin_clz(b & 0x7fffffu) - 9);  // fp32 subnormal
    const int se = e - 8;
    return se < -127 ? -127 : (se > 127 ? 127 : se);
}

// Codes of 32 values v (fp32) into 8 words, with the block's scale byte.
__device__ __forceinline__ uint32_t mx_quantize32(const float (&v)[32], uint32_t (&w)[8]) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const int se = mx_block_exp(amax);
#pragma unroll
    for (int k = 0; k < 8; ++k)
        w[k] = e4m3_encode4(__builtin_amdgcn_ldexpf(v[4 * k], -se), __builtin_amdgcn_ldexpf(v[4 * k + 1], -se),
                            __builtin_amdgcn_ldexpf(v[4 * k + 2], -se), __builtin_amdgcn_ldexpf(v[4 * k + 3], -se));
    return (uint32_t)(se + 127);
}

// Row-wise quantization of bf16 [rows][K]: block b (of rows * K / 32) per call.
__device__ __forceinline__ void mx_quantize_block_bf16(const uint16_t *src, int K, uint8_t *q, uint8_t *s,
                                                       int64_t b) {
    const int64_t row = b / (K / 32), blk = b % (K / 32);
    const u32x4 *in = reinterpret_cast<const u32x4 *>(src + row * K + blk * 32);
    float v[32];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const u32x4 x = in[c];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            v[8 * c + 2 * d] = __uint_as_float(x[d] << 16);
            v[8 * c + 2 * d + 1] = __uint_as_float(x[d] & 0xffff0000u);
        }
    }
    uint32_t w[8];
    const uint32_t sb = mx_quantize32(v, w);
    u32x4 *out = reinterpret_cast<u32x4 *>(q + row * K + blk * 32);
    out[0] = u32x4{w[0], w[1], w[2], w[3]};
    out[1] = u32x4{w[4], w[5], w[6], w[7]};
    s[row * (K / 32) + blk] = (uint8_t)sb;
}

// Scale rows of an MX operand window, parallel to a KOp: row i's scale bytes
// start at (rows ? gathered row : (i < 128 ? lo : hi) + (i & 127) * ld).
struct SOp {
    const uint8_t *lo, *hi;
    int64_t ld;  // bytes per row = K / 32
    const moe_src *rows;
    const uint8_t *src;
    int32_t np;
};

// A padding row of a gathered operand reads zero codes (the zero row), so any
// scale serves it: it takes source row 0's.
__device__ __forceinline__ const uint8_t *mx_scale_row(const SOp &op, int row) {
    const uint8_t *base;
    if (op.rows) {
        const uint2 s = reinterpret_cast<const uint2 *>(op.rows)[row];
        const int64_t src_row = (int32_t)s.x >= 0 ? (int64_t)(int32_t)s.x * op.np + (int32_t)s.y : 0;
        base = op.src + src_row * op.ld;
    } else {
        base = (row < 128 ? op.lo : op.hi) + (int64_t)(row & 127) * op.ld;
    }
    return base;
}

// dma_src_w for an MX operand tile, kept out of line: inlined into the MX
// main loop together with a gathered operand, its branch makes this
// compiler's CFG simplification crash.  It runs once per tile and lane.
template <int NW>
__device__ __attribute__((noinline)) const uint16_t *mx_dma_src(const KOp &op, int i) {
    return dma_src_w<64, 3, NW>(op, i);
}

// The same for an operand read in place (never gathered), inline: the
// out-of-line call takes the operand through scratch memory, and reading it
// back waits for every vector-memory operation in flight.
template <int NW>
__device__ __forceinline__ const uint16_t *mx_dma_src_plain(const KOp &op, int i) {
    return dma_src_w<64, 3, NW>(KOp{op.lo, op.hi, op.ld, nullptr, nullptr, 0}, i);
}

template <int OPSEL>
__device__ __forceinline__ f32x16 mfma_mx(const i32x8 &a, const i32x8 &b, const f32x16 &c, uint32_t sa, uint32_t sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, OPSEL, (int)sa, OPSEL, (int)sb);
}

// Two 16-byte chunks of an operand tile row as one MFMA fragment.
__device__ __forceinline__ i32x8 mx_frag(const char *tile, int row, int c0, int c1) {
    const u32x4 x = *reinterpret_cast<const u32x4 *>(tile + tile_off_t<64, 3>(row, c0));
    const u32x4 y = *reinterpret_cast<const u32x4 *>(tile + tile_off_t<64, 3>(row, c1));
    return i32x8{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
}

// One 64-deep sub-step S (0 or 1) of an MX step: fragment reads and the
// MI x NI MFMAs (op_sel S*2 picks this sub-step's scale byte); in sub-step 0
// one DMA instruction of the next stage follows every EVERY MFMAs.
template <int WM, int WN, int S, int EVERY, int GH, bool FILL>
__device__ __forceinline__ void mx_substep(const char *stage, int arow, const int (&brow)[WaveGrid<WM, WN>::NI], int h,
                                           const uint32_t (&ca)[WaveGrid<WM, WN>::MI],
                                           const uint32_t (&cb)[WaveGrid<WM, WN>::NI], AccW<WM, WN> &acc,
                                           const uint16_t *const (&asrc)[GH], const uint16_t *const (&bsrc)[GH],
                                           int k0, char *dst) {
    using WG = WaveGrid<WM, WN>;
    constexpr int MI = WG::MI, NI = WG::NI, NW = WG::NW;
    constexpr int tile_bytes = 256 * 128;
    i32x8 fa[MI], fb[NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) fa[mi] = mx_frag(stage, arow + mi * 32, 4 * S + h, 4 * S + 2 + h);
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) fb[ni] = mx_frag(stage + tile_bytes, brow[ni], 4 * S + h, 4 * S + 2 + h);
#pragma unroll
    for (int q = 0; q < MI * NI; ++q) {
        const int mi = q / NI, ni = q % NI;
        acc[mi][ni] = mfma_mx<2 * S>(fa[mi], fb[ni], acc[mi][ni], ca[mi], cb[ni]);
        if constexpr (S == 0 && FILL) {
            if ((q + 1) % EVERY == 0) {
                const int g = (q + 1) / EVERY - 1;
                const bool isa = g < GH;
                dma_blk_w<64, NW>(isa ? asrc[g] : bsrc[g - GH], k0, isa ? dst : dst + tile_bytes, isa ? g : g - GH);
            }
        }
    }
    if constexpr (S == 0 && FILL) {
#pragma unroll
        for (int j = 0; j < 2 * GH; ++j) {
            __builtin_amdgcn_sched_group_barrier(0x008, EVERY, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
    }
}

// LDS of an MX GEMM: two 64 KiB stages of operand codes, then the scale
// words in two buffers of SG-step groups: [2][A, B][256 rows][SG] u32.
constexpr int kMxScaleBytes = 2 * 2 * 256 * 16;
constexpr int kMxLds = kGemmLds + kMxScaleBytes;

// Scale group buffer b (0/1) of operand o (0 = A, 1 = B).
template <int SG>
__device__ __forceinline__ char *mx_scale_buf(char *lds, int b, int o) {
    return lds + kGemmLds + b * (2 * 256 * 4 * SG) + o * (256 * 4 * SG);
}

// This wave's gather DMA of one scale group: lane = operand row (waves 0-3
// the A rows 64w + lane, waves 4-7 the B rows), SG consecutive step words.
template <int SG>
__device__ __forceinline__ void mx_scale_dma(const uint32_t *ssrc, int step, char *lds, int b) {
    const int w = threadIdx.x >> 6;
    const void *src = reinterpret_cast<const void *>(ssrc + step);
    lds_void_t *dst = (lds_void_t *)(mx_scale_buf<SG>(lds, b, w >> 2) + (w & 3) * (64 * 4 * SG));
    if constexpr (SG == 4)
        __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
    else
        __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
}

// This lane's scale words of step kt (A rows arow + 32 mi, B rows brow[ni]),
// shifted so that op_sel 0 / 2 pick its lane half's block of each sub-step.
template <int WM, int WN, int SG>
__device__ __forceinline__ void mx_read_scales(char *lds, int kt, int arow, const int (&brow)[WaveGrid<WM, WN>::NI],
                                               int h, uint32_t (&ca)[WaveGrid<WM, WN>::MI],
                                               uint32_t (&cb)[WaveGrid<WM, WN>::NI]) {
    const int grp = kt / SG, j = kt % SG;
    const uint32_t *swa = reinterpret_cast<const uint32_t *>(mx_scale_buf<SG>(lds, grp & 1, 0));
    const uint32_t *swb = reinterpret_cast<const uint32_t *>(mx_scale_buf<SG>(lds, grp & 1, 1));
#pragma unroll
    for (int mi = 0; mi < WaveGrid<WM, WN>::MI; ++mi) ca[mi] = swa[(arow + mi * 32) * SG + j] >> (8 * h);
#pragma unroll
    for (int ni = 0; ni < WaveGrid<WM, WN>::NI; ++ni) cb[ni] = swb[brow[ni] * SG + j] >> (8 * h);
}

// One 128-deep K step kt on stage `slot`: wait for the stage (TAIL: the
// caller's prologue or the previous step did); on the first step of an
// SG-step group that has a successor, fetch that group's scale words (their
// buffer was last read in the previous group, which every wave has left by
// that barrier); with FILL spread the next stage's DMA over sub-step 0 (and
// with TAIL end with the wait and barrier for it).  The scale fetch comes
// before the sub-steps so that its branch does not split them: the MFMA /
// DMA interleave is pinned only within one basic block.  ca / cb hold this
// step's scale words on entry when SG > 1 (read one step ahead, between the
// sub-steps: step kt + 1's group is in LDS since step kt's barrier) and the
// next step's on return; with SG = 1 the next group is this step's DMA, so
// the words are read after the barrier.
template <int WM, int WN, int EVERY, int GH, int SG, bool FILL, bool TAIL>
__device__ __forceinline__ void mx_step(char *lds, int slot, int kt, int nk, int arow,
                                        const int (&brow)[WaveGrid<WM, WN>::NI], int h, const uint32_t *ssrc,
                                        uint32_t (&ca)[WaveGrid<WM, WN>::MI], uint32_t (&cb)[WaveGrid<WM, WN>::NI],
                                        AccW<WM, WN> &acc, const uint16_t *const (&asrc)[GH],
                                        const uint16_t *const (&bsrc)[GH]) {
    using WG = WaveGrid<WM, WN>;
    constexpr int MI = WG::MI, NI = WG::NI;
    constexpr int stage_bytes = 2 * 256 * 128;
    if constexpr (!TAIL) wait_vm_barrier<0>();
    if (FILL && kt % SG == 0 && kt + SG < nk) mx_scale_dma<SG>(ssrc, kt + SG, lds, (kt / SG + 1) & 1);
    char *dst = lds + (slot ^ 1) * stage_bytes;
    const char *stage = lds + slot * stage_bytes;
    if constexpr (SG == 1) mx_read_scales<WM, WN, SG>(lds, kt, arow, brow, h, ca, cb);
    mx_substep<WM, WN, 0, EVERY, GH, FILL>(stage, arow, brow, h, ca, cb, acc, asrc, bsrc, (kt + 1) * 64, dst);
    uint32_t na[MI], nb[NI];
    if constexpr (SG > 1 && FILL) mx_read_scales<WM, WN, SG>(lds, kt + 1, arow, brow, h, na, nb);
    mx_substep<WM, WN, 1, EVERY, GH, FILL>(stage, arow, brow, h, ca, cb, acc, asrc, bsrc, (kt + 1) * 64, dst);
    if constexpr (SG > 1 && FILL) {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) ca[mi] = na[mi];
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) cb[ni] = nb[ni];
    }
    if constexpr (FILL && TAIL) {
        __builtin_amdgcn_sched_barrier(0);  // every MFMA of the step issued before the wave waits
        wait_vm_barrier<0>();
    }
}

// MX main loop: 256 x 256 tile, K steps of 128 codes (one [256][128]-byte
// operand tile each, the bf16 loop's DMA and swizzle), two 64-deep MFMA
// sub-steps per step, double buffered.  ak/bk address the codes as 16-bit
// units (ld = K / 2); as/bs the scale bytes.  Scale words reach LDS by a
// gather DMA (lane = operand row, SG steps' words per lane) rather than by
// per-lane loads: a 4-byte load per lane, row and step costs three times the
// vector-memory requests of the operand tiles.  SG = 4 (16-byte lanes) needs
// nk % 4 == 0 and 16-byte aligned scale rows, SG = 1 4-byte aligned ones.
// Needs 8 waves (4 x 64 rows per operand); lds holds kMxLds bytes.
//
// PLAIN: both operands are read in place (no gathered rows): their DMA
// addresses are computed inline, each step's wait sits at the end of the
// step before it (the prologue's for step 0), and pre may be set.
//
// pre (PLAIN only): step 0's operand and scale DMAs were issued by
// mx_prefetch_stage0, followed by at least 64 more vector-memory operations
// of this wave (a previous tile's stores).  A wave's vector-memory
// operations complete in issue order, so once no more than the last 63 are
// in flight those DMAs have landed: the prologue waits for vmcnt 63, not for
// the stores to be written.  Read in the prologue only, so the loop carries
// no flag.
template <int WM, int WN, int SG, bool PLAIN = false>
__device__ __forceinline__ void gemm_mainloop_mx(const KOp &ak, const KOp &bk, const SOp &as, const SOp &bs, int nk,
                                                 bool swiglu, char *lds, AccW<WM, WN> &acc, bool pre = false) {
    using WG = WaveGrid<WM, WN>;
    constexpr int MI = WG::MI, NI = WG::NI, NW = WG::NW;
    static_assert(NW == 8, "one scale DMA per wave: waves 0-3 A rows, 4-7 B rows");
    static_assert(SG == 1 || SG == 4, "scale DMA lanes of 4 or 16 bytes");
    constexpr int tile_bytes = 256 * 128;
    constexpr int GH = tile_bytes / 1024 / NW;
    constexpr int G = 2 * GH;
    static_assert((MI * NI) % G == 0, "DMA slots in one sub-step");
    constexpr int EVERY = MI * NI / G;
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
    const int wm = wave / WN, wn = wave % WN, h = lane >> 5;
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
    const uint16_t *asrc[GH], *bsrc[GH];
#pragma unroll
    for (int i = 0; i < GH; ++i) {
        asrc[i] = PLAIN ? mx_dma_src_plain<NW>(ak, i) : mx_dma_src<NW>(ak, i);
        bsrc[i] = PLAIN ? mx_dma_src_plain<NW>(bk, i) : mx_dma_src<NW>(bk, i);
    }
    const uint32_t *ssrc = reinterpret_cast<const uint32_t *>(
        wave < 4 ? mx_scale_row(as, 64 * wave + lane) : mx_scale_row(bs, 64 * (wave - 4) + lane));
    if (!(PLAIN && pre)) {
        __syncthreads();  // the previous tile's epilogue may still read LDS
        mx_scale_dma<SG>(ssrc, 0, lds, 0);
#pragma unroll
        for (int i = 0; i < GH; ++i) {
            dma_blk_w<64, NW>(asrc[i], 0, lds, i);
            dma_blk_w<64, NW>(bsrc[i], 0, lds + tile_bytes, i);
        }
        if constexpr (PLAIN) wait_vm_barrier<0>();
    } else {
        wait_vm_barrier<63>();
    }
    uint32_t ca[MI], cb[NI];
    if constexpr (SG > 1) {  // step 0's words: wait for the first group
        if constexpr (!PLAIN) wait_vm_barrier<0>();
        mx_read_scales<WM, WN, SG>(lds, 0, arow, brow, h, ca, cb);
    }
    int slot = 0;
    for (int kt = 0; kt + 1 < nk; ++kt) {
        mx_step<WM, WN, EVERY, GH, SG, true, PLAIN>(lds, slot, kt, nk, arow, brow, h, ssrc, ca, cb, acc, asrc, bsrc);
        slot ^= 1;
    }
    mx_step<WM, WN, EVERY, GH, SG, false, PLAIN>(lds, slot, nk - 1, nk, arow, brow, h, ssrc, ca, cb, acc, asrc, bsrc);
    __syncthreads();
}

// Step 0's DMAs of an MX tile whose operands are read in place (operands and
// scale words), issued ahead of gemm_mainloop_mx(..., pre = true) on the
// same operands; LDS must be free (after a main loop's closing barrier, with
// no LDS use since).
template <int WM, int WN, int SG>
__device__ __forceinline__ void mx_prefetch_stage0(const KOp &ak, const KOp &bk, const SOp &as, const SOp &bs,
                                                   char *lds) {
    constexpr int NW = WaveGrid<WM, WN>::NW;
    constexpr int tile_bytes = 256 * 128;
    constexpr int GH = tile_bytes / 1024 / NW;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const uint32_t *ssrc = reinterpret_cast<const uint32_t *>(
        wave < 4 ? mx_scale_row(as, 64 * wave + lane) : mx_scale_row(bs, 64 * (wave - 4) + lane));
    mx_scale_dma<SG>(ssrc, 0, lds, 0);
#pragma unroll
    for (int i = 0; i < GH; ++i) {
        dma_blk_w<64, NW>(mx_dma_src_plain<NW>(ak, i), 0, lds, i);
        dma_blk_w<64, NW>(mx_dma_src_plain<NW>(bk, i), 0, lds + tile_bytes, i);
    }
}

// Gate/up tile -> a = silu(gate) * up (256 rows x 128 columns), MX-quantized
// along the columns: codes Aq[row][0..128) and 4 scale bytes per row.  The fp32
// tile goes through LDS (128 KiB); then every thread quantizes whole 32-column
// blocks of a row.  With HUg set, h and u are also stored as bf16 (the
// backward's saved pre-activations): gate columns at HUg, up at HUu.
template <int WM, int WN>
__device__ __forceinline__ void epilogue_swiglu_mx(AccW<WM, WN> &acc, char *lds, uint8_t *Aq, int64_t ldq,
                                                   uint8_t *As, int64_t lds_row, uint16_t *HUg, uint16_t *HUu,
                                                   int64_t ldHU) {
    using WG = WaveGrid<WM, WN>;
    constexpr int NT = WG::THREADS, half = WG::NI / 2;
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63, wm = wave / WN, wn = wave % WN;
    float *st = reinterpret_cast<float *>(lds);  // [256][128]
    __syncthreads();
    float *base = st + (wm * (WG::MI * 32) + 4 * (lane >> 5)) * 128 + wn * (half * 32) + (lane & 31);
#pragma unroll
    for (int mi = 0; mi < WG::MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < half; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                base[(mi * 32 + 8 * (e >> 2) + (e & 3)) * 128 + ni * 32] =
                    silu_f(acc[mi][ni][e]) * acc[mi][ni + half][e];
    __syncthreads();
    for (int b = t; b < 256 * 4; b += NT) {
        const int row = b >> 2, blk = b & 3;
        float v[32];
        const float4 *src = reinterpret_cast<const float4 *>(st + row * 128 + blk * 32);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float4 x = src[c];
            v[4 * c] = x.x;
            v[4 * c + 1] = x.y;
            v[4 * c + 2] = x.z;
            v[4 * c + 3] = x.w;
        }
        uint32_t w[8];
        const uint32_t sb = mx_quantize32(v, w);
        u32x4 *out = reinterpret_cast<u32x4 *>(Aq + row * ldq + blk * 32);
        out[0] = u32x4{w[0], w[1], w[2], w[3]};
        out[1] = u32x4{w[4], w[5], w[6], w[7]};
        As[row * lds_row + blk] = (uint8_t)sb;
    }
    if (HUg) {
        const LaneStageW<128, WM> sg(lds, 0, wm, lane, wn * half * 32), su(lds, 32768, wm, lane, wn * half * 32);
        __syncthreads();  // every thread is done reading the fp32 tile
#pragma unroll
        for (int mi = 0; mi < WG::MI; ++mi) {
#pragma unroll
            for (int ni = 0; ni < half; ++ni)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    sg.put(mi, e, ni * 32, acc[mi][ni][e]);
                    su.put(mi, e, ni * 32, acc[mi][ni + half][e]);
                }
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
        const int tt = opaque_tid();
        copy_staged<128, NT, false>(lds, HUg, ldHU, 128, tt);
        copy_staged<128, NT, false>(lds + 32768, HUu, ldHU, 128, tt);
    }
}

}  // namespace moe
