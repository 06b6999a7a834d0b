// MXFP8 backward of the routed experts ("Beyond Peak TFLOPs" section 3 and
// the Mixture-of-Kittens notes section 6 report an MXFP8 backward; section 5
// of the notes fuses the quantization into the loads, the grouped GEMMs and
// SwiGLU).
//
// Every product of the backward takes MX operands blocked along its own
// reduction dimension, quantized from the value the bf16 backward uses there:
//   down dgrad     dA' = dO_d W2[l]     over H:  dO_d rows along H (row
//                  quantization), W2[l] columns along H (weights quantized
//                  transposed once per update, [L][I][H]);
//   gate/up dgrad  dXd = dHU W13[l]     over 2I: dHU rows along 2I, W13[l]
//                  columns along 2I ([L][H][2I]);
//   dW2[l]  = (w dO_d)^T a              over the expert's rows;
//   dW13[l] = dHU^T Xd                  over the expert's rows:
// the four row-dimension operands are quantized along the rows in blocks of
// 32 dispatched rows and stored transposed per expert segment ([C][rows of
// the segment]), so every MX product reads both operands K-contiguous through
// the forward's scaled-MFMA loop.
// The SwiGLU backward and dw stay those of the bf16 path, with a read from
// the forward's MX codes (exactly: an E4M3 value times a power of two is an
// fp32 number).
#pragma once

#include "common.hpp"
#include "gemm.hpp"
#include "layer.hpp"
#include "mx.hpp"

namespace moe {

// Value of an E4M3 code (s.eeee.mmm, bias 7, subnormals; the encoder never
// writes the NaN codes) times 2^(sbyte - 127).  Exact in fp32: the smallest
// magnitude, 2^-9 * 2^-127, is above fp32's smallest subnormal.
__device__ __forceinline__ float mx_decode(uint32_t code, uint32_t sbyte) {
    const uint32_t e = (code >> 3) & 15u, m = code & 7u;
    const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
    const float v = __builtin_amdgcn_ldexpf(mag, (int)sbyte - 127);
    return (code & 0x80u) ? -v : v;
}

// The activation a as the down-dgrad epilogue reads it (the interface of
// ARowsBf16), from MX codes [rows][ld] and scale bytes [rows][ld/32]: 8
// codes and their block's scale byte.
struct ARowsMx {
    const uint8_t *q, *s;
    int64_t ld;
    struct Raw {
        uint2 c;
        uint32_t sb;
    };
    __device__ __forceinline__ Raw load(int row, int col) const {
        return Raw{*reinterpret_cast<const uint2 *>(q + (int64_t)row * ld + col), s[(int64_t)row * (ld / 32) + col / 32]};
    }
    __device__ __forceinline__ static float at(const Raw &v, int i) {
        return mx_decode(((i < 4 ? v.c.x : v.c.y) >> (8 * (i & 3))) & 0xffu, v.sb);
    }
};

// ---------------------------------------------------------------------------
// Quantization passes.
// ---------------------------------------------------------------------------

// Column quantization: the codes of column c of a [R][C] source in blocks
// of 32 consecutive rows.  Outputs: without seg_off, out[c][r] with ldq codes
// per c (scale bytes [c][r / 32]), batch b at b * out_bstride codes
// (b * out_bstride / 32 scale bytes); with seg_off (the dispatched rows of a
// table), segment-major: local expert l's rows [S, S + n) (S = seg_off[l],
// n = seg_off[l+1] - S) form a [C][n] block at code C * S, scales [C][n / 32]
// at byte C * S / 32, so the weight-gradient tiles of one expert read compact
// rows.  Sources:
//   bf16 rows src + r * ld (+ b * in_bstride), or, with phi, row r taken from
//   source row part * Np + tok of phi[r] (padding rows zero);
//   or MX codes srcq / srcs [R][C] (+ [R][C/32]), decoded exactly.
// With wrow (bf16 sources), column codes are taken of bf16(value * wrow[r])
// (an fp32 product rounded once, as the bf16 backward's dO_d w), and with rq
// the same pass also writes the row codes of the unscaled values ([R][C],
// scales rs [R][C/32]): one read of the source for both encodings.
// Rows at or past *nrows (if given, else R) read as zero; only whole blocks
// below the row count (rounded up to 32) are written.
struct ColQArgs {
    const uint16_t *src;
    int64_t ld, in_bstride;
    const moe_src *phi;
    int32_t Np;
    const uint8_t *srcq, *srcs;
    const int32_t *nrows;
    const int32_t *seg_off;
    int L;
    const float *wrow;
    uint8_t *rq, *rs;
    int64_t R;
    int C, batch;
    uint8_t *q, *s;
    int64_t ldq, out_bstride;
};

constexpr int kColqRows = 128, kColqCols = 64, kColqThreads = 256;
constexpr int kColqLd = kColqRows + 4;  // floats per staged column (float4-aligned)
constexpr int kColqLds = kColqCols * kColqLd * 4;

__device__ __forceinline__ void mx_colq_body(const ColQArgs &a, float *st) {
    const int64_t rows = a.nrows ? (int64_t)(*a.nrows) : a.R;
    const int64_t rt = (rows + kColqRows - 1) / kColqRows, ct = (a.C + kColqCols - 1) / kColqCols;
    const int64_t per = rt * ct, total = per * a.batch;
    const int t = threadIdx.x;
    for (int64_t it = blockIdx.x; it < total; it += gridDim.x) {
        const int64_t b = it / per, in = it % per;
        const int64_t r0 = (in / ct) * kColqRows;
        const int c0 = (int)(in % ct) * kColqCols;
        __syncthreads();  // the previous tile's readers are done with st
        if (a.srcq) {
            // 128 rows x 64 codes: 16 codes (one half block) per chunk, two
            // chunks per thread, both loads issued before either is decoded
            constexpr int N = kColqRows * 4 / kColqThreads;
            const int cc = (t & 3) * 16;
            u32x4 x[N];
            uint32_t sb[N];
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const int64_t r = r0 + (t >> 2) + i * (kColqThreads / 4);
                const bool ok = r < rows && c0 + cc < a.C;
                x[i] = ok ? *reinterpret_cast<const u32x4 *>(a.srcq + r * a.C + c0 + cc) : u32x4{0u, 0u, 0u, 0u};
                sb[i] = ok ? a.srcs[r * (a.C / 32) + (c0 + cc) / 32] : 0u;
            }
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const int row = (t >> 2) + i * (kColqThreads / 4);
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    st[(cc + j) * kColqLd + row] = mx_decode((x[i][j >> 2] >> (8 * (j & 3))) & 0xffu, sb[i]);
            }
        } else {
            // 128 rows x 64 bf16: 8 values per 16-byte chunk, four chunks per
            // thread (rows t/8 + 32 i, the same 8 columns); the row sources
            // (a table lookup when gathered) and then all four loads are
            // issued before any value is used
            constexpr int N = kColqRows * 8 / kColqThreads;
            const int cc = (t & 7) * 8;
            const uint16_t *p[N];
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const int64_t r = r0 + (t >> 3) + i * (kColqThreads / 8);
                p[i] = nullptr;
                if (r < rows && c0 + cc < a.C) {
                    if (a.phi) {
                        const int2 e = reinterpret_cast<const int2 *>(a.phi)[r];
                        if (e.x >= 0) p[i] = a.src + ((int64_t)e.x * a.Np + e.y) * a.ld + c0 + cc;
                    } else {
                        p[i] = a.src + b * a.in_bstride + r * a.ld + c0 + cc;
                    }
                }
            }
            u32x4 x[N];
            float wr[N];
#pragma unroll
            for (int i = 0; i < N; ++i) {
                x[i] = p[i] ? *reinterpret_cast<const u32x4 *>(p[i]) : u32x4{0u, 0u, 0u, 0u};
                const int64_t r = r0 + (t >> 3) + i * (kColqThreads / 8);
                wr[i] = a.wrow && r < rows ? a.wrow[r] : 0.f;
            }
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const int row = (t >> 3) + i * (kColqThreads / 8);
                const int64_t r = r0 + row;
                float v[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v[2 * j] = __uint_as_float(x[i][j] << 16);
                    v[2 * j + 1] = __uint_as_float(x[i][j] & 0xffff0000u);
                }
                if (a.rq) {
                    // row codes: lanes with t & 3 = 0 .. 3 (adjacent lanes of
                    // one wave) hold one 32-column block of the row
                    float am = 0.f;
#pragma unroll
                    for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(v[j]));
                    am = fmaxf(am, __shfl_xor(am, 1, 64));
                    am = fmaxf(am, __shfl_xor(am, 2, 64));
                    const int se = mx_block_exp(am);
                    float y[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) y[j] = __builtin_amdgcn_ldexpf(v[j], -se);
                    const uint32_t w0 = e4m3_encode4(y[0], y[1], y[2], y[3]);
                    const uint32_t w1 = e4m3_encode4(y[4], y[5], y[6], y[7]);
                    if (r < rows && c0 + cc < a.C) {
                        *reinterpret_cast<uint2 *>(a.rq + r * a.C + c0 + cc) = make_uint2(w0, w1);
                        if ((t & 3) == 0) a.rs[r * (a.C / 32) + (c0 + cc) / 32] = (uint8_t)(se + 127);
                    }
                }
                if (a.wrow) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) v[j] = __uint_as_float((uint32_t)f2bf(v[j] * wr[i]) << 16);
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) st[(cc + j) * kColqLd + row] = v[j];
            }
        }
        __syncthreads();
        // where column c0 + c of rows [r0, r0 + 128) goes: a [C][ld] block at
        // `base` whose first row is `first` (a tile lies inside one segment:
        // segments are multiples of 256 rows)
        int64_t base = b * a.out_bstride, ld = a.ldq, first = 0;
        if (a.seg_off) {
            const int l = expert_of(a.seg_off, a.L, (int)r0);
            first = a.seg_off[l];
            ld = a.seg_off[l + 1] - first;
            base = (int64_t)a.C * first;
        }
        // one 32-row block of one column per thread
        const int c = t >> 2, blk = t & 3;
        const int64_t rb = r0 + 32 * blk;
        if (c0 + c < a.C && rb < rows) {
            float v[32];
            const float4 *src = reinterpret_cast<const float4 *>(st + c * kColqLd + 32 * blk);
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const float4 x = src[m];
                v[4 * m] = x.x;
                v[4 * m + 1] = x.y;
                v[4 * m + 2] = x.z;
                v[4 * m + 3] = x.w;
            }
            uint32_t w[8];
            const uint32_t sb = mx_quantize32(v, w);
            const int64_t o = base + (int64_t)(c0 + c) * ld + (rb - first);
            reinterpret_cast<u32x4 *>(a.q + o)[0] = u32x4{w[0], w[1], w[2], w[3]};
            reinterpret_cast<u32x4 *>(a.q + o)[1] = u32x4{w[4], w[5], w[6], w[7]};
            a.s[o / 32] = (uint8_t)sb;
        }
    }
}

// ---------------------------------------------------------------------------
// MX backward GEMMs (256 x 256 tiles, the forward's scaled-MFMA loop).
// ---------------------------------------------------------------------------

struct MxBwdArgs {
    const uint8_t *dOq, *dOs;      // dO_d rows along H: [cap][H], [cap][H/32]
    const uint8_t *W2tq, *W2ts;    // W2 columns along H: [L][I][H], [L][I][H/32]
    const uint8_t *Aq, *As;        // the forward's a: [cap][I], [cap][I/32]
    const uint16_t *HU;            // the forward's h, u (bf16 [cap][2I])
    const float *wrow;             // router weight per dispatched row
    uint16_t *dHU;                 // bf16 [cap][2I]
    float *part;                   // dw partials [cap][nparts]
    const uint8_t *dHUq, *dHUs;    // dHU rows along 2I: [cap][2I], [cap][2I/32]
    const uint8_t *W13tq, *W13ts;  // W13 columns along 2I: [L][H][2I], [L][H][2I/32]
    uint16_t *dXd;                 // bf16 [cap][H]
    const int32_t *seg_off;
    int L, H, I, nparts;
};

// B2 with MX operands: dA' = dOq W2t[l]^T over H, SwiGLU backward and dw
// partials in the epilogue.  A last column tile of 128 (I % 256 == 128)
// reads its B rows 0-127 twice; the epilogue keeps the valid columns.
template <int SG>
__device__ __forceinline__ void mx_bwd_down_tile(const MxBwdArgs &a, int mt, int nt, char *lds) {
    const int H = a.H, I = a.I;
    const int m0 = mt * kBM, n0 = nt * 256;
    const int l = expert_of(a.seg_off, a.L, m0);
    const uint8_t *gq = a.dOq + (int64_t)m0 * H;
    const uint8_t *gs = a.dOs + (int64_t)m0 * (H / 32);
    const KOp ak{as_u16(gq), as_u16(gq + 128ll * H), H / 2, nullptr, nullptr, 0};
    const SOp as{gs, gs + 128ll * (H / 32), H / 32, nullptr, nullptr, 0};
    const int hi = I - n0 > 128 ? 128 : 0;
    const uint8_t *wq = a.W2tq + ((int64_t)l * I + n0) * H;
    const uint8_t *ws = a.W2ts + ((int64_t)l * I + n0) * (H / 32);
    const KOp bk{as_u16(wq), as_u16(wq + (int64_t)hi * H), H / 2, nullptr, nullptr, 0};
    const SOp bs{ws, ws + (int64_t)hi * (H / 32), H / 32, nullptr, nullptr, 0};
    AccW<kFwdWM, kFwdWN> acc;
    gemm_mainloop_mx<kFwdWM, kFwdWN, SG>(ak, bk, as, bs, H / 128, false, lds, acc);
    epilogue_swiglu_bwd_w<kFwdWM, kFwdWN>(acc, lds, ARowsMx{a.Aq + (int64_t)m0 * I, a.As + (int64_t)m0 * (I / 32), I},
                                          a.HU + (int64_t)m0 * 2 * I, a.wrow + m0, a.dHU + (int64_t)m0 * 2 * I,
                                          a.part + (int64_t)m0 * a.nparts, a.nparts, I, n0);
}

template <int SG>
__device__ __forceinline__ void mx_bwd_down_phase(const MxBwdArgs &a, char *lds) {
    const int mtiles = a.seg_off[a.L] / kBM, ntiles = (a.I + 255) / 256;
    const int64_t total = (int64_t)mtiles * ntiles;
    for (int64_t it = blockIdx.x; it - blockIdx.x < total; it += gridDim.x) {
        const int64_t lid = logical_tile(it);
        if (lid >= total) continue;
        int m, n;
        grouped_mn<4>(lid, mtiles, ntiles, m, n);
        mx_bwd_down_tile<SG>(a, m, n, lds);
    }
}

// B3 with MX operands: dXd = dHUq W13t[l]^T over 2I.
template <int SG>
__device__ __forceinline__ void mx_bwd_gateup_tile(const MxBwdArgs &a, int mt, int nt, char *lds) {
    const int H = a.H, I = a.I;
    const int m0 = mt * kBM;
    const int l = expert_of(a.seg_off, a.L, m0);
    const uint8_t *gq = a.dHUq + (int64_t)m0 * 2 * I;
    const uint8_t *gs = a.dHUs + (int64_t)m0 * (2 * I / 32);
    const KOp ak{as_u16(gq), as_u16(gq + 256ll * I), I, nullptr, nullptr, 0};
    const SOp as{gs, gs + 128ll * (2 * I / 32), 2 * I / 32, nullptr, nullptr, 0};
    const uint8_t *wq = a.W13tq + ((int64_t)l * H + nt * 256) * 2 * I;
    const uint8_t *ws = a.W13ts + ((int64_t)l * H + nt * 256) * (2 * I / 32);
    const KOp bk{as_u16(wq), as_u16(wq + 256ll * I), I, nullptr, nullptr, 0};
    const SOp bs{ws, ws + 128ll * (2 * I / 32), 2 * I / 32, nullptr, nullptr, 0};
    AccW<kFwdWM, kFwdWN> acc;
    gemm_mainloop_mx<kFwdWM, kFwdWN, SG>(ak, bk, as, bs, 2 * I / 128, false, lds, acc);
    epilogue_store_bf16_w<kFwdWM, kFwdWN>(acc, lds, a.dXd + (int64_t)m0 * H + nt * 256, H, 256);
}

template <int SG>
__device__ __forceinline__ void mx_bwd_gateup_phase(const MxBwdArgs &a, char *lds) {
    const int mtiles = a.seg_off[a.L] / kBM, ntiles = a.H / 256;
    const int64_t total = (int64_t)mtiles * ntiles;
    for (int64_t it = blockIdx.x; it - blockIdx.x < total; it += gridDim.x) {
        const int64_t lid = logical_tile(it);
        if (lid >= total) continue;
        int m, n;
        grouped_mn<4>(lid, mtiles, ntiles, m, n);
        mx_bwd_gateup_tile<SG>(a, m, n, lds);
    }
}

// B5 with MX operands: the column-quantized activations, segment-major
// (expert l: a [C][n_l] block of codes at C * seg_off[l], its scales
// [C][n_l / 32] at C * seg_off[l] / 32).
struct MxWgradArgs {
    const uint8_t *dOwTq, *dOwTs;  // (w dO_d)^T, C = H
    const uint8_t *aTq, *aTs;      // a^T, C = I
    const uint8_t *dHUTq, *dHUTs;  // dHU^T, C = 2I
    const uint8_t *XdTq, *XdTs;    // Xd^T, C = H
    const int32_t *seg_off;
    float *dW13, *dW2;
    int L, H, I;
};

// The operands of one 256 x 256 output tile of dW2[l] (w2) or dW13[l] over
// the expert's kext rows (a multiple of 256; scale rows of kext / 32 bytes, a
// multiple of 8, hence 4-byte scale DMAs).
struct MxWgradTile {
    KOp ak, bk;
    SOp as, bs;
    int nk;
};

// seg_off[l] for a uniform l by a scalar load: it adds nothing to the vector
// memory counter, so reading it does not wait for the previous tile's stores.
__device__ __forceinline__ int seg_uniform(const int32_t *seg_off, int l) {
    using cint = __attribute__((address_space(4))) const int32_t;
    return ((cint *)seg_off)[l];
}

__device__ __forceinline__ MxWgradTile mx_wgrad_operands(const MxWgradArgs &a, bool w2, int l, int mt, int nt) {
    const int H = a.H, I = a.I;
    const int64_t S = seg_uniform(a.seg_off, l);
    const int kext = seg_uniform(a.seg_off, l + 1) - (int)S;
    const int64_t ld = kext, lds_s = kext / 32;
    // an operand's row r: the expert's block (at C * S) plus r * kext
    const int Ca = w2 ? H : 2 * I, Cb = w2 ? I : H;
    const uint8_t *aq = (w2 ? a.dOwTq : a.dHUTq) + Ca * S + (int64_t)mt * 256 * ld;
    const uint8_t *as_ = (w2 ? a.dOwTs : a.dHUTs) + Ca * S / 32 + (int64_t)mt * 256 * lds_s;
    const uint8_t *bq = (w2 ? a.aTq : a.XdTq) + Cb * S + (int64_t)nt * 256 * ld;
    const uint8_t *bs_ = (w2 ? a.aTs : a.XdTs) + Cb * S / 32 + (int64_t)nt * 256 * lds_s;
    const int bhi = (w2 && I - nt * 256 <= 128) ? 0 : 128;
    return {KOp{as_u16(aq), as_u16(aq + 128 * ld), ld / 2, nullptr, nullptr, 0},
            KOp{as_u16(bq), as_u16(bq + bhi * ld), ld / 2, nullptr, nullptr, 0},
            SOp{as_, as_ + 128 * lds_s, lds_s, nullptr, nullptr, 0},
            SOp{bs_, bs_ + bhi * lds_s, lds_s, nullptr, nullptr, 0}, kext / 128};
}

// Work item lid of the weight-gradient launch: a tile (w2, l, mt, nt) when
// lid < L * per, else a reverse-dispatch item.
struct MxWgradItem {
    bool w2;
    int l, mt, nt;
};

__device__ __forceinline__ MxWgradItem mx_wgrad_item(int64_t lid, int L, int per, int mt2, int nt2, int mt13, int nt13,
                                                     const int *s_order) {
    const int pos = (int)((uint32_t)lid / (uint32_t)per), in = (int)((uint32_t)lid - (uint32_t)pos * (uint32_t)per);
    MxWgradItem t;
    t.l = L <= 256 ? __builtin_amdgcn_readfirstlane(s_order[pos]) : pos;  // uniform: keep it scalar
    t.w2 = in < mt2 * nt2;
    if (t.w2)
        grouped_mn<4>(in, mt2, nt2, t.mt, t.nt);
    else
        grouped_mn<4>(in - mt2 * nt2, mt13, nt13, t.mt, t.nt);
    return t;
}

// One weight-gradient tile; pre: its first stage is in flight.  When the
// block's next item (nlid, if nxt) is a tile, its first stage's DMAs go out
// before this tile's stores; returns whether they did.
template <bool W2>
__device__ __forceinline__ bool mx_wgrad_tile(const MxWgradArgs &a, const MxWgradItem &t, bool pre, bool nxt,
                                              int64_t nlid, int L, int per, int mt2, int nt2, int mt13, int nt13,
                                              const int *s_order, char *lds) {
    const int H = a.H, I = a.I;
    AccW<kFwdWM, kFwdWN> acc;
    {
        const MxWgradTile o = mx_wgrad_operands(a, W2, t.l, t.mt, t.nt);
        gemm_mainloop_mx<kFwdWM, kFwdWN, 1, true>(o.ak, o.bk, o.as, o.bs, o.nk, false, lds, acc, pre);
    }
    const int nvalid = W2 ? min(256, I - t.nt * 256) : 256;
    bool issued = false;
    if (nvalid == 256 && nxt) {
        const MxWgradItem u = mx_wgrad_item(nlid, L, per, mt2, nt2, mt13, nt13, s_order);
        const MxWgradTile o = mx_wgrad_operands(a, u.w2, u.l, u.mt, u.nt);
        if (o.nk > 0) {
            mx_prefetch_stage0<kFwdWM, kFwdWN, 1>(o.ak, o.bk, o.as, o.bs, lds);
            issued = true;
        }
    }
    if constexpr (W2)
        epilogue_store_f32_w<kFwdWM, kFwdWN>(acc, a.dW2 + (int64_t)t.l * H * I + (int64_t)t.mt * 256 * I + t.nt * 256, I,
                                             256, nvalid);
    else
        epilogue_store_f32_w<kFwdWM, kFwdWN>(
            acc, a.dW13 + (int64_t)t.l * 2 * I * H + (int64_t)t.mt * 256 * H + t.nt * 256, H, 256, 256);
    return issued;
}

// All weight-gradient tiles, longest experts first, then the reverse-dispatch
// items of `c` (as the bf16 weight-gradient launch).  A tile's 256 KB of fp32
// stores drain slowly (the workgroups write their tiles at about the same
// time), and a wave's vector-memory operations complete in order, so a DMA
// issued after the stores is seen to land only once they have drained.  When
// the block's next item is a tile, its first stage's DMAs therefore go out
// before this tile's stores (LDS is free after the main loop; the store
// epilogue uses none): the next main loop starts once all but the last 63
// stores have drained, and its first step's MFMAs overlap the rest.  Only
// after a whole tile (128 stores per wave).  Nothing between the stores and
// that wait may wait for the counter: the tile operands come from scalar
// loads and inline address arithmetic, no vector loads or scratch.  The
// expert order sits past the GEMM's LDS in the same array: with a second LDS
// variable the compiler gives LDS accesses alias scopes and then waits for
// every outstanding DMA before the scale and fragment reads of each step.
__device__ __forceinline__ void mx_wgrad_phase(const MxWgradArgs &a, const WindowCombine &c, char *lds) {
    const int H = a.H, I = a.I, L = a.L;
    int *s_order = reinterpret_cast<int *>(lds + kMxLds);
    experts_by_rows(a.seg_off, L, 1, s_order);
    const int mt2 = H / 256, nt2 = (I + 255) / 256;  // dW2 [H][I]
    const int mt13 = 2 * I / 256, nt13 = H / 256;     // dW13 [2I][H]
    const int per = mt2 * nt2 + mt13 * nt13;
    const int64_t ntiles = (int64_t)L * per;
    const int64_t ncb = c.Y ? (c.ntok + kCombineItem - 1) / kCombineItem : 0;
    const int64_t total = ntiles + ncb;
    bool pre = false;  // this item's first stage is in flight
    for (int64_t it = blockIdx.x; it - blockIdx.x < total; it += gridDim.x) {
        const int64_t lid = logical_tile(it);
        if (lid >= total) continue;
        if (lid >= ntiles) {
            const int64_t g0 = (lid - ntiles) * kCombineItem;
            combine_body<kRowUnrollWide>(c.Y, c.route_row, c.w, c.out, c.K, c.H, g0, min(g0 + kCombineItem, c.ntok),
                                         threadIdx.x / kWave, blockDim.x / kWave, c.tpp, c.tstride);
            continue;
        }
        const MxWgradItem t = mx_wgrad_item(lid, L, per, mt2, nt2, mt13, nt13, s_order);
        const int64_t nx = it + gridDim.x, nlid = logical_tile(nx);
        const bool nxt = nx - blockIdx.x < total && nlid < ntiles;
        if (t.w2)
            pre = mx_wgrad_tile<true>(a, t, pre, nxt, nlid, L, per, mt2, nt2, mt13, nt13, s_order, lds);
        else
            pre = mx_wgrad_tile<false>(a, t, pre, nxt, nlid, L, per, mt2, nt2, mt13, nt13, s_order, lds);
    }
}

}  // namespace moe
