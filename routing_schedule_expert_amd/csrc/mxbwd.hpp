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
// 32 dispatched rows and stored transposed ([C][ld_t]), so every MX product
// reads both operands K-contiguous through the forward's scaled-MFMA loop.
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

// Row quantization of bf16 [rows][K] for the rows below *nrows (the
// dispatched rows of a table): one 32-element block per thread.
__device__ __forceinline__ void mx_quantize_rows_body(const uint16_t *src, const int32_t *nrows, int K, uint8_t *q,
                                                      uint8_t *s) {
    const int64_t nblocks = (int64_t)(*nrows) * (K / 32);
    for (int64_t b = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; b < nblocks; b += (int64_t)gridDim.x * blockDim.x)
        mx_quantize_block_bf16(src, K, q, s, b);
}

// Column quantization: out[c][r] = codes of column c of a [R][C] source in
// blocks of 32 consecutive rows (scale bytes [c][r / 32]), for batch b at
// b * out_bstride codes (b * out_bstride / 32 scale bytes).  Sources:
//   bf16 rows src + r * ld (+ b * in_bstride), or, with phi, row r taken from
//   source row part * Np + tok of phi[r] (padding rows zero);
//   or MX codes srcq / srcs [R][C] (+ [R][C/32]), decoded exactly.
// Rows at or past *nrows (if given, else R) read as zero; only whole blocks
// below the row count (rounded up to 32) are written.
struct ColQArgs {
    const uint16_t *src;
    int64_t ld, in_bstride;
    const moe_src *phi;
    int32_t Np;
    const uint8_t *srcq, *srcs;
    const int32_t *nrows;
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
            // 128 rows x 64 codes: 16 codes (one half block) per chunk
            for (int k = t; k < kColqRows * 4; k += kColqThreads) {
                const int row = k >> 2, cc = (k & 3) * 16;
                float v[16];
                const int64_t r = r0 + row;
                if (r < rows && c0 + cc < a.C) {
                    const u32x4 c = *reinterpret_cast<const u32x4 *>(a.srcq + r * a.C + c0 + cc);
                    const uint32_t sb = a.srcs[r * (a.C / 32) + (c0 + cc) / 32];
#pragma unroll
                    for (int j = 0; j < 16; ++j) v[j] = mx_decode((c[j >> 2] >> (8 * (j & 3))) & 0xffu, sb);
                } else {
#pragma unroll
                    for (int j = 0; j < 16; ++j) v[j] = 0.f;
                }
#pragma unroll
                for (int j = 0; j < 16; ++j) st[(cc + j) * kColqLd + row] = v[j];
            }
        } else {
            // 128 rows x 64 bf16: 8 values per 16-byte chunk
            for (int k = t; k < kColqRows * 8; k += kColqThreads) {
                const int row = k >> 3, cc = (k & 7) * 8;
                const int64_t r = r0 + row;
                const uint16_t *p = nullptr;
                if (r < rows && c0 + cc < a.C) {
                    if (a.phi) {
                        const int2 e = reinterpret_cast<const int2 *>(a.phi)[r];
                        if (e.x >= 0) p = a.src + ((int64_t)e.x * a.Np + e.y) * a.ld;
                    } else {
                        p = a.src + b * a.in_bstride + r * a.ld;
                    }
                }
                u32x4 x = {0u, 0u, 0u, 0u};
                if (p) x = *reinterpret_cast<const u32x4 *>(p + c0 + cc);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    st[(cc + 2 * j) * kColqLd + row] = __uint_as_float(x[j] << 16);
                    st[(cc + 2 * j + 1) * kColqLd + row] = __uint_as_float(x[j] & 0xffff0000u);
                }
            }
        }
        __syncthreads();
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
            uint8_t *out = a.q + b * a.out_bstride + (int64_t)(c0 + c) * a.ldq + rb;
            reinterpret_cast<u32x4 *>(out)[0] = u32x4{w[0], w[1], w[2], w[3]};
            reinterpret_cast<u32x4 *>(out)[1] = u32x4{w[4], w[5], w[6], w[7]};
            a.s[b * (a.out_bstride / 32) + (int64_t)(c0 + c) * (a.ldq / 32) + rb / 32] = (uint8_t)sb;
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

// B5 with MX operands: the column-quantized activations, stored transposed
// with ld_t codes per row (ld_t a multiple of 512, so scale rows of ld_t / 32
// bytes stay 16-byte aligned).
struct MxWgradArgs {
    const uint8_t *dOwTq, *dOwTs;  // (w dO_d)^T: [H][ld_t]
    const uint8_t *aTq, *aTs;      // a^T: [I][ld_t]
    const uint8_t *dHUTq, *dHUTs;  // dHU^T: [2I][ld_t]
    const uint8_t *XdTq, *XdTs;    // Xd^T: [H][ld_t]
    int64_t ld_t;
    const int32_t *seg_off;
    float *dW13, *dW2;
    int L, H, I;
};

// One 256 x 256 output tile of dW2[l] (W2) or dW13[l] over the expert's rows
// [seg_off[l], seg_off[l+1]) (a multiple of 256; the scale rows start at a
// multiple of 8 bytes, hence 4-byte scale DMAs).
template <bool W2>
__device__ __forceinline__ void mx_wgrad_tile(const MxWgradArgs &a, int l, int mt, int nt, char *lds) {
    const int H = a.H, I = a.I;
    const int64_t ld = a.ld_t, lds_s = ld / 32;
    const int S = a.seg_off[l], kext = a.seg_off[l + 1] - S;
    const uint8_t *aq, *as_, *bq, *bs_;
    int bhi;
    if constexpr (W2) {
        aq = a.dOwTq + (int64_t)mt * 256 * ld + S;
        as_ = a.dOwTs + (int64_t)mt * 256 * lds_s + S / 32;
        bq = a.aTq + (int64_t)nt * 256 * ld + S;
        bs_ = a.aTs + (int64_t)nt * 256 * lds_s + S / 32;
        bhi = I - nt * 256 > 128 ? 128 : 0;
    } else {
        aq = a.dHUTq + (int64_t)mt * 256 * ld + S;
        as_ = a.dHUTs + (int64_t)mt * 256 * lds_s + S / 32;
        bq = a.XdTq + (int64_t)nt * 256 * ld + S;
        bs_ = a.XdTs + (int64_t)nt * 256 * lds_s + S / 32;
        bhi = 128;
    }
    const KOp ak{as_u16(aq), as_u16(aq + 128 * ld), ld / 2, nullptr, nullptr, 0};
    const SOp as{as_, as_ + 128 * lds_s, lds_s, nullptr, nullptr, 0};
    const KOp bk{as_u16(bq), as_u16(bq + bhi * ld), ld / 2, nullptr, nullptr, 0};
    const SOp bs{bs_, bs_ + bhi * lds_s, lds_s, nullptr, nullptr, 0};
    AccW<kFwdWM, kFwdWN> acc;
    gemm_mainloop_mx<kFwdWM, kFwdWN, 1>(ak, bk, as, bs, kext / 128, false, lds, acc);
    if constexpr (W2)
        epilogue_store_f32_w<kFwdWM, kFwdWN>(acc, a.dW2 + (int64_t)l * H * I + (int64_t)mt * 256 * I + nt * 256, I, 256,
                                             I - nt * 256);
    else
        epilogue_store_f32_w<kFwdWM, kFwdWN>(acc, a.dW13 + (int64_t)l * 2 * I * H + (int64_t)mt * 256 * H + nt * 256, H,
                                             256, 256);
}

// All weight-gradient tiles, longest experts first, then the reverse-dispatch
// items of `c` (as the bf16 weight-gradient launch).
__device__ __forceinline__ void mx_wgrad_phase(const MxWgradArgs &a, const WindowCombine &c, char *lds) {
    const int H = a.H, I = a.I, L = a.L;
    __shared__ int s_order[256];
    experts_by_rows(a.seg_off, L, 1, s_order);
    const int mt2 = H / 256, nt2 = (I + 255) / 256;  // dW2 [H][I]
    const int mt13 = 2 * I / 256, nt13 = H / 256;     // dW13 [2I][H]
    const int per = mt2 * nt2 + mt13 * nt13;
    const int64_t ntiles = (int64_t)L * per;
    const int64_t ncb = c.Y ? (c.ntok + kCombineItem - 1) / kCombineItem : 0;
    const int64_t total = ntiles + ncb;
    for (int64_t it = blockIdx.x; it - blockIdx.x < total; it += gridDim.x) {
        const int64_t lid = logical_tile(it);
        if (lid >= total) continue;
        if (lid >= ntiles) {
            const int64_t g0 = (lid - ntiles) * kCombineItem;
            combine_body<kRowUnrollWide>(c.Y, c.route_row, c.w, c.out, c.K, c.H, g0, min(g0 + kCombineItem, c.ntok),
                                         threadIdx.x / kWave, blockDim.x / kWave, c.tpp, c.tstride);
            continue;
        }
        const int pos = (int)((uint32_t)lid / (uint32_t)per), in = (int)((uint32_t)lid - (uint32_t)pos * (uint32_t)per);
        const int l = L <= 256 ? s_order[pos] : pos;
        int mt, nt;
        if (in < mt2 * nt2) {
            grouped_mn<4>(in, mt2, nt2, mt, nt);
            mx_wgrad_tile<true>(a, l, mt, nt, lds);
        } else {
            grouped_mn<4>(in - mt2 * nt2, mt13, nt13, mt, nt);
            mx_wgrad_tile<false>(a, l, mt, nt, lds);
        }
    }
}

}  // namespace moe
