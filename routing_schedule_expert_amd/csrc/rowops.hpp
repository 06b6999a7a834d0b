// Row-streaming kernels: the pull gather, the fixed-order combine, and the two
// small per-row helpers of the backward.  All are HBM-bound copies: one wave
// moves one row with 16-byte lane accesses (a row of H bf16 is H/8 chunks),
// loads are issued before stores so each lane has several in flight.
//
//  gather   pull dispatch of "Beyond Peak TFLOPs" section 2.A / the
//           Mixture-of-Kittens notes section 2: the destination reads each row
//           through the two-column table {part, tok}; the backward's
//           reverse-combine is the same gather of dOut.
//  combine  push combine of the notes' section 2 done locally: per token, the
//           local slots' rows weighted and summed in ascending slot order in
//           fp32, rounded once; with no weights it is the reverse-dispatch sum.
#pragma once

#include "common.hpp"

namespace moe {

constexpr int kRowUnroll = 4;
constexpr int kRowUnrollWide = 8;

// Rows [0, Npad) of dst get src[phi.part][phi.tok] (or zeros on padding).
// Persistent over rows: Npad is read on the device.
__device__ void gather_rows_body(const uint16_t *__restrict__ src, const moe_src *__restrict__ phi,
                                 const int32_t *__restrict__ npad_ptr, uint16_t *__restrict__ dst,
                                 int Np, int H, int64_t row_begin, int64_t row_end_cap,
                                 int wave_global, int nwaves) {
    const int lane = lane_id();
    const int64_t npad = min((int64_t)*npad_ptr, row_end_cap);
    const int chunks = H / 8;
    for (int64_t row = row_begin + wave_global; row < npad; row += nwaves) {
        const uint2 s = reinterpret_cast<const uint2 *>(phi)[row];
        const int32_t part = (int32_t)s.x, tok = (int32_t)s.y;
        u32x4 *out = reinterpret_cast<u32x4 *>(dst + row * (int64_t)H);
        if (part < 0) {
            for (int c = lane; c < chunks; c += kWave) out[c] = u32x4{0, 0, 0, 0};
            continue;
        }
        const u32x4 *in = reinterpret_cast<const u32x4 *>(src + ((int64_t)part * Np + tok) * H);
        int c = lane;
        for (; c + (kRowUnroll - 1) * kWave < chunks; c += kRowUnroll * kWave) {
            u32x4 v[kRowUnroll];
#pragma unroll
            for (int u = 0; u < kRowUnroll; ++u) v[u] = __builtin_nontemporal_load(in + c + u * kWave);
#pragma unroll
            for (int u = 0; u < kRowUnroll; ++u) out[c + u * kWave] = v[u];
        }
        for (; c < chunks; c += kWave) out[c] = __builtin_nontemporal_load(in + c);
    }
}

// Token g' of a window of tpp tokens in each partition, partitions tstride
// tokens apart, as an index into the whole [P][tstride] token array
// (tpp == 0: the identity).
__device__ __forceinline__ int64_t window_token(int64_t g, int tpp, int64_t tstride) {
    return tpp ? (g / tpp) * tstride + g % tpp : g;
}

// The backward's reverse-combine gather: rows [0, Npad) of dst get
// src[phi.part][phi.tok] (zeros on padding) and rows of dst_w the same row
// times wrow[row], each element rounded once to bf16 (the weight gradient's
// operand, so the router weight is applied once per row, not per product).
__device__ void gather_rows_scaled_body(const uint16_t *__restrict__ src, const moe_src *__restrict__ phi,
                                        const int32_t *__restrict__ npad_ptr, const float *__restrict__ wrow,
                                        uint16_t *__restrict__ dst, uint16_t *__restrict__ dst_w, int Np, int H,
                                        int64_t row_end_cap, int wave_global, int nwaves) {
    const int lane = lane_id();
    const int64_t npad = min((int64_t)*npad_ptr, row_end_cap);
    const int chunks = H / 8;
    for (int64_t row = wave_global; row < npad; row += nwaves) {
        const uint2 s = reinterpret_cast<const uint2 *>(phi)[row];
        const int32_t part = (int32_t)s.x, tok = (int32_t)s.y;
        u32x4 *out = reinterpret_cast<u32x4 *>(dst + row * (int64_t)H);
        u32x4 *outw = reinterpret_cast<u32x4 *>(dst_w + row * (int64_t)H);
        if (part < 0) {
            for (int c = lane; c < chunks; c += kWave) out[c] = outw[c] = u32x4{0, 0, 0, 0};
            continue;
        }
        const float sc = wrow[row];
        const u32x4 *in = reinterpret_cast<const u32x4 *>(src + ((int64_t)part * Np + tok) * H);
        for (int c0 = lane; c0 < chunks; c0 += kRowUnroll * kWave) {
            u32x4 v[kRowUnroll];
#pragma unroll
            for (int u = 0; u < kRowUnroll; ++u)
                if (c0 + u * kWave < chunks) v[u] = __builtin_nontemporal_load(in + c0 + u * kWave);
#pragma unroll
            for (int u = 0; u < kRowUnroll; ++u) {
                const int c = c0 + u * kWave;
                if (c < chunks) {
                    out[c] = v[u];
                    u32x4 x;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        x[e] = pack_bf2(__uint_as_float(v[u][e] << 16) * sc, __uint_as_float(v[u][e] & 0xffff0000u) * sc);
                    outw[c] = x;
                }
            }
        }
    }
}

// out[g] = sum_{j asc, rows[g][j] >= 0} w[g][j] * Y[rows[g][j]] (+ S[g]) for
// tokens g in [g_begin, g_end) (through window_token when tpp > 0: route_row,
// w and out then point at the window's first token of partition 0); one wave
// per token, U 16-byte chunks per lane in flight.  w == nullptr means every
// weight is 1.  S (nullable, [tokens][H]) is the shared expert's output, added
// after the slots, before the one rounding.
// U trades registers for bytes in flight: the standalone combine kernel keeps
// many waves per CU and U = kRowUnroll; a combine that runs inside a GEMM
// kernel (eight waves per CU) takes U = kRowUnrollWide, a whole 7,168-wide
// row per wave, so the CU still keeps enough row loads in flight.
// skip_single: tokens with exactly one local route are left alone (the down
// GEMM's epilogue wrote them: RowCombine).
template <int U = kRowUnroll>
__device__ void combine_body(const uint16_t *__restrict__ Y, const int32_t *__restrict__ route_row,
                             const float *__restrict__ w, uint16_t *__restrict__ out, int K, int H,
                             int64_t g_begin, int64_t g_end, int wave_global, int nwaves, int tpp = 0,
                             int64_t tstride = 0, const uint16_t *__restrict__ S = nullptr,
                             bool skip_single = false) {
    const int lane = lane_id();
    const int chunks = H / 8;
    for (int64_t gw = g_begin + wave_global; gw < g_end; gw += nwaves) {
        const int64_t g = window_token(gw, tpp, tstride);
        if (skip_single) {
            int n = 0;
            for (int j0 = 0; j0 < K; j0 += kWave) {
                const int j = j0 + lane;
                n += __popcll(ballot(j < K && route_row[g * K + j] >= 0));
            }
            if (n == 1) continue;
        }
        u32x4 *o = reinterpret_cast<u32x4 *>(out + g * (int64_t)H);
        for (int c0 = 0; c0 < chunks; c0 += U * kWave) {
            float acc[U][8];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[u][e] = 0.f;
            for (int j = 0; j < K; ++j) {
                const int32_t rw = route_row[g * K + j];
                if (rw < 0) continue;
                const float wq = w ? w[g * K + j] : 1.0f;
                const u32x4 *yr = reinterpret_cast<const u32x4 *>(Y + (int64_t)rw * H);
                u32x4 v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    int c = c0 + u * kWave + lane;
                    v[u] = c < chunks ? __builtin_nontemporal_load(yr + c) : u32x4{0, 0, 0, 0};
                }
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc[u][2 * e] = fmaf(wq, __uint_as_float(v[u][e] << 16), acc[u][2 * e]);
                        acc[u][2 * e + 1] = fmaf(wq, __uint_as_float(v[u][e] & 0xffff0000u), acc[u][2 * e + 1]);
                    }
            }
            if (S) {
                const u32x4 *sr = reinterpret_cast<const u32x4 *>(S + g * (int64_t)H);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    int c = c0 + u * kWave + lane;
                    const u32x4 v = c < chunks ? __builtin_nontemporal_load(sr + c) : u32x4{0, 0, 0, 0};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc[u][2 * e] += __uint_as_float(v[e] << 16);
                        acc[u][2 * e + 1] += __uint_as_float(v[e] & 0xffff0000u);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                int c = c0 + u * kWave + lane;
                if (c < chunks)
                    o[c] = u32x4{pack_bf2(acc[u][0], acc[u][1]), pack_bf2(acc[u][2], acc[u][3]),
                                 pack_bf2(acc[u][4], acc[u][5]), pack_bf2(acc[u][6], acc[u][7])};
            }
        }
    }
}

// tab[row] for the local routes of token g: (g, bits of w_gj) when the token
// has exactly one local route, at slot j (its combine is then a single term,
// which the down GEMM's epilogue computes: RowCombine), else (-1, 0).
// Padding rows are marked by single_route_pad.
__device__ void single_route_body(const int32_t *__restrict__ route_row, const float *__restrict__ w,
                                  int2 *__restrict__ tab, int K, int64_t g) {
    int n = 0, jj = -1;
    for (int j = 0; j < K; ++j)
        if (route_row[g * K + j] >= 0) ++n, jj = j;
    const int2 e = n == 1 ? make_int2((int)g, __float_as_int(w[g * K + jj])) : make_int2(-1, 0);
    for (int j = 0; j < K; ++j) {
        const int32_t r = route_row[g * K + j];
        if (r >= 0) tab[r] = e;
    }
}

// tab[row] = (-1, 0) for a padding row (phi partition < 0) below seg_off[L]:
// such a row belongs to no token.
__device__ __forceinline__ void single_route_pad(const moe_src *__restrict__ phi, int2 *__restrict__ tab,
                                                 int64_t row) {
    if (phi[row].part < 0) tab[row] = make_int2(-1, 0);
}

// wrow[i] = router weight of the route placed at row i (0 on padding rows).
__device__ void row_weight_body(const moe_src *__restrict__ phi, const int32_t *__restrict__ npad_ptr,
                                const int32_t *__restrict__ route_row, const float *__restrict__ w,
                                float *__restrict__ wrow, int Np, int K, int64_t i) {
    if (i >= *npad_ptr) return;
    const uint2 s = reinterpret_cast<const uint2 *>(phi)[i];
    float v = 0.f;
    if ((int32_t)s.x >= 0) {
        const int64_t g = (int64_t)(int32_t)s.x * Np + (int32_t)s.y;
        for (int j = 0; j < K; ++j)
            if (route_row[g * K + j] == (int32_t)i) v = w[g * K + j];
    }
    wrow[i] = v;
}

// dw[slot] = sum_q part[row][q] in ascending q (0 for non-local slots); slot
// is mapped like a token by window_token, in units of slots (tpp K per
// partition, tstride K apart).
__device__ void dw_finalize_body(const int32_t *__restrict__ route_row, const float *__restrict__ part,
                                 int nparts, float *__restrict__ dw, int64_t slot_w, int spp = 0,
                                 int64_t sstride = 0) {
    const int64_t slot = window_token(slot_w, spp, sstride);
    int32_t row = route_row[slot];
    float s = 0.f;
    if (row >= 0) {
        const float *p = part + (int64_t)row * nparts;
        for (int q = 0; q < nparts; ++q) s += p[q];
    }
    dw[slot] = s;
}

}  // namespace moe
