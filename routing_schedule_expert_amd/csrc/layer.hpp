// Layer-level device code: the expert FFN phases, the chunked persistent FFN,
// the persistent whole-forward launch, and the backward phases.
//
//  * Expert FFN ("Mixture-of-Kittens: A MoE Megakernel for GB300 NVL72",
//    sections 3 and 5): gate/up projection with SwiGLU fused into its
//    epilogue, then the down projection, over 256-row tiles of the expert
//    segments.  Npad is read on the device; every persistent workgroup loops
//    over the tiles of a phase.
//  * Chunked FFN (section 3, the minibatch T): rows are processed in chunks of
//    T dispatched rows; phase p runs the gate/up tiles of chunk p together
//    with the down tiles of chunk p-1, separated by device-wide barriers.
//  * Persistent forward (section 5, megakernel fusion): schedule, gather, FFN
//    and combine in one cooperative launch with device-side barriers between
//    stages, so no host launch sits between them.
//  * Backward (section 2: pull reverse-combine / push reverse-dispatch; section
//    5: router-weight gradient from the SwiGLU activations and the down
//    dgrad; "Beyond Peak TFLOPs" section 2.C: weight gradients after the data
//    gradients, accumulated over tokens in one fixed-order pass).
#pragma once

#include "common.hpp"
#include "gemm.hpp"
#include "mx.hpp"
#include "rowops.hpp"
#include "schedule.hpp"
#include "wide.hpp"

namespace moe {

// Forward GEMM configuration: 8 waves (4 x 2, two per SIMD) on a 256 x 256
// tile, 64-deep steps double buffered by DMA, window-swizzled LDS.
constexpr int kFwdWM = 4, kFwdWN = 2;
constexpr int kFwdThreads = 64 * kFwdWM * kFwdWN;

// Xd == nullptr: the gate/up GEMM pulls its A rows straight from X through
// the table phi (the dispatch fused into the operand loads) and no dispatched
// copy is written.
struct FfnArgs {
    const uint16_t *Xd, *W13, *W2;
    const int32_t *seg_off;
    uint16_t *HU, *A, *Y;
    int L, H, I;
    int32_t chunk_rows;
    uint32_t *bar;
    const uint16_t *X;
    const moe_src *phi;
    int32_t Np;
    RowCombine rc;  // the wide down tiles' combine of single-route tokens (rc.out null: none)
};

__device__ __forceinline__ void ffn_gateup_tile(const FfnArgs &a, int mt, int nt, char *lds) {
    const int H = a.H, I = a.I;
    const int m0 = mt * kBM;
    const int l = expert_of(a.seg_off, a.L, m0);
    const uint16_t *w = a.W13 + (int64_t)l * 2 * I * H;
    KOp ak;
    if (a.Xd) {
        const uint16_t *xa = a.Xd + (int64_t)m0 * H;
        ak = KOp{xa, xa + 128ll * H, H, nullptr, nullptr, 0};
    } else {
        ak = KOp{nullptr, nullptr, H, a.phi + m0, a.X, a.Np};
    }
    KOp bk{w + (int64_t)nt * 128 * H, w + ((int64_t)I + nt * 128) * H, H};
    AccW<kFwdWM, kFwdWN> acc;
    gemm_mainloop_x<kFwdWM, kFwdWN, false, false>(ak, bk, H / 64, true, lds, acc);
    uint16_t *hu = a.HU ? a.HU + (int64_t)m0 * 2 * I : nullptr;
    epilogue_swiglu_w<kFwdWM, kFwdWN>(acc, lds, a.A + (int64_t)m0 * I + nt * 128, I, hu ? hu + nt * 128 : nullptr,
                                      hu ? hu + I + nt * 128 : nullptr, 2ll * I);
}

__device__ __forceinline__ void ffn_down_tile(const FfnArgs &a, int mt, int nt, char *lds) {
    const int H = a.H, I = a.I;
    const int m0 = mt * kBM;
    const int l = expert_of(a.seg_off, a.L, m0);
    const uint16_t *aa = a.A + (int64_t)m0 * I;
    const uint16_t *w = a.W2 + (int64_t)l * H * I + (int64_t)nt * 256 * I;
    KOp ak{aa, aa + 128ll * I, I};
    KOp bk{w, w + 128ll * I, I};
    AccW<kFwdWM, kFwdWN> acc;
    gemm_mainloop_x<kFwdWM, kFwdWN, false, false>(ak, bk, I / 64, false, lds, acc);
    epilogue_store_bf16_comb<kFwdWM, kFwdWN>(acc, lds, a.Y + (int64_t)m0 * H + nt * 256, H, a.rc, m0, nt * 256,
                                             lds + kGemmLds);
}

// One persistent pass over the tiles of rows [r0, r1) (multiples of 256).
// The whole table's gate/up tiles, in expert-aligned order.
__device__ __forceinline__ void ffn_gateup_phase(const FfnArgs &a, char *lds) {
    const int mtiles = a.seg_off[a.L] / kBM, ntiles = a.I / 128;
    const int64_t total = (int64_t)mtiles * ntiles;
    for (int64_t it = blockIdx.x; it - blockIdx.x < total; it += gridDim.x) {
        const int64_t lid = logical_tile(it);
        if (lid >= total) continue;
        int m, n;
        expert_mn(lid, a.seg_off, a.L, ntiles, m, n);
        ffn_gateup_tile(a, m, n, lds);
    }
}

// The whole table's down tiles (256 x 256): groups of 4 M tiles sweep the N
// tiles (the expert-aligned order measured 1-4% slower on the down-shaped
// products, K = I).
__device__ __forceinline__ void ffn_down_phase(const FfnArgs &a, char *lds) {
    const int mtiles = a.seg_off[a.L] / kBM, ntiles = a.H / 256;
    const int64_t total = (int64_t)mtiles * ntiles;
    for (int64_t it = blockIdx.x; it - blockIdx.x < total; it += gridDim.x) {
        const int64_t lid = logical_tile(it);
        if (lid >= total) continue;
        int m, n;
        grouped_mn<4>(lid, mtiles, ntiles, m, n);
        ffn_down_tile(a, m, n, lds);
    }
}

// Wide-tile down projection (wide.hpp): 256 x 384 tiles of Y, narrow
// 256 x 256 tiles for the rest.  (The same tile on the gate/up projection,
// with SwiGLU in its epilogue, measured 3.61 ms against 3.09 ms for the
// 256 x 256 tile: its 7,168-deep K loops stream 3.7 and 5.5 MB operand
// strips through a 4 MB L2, and it fetched 9.9 against 8.5 GB into L2.)
template <int BN>
__device__ __forceinline__ void wide_down_tile(const FfnArgs &a, int mt, int n0, char *lds) {
    const int H = a.H, I = a.I;
    const int m0 = mt * kBM;
    const int l = expert_of(a.seg_off, a.L, m0);
    AccWide<BN> acc;
    wide_mainloop<BN>(a.A + (int64_t)m0 * I, I, a.W2 + ((int64_t)l * H + n0) * I, I, I / kWBK, lds, acc);
    wide_epilogue_store<BN>(acc, lds, a.Y + (int64_t)m0 * H + n0, H, a.rc, m0, n0);
}

// All wide tiles (groups of 4 M tiles sweep the N tiles), then the narrow ones.
__device__ __forceinline__ void wide_down_phase(const FfnArgs &a, char *lds) {
    const int mtiles = a.seg_off[a.L] / kBM;
    const WideSplit sp = wide_split(a.H, kWideBN, 256);
    const int64_t nwide = (int64_t)mtiles * sp.nw, total = nwide + (int64_t)mtiles * sp.nn;
    for (int64_t it = blockIdx.x; it - blockIdx.x < total; it += gridDim.x) {
        const int64_t lid = logical_tile(it);
        if (lid >= total) continue;
        int m, n;
        if (lid < nwide) {
            grouped_mn<4>(lid, mtiles, sp.nw, m, n);
            wide_down_tile<kWideBN>(a, m, sp.col(n), lds);
        } else {
            grouped_mn<4>(lid - nwide, mtiles, sp.nn, m, n);
            wide_down_tile<256>(a, m, sp.col(sp.nw + n), lds);
        }
    }
}

// Chunked pipeline: phase p = gate/up of chunk p and down of chunk p-1.
__device__ __forceinline__ void ffn_chunked_body(const FfnArgs &a, char *lds, GridBarrier &gb) {
    const int npad = a.seg_off[a.L];
    const int T = a.chunk_rows;
    const int nchunks = (npad + T - 1) / T;
    for (int p = 0; p <= nchunks; ++p) {
        const int gu0 = min(p * T, npad), gu1 = min((p + 1) * T, npad);
        const int dn0 = p > 0 ? min((p - 1) * T, npad) : 0, dn1 = p > 0 ? gu0 : 0;
        const int64_t ngu = (int64_t)((gu1 - gu0) / kBM) * (a.I / 128);
        const int64_t ndn = (int64_t)((dn1 - dn0) / kBM) * (a.H / 256);
        const int64_t total = ngu + ndn;
        for (int64_t it = blockIdx.x; it - blockIdx.x < total; it += gridDim.x) {
            const int64_t lid = logical_tile(it);
            if (lid >= total) continue;
            int m, n;
            if (lid < ngu) {
                grouped_mn<4>(lid, (gu1 - gu0) / kBM, a.I / 128, m, n);
                ffn_gateup_tile(a, gu0 / kBM + m, n, lds);
            } else {
                grouped_mn<4>(lid - ngu, (dn1 - dn0) / kBM, a.H / 256, m, n);
                ffn_down_tile(a, dn0 / kBM + m, n, lds);
            }
        }
        gb.sync();
    }
}

// ---------------------------------------------------------------------------
// MXFP8 expert FFN.
// ---------------------------------------------------------------------------

struct MxFfnArgs {
    const uint8_t *Xq, *Xs;  // MX codes [P*Np][H] and scale bytes [P*Np][H/32] of X
    const moe_src *phi;      // the pull table: dispatched row -> X row
    int32_t Np;
    const uint8_t *W13q, *W13s, *W2q, *W2s;  // [L][2I][H] (+/32), [L][H][I] (+/32)
    const int32_t *seg_off;
    uint8_t *Aq, *As;  // MX codes [cap][I] and scale bytes [cap][I/32] of a
    uint16_t *HU;      // nullable: bf16 [cap][2I], h then u (saved for the backward)
    uint16_t *Y;       // bf16 [cap][H]
    int L, H, I;
    RowCombine rc;  // the down tiles' combine of single-route tokens (rc.out null: none)
};

__device__ __forceinline__ const uint16_t *as_u16(const uint8_t *p) { return reinterpret_cast<const uint16_t *>(p); }

template <int SG>
__device__ __forceinline__ void mx_gateup_tile(const MxFfnArgs &a, int mt, int nt, char *lds) {
    const int H = a.H, I = a.I;
    const int m0 = mt * kBM;
    const int l = expert_of(a.seg_off, a.L, m0);
    const KOp ak{nullptr, nullptr, H / 2, a.phi + m0, as_u16(a.Xq), a.Np};
    const SOp as{nullptr, nullptr, H / 32, a.phi + m0, a.Xs, a.Np};
    const uint8_t *w = a.W13q + (int64_t)l * 2 * I * H;
    const uint8_t *ws = a.W13s + (int64_t)l * 2 * I * (H / 32);
    const KOp bk{as_u16(w + (int64_t)nt * 128 * H), as_u16(w + ((int64_t)I + nt * 128) * H), H / 2, nullptr, nullptr, 0};
    const SOp bs{ws + (int64_t)nt * 128 * (H / 32), ws + ((int64_t)I + nt * 128) * (H / 32), H / 32, nullptr, nullptr,
                 0};
    AccW<kFwdWM, kFwdWN> acc;
    gemm_mainloop_mx<kFwdWM, kFwdWN, SG>(ak, bk, as, bs, H / 128, true, lds, acc);
    uint16_t *hu = a.HU ? a.HU + (int64_t)m0 * 2 * I + nt * 128 : nullptr;
    epilogue_swiglu_mx<kFwdWM, kFwdWN>(acc, lds, a.Aq + (int64_t)m0 * I + nt * 128, I,
                                       a.As + (int64_t)m0 * (I / 32) + nt * 4, I / 32, hu, hu ? hu + I : nullptr,
                                       2ll * I);
}

template <int SG>
__device__ __forceinline__ void mx_down_tile(const MxFfnArgs &a, int mt, int nt, char *lds) {
    const int H = a.H, I = a.I;
    const int m0 = mt * kBM;
    const int l = expert_of(a.seg_off, a.L, m0);
    const uint8_t *aq = a.Aq + (int64_t)m0 * I;
    const uint8_t *asc = a.As + (int64_t)m0 * (I / 32);
    const KOp ak{as_u16(aq), as_u16(aq + 128ll * I), I / 2, nullptr, nullptr, 0};
    const SOp as{asc, asc + 128ll * (I / 32), I / 32, nullptr, nullptr, 0};
    const uint8_t *w = a.W2q + ((int64_t)l * H + nt * 256) * I;
    const uint8_t *ws = a.W2s + ((int64_t)l * H + nt * 256) * (I / 32);
    const KOp bk{as_u16(w), as_u16(w + 128ll * I), I / 2, nullptr, nullptr, 0};
    const SOp bs{ws, ws + 128ll * (I / 32), I / 32, nullptr, nullptr, 0};
    AccW<kFwdWM, kFwdWN> acc;
    gemm_mainloop_mx<kFwdWM, kFwdWN, SG>(ak, bk, as, bs, I / 128, false, lds, acc);
    epilogue_store_bf16_comb<kFwdWM, kFwdWN>(acc, lds, a.Y + (int64_t)m0 * H + nt * 256, H, a.rc, m0, nt * 256,
                                             lds + kGemmLds);
}

template <int SG>
__device__ __forceinline__ void mx_gateup_phase(const MxFfnArgs &a, char *lds) {
    const int mtiles = a.seg_off[a.L] / kBM, ntiles = a.I / 128;
    const int64_t total = (int64_t)mtiles * ntiles;
    for (int64_t it = blockIdx.x; it - blockIdx.x < total; it += gridDim.x) {
        const int64_t lid = logical_tile(it);
        if (lid >= total) continue;
        int m, n;
        expert_mn(lid, a.seg_off, a.L, ntiles, m, n);
        mx_gateup_tile<SG>(a, m, n, lds);
    }
}

template <int SG>
__device__ __forceinline__ void mx_down_phase(const MxFfnArgs &a, char *lds) {
    const int mtiles = a.seg_off[a.L] / kBM, ntiles = a.H / 256;
    const int64_t total = (int64_t)mtiles * ntiles;
    for (int64_t it = blockIdx.x; it - blockIdx.x < total; it += gridDim.x) {
        const int64_t lid = logical_tile(it);
        if (lid >= total) continue;
        int m, n;
        grouped_mn<4>(lid, mtiles, ntiles, m, n);
        mx_down_tile<SG>(a, m, n, lds);
    }
}

// ---------------------------------------------------------------------------
// Shared expert ("Beyond Peak TFLOPs" section 2.C; the Mixture-of-Kittens
// notes, section 5: a dense bf16 expert over every token).  It is one more
// grouped GEMM with a single segment whose table is the identity over the
// tokens, and its tiles share the routed GEMM's launches: the two work lists
// are concatenated, shared tiles first, so neither waits for the other's
// tail.
// ---------------------------------------------------------------------------

__device__ __forceinline__ void dual_gateup_body(const FfnArgs &s, const FfnArgs &r, char *lds) {
    const int ms = s.seg_off[s.L] / kBM, ns = s.I / 128;
    const int mr = r.seg_off[r.L] / kBM, nr = r.I / 128;
    const int64_t ts = (int64_t)ms * ns, total = ts + (int64_t)mr * nr;
    for (int64_t it = blockIdx.x; it - blockIdx.x < total; it += gridDim.x) {
        const int64_t lid = logical_tile(it);
        if (lid >= total) continue;
        int m, n;
        if (lid < ts) {
            grouped_mn<4>(lid, ms, ns, m, n);
            ffn_gateup_tile(s, m, n, lds);
        } else {
            expert_mn(lid - ts, r.seg_off, r.L, nr, m, n);
            ffn_gateup_tile(r, m, n, lds);
        }
    }
}

__device__ __forceinline__ void dual_down_body(const FfnArgs &s, const FfnArgs &r, char *lds) {
    const int ms = s.seg_off[s.L] / kBM, nt = s.H / 256;
    const int mr = r.seg_off[r.L] / kBM;
    const int64_t ts = (int64_t)ms * nt, total = ts + (int64_t)mr * nt;
    for (int64_t it = blockIdx.x; it - blockIdx.x < total; it += gridDim.x) {
        const int64_t lid = logical_tile(it);
        if (lid >= total) continue;
        int m, n;
        if (lid < ts) {
            grouped_mn<4>(lid, ms, nt, m, n);
            ffn_down_tile(s, m, n, lds);
        } else {
            grouped_mn<4>(lid - ts, mr, nt, m, n);
            ffn_down_tile(r, m, n, lds);
        }
    }
}

// ---------------------------------------------------------------------------
// Macrobatch ring ("Beyond Peak TFLOPs" section 2.B; the Mixture-of-Kittens
// notes, section 4): the combine of one macrobatch runs in the same launch as
// the gate/up GEMM of the next, so a slot's rows are consumed while the next
// macrobatch's rows are produced.
// ---------------------------------------------------------------------------

// The combine of one token window (tpp tokens in each of the partitions,
// tstride apart); Y == nullptr: nothing to combine.
struct WindowCombine {
    const uint16_t *Y;
    const int32_t *route_row;  // at the window's first token of partition 0
    const float *w;
    uint16_t *out;
    int K, H, tpp;
    int64_t ntok, tstride;
    int skip_single;  // leave the tokens with one local route (the down epilogue wrote them)
};

constexpr int kCombineItem = 64;  // tokens per combine work item (8 per wave)

// Work items: the gate/up tiles of `a` then the combine items of `c`.  Each
// workgroup takes whole items, so the HBM-bound combine fills the CUs the
// last round of MFMA tiles leaves idle.
__device__ __forceinline__ void ring_gateup_combine_body(const FfnArgs &a, const WindowCombine &c, char *lds) {
    const int npad = a.seg_off[a.L];
    const int mtiles = npad / kBM, ntiles = a.I / 128;
    const int64_t ngu = (int64_t)mtiles * ntiles;
    const int64_t ncb = c.Y ? (c.ntok + kCombineItem - 1) / kCombineItem : 0;
    const int64_t total = ngu + ncb;
    const int waves = blockDim.x / kWave;
    for (int64_t it = blockIdx.x; it - blockIdx.x < total; it += gridDim.x) {
        const int64_t lid = logical_tile(it);
        if (lid >= total) continue;
        if (lid < ngu) {
            int m, n;
            expert_mn(lid, a.seg_off, a.L, ntiles, m, n);
            ffn_gateup_tile(a, m, n, lds);
        } else {
            const int64_t g0 = (lid - ngu) * kCombineItem;
            combine_body<kRowUnrollWide>(c.Y, c.route_row, c.w, c.out, c.K, c.H, g0, min(g0 + kCombineItem, c.ntok),
                         threadIdx.x / kWave, waves, c.tpp, c.tstride, nullptr, c.skip_single != 0);
        }
    }
}

// ---------------------------------------------------------------------------
// Persistent forward.
// ---------------------------------------------------------------------------

struct LayerFwdArgs {
    SchedArgs sched;
    FfnArgs ffn;
    const uint16_t *X;
    const float *w;
    uint16_t *out;
    int Np, K;
    int64_t ntok, cap;
};

__device__ __forceinline__ void layer_fwd_persistent_body(const LayerFwdArgs &a, char *lds) {
    const SchedArgs &s = a.sched;
    const int nitems = s.P * s.wg_per_part;
    int32_t *smem = reinterpret_cast<int32_t *>(lds);
    GridBarrier gb(a.ffn.bar);
    for (int x = blockIdx.x; x < nitems; x += gridDim.x) sched_count_body(s, smem, x);
    gb.sync();
    if (blockIdx.x == 0) sched_finalize(s, 0, smem);
    gb.sync();
    for (int x = blockIdx.x; x < nitems; x += gridDim.x) sched_scatter_body(s, smem, x);
    gb.sync();
    const int waves = blockDim.x / kWave;
    if (a.ffn.Xd) {
        gather_rows_body(a.X, s.phi, s.seg_off + s.L, const_cast<uint16_t *>(a.ffn.Xd), a.Np, a.ffn.H, 0, a.cap,
                         blockIdx.x * waves + threadIdx.x / kWave, gridDim.x * waves);
        gb.sync();
    }
    if (a.ffn.chunk_rows > 0) {
        ffn_chunked_body(a.ffn, lds, gb);
    } else {
        ffn_gateup_phase(a.ffn, lds);
        gb.sync();
        ffn_down_phase(a.ffn, lds);
        gb.sync();
    }
    combine_body<kRowUnrollWide>(a.ffn.Y, s.route_row, a.w, a.out, a.K, a.ffn.H, 0, a.ntok,
                 blockIdx.x * waves + threadIdx.x / kWave, gridDim.x * waves);
}

// ---------------------------------------------------------------------------
// Backward.
// ---------------------------------------------------------------------------

// The weights and the row activations are read as they lie: the data
// gradients take W2[l] and W13[l] as MN-contiguous operands, the weight
// gradients take the activation rows as MN-contiguous operands on both sides
// (their K is the row index), so no transposed copy is made.
// Data-gradient GEMMs: their B operand is MN-contiguous, and each of its
// fragments takes two transposing LDS reads against one plain read for a
// K-contiguous fragment, so the wave grid is 2 x 4 (4 A blocks, 2 B blocks
// per wave) rather than the forward's 4 x 2: 8 LDS reads per sub-step, not 10.
constexpr int kBwdWM = 2, kBwdWN = 4;

// The data-gradient GEMMs of one table (B2, B3).
struct BwdArgs {
    const uint16_t *dOd;
    uint16_t *dXd, *dHU;
    const float *wrow;
    float *part;
    const uint16_t *HU, *A, *W13, *W2;
    const int32_t *seg_off;
    int L, H, I, nparts;
};

// B2: dA' = dO_d W2[l], SwiGLU backward in the epilogue.
__device__ __forceinline__ void bwd_down_phase(const BwdArgs &a, char *lds) {
    const int H = a.H, I = a.I;
    const int npad = a.seg_off[a.L];
    const int mtiles = npad / kBM, ntiles = (I + 255) / 256;
    const int64_t total = (int64_t)mtiles * ntiles;
    for (int64_t it = blockIdx.x; it - blockIdx.x < total; it += gridDim.x) {
        const int64_t lid = logical_tile(it);
        if (lid >= total) continue;
        int mt, nt;
        grouped_mn<4>(lid, mtiles, ntiles, mt, nt);
        const int m0 = mt * kBM;
        const int l = expert_of(a.seg_off, a.L, m0);
        const uint16_t *g = a.dOd + (int64_t)m0 * H;
        const KOp ak{g, g + 128ll * H, H};
        const TOp bk{a.W2 + (int64_t)l * H * I + nt * 256, I, min(256, I - nt * 256)};  // [k = h][i]
        AccW<kBwdWM, kBwdWN> acc;
        gemm_mainloop_x<kBwdWM, kBwdWN, false, true>(ak, bk, H / 64, false, lds, acc);
        epilogue_swiglu_bwd_w<kBwdWM, kBwdWN>(acc, lds, ARowsBf16{a.A + (int64_t)m0 * I, I}, a.HU + (int64_t)m0 * 2 * I, a.wrow + m0,
                                              a.dHU + (int64_t)m0 * 2 * I, a.part + (int64_t)m0 * a.nparts, a.nparts, I,
                                              nt * 256);
    }
}

// B3: dXd = dHU W13[l].
__device__ __forceinline__ void bwd_gateup_phase(const BwdArgs &a, char *lds) {
    const int H = a.H, I = a.I;
    const int npad = a.seg_off[a.L];
    const int mtiles = npad / kBM, ntiles = H / 256;
    const int64_t total = (int64_t)mtiles * ntiles;
    for (int64_t it = blockIdx.x; it - blockIdx.x < total; it += gridDim.x) {
        const int64_t lid = logical_tile(it);
        if (lid >= total) continue;
        int mt, nt;
        grouped_mn<4>(lid, mtiles, ntiles, mt, nt);
        const int m0 = mt * kBM;
        const int l = expert_of(a.seg_off, a.L, m0);
        const uint16_t *g = a.dHU + (int64_t)m0 * 2 * I;
        const KOp ak{g, g + 128ll * 2 * I, 2ll * I};
        const TOp bk{a.W13 + (int64_t)l * 2 * I * H + nt * 256, H, 256};  // [k = j][h]
        AccW<kBwdWM, kBwdWN> acc;
        gemm_mainloop_x<kBwdWM, kBwdWN, false, true>(ak, bk, 2 * I / 64, false, lds, acc);
        epilogue_store_bf16_w<kBwdWM, kBwdWN>(acc, lds, a.dXd + (int64_t)m0 * H + nt * 256, H, 256);
    }
}

// B5 operands: the activation rows of G tables (the backward of one table,
// or of a group of macrobatches whose weight gradients are taken together).
// Table g's buffers are at fixed strides from table 0's (kernel arguments are
// not indexed at run time, which would copy them to scratch); its A rows are
// either in a ring slot (bit g of a_in_ring) or at A + g * a_stride.
constexpr int kMaxWgradGroup = 16;
struct WgradArgs {
    const uint16_t *dOw, *dHU, *Xd, *A;
    int64_t stride;           // elements between consecutive tables' dOw, dHU, Xd and A buffers
    const int32_t *seg_off;   // table g: seg_off + g * (L + 1)
    const uint16_t *A_ring;   // ring slots of A, slot_elems apart
    int64_t slot_elems;
    int ring_slots, m0, M;    // table g is macrobatch m0 + g, in slot (M - 1 - m) % ring_slots
    uint32_t a_in_ring;
    int G;
    float *dW13, *dW2;
    int L, H, I;
    int accumulate;  // add to dW13 / dW2 instead of overwriting them
};

__device__ __forceinline__ const uint16_t *wgrad_A(const WgradArgs &a, int g) {
    if ((a.a_in_ring >> g) & 1u)
        return a.A_ring + (int64_t)((a.M - 1 - (a.m0 + g)) % a.ring_slots) * a.slot_elems;
    return a.A + g * a.stride;
}

// One output tile of dW2[l] (W2) or dW13[l]: the K loop over the expert's rows
// of every table of the group, then the fp32 store.
template <bool W2>
__device__ __forceinline__ void wgrad_tile(const WgradArgs &a, int l, int mt, int nt, char *lds) {
    const int H = a.H, I = a.I, L = a.L;
    AccW<kFwdWM, kFwdWN> acc;
    for (int g = 0; g < a.G; ++g) {
        const int32_t *so = a.seg_off + g * (L + 1);
        const int S = so[l];
        const int kext = so[l + 1] - S;  // padded: padding rows are zero in every operand
        const int64_t off = g * a.stride;
        if constexpr (W2) {
            const TOp ak{a.dOw + off + (int64_t)S * H + mt * 256, H, 256};
            const TOp bk{wgrad_A(a, g) + (int64_t)S * I + nt * 256, I, min(256, I - nt * 256)};
            gemm_mainloop_x<kFwdWM, kFwdWN, true, true>(ak, bk, kext / 64, false, lds, acc, g == 0);
        } else {
            const TOp ak{a.dHU + off + (int64_t)S * 2 * I + mt * 256, 2ll * I, 256};
            const TOp bk{a.Xd + off + (int64_t)S * H + nt * 256, H, 256};
            gemm_mainloop_x<kFwdWM, kFwdWN, true, true>(ak, bk, kext / 64, false, lds, acc, g == 0);
        }
    }
    if constexpr (W2)
        epilogue_store_f32_w<kFwdWM, kFwdWN>(acc, a.dW2 + (int64_t)l * H * I + (int64_t)mt * 256 * I + nt * 256, I, 256,
                                             I - nt * 256, a.accumulate);
    else
        epilogue_store_f32_w<kFwdWM, kFwdWN>(acc, a.dW13 + (int64_t)l * 2 * I * H + (int64_t)mt * 256 * H + nt * 256, H,
                                             256, 256, a.accumulate);
}

// B5: per expert, dW2[l] = sum_rows (w dO_d)^T a  and  dW13[l] = sum_rows dHU^T Xd,
// both operands the segment's activation rows read MN-contiguous (K = row).
// The K loop of an output tile runs over the expert's rows of table 0, then
// table 1, ... in ascending row order inside one workgroup, so the weight
// gradients of a group of tables take one pass ("Beyond Peak TFLOPs"
// section 2.C: deferred weight gradients accumulated over the token dimension
// in one pass).  Longest experts first.  The reverse-dispatch sum `c` (B4,
// HBM-bound) shares the launch as 64-token work items after the tiles (the
// deferred weight gradients overlap the last reverse-dispatch rounds).
// s_order[rank] = the local expert with the rank-th most rows over G tables
// (ties by ascending id); only for L <= 256.
__device__ __forceinline__ void experts_by_rows(const int32_t *seg_off, int L, int G, int *s_order) {
    __syncthreads();
    if (L <= 256) {
        for (int l = threadIdx.x; l < L; l += blockDim.x) {
            auto total = [&](int e) {
                int n = 0;
                for (int g = 0; g < G; ++g) n += seg_off[g * (L + 1) + e + 1] - seg_off[g * (L + 1) + e];
                return n;
            };
            const int len = total(l);
            int rank = 0;
            for (int q = 0; q < L; ++q) {
                const int lq = total(q);
                rank += (lq > len || (lq == len && q < l)) ? 1 : 0;
            }
            s_order[rank] = l;
        }
    }
    __syncthreads();
}

__device__ __forceinline__ void wgrad_phase(const WgradArgs &a, const WindowCombine &c, char *lds) {
    const int H = a.H, I = a.I, L = a.L, G = a.G;
    __shared__ int s_order[256];
    experts_by_rows(a.seg_off, L, G, s_order);
    const int mt2 = H / 256, nt2 = (I + 255) / 256;   // dW2 [H][I]
    const int mt13 = 2 * I / 256, nt13 = H / 256;      // dW13 [2I][H]
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
            wgrad_tile<true>(a, l, mt, nt, lds);
        } else {
            grouped_mn<4>(in - mt2 * nt2, mt13, nt13, mt, nt);
            wgrad_tile<false>(a, l, mt, nt, lds);
        }
    }
}

}  // namespace moe
