// On-device pull schedule: counting sort of routes into padded expert segments.
//
// Method ("Mixture-of-Kittens: A MoE Megakernel for GB300 NVL72", section 2,
// on-device schedule generation; "Scan once, scatter once", section "The fix
// is a counting sort"):
//   1. count routes per (local expert, partition, logical thread),
//   2. prefix the per-thread counts into thread-major offsets,
//   3. pad every expert segment to pad_rows and take its base row S[l],
//   4. scatter every route once to Phi[S[l] + p] with the stable cross-rank
//      position p = sum_r' min(M[l][r'], o) + #{r' < r : M[l][r'] > o}.
//
// CDNA4 mapping.  A logical thread is one wavefront that owns a contiguous
// chunk of kChunk routes of one partition (contiguous ownership is what makes
// the order stable, so the table does not depend on how many logical threads
// there are).  Inside a wave, 64 consecutive routes are ranked at once: lanes
// holding the same local expert find each other with one ballot per bit of the
// expert id, and a route's rank among them is a masked popcount, so the
// ordinal o of every route is its index order with no atomics.  Per-wave
// counters live in LDS.  A second pass (one workgroup per batch) turns the
// per-wave counts into exclusive offsets, the per-(expert, partition) counts
// M and the padded segment offsets S; a third places every route.  The count
// stage also leaves every route's local id as one byte, so the scatter reads
// a quarter of the ids' bytes the second time (the pages' design reads the
// ids twice).
#pragma once

#include "common.hpp"

namespace moe {

constexpr int kSchedUnroll = 16;                    // route loads in flight per lane
constexpr int kSchedBlock = kWave * kSchedUnroll;   // routes ranked per pass of a wave
constexpr int kSchedWaves = 4;                      // waves per workgroup of the standalone kernels
constexpr int kSchedPMax = 8;                       // partitions handled by the unrolled position formula

struct SchedArgs {
    const int32_t *routes;  // table b, partition r: R routes at b * bstride + r * pstride
    int32_t *counts;        // [nb][L][P]
    int32_t *seg_off;       // [nb][L+1]
    moe_src *phi;           // [nb][cap]
    int32_t *route_row;     // same layout as routes
    int32_t *wcnt;          // ws: [nb][P][W][L] counts, then exclusive offsets
    // Route ids outside [0, E): per chunk (ws, [nb][P][W], written by the
    // count stage) and per table (ws, [nb], their sum, written by the
    // finalize).  Such ids are never local; the sum lets a caller detect a
    // corrupt routing tensor without a host round trip.
    int32_t *winv;
    int32_t *invalid_ids;
    int32_t P, R, K, L, base, pad, nb, W, wg_per_part, nbits;
    int32_t E;
    int32_t wpw;  // waves per workgroup (chunks handled by one workgroup)
    int32_t cb;   // 1024-route blocks per chunk (a chunk is one logical thread)
    int64_t cap;
    // Element strides between tables and between partitions of a table: P * R
    // and R for nb whole routing tensors; B * K and Np * K when the tables are
    // the token windows [m B, (m + 1) B) of one [P][Np][K] tensor (macrobatches).
    int64_t bstride, pstride;
    // Local ids of every route as bytes, written by the count stage and read
    // by the scatter instead of the 4-byte ids (nullptr when L > 255: the
    // scatter then reads the ids again).  Block k of partition r of table b
    // is 1,024 bytes at ((b * P + r) * nblk + k) * 1024, lane l's 16 ids (its
    // routes lo + u * 64 + l) one 16-byte word at l * 16.
    uint8_t *ids8;
    int32_t nblk;  // blocks of kSchedBlock routes per partition
};

__device__ __forceinline__ uint8_t *ids8_block(const SchedArgs &a, int b, int r, int64_t blk) {
    return a.ids8 + (((int64_t)b * a.P + r) * a.nblk + blk) * kSchedBlock;
}

// Workgroup index -> (batch, partition, first chunk).  For eight or more
// batches the workgroups of one batch share an XCD (hardware deals workgroup
// ids round-robin over the 8 XCDs), so its table rows merge in one L2.
__device__ __forceinline__ bool sched_locate(const SchedArgs &a, int x, int &b, int &r, int &q) {
    int wg_per_batch = a.P * a.wg_per_part;
    int k;
    if (a.nb >= 8) {
        int xcd = x & 7, s = x >> 3;
        b = xcd + 8 * (s / wg_per_batch);
        k = s % wg_per_batch;
    } else {
        b = x / wg_per_batch;
        k = x % wg_per_batch;
    }
    if (b >= a.nb) return false;
    r = k / a.wg_per_part;
    q = k % a.wg_per_part;
    return true;
}

__device__ __forceinline__ uint32_t local_id(int32_t e, int base, int L) {
    uint32_t l = (uint32_t)(e - base);
    return l < (uint32_t)L ? l : (uint32_t)L;  // L = not local
}

// Exclusive prefix sum over the threads of the workgroup, in thread order
// (wave-level shuffles, then the per-wave totals through LDS).
__device__ __forceinline__ int32_t block_exclusive_scan(int32_t v, int32_t *tmp /* >= 16 ints */) {
    const int lane = lane_id(), w = threadIdx.x >> 6;
    int32_t x = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int32_t y = __shfl_up(x, off, kWave);
        if (lane >= off) x += y;
    }
    __syncthreads();
    if (lane == kWave - 1) tmp[w] = x;
    __syncthreads();
    int32_t base = 0;
    for (int i = 0; i < w; ++i) base += tmp[i];
    return base + x - v;
}

// Stages 2 and 3 for batch b: per (partition, expert) exclusive prefix of the
// per-chunk counts (in place), M[l][r], and the padded segment offsets S.
// smem: P*L + L + 17 ints.
__device__ void sched_finalize(const SchedArgs &a, int b, int32_t *smem) {
    const int L = a.L, P = a.P, W = a.W;
    int32_t *wc = a.wcnt + (int64_t)b * P * W * L;
    int32_t *cnt = a.counts + (int64_t)b * L * P;
    int32_t *s_tot = smem;          // [P][L]
    int32_t *s_len = s_tot + P * L; // [L]
    int32_t *s_tmp = s_len + L;     // [16]
    int32_t *s_inv = s_tmp + 16;    // [1]
    __syncthreads();
    if (threadIdx.x == 0) *s_inv = 0;
    __syncthreads();
    {  // ids outside [0, E) over the table's chunks (integer sum, exact in any order)
        const int32_t *wi = a.winv + (int64_t)b * P * W;
        int32_t n = 0;
        for (int i = threadIdx.x; i < P * W; i += blockDim.x) n += wi[i];
        if (n) __hip_atomic_fetch_add(s_inv, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    for (int pr = threadIdx.x; pr < P * L; pr += blockDim.x) {
        const int r = pr / L, l = pr % L;
        int32_t *col = wc + (int64_t)r * W * L + l;
        int32_t acc = 0;
        // batches of 16 chunks, loads first (predicated), so a column costs one
        // memory round trip per 16 chunks
        for (int w = 0; w < W; w += 16) {
            int32_t v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = w + u < W ? col[(int64_t)(w + u) * L] : 0;
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                if (w + u < W) col[(int64_t)(w + u) * L] = acc;
                acc += v[u];
            }
        }
        cnt[l * P + r] = acc;
        s_tot[pr] = acc;
    }
    __syncthreads();
    for (int l = threadIdx.x; l < L; l += blockDim.x) {
        int32_t t = 0;
        for (int r = 0; r < P; ++r) t += s_tot[r * L + l];
        s_len[l] = (t + a.pad - 1) / a.pad * a.pad;
    }
    __syncthreads();
    // each thread owns a contiguous run of experts; scan the run sums
    const int per = (L + blockDim.x - 1) / blockDim.x;
    const int lo = min(L, (int)threadIdx.x * per), hi = min(L, lo + per);
    int32_t sum = 0;
    for (int l = lo; l < hi; ++l) sum += s_len[l];
    int32_t acc = block_exclusive_scan(sum, s_tmp);
    int32_t *so = a.seg_off + (int64_t)b * (L + 1);
    for (int l = lo; l < hi; ++l) {
        so[l] = acc;
        acc += s_len[l];
    }
    if (threadIdx.x == blockDim.x - 1) so[L] = acc;  // the last thread's run ends at L
    __syncthreads();
    if (threadIdx.x == 0) a.invalid_ids[b] = *s_inv;
}

// Stage 1: per-chunk counts.  x is the workgroup's index in the schedule grid
// (a persistent caller loops over it).  Counting needs no ranks: every local
// lane adds one to its expert's LDS counter (integer adds, exact in any order).
__device__ void sched_count_body(const SchedArgs &a, int32_t *smem, int x) {
    int b, r, q;
    if (!sched_locate(a, x, b, r, q)) return;
    __syncthreads();  // LDS may still be in use by the caller's previous item
    const int lane = lane_id();
    const int wv = threadIdx.x / kWave;
    const int w = q * a.wpw + wv;  // chunk (logical thread) index in the partition
    const int L = a.L;
    int32_t *cnt = smem + wv * (L + 1);
    for (int l = lane; l <= L; l += kWave) cnt[l] = 0;
    __syncthreads();
    if (w < a.W) {
        const int32_t *src = a.routes + (int64_t)b * a.bstride + (int64_t)r * a.pstride;
        // the next block's ids are loaded while this one is counted
        auto load_block = [&](int64_t lo, int32_t (&e)[kSchedUnroll]) {
#pragma unroll
            for (int u = 0; u < kSchedUnroll; ++u) {
                const int64_t i = lo + u * kWave + lane;
                e[u] = i < a.R ? __builtin_nontemporal_load(src + i) : -1;
            }
        };
        int32_t e[kSchedUnroll];
        load_block((int64_t)w * a.cb * kSchedBlock, e);
        int32_t ninv = 0;
        for (int blk = 0; blk < a.cb; ++blk) {
            const int64_t lo = ((int64_t)w * a.cb + blk) * kSchedBlock;
            if (lo >= a.R) break;
            int32_t en[kSchedUnroll];
            if (blk + 1 < a.cb) load_block(lo + kSchedBlock, en);
            u32x4 word = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int u = 0; u < kSchedUnroll; ++u) {
                const uint32_t v = local_id(e[u], a.base, L);
                word[u >> 2] |= v << (8 * (u & 3));
                if (v < (uint32_t)L)
                    __hip_atomic_fetch_add(cnt + v, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                // ids outside [0, E) among the routes that exist (past R the
                // loads filled -1)
                ninv += (lo + u * kWave + lane < a.R && (uint32_t)e[u] >= (uint32_t)a.E) ? 1 : 0;
            }
            if (a.ids8)
                *reinterpret_cast<u32x4 *>(ids8_block(a, b, r, (int64_t)w * a.cb + blk) + lane * 16) = word;
#pragma unroll
            for (int u = 0; u < kSchedUnroll; ++u) e[u] = en[u];
        }
        if (ninv) __hip_atomic_fetch_add(cnt + L, ninv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    __syncthreads();
    if (w < a.W) {
        int32_t *dst = a.wcnt + (((int64_t)b * a.P + r) * a.W + w) * L;
        for (int l = lane; l < L; l += kWave) dst[l] = cnt[l];
        if (lane == 0) a.winv[((int64_t)b * a.P + r) * a.W + w] = cnt[L];
    }
}

// Places the routes of one block of kSchedBlock routes starting at route lo
// of partition r: lane l holds the local ids v[u] (L = not local) of routes
// lo + u * 64 + l.  (A) the local routes are compacted, in index order, into
// an LDS list (ballot + masked popcount give each local lane its slot); (B)
// the list is processed 64 entries at a time: lanes holding the same expert
// find each other with one ballot per bit of the expert id, the group leader
// advances the wave's running count for that expert with an LDS atomic
// (integer, program order) and the returned old value plus the lane's rank in
// its group is the ordinal o; then p and the row follow, Phi[row] is written
// and the row is staged in LDS at the route's place; (C) each lane writes its
// routes' rows, coalesced (-1 for the routes that are not local, which never
// touch LDS).  Only local routes pay for ranking and placement.  NB: bits of
// the expert ids ranked by an unrolled match (0: a runtime loop over a.nbits).
template <int NB>
__device__ __forceinline__ void place_block_n(const SchedArgs &a, const uint32_t (&v)[kSchedUnroll], int32_t lo,
                                              int r, const int32_t *sM, const int32_t *sS, int32_t *run,
                                              int32_t *list, int32_t *rowbuf, moe_src *phi, int32_t *rrow) {
    const int lane = lane_id();
    const int L = a.L, P = a.P;
    const uint32_t K = (uint32_t)a.K;
    const bool fast = P <= kSchedPMax;
    int nloc = 0;
#pragma unroll
    for (int u = 0; u < kSchedUnroll; ++u) {
        const bool local = v[u] < (uint32_t)L;
        const uint64_t lm = ballot(local);
        if (local) list[nloc + lanes_below(lm)] = (int32_t)((v[u] << 16) | (uint32_t)(u * kWave + lane));
        nloc += __popcll(lm);
    }
    const uint32_t t0 = (uint32_t)lo / K;  // lo >= 0
    const uint32_t j0 = (uint32_t)lo - t0 * K;
    for (int c0 = 0; c0 < nloc; c0 += kWave) {
        const bool valid = c0 + lane < nloc;
        const int32_t ent = valid ? list[c0 + lane] : (int32_t)((uint32_t)L << 16);
        const uint32_t e = (uint32_t)ent >> 16;
        const int32_t ib = ent & 0xffff;  // index inside the block
        uint64_t peers;
        if constexpr (NB > 0) peers = match_lanes_n<NB>(e);
        else peers = match_lanes(e, a.nbits);
        const int rank = lanes_below(peers);
        int32_t old = 0;
        if (rank == 0 && valid)
            old = __hip_atomic_fetch_add(run + e, (int32_t)__popcll(peers), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_WORKGROUP);
        const int32_t o = __shfl(old, (int)__builtin_ctzll(peers), kWave) + rank;
        if (valid) {
            int32_t p = 0;
            if (fast) {
                // min(m, o) + [m > o] = min(m, o + 1): partitions before r
                // count up to o + 1, the others up to o (r is wave-uniform)
                const int4 m0 = *reinterpret_cast<const int4 *>(sM + e * kSchedPMax);
                const int4 m1 = *reinterpret_cast<const int4 *>(sM + e * kSchedPMax + 4);
                const int32_t m[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
                for (int rr = 0; rr < kSchedPMax; ++rr) p += min(m[rr], rr < r ? o + 1 : o);
            } else {
                const int32_t *Ml = sM + e * P;
                for (int rr = 0; rr < P; ++rr) p += min(Ml[rr], rr < r ? o + 1 : o);
            }
            const int32_t row = sS[e] + p;
            const uint32_t jj = j0 + (uint32_t)ib;  // slot offset from token t0, < K + 1024
            const uint32_t t = t0 + jj / K;
            if ((uint32_t)row < (uint32_t)a.cap)  // always true for a consistent table
                reinterpret_cast<uint2 *>(phi)[row] = make_uint2((uint32_t)r, t);
            rowbuf[ib] = row;
        }
    }
    // (C) route rows of the block, coalesced; streamed past L2 (nontemporal) so
    // the partly written lines of Phi, which other partitions' workgroups fill
    // in, stay there longer
    const int32_t nb_routes = min(kSchedBlock, a.R - lo);
    int32_t rows[kSchedUnroll];
#pragma unroll
    for (int u = 0; u < kSchedUnroll; ++u) rows[u] = v[u] < (uint32_t)L ? rowbuf[u * kWave + lane] : -1;
#pragma unroll
    for (int u = 0; u < kSchedUnroll; ++u)
        if (u * kWave + lane < nb_routes) __builtin_nontemporal_store(rows[u], rrow + lo + u * kWave + lane);
}

__device__ __forceinline__ void place_block(const SchedArgs &a, const uint32_t (&v)[kSchedUnroll], int32_t lo, int r,
                                            const int32_t *sM, const int32_t *sS, int32_t *run, int32_t *list,
                                            int32_t *rowbuf, moe_src *phi, int32_t *rrow) {
    if (a.nbits <= 6) place_block_n<6>(a, v, lo, r, sM, sS, run, list, rowbuf, phi, rrow);
    else if (a.nbits <= 9) place_block_n<9>(a, v, lo, r, sM, sS, run, list, rowbuf, phi, rrow);
    else place_block_n<0>(a, v, lo, r, sM, sS, run, list, rowbuf, phi, rrow);
}

// Padding rows (-1, -1) of segments l = first, first + step, ... < L.
__device__ __forceinline__ void pad_segments(const SchedArgs &a, const int32_t *sM, int mstride, const int32_t *sS,
                                             moe_src *phi, int first, int step) {
    for (int l = first; l < a.L; l += step) {
        int32_t t = 0;
        for (int rr = 0; rr < a.P; ++rr) t += sM[l * mstride + rr];
        const int32_t hi = min(sS[l + 1], (int32_t)a.cap);  // sS[l + 1] <= cap for a consistent table
        for (int32_t row = max(sS[l] + t, 0) + threadIdx.x; row < hi; row += blockDim.x)
            reinterpret_cast<uint2 *>(phi)[row] = make_uint2(0xffffffffu, 0xffffffffu);
    }
}

// Stage 4: place every route once (place_block per block of the chunk).
__device__ void sched_scatter_body(const SchedArgs &a, int32_t *smem, int x) {
    int b, r, q;
    if (!sched_locate(a, x, b, r, q)) return;
    __syncthreads();
    const int lane = lane_id();
    const int wv = threadIdx.x / kWave;
    const int w = q * a.wpw + wv;
    const int L = a.L, P = a.P;
    const int mstride = P <= kSchedPMax ? kSchedPMax : P;
    // LDS: M [L][mstride] (zero-padded), S [L+1], then per wave: running
    // offsets [L], the compacted list [1024] and the staged route rows [1024]
    int32_t *sM = smem;
    int32_t *sS = sM + L * mstride;
    int32_t *wave_base = sS + L + 1 + wv * (L + 2 * kSchedBlock);
    int32_t *run = wave_base;
    int32_t *list = run + L;
    int32_t *rowbuf = list + kSchedBlock;
    const int32_t *cnt = a.counts + (int64_t)b * L * P;
    const int32_t *so = a.seg_off + (int64_t)b * (L + 1);
    for (int i = threadIdx.x; i < L * mstride; i += blockDim.x) {
        const int l = i / mstride, rr = i % mstride;
        sM[i] = rr < P ? cnt[l * P + rr] : 0;
    }
    for (int i = threadIdx.x; i <= L; i += blockDim.x) sS[i] = so[i];
    if (w < a.W) {
        const int32_t *off = a.wcnt + (((int64_t)b * P + r) * a.W + w) * L;
        for (int l = lane; l < L; l += kWave) run[l] = off[l];
    }
    __syncthreads();
    moe_src *phi = a.phi + (int64_t)b * a.cap;
    if (w < a.W) {
        const int32_t *src = a.routes + (int64_t)b * a.bstride + (int64_t)r * a.pstride;
        int32_t *rrow = a.route_row + (int64_t)b * a.bstride + (int64_t)r * a.pstride;
        for (int blk = 0; blk < a.cb; ++blk) {
            // 64-bit before the bound check: near R = 2^31 the block start of
            // a trailing block would not fit in 32 bits
            const int64_t lo64 = ((int64_t)w * a.cb + blk) * kSchedBlock;
            if (lo64 >= a.R) break;
            const int32_t lo = (int32_t)lo64;  // < R < 2^31
            uint32_t v[kSchedUnroll];
            if (a.ids8) {  // the count stage's bytes: a quarter of the ids' traffic
                const u32x4 word = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4 *>(ids8_block(a, b, r, w * a.cb + blk) + lane * 16));
#pragma unroll
                for (int u = 0; u < kSchedUnroll; ++u) v[u] = (word[u >> 2] >> (8 * (u & 3))) & 0xffu;
            } else {
                int32_t e[kSchedUnroll];
#pragma unroll
                for (int u = 0; u < kSchedUnroll; ++u) {
                    const int64_t i = lo64 + u * kWave + lane;
                    e[u] = i < a.R ? __builtin_nontemporal_load(src + i) : -1;
                }
#pragma unroll
                for (int u = 0; u < kSchedUnroll; ++u) v[u] = local_id(e[u], a.base, L);
            }
            place_block(a, v, lo, r, sM, sS, run, list, rowbuf, phi, rrow);
        }
    }
    // padding rows of the segments this workgroup owns
    __syncthreads();
    pad_segments(a, sM, mstride, sS, phi, r * a.wg_per_part + q, P * a.wg_per_part);
}

}  // namespace moe
