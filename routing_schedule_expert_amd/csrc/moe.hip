// C-ABI entry points and kernels of the MoE layer share (gfx950).
// The operations, their arguments and error behaviour are documented in
// include/moe.h; the device code lives in schedule.hpp, rowops.hpp, gemm.hpp
// and layer.hpp.
#include <hip/hip_runtime.h>

#include <string.h>

#include <mutex>
#include <vector>

#include "common.hpp"
#include "gemm.hpp"
#include "layer.hpp"
#include "mxbwd.hpp"
#include "rowops.hpp"
#include "schedule.hpp"

using namespace moe;

// ---------------------------------------------------------------------------
// Kernels.
// ---------------------------------------------------------------------------

__global__ void k_zero_u32(uint32_t *p, int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

__global__ __launch_bounds__(256) void k_sched_count(SchedArgs a) {
    extern __shared__ __attribute__((aligned(16))) int32_t sched_smem[];
    sched_count_body(a, sched_smem, blockIdx.x);
}

__global__ __launch_bounds__(256) void k_sched_finalize(SchedArgs a) {
    extern __shared__ __attribute__((aligned(16))) int32_t sched_smem[];
    sched_finalize(a, blockIdx.x, sched_smem);
}

__global__ __launch_bounds__(256) void k_sched_scatter(SchedArgs a) {
    extern __shared__ __attribute__((aligned(16))) int32_t sched_smem[];
    sched_scatter_body(a, sched_smem, blockIdx.x);
}

__global__ __launch_bounds__(256) void k_gather(const uint16_t *src, const moe_src *phi, const int32_t *npad_ptr,
                                                uint16_t *dst, int Np, int H, int64_t cap) {
    const int waves = blockDim.x / kWave;
    gather_rows_body(src, phi, npad_ptr, dst, Np, H, 0, cap, blockIdx.x * waves + threadIdx.x / kWave,
                     gridDim.x * waves);
}

__global__ __launch_bounds__(256) void k_gather_scaled(const uint16_t *src, const moe_src *phi,
                                                       const int32_t *npad_ptr, const float *wrow, uint16_t *dst,
                                                       uint16_t *dst_w, int Np, int H, int64_t cap) {
    const int waves = blockDim.x / kWave;
    gather_rows_scaled_body(src, phi, npad_ptr, wrow, dst, dst_w, Np, H, cap, blockIdx.x * waves + threadIdx.x / kWave,
                            gridDim.x * waves);
}

__global__ __launch_bounds__(256) void k_combine(const uint16_t *Y, const int32_t *route_row, const float *w,
                                                 uint16_t *out, int K, int H, int64_t ntok, int tpp,
                                                 int64_t tstride, const uint16_t *S, int skip_single) {
    const int waves = blockDim.x / kWave;
    combine_body(Y, route_row, w, out, K, H, 0, ntok, blockIdx.x * waves + threadIdx.x / kWave, gridDim.x * waves,
                 tpp, tstride, S, skip_single != 0);
}

// tab (see single_route_body) for every token of one table, (-1, 0) on its
// padding rows.
// With tpp > 0 the tokens are a window of tpp tokens per partition,
// partitions tstride apart (window_token).
__global__ __launch_bounds__(256) void k_single_route(const int32_t *route_row, const float *w, const moe_src *phi,
                                                      const int32_t *npad_ptr, int2 *tab, int K, int64_t ntok,
                                                      int tpp, int64_t tstride) {
    const int64_t npad = *npad_ptr, stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < ntok || i < npad; i += stride) {
        if (i < ntok) single_route_body(route_row, w, tab, K, window_token(i, tpp, tstride));
        if (i < npad) single_route_pad(phi, tab, i);
    }
}

// The shared expert's table: row g < ntok pulls token g (partition g / Np,
// token g % Np), rows [ntok, ntokp) are padding; one segment [0, ntokp).
__global__ __launch_bounds__(256) void k_identity_table(moe_src *phi, int32_t *seg_off, int Np, int64_t ntok,
                                                        int64_t ntokp) {
    for (int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; g < ntokp; g += (int64_t)gridDim.x * blockDim.x)
        reinterpret_cast<int2 *>(phi)[g] =
            g < ntok ? make_int2((int)(g / Np), (int)(g % Np)) : make_int2(-1, -1);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        seg_off[0] = 0;
        seg_off[1] = (int32_t)ntokp;
    }
}

__global__ __launch_bounds__(kFwdThreads) void k_dual_gateup(FfnArgs sh, FfnArgs r) {
    __shared__ __attribute__((aligned(16))) char lds[kGemmLds];
    dual_gateup_body(sh, r, lds);
}

__global__ __launch_bounds__(kFwdThreads) void k_dual_down(FfnArgs sh, FfnArgs r) {
    __shared__ __attribute__((aligned(16))) char lds[kGemmLds];
    dual_down_body(sh, r, lds);
}

__global__ __launch_bounds__(256) void k_row_weight(const moe_src *phi, const int32_t *npad_ptr,
                                                    const int32_t *route_row, const float *w, float *wrow, int Np,
                                                    int K, int64_t cap) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < cap; i += (int64_t)gridDim.x * blockDim.x)
        row_weight_body(phi, npad_ptr, route_row, w, wrow, Np, K, i);
}

__global__ __launch_bounds__(256) void k_dw_finalize(const int32_t *route_row, const float *part, int nparts,
                                                     float *dw, int64_t nslots, int spp, int64_t sstride) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nslots;
         i += (int64_t)gridDim.x * blockDim.x)
        dw_finalize_body(route_row, part, nparts, dw, i, spp, sstride);
}

__global__ __launch_bounds__(kFwdThreads) void k_ring_gateup_combine(FfnArgs a, WindowCombine c) {
    __shared__ __attribute__((aligned(16))) char lds[kGemmLds];
    ring_gateup_combine_body(a, c, lds);
}

__global__ __launch_bounds__(kFwdThreads) void k_ffn_gateup(FfnArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[kGemmLds];
    ffn_gateup_phase(a, lds);
}

__global__ __launch_bounds__(kFwdThreads) void k_ffn_down(FfnArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[kGemmLds];
    ffn_down_phase(a, lds);
}

// Wide-tile down projection: 8 waves, all 160 KiB of LDS, one workgroup per CU.
__global__ __launch_bounds__(kWideThreads) void k_ffn_down_w(FfnArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[kWideLds];
    wide_down_phase(a, lds);
}

__global__ __launch_bounds__(kFwdThreads) void k_ffn_chunked(FfnArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[kGemmLds];
    GridBarrier gb(a.bar);
    ffn_chunked_body(a, lds, gb);
}

__global__ __launch_bounds__(kFwdThreads) void k_layer_fwd_persistent(LayerFwdArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[kGemmLds];
    layer_fwd_persistent_body(a, lds);
}

__global__ __launch_bounds__(256) void k_mx_quantize(const uint16_t *src, int64_t nblocks, int K, uint8_t *q,
                                                    uint8_t *s) {
    for (int64_t b = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; b < nblocks; b += (int64_t)gridDim.x * blockDim.x)
        mx_quantize_block_bf16(src, K, q, s, b);
}

template <int SG>
__global__ __launch_bounds__(kFwdThreads) void k_mx_gateup(MxFfnArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[kMxLds];
    mx_gateup_phase<SG>(a, lds);
}

template <int SG>
__global__ __launch_bounds__(kFwdThreads) void k_mx_down(MxFfnArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[kMxLds];
    mx_down_phase<SG>(a, lds);
}

__global__ __launch_bounds__(kColqThreads) void k_mx_colq(ColQArgs a) {
    __shared__ __attribute__((aligned(16))) float st[kColqLds / 4];
    mx_colq_body(a, st);
}

template <int SG>
__global__ __launch_bounds__(kFwdThreads) void k_mx_bwd_down(MxBwdArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[kMxLds];
    mx_bwd_down_phase<SG>(a, lds);
}

template <int SG>
__global__ __launch_bounds__(kFwdThreads) void k_mx_bwd_gateup(MxBwdArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[kMxLds];
    mx_bwd_gateup_phase<SG>(a, lds);
}

__global__ __launch_bounds__(kFwdThreads) void k_mx_wgrad(MxWgradArgs a, WindowCombine c) {
    __shared__ __attribute__((aligned(16))) char lds[kMxLds + 256 * sizeof(int)];
    mx_wgrad_phase(a, c, lds);
}

__global__ __launch_bounds__(kFwdThreads) void k_bwd_down(BwdArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[kGemmLds];
    bwd_down_phase(a, lds);
}

__global__ __launch_bounds__(kFwdThreads) void k_bwd_gateup(BwdArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[kGemmLds];
    bwd_gateup_phase(a, lds);
}

__global__ __launch_bounds__(kFwdThreads) void k_wgrad(WgradArgs a, WindowCombine c) {
    __shared__ __attribute__((aligned(16))) char lds[kGemmLds];
    wgrad_phase(a, c, lds);
}

// ---------------------------------------------------------------------------
// Launch trace.
// ---------------------------------------------------------------------------

namespace {

struct TraceRec {
    char name[32];
    hipEvent_t start, stop;
};

std::mutex g_trace_mu;
std::vector<TraceRec> g_trace;
int g_trace_cap = 0;
int g_trace_used = 0;

struct TraceScope {
    TraceRec *rec = nullptr;
    hipStream_t stream;
    TraceScope(const char *name, hipStream_t s) : stream(s) {
        if (g_trace_used < g_trace_cap) {
            rec = &g_trace[g_trace_used++];
            strncpy(rec->name, name, 31);
            rec->name[31] = 0;
            (void)hipEventRecord(rec->start, s);
        }
    }
    ~TraceScope() {
        if (rec) (void)hipEventRecord(rec->stop, stream);
    }
};

// Per-device compute-unit count (the persistent grids are sized to it).
int device_cus() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

// Persistent GEMM grid: one workgroup per CU, rounded down to a multiple of 8
// (one per XCD) so the XCD-aware tile order stays exact.
int gemm_grid() {
    int g = device_cus();
    g -= g % 8;
    return g > 0 ? g : 8;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int check_desc(const moe_desc *d, bool need_ffn) {
    if (!d) return MOE_EINVAL;
    if (d->P < 1 || d->Np < 1 || d->K < 1 || d->E < 1 || d->L < 1 || d->pad_rows < 1 || d->sched_threads < 1)
        return MOE_EINVAL;
    if (d->expert_base < 0 || (int64_t)d->expert_base + d->L > d->E) return MOE_EINVAL;
    if (d->num_batches < 1) return MOE_EINVAL;
    const int64_t R = (int64_t)d->Np * d->K;
    const int64_t cap = (int64_t)d->P * R + (int64_t)d->L * (d->pad_rows - 1);
    if (R >= (1ll << 31) || cap >= (1ll << 31) - 256) return MOE_EUNSUPPORTED;
    if (d->L > 4096 || d->P > 4096 || (int64_t)d->L * d->P > 16384) return MOE_EUNSUPPORTED;
    if (need_ffn) {
        if (d->H < 1 || d->I < 1) return MOE_EINVAL;
        if (d->H % 256 || d->I % 128 || d->pad_rows % 256) return MOE_EUNSUPPORTED;
        // the GEMM launches number their tiles with 32-bit integers (far past
        // any shape whose buffers fit in device memory)
        const int64_t row_tiles = cap / 256 + 1, col_tiles = d->H / 128 + 2 * (int64_t)d->I / 128 + 2;
        const int64_t wgrad_tiles = (int64_t)d->L * (d->H / 256) * 3 * (d->I / 256 + 1);
        if (row_tiles * col_tiles + wgrad_tiles >= (1ll << 30)) return MOE_EUNSUPPORTED;
        // the wide down tiles address 384 rows of W2 and 256 rows of A with
        // 32-bit byte offsets below 1 GiB
        if (768ll * d->I >= (1ll << 30)) return MOE_EUNSUPPORTED;
    }
    return MOE_OK;
}

int64_t cap_rows(const moe_desc *d) {
    return (int64_t)d->P * d->Np * d->K + (int64_t)d->L * (d->pad_rows - 1);
}

// Rows of the shared expert's buffers: every token, rounded up to a tile.
int64_t shared_rows(const moe_desc *d) { return ((int64_t)d->P * d->Np + 255) / 256 * 256; }


// Blocks of kSchedBlock routes per logical thread: 1,024 routes for a single
// routing tensor (most parallelism), 4,096 when many tensors are scheduled
// together (fewer chunks).
int sched_cb(const moe_desc *d) { return (d->num_batches >= 8 ? 4096 : 1024) / kSchedBlock; }
static_assert(1024 % kSchedBlock == 0, "a logical thread holds whole blocks");
int sched_chunks(const moe_desc *d) {
    const int64_t chunk = (int64_t)kSchedBlock * sched_cb(d);
    return (int)(((int64_t)d->Np * d->K + chunk - 1) / chunk);
}
int sched_wg_per_part(const moe_desc *d) { return (sched_chunks(d) + kSchedWaves - 1) / kSchedWaves; }

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// Workspace of the shared expert's identity table: 2 offsets, then the rows.
int64_t shared_table_bytes(const moe_desc *d) { return 256 + align256(shared_rows(d) * 8); }

// Schedule workspace: the per-table count of route ids outside [0, E) (int32
// [nb], at byte 0, documented in moe.h), the per-chunk counts, the per-chunk
// invalid-id counts, then (L <= 255) every route's local id as a byte in
// blocks of kSchedBlock (SchedArgs::ids8).
int64_t sched_invalid_bytes(const moe_desc *d) { return align256(4ll * d->num_batches); }
int64_t sched_counts_bytes(const moe_desc *d) { return align256(4ll * d->num_batches * d->P * sched_chunks(d) * d->L); }
int64_t sched_winv_bytes(const moe_desc *d) { return align256(4ll * d->num_batches * d->P * sched_chunks(d)); }
int64_t sched_nblk(const moe_desc *d) { return ((int64_t)d->Np * d->K + kSchedBlock - 1) / kSchedBlock; }
int64_t sched_ids8_offset(const moe_desc *d) {
    return sched_invalid_bytes(d) + sched_counts_bytes(d) + sched_winv_bytes(d);
}
int64_t sched_ws_bytes(const moe_desc *d) {
    const int64_t ids = d->L <= 255 ? align256((int64_t)d->num_batches * d->P * sched_nblk(d) * kSchedBlock) : 0;
    return sched_ids8_offset(d) + ids;
}

// The forward's per-row table of single-route tokens (k_single_route): 8
// bytes per row of capacity, after the schedule's workspace.
int64_t single_route_bytes(const moe_desc *d) { return align256(cap_rows(d) * 8); }

int bwd_nparts(const moe_desc *d) { return (d->I + 255) / 256; }  // one dw partial per 256-column tile

// Backward workspace: dO_d, dXd, dO_d * w (bf16 [cap][H] each), dHU (bf16
// [cap][2I]), the row weights and the dw partials (fp32).
int64_t bwd_ws_bytes(const moe_desc *d) {
    const int64_t cap = cap_rows(d), H = d->H, I = d->I;
    return align256(cap * H * 2) * 3 + align256(cap * 2 * I * 2) + align256(cap * 4) +
           align256(cap * 4ll * bwd_nparts(d));
}

// MX backward workspace, after the bf16 backward's buffers: the row-quantized
// dO_d and dHU, and the four column-quantized operands of the weight
// gradients, transposed per expert segment (C codes per dispatched row).

// The MX buffers in carving order (the workspace fields MOE_WS_MX_*_Q / _S
// name them in this order from MOE_WS_MX_DHU_Q on).
enum MxBuf { kDOq, kDOs, kDHUq, kDHUs, kDOwTq, kDOwTs, kATq, kATs, kXdTq, kXdTs, kDHUTq, kDHUTs, kMxBufs };
static_assert(MOE_WS_MX_DHUT_S - MOE_WS_MX_DO_Q + 1 == kMxBufs, "one workspace field per MX buffer");

// The MX backward's bf16 / fp32 buffers: dXd [cap][H], dHU [cap][2I] (bf16),
// the row weights and the dw partials (fp32), at these offsets.
int64_t mx_dhu_offset(const moe_desc *d) { return align256(cap_rows(d) * d->H * 2); }
int64_t mx_wrow_offset(const moe_desc *d) { return mx_dhu_offset(d) + align256(cap_rows(d) * 2 * d->I * 2); }
int64_t mx_part_offset(const moe_desc *d) { return mx_wrow_offset(d) + align256(cap_rows(d) * 4); }

// Byte offsets of the MX code buffers after those; returns the total.
int64_t mx_bwd_offsets(const moe_desc *d, int64_t (&off)[kMxBufs]) {
    const int64_t cap = cap_rows(d), H = d->H, I = d->I;
    const int64_t bytes[kMxBufs] = {cap * H, cap * H / 32, cap * 2 * I, cap * 2 * I / 32,
                                    cap * H, cap * H / 32, cap * I,     cap * I / 32,
                                    cap * H, cap * H / 32, cap * 2 * I, cap * 2 * I / 32};
    int64_t o = mx_part_offset(d) + align256(cap * 4ll * bwd_nparts(d));
    for (int i = 0; i < kMxBufs; ++i) {
        off[i] = o;
        o += align256(bytes[i]);
    }
    return o;
}

struct MxBwdBufs {
    uint8_t *b[kMxBufs];
};

MxBwdBufs carve_mx_bwd(char *ws, const moe_desc *d) {
    int64_t off[kMxBufs];
    mx_bwd_offsets(d, off);
    MxBwdBufs m;
    for (int i = 0; i < kMxBufs; ++i) m.b[i] = reinterpret_cast<uint8_t *>(ws + off[i]);
    return m;
}

int64_t mx_bwd_ws_bytes(const moe_desc *d) {
    int64_t off[kMxBufs];
    return mx_bwd_offsets(d, off);
}

constexpr int64_t kBarrierBytes = 256;

int launch_status() { return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP; }

void fill_sched_args(SchedArgs &a, const moe_desc *d, const int32_t *routes, int32_t *counts, int32_t *seg_off,
                     moe_src *phi, int32_t *route_row, char *ws, int wpw) {
    a.routes = routes;
    a.counts = counts;
    a.seg_off = seg_off;
    a.phi = phi;
    a.route_row = route_row;
    a.invalid_ids = reinterpret_cast<int32_t *>(ws);
    a.wcnt = reinterpret_cast<int32_t *>(ws + sched_invalid_bytes(d));
    a.winv = reinterpret_cast<int32_t *>(ws + sched_invalid_bytes(d) + sched_counts_bytes(d));
    a.E = d->E;
    a.P = d->P;
    a.R = d->Np * d->K;
    a.K = d->K;
    a.L = d->L;
    a.base = d->expert_base;
    a.pad = d->pad_rows;
    a.nb = d->num_batches;
    a.W = sched_chunks(d);
    a.wpw = wpw;
    a.cb = sched_cb(d);
    a.wg_per_part = (a.W + wpw - 1) / wpw;
    a.nbits = 32 - __builtin_clz((unsigned)d->L | 1u);
    a.cap = cap_rows(d);
    a.pstride = a.R;
    a.bstride = (int64_t)a.P * a.R;
    a.ids8 = d->L <= 255 ? reinterpret_cast<uint8_t *>(ws + sched_ids8_offset(d)) : nullptr;
    a.nblk = (int32_t)sched_nblk(d);
}

constexpr size_t kMaxLds = 160 * 1024;  // LDS of one gfx950 workgroup

// LDS (bytes) of each schedule body for `wpw` waves per workgroup (stage 0
// count, 1 finalize, 2 scatter; -1: the largest, for a caller running all three).
size_t sched_lds_bytes(const moe_desc *d, int wpw, int stage = -1) {
    const size_t L = d->L, P = d->P;
    const size_t mstride = P <= (size_t)kSchedPMax ? (size_t)kSchedPMax : P;
    size_t count = wpw * (L + 1), fin = P * L + L + 17, scat = L * mstride + L + 1 + wpw * (L + 2 * kSchedBlock);
    if (stage == 0) return 4 * count;
    if (stage == 1) return 4 * fin;
    if (stage == 2) return 4 * scat;
    return 4 * std::max(count, std::max(fin, scat));
}

// pstride / bstride > 0: the tables are token windows of one routing tensor
// (SchedArgs); 0 keeps whole tensors.
int launch_schedule(const moe_desc *d, const int32_t *routes, int32_t *counts, int32_t *seg_off, moe_src *phi,
                    int32_t *route_row, char *ws, hipStream_t s, int64_t pstride = 0, int64_t bstride = 0) {
    SchedArgs a;
    fill_sched_args(a, d, routes, counts, seg_off, phi, route_row, ws, kSchedWaves);
    if (pstride > 0) a.pstride = pstride;
    if (bstride > 0) a.bstride = bstride;
    const int wg_per_batch = a.P * a.wg_per_part;
    const int grid = a.nb >= 8 ? 8 * ((a.nb + 7) / 8) * wg_per_batch : a.nb * wg_per_batch;
    if (sched_lds_bytes(d, kSchedWaves) > kMaxLds) return MOE_EUNSUPPORTED;
    {
        TraceScope tr("sched_count", s);
        hipLaunchKernelGGL(k_sched_count, dim3(grid), dim3(64 * kSchedWaves), sched_lds_bytes(d, kSchedWaves, 0), s,
                           a);
    }
    if (launch_status() != MOE_OK) return MOE_EHIP;
    {
        TraceScope tr("sched_finalize", s);
        hipLaunchKernelGGL(k_sched_finalize, dim3(a.nb), dim3(256), sched_lds_bytes(d, kSchedWaves, 1), s, a);
    }
    if (launch_status() != MOE_OK) return MOE_EHIP;
    {
        TraceScope tr("sched_scatter", s);
        hipLaunchKernelGGL(k_sched_scatter, dim3(grid), dim3(64 * kSchedWaves), sched_lds_bytes(d, kSchedWaves, 2),
                           s, a);
    }
    return launch_status();
}

// np_stride > 0: source rows part * np_stride + tok (a token window of a
// larger [P][np_stride] array, src pointing at the window's first token).
int launch_gather(const moe_desc *d, const uint16_t *src, const moe_src *phi, const int32_t *seg_off, uint16_t *dst,
                  hipStream_t s, const char *name, int np_stride = 0) {
    const int64_t cap = cap_rows(d);
    const int grid = (int)std::min<int64_t>((cap + 3) / 4, 16ll * device_cus());
    TraceScope tr(name, s);
    hipLaunchKernelGGL(k_gather, dim3(grid), dim3(256), 0, s, src, phi, seg_off + d->L, dst,
                       np_stride > 0 ? np_stride : d->Np, d->H, cap);
    return launch_status();
}

// tstride > d->Np: the d->Np tokens of each partition are a window of a
// [P][tstride] token array (route_row, w, out pointing at its first token).
// S (nullable): the shared expert's output rows [P*Np][H], added per token.
int launch_combine(const moe_desc *d, const uint16_t *Y, const int32_t *route_row, const float *w, uint16_t *out,
                   hipStream_t s, const char *name, int64_t tstride = 0, const uint16_t *S = nullptr,
                   bool skip_single = false) {
    const int64_t ntok = (int64_t)d->P * d->Np;
    const int grid = (int)std::min<int64_t>((ntok + 3) / 4, 16ll * device_cus());
    const int tpp = tstride > d->Np ? d->Np : 0;
    TraceScope tr(name, s);
    hipLaunchKernelGGL(k_combine, dim3(grid), dim3(256), 0, s, Y, route_row, w, out, d->K, d->H, ntok, tpp,
                       tpp ? tstride : (int64_t)0, S, skip_single ? 1 : 0);
    return launch_status();
}

// The per-row table of the tokens with one local route (in the workspace
// after the schedule's part) and the epilogue arguments that use it.
int launch_single_route(const moe_desc *d, const int32_t *route_row, const moe_src *phi, const int32_t *seg_off,
                        const float *w, uint16_t *out, char *ws, hipStream_t s, RowCombine &rcomb,
                        int64_t tstride = 0) {
    int2 *tab = reinterpret_cast<int2 *>(ws);
    const int64_t ntok = (int64_t)d->P * d->Np, n = std::max<int64_t>(ntok, cap_rows(d));
    const int tpp = tstride > d->Np ? d->Np : 0;
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 4ll * device_cus()));
    TraceScope tr("single_route", s);
    hipLaunchKernelGGL(k_single_route, dim3(grid), dim3(256), 0, s, route_row, w, phi, seg_off + d->L, tab, d->K,
                       ntok, tpp, tpp ? tstride : (int64_t)0);
    rcomb = RowCombine{out, tab};
    return launch_status();
}

FfnArgs make_ffn_args(const moe_desc *d, const uint16_t *Xd, const uint16_t *W13, const uint16_t *W2,
                      const int32_t *seg_off, uint16_t *HU, uint16_t *A, uint16_t *Y, int32_t chunk_rows,
                      uint32_t *bar, const uint16_t *X = nullptr, const moe_src *phi = nullptr) {
    FfnArgs a;
    a.Xd = Xd;
    a.X = X;
    a.phi = phi;
    a.Np = d->Np;
    a.W13 = W13;
    a.W2 = W2;
    a.seg_off = seg_off;
    a.HU = HU;
    a.A = A;
    a.Y = Y;
    a.L = d->L;
    a.H = d->H;
    a.I = d->I;
    a.chunk_rows = chunk_rows;
    a.bar = bar;
    a.rc = RowCombine{nullptr, nullptr};
    return a;
}

int launch_cooperative(const void *fn, int grid, void **args, hipStream_t s) {
    hipError_t e = hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kFwdThreads), args, 0, s);
    return e == hipSuccess ? MOE_OK : MOE_EHIP;
}

int launch_ffn(const moe_desc *d, const FfnArgs &a, hipStream_t s) {
    const int grid = gemm_grid();
    if (a.chunk_rows <= 0) {
        {
            TraceScope tr("ffn_gateup", s);
            hipLaunchKernelGGL(k_ffn_gateup, dim3(grid), dim3(kFwdThreads), 0, s, a);
        }
        if (launch_status() != MOE_OK) return MOE_EHIP;
        TraceScope tr("ffn_down", s);
        hipLaunchKernelGGL(k_ffn_down_w, dim3(grid), dim3(kWideThreads), 0, s, a);
        return launch_status();
    }
    {
        TraceScope tr("ffn_barrier_zero", s);
        hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(64), 0, s, a.bar, (int64_t)(kBarrierBytes / 4));
    }
    if (launch_status() != MOE_OK) return MOE_EHIP;
    FfnArgs copy = a;
    void *args[] = {&copy};
    TraceScope tr("ffn_chunked", s);
    return launch_cooperative(reinterpret_cast<const void *>(k_ffn_chunked), grid, args, s);
}

bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; }

int launch_mx_quantize(const uint16_t *src, int64_t rows, int32_t K, uint8_t *q, uint8_t *sc, hipStream_t s,
                       const char *name) {
    const int64_t nblocks = rows * (K / 32);
    if (nblocks == 0) return MOE_OK;
    const int grid = (int)std::min<int64_t>((nblocks + 255) / 256, 16ll * device_cus());
    TraceScope tr(name, s);
    hipLaunchKernelGGL(k_mx_quantize, dim3(grid), dim3(256), 0, s, src, nblocks, (int)K, q, sc);
    return launch_status();
}

// Workspace of moe_layer_fwd_noalloc: a static device array, one copy per GPU
// the library runs on, held until the process ends.  Host code never passes
// `scratch` itself to a kernel (in host code the name is only a stand-in for
// the symbol): the device address comes from hipGetSymbolAddress, once per
// device, with that device current.
constexpr int64_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte workspace blocks");
static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[64] = {};

int scratch_for_current_device(char **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_EHIP;
    if (dev < 0 || dev >= 64) return MOE_EUNSUPPORTED;
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_EHIP;
        g_scratch_ptr[dev] = p;
    }
    *out = static_cast<char *>(g_scratch_ptr[dev]);
    return MOE_OK;
}

// status[0] = the invalid-id count, status[1] = the barrier word when the
// call waited across workgroups (else 0: the word is left from earlier calls).
__global__ void k_copy_status(const char *ws, int64_t inv_off, int64_t bar_off, int waited, int32_t *status) {
    if (threadIdx.x == 0) {
        status[0] = *reinterpret_cast<const int32_t *>(ws + inv_off);
        status[1] = waited ? *reinterpret_cast<const int32_t *>(ws + bar_off) : 0;
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI.
// ---------------------------------------------------------------------------

extern "C" {

const char *moe_strerror(int code) {
    switch (code) {
        case MOE_OK: return "ok";
        case MOE_EINVAL: return "invalid argument (dimension, NULL or misaligned pointer)";
        case MOE_ENOSPC: return "workspace or capacity too small";
        case MOE_EUNSUPPORTED: return "unsupported shape";
        case MOE_EHIP: return "HIP launch or runtime error";
        default: return "unknown error";
    }
}

int64_t moe_capacity_rows(const moe_desc *d) {
    if (check_desc(d, false) != MOE_OK) return -1;
    return cap_rows(d);
}

int64_t moe_workspace_bytes(const moe_desc *d, int op) {
    const bool ffn = op == MOE_OP_EXPERT_FFN || op == MOE_OP_LAYER_FWD || op == MOE_OP_LAYER_BWD ||
                     op == MOE_OP_DISPATCH || op == MOE_OP_COMBINE || op == MOE_OP_LAYER_FWD_SHARED ||
                     op == MOE_OP_LAYER_BWD_MX;
    if (check_desc(d, ffn) != MOE_OK) return -1;
    switch (op) {
        case MOE_OP_SCHEDULE: return sched_ws_bytes(d);
        case MOE_OP_DISPATCH:
        case MOE_OP_COMBINE: return 0;
        case MOE_OP_EXPERT_FFN: return kBarrierBytes;
        case MOE_OP_LAYER_FWD: {
            moe_desc one = *d;
            one.num_batches = 1;
            return kBarrierBytes + sched_ws_bytes(&one) + single_route_bytes(d);
        }
        case MOE_OP_LAYER_BWD: return bwd_ws_bytes(d);
        case MOE_OP_LAYER_BWD_MX: return mx_bwd_ws_bytes(d);
        case MOE_OP_LAYER_FWD_SHARED: {
            moe_desc one = *d;
            one.num_batches = 1;
            return kBarrierBytes + sched_ws_bytes(&one) + shared_table_bytes(d);
        }
        default: return -1;
    }
}

int64_t moe_workspace_field(const moe_desc *d, int op, int field) {
    if (moe_workspace_bytes(d, op) < 0) return -1;
    // barrier words (LAYER_FWD, EXPERT_FFN) at byte 0, word 2 the give-up
    // flag; the schedule's workspace after them (LAYER_FWD, LAYER_FWD_SHARED)
    // or alone (SCHEDULE), its invalid-id counts at its byte 0
    if (field == MOE_WS_INVALID_IDS) {
        if (op == MOE_OP_SCHEDULE) return 0;
        if (op == MOE_OP_LAYER_FWD || op == MOE_OP_LAYER_FWD_SHARED) return kBarrierBytes;
        return -1;
    }
    if (field == MOE_WS_BARRIER_STATUS) {
        if (op == MOE_OP_LAYER_FWD || op == MOE_OP_EXPERT_FFN) return 8;
        return -1;
    }
    if (field == MOE_WS_SINGLE_ROUTE) {
        if (op != MOE_OP_LAYER_FWD) return -1;
        moe_desc one = *d;
        one.num_batches = 1;
        return kBarrierBytes + sched_ws_bytes(&one);
    }
    if (op == MOE_OP_LAYER_BWD_MX) {
        // the bf16 backward's dHU follows dO_d, dXd and dO_d w
        if (field == MOE_WS_MX_DHU) return mx_dhu_offset(d);
        int64_t off[kMxBufs];
        mx_bwd_offsets(d, off);
        if (field >= MOE_WS_MX_DO_Q && field < MOE_WS_MX_DO_Q + kMxBufs) return off[field - MOE_WS_MX_DO_Q];
    }
    return -1;
}

int moe_schedule(const moe_desc *d, const int32_t *routes, int32_t *counts, int32_t *seg_off, moe_src *phi,
                 int32_t *route_row, void *ws, size_t ws_bytes, void *stream) {
    int rc = check_desc(d, false);
    if (rc != MOE_OK) return rc;
    if (!routes || !counts || !seg_off || !phi || !route_row || !ws) return MOE_EINVAL;
    if (!aligned16(routes) || !aligned16(counts) || !aligned16(seg_off) || !aligned16(phi) ||
        !aligned16(route_row) || !aligned16(ws))
        return MOE_EINVAL;
    if ((int64_t)ws_bytes < sched_ws_bytes(d)) return MOE_ENOSPC;
    return launch_schedule(d, routes, counts, seg_off, phi, route_row, static_cast<char *>(ws),
                           static_cast<hipStream_t>(stream));
}

int moe_dispatch(const moe_desc *d, const uint16_t *X, const moe_src *phi, const int32_t *seg_off, uint16_t *Xd,
                 void *stream) {
    if (!d) return MOE_EINVAL;
    int rc = check_desc(d, false);
    if (rc != MOE_OK) return rc;
    if (d->H < 8 || d->H % 8) return d->H < 1 ? MOE_EINVAL : MOE_EUNSUPPORTED;
    if (!X || !phi || !seg_off || !Xd) return MOE_EINVAL;
    if (!aligned16(X) || !aligned16(phi) || !aligned16(Xd)) return MOE_EINVAL;
    return launch_gather(d, X, phi, seg_off, Xd, static_cast<hipStream_t>(stream), "dispatch");
}

int moe_combine(const moe_desc *d, const uint16_t *Y, const int32_t *route_row, const float *w, uint16_t *out,
                void *stream) {
    if (!d) return MOE_EINVAL;
    int rc = check_desc(d, false);
    if (rc != MOE_OK) return rc;
    if (d->H < 8 || d->H % 8) return d->H < 1 ? MOE_EINVAL : MOE_EUNSUPPORTED;
    if (!Y || !route_row || !out) return MOE_EINVAL;
    if (!aligned16(Y) || !aligned16(out)) return MOE_EINVAL;
    return launch_combine(d, Y, route_row, w, out, static_cast<hipStream_t>(stream), w ? "combine" : "combine_unweighted");
}

int moe_expert_ffn(const moe_desc *d, const uint16_t *Xd, const uint16_t *W13, const uint16_t *W2,
                   const int32_t *seg_off, uint16_t *HU, uint16_t *A, uint16_t *Y, int32_t chunk_rows, void *ws,
                   size_t ws_bytes, void *stream) {
    int rc = check_desc(d, true);
    if (rc != MOE_OK) return rc;
    if (!Xd || !W13 || !W2 || !seg_off || !A || !Y) return MOE_EINVAL;
    if (!aligned16(Xd) || !aligned16(W13) || !aligned16(W2) || !aligned16(A) || !aligned16(Y) ||
        (HU && !aligned16(HU)))
        return MOE_EINVAL;
    if (chunk_rows < 0 || chunk_rows % 256) return MOE_EINVAL;
    if (chunk_rows > 0 && (!ws || !aligned16(ws) || ws_bytes < (size_t)kBarrierBytes)) return ws ? MOE_ENOSPC : MOE_EINVAL;
    FfnArgs a = make_ffn_args(d, Xd, W13, W2, seg_off, HU, A, Y, chunk_rows, static_cast<uint32_t *>(ws));
    return launch_ffn(d, a, static_cast<hipStream_t>(stream));
}

int moe_layer_fwd_noalloc(const moe_desc *d, const int32_t *routes, const float *w, const uint16_t *X,
                          const uint16_t *W13, const uint16_t *W2, int32_t *counts, int32_t *seg_off, moe_src *phi,
                          int32_t *route_row, uint16_t *Xd, uint16_t *HU, uint16_t *A, uint16_t *Y, uint16_t *out,
                          int32_t flags, int32_t chunk_rows, int32_t *status, void *stream) {
    int rc = check_desc(d, true);
    if (rc != MOE_OK) return rc;
    if (moe_workspace_bytes(d, MOE_OP_LAYER_FWD) > kScratchBytes) return MOE_ENOSPC;
    if (status && ((uintptr_t)status & 3u)) return MOE_EINVAL;
    char *ws = nullptr;
    rc = scratch_for_current_device(&ws);
    if (rc != MOE_OK) return rc;
    rc = moe_layer_fwd(d, routes, w, X, W13, W2, counts, seg_off, phi, route_row, Xd, HU, A, Y, out, flags,
                       chunk_rows, ws, (size_t)kScratchBytes, stream);
    if (rc != MOE_OK || !status) return rc;
    const int waited = (flags & MOE_PERSISTENT) || chunk_rows > 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    TraceScope tr("noalloc_status", s);
    hipLaunchKernelGGL(k_copy_status, dim3(1), dim3(64), 0, s, ws,
                       moe_workspace_field(d, MOE_OP_LAYER_FWD, MOE_WS_INVALID_IDS),
                       moe_workspace_field(d, MOE_OP_LAYER_FWD, MOE_WS_BARRIER_STATUS), waited, status);
    return launch_status();
}

int moe_layer_fwd(const moe_desc *d, const int32_t *routes, const float *w, const uint16_t *X, const uint16_t *W13,
                  const uint16_t *W2, int32_t *counts, int32_t *seg_off, moe_src *phi, int32_t *route_row,
                  uint16_t *Xd, uint16_t *HU, uint16_t *A, uint16_t *Y, uint16_t *out, int32_t flags,
                  int32_t chunk_rows, void *ws, size_t ws_bytes, void *stream) {
    int rc = check_desc(d, true);
    if (rc != MOE_OK) return rc;
    if (d->num_batches != 1) return MOE_EINVAL;
    if (!routes || !w || !X || !W13 || !W2 || !counts || !seg_off || !phi || !route_row || !A || !Y || !out || !ws)
        return MOE_EINVAL;
    const void *ptrs[] = {routes, w, X, W13, W2, counts, seg_off, phi, route_row, A, Y, out, ws};
    for (const void *p : ptrs)
        if (!aligned16(p)) return MOE_EINVAL;
    if ((HU && !aligned16(HU)) || (Xd && !aligned16(Xd))) return MOE_EINVAL;
    if (!Xd && d->H > kZeroRowElems) return MOE_EUNSUPPORTED;  // padding rows read the static zero row
    if (chunk_rows < 0 || chunk_rows % 256) return MOE_EINVAL;
    if (flags & ~MOE_PERSISTENT) return MOE_EINVAL;
    if ((int64_t)ws_bytes < moe_workspace_bytes(d, MOE_OP_LAYER_FWD)) return MOE_ENOSPC;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *wsb = static_cast<char *>(ws);
    uint32_t *bar = reinterpret_cast<uint32_t *>(wsb);
    char *sched_ws = wsb + kBarrierBytes;
    if (flags & MOE_PERSISTENT) {
        LayerFwdArgs la;
        moe_desc one = *d;
        one.num_batches = 1;
        if (sched_lds_bytes(&one, kFwdThreads / 64) > (size_t)kGemmLds) return MOE_EUNSUPPORTED;
        fill_sched_args(la.sched, &one, routes, counts, seg_off, phi, route_row, sched_ws, kFwdThreads / 64);
        la.ffn = make_ffn_args(d, Xd, W13, W2, seg_off, HU, A, Y, chunk_rows, bar, X, phi);
        la.X = X;
        la.w = w;
        la.out = out;
        la.Np = d->Np;
        la.K = d->K;
        la.ntok = (int64_t)d->P * d->Np;
        la.cap = cap_rows(d);
        {
            TraceScope tr("layer_zero", s);
            hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(64), 0, s, bar, (int64_t)(kBarrierBytes / 4));
        }
        if (launch_status() != MOE_OK) return MOE_EHIP;
        void *args[] = {&la};
        TraceScope tr("layer_fwd_persistent", s);
        return launch_cooperative(reinterpret_cast<const void *>(k_layer_fwd_persistent), gemm_grid(), args, s);
    }
    moe_desc one = *d;
    one.num_batches = 1;
    rc = launch_schedule(&one, routes, counts, seg_off, phi, route_row, sched_ws, s);
    if (rc != MOE_OK) return rc;
    if (Xd) {
        rc = launch_gather(d, X, phi, seg_off, Xd, s, "dispatch");
        if (rc != MOE_OK) return rc;
    }
    FfnArgs a = make_ffn_args(d, Xd, W13, W2, seg_off, HU, A, Y, chunk_rows, bar, X, phi);
    // with the wide down tiles, the tokens that have one local route are
    // combined in the down GEMM's epilogue and the combine launch skips them
    const bool fused = chunk_rows <= 0;
    if (fused) {
        rc = launch_single_route(d, route_row, phi, seg_off, w, out, sched_ws + sched_ws_bytes(&one), s, a.rc);
        if (rc != MOE_OK) return rc;
    }
    rc = launch_ffn(d, a, s);
    if (rc != MOE_OK) return rc;
    return launch_combine(d, Y, route_row, w, out, s, "combine", 0, nullptr, fused);
}

}  // extern "C"

namespace {

// Per-table backward buffers: the gathered output gradient and its rows times
// w, the row gradients, the row weights and the dw partials.
struct BwdBufs {
    uint16_t *dOd, *dOw, *dXd, *dHU;
    float *wrow, *part;
};

BwdBufs carve_bwd(char *p, const moe_desc *d) {
    const int64_t cap = cap_rows(d), H = d->H, I = d->I;
    BwdBufs b;
    b.dOd = reinterpret_cast<uint16_t *>(p);
    p += align256(cap * H * 2);
    b.dXd = reinterpret_cast<uint16_t *>(p);
    p += align256(cap * H * 2);
    b.dOw = reinterpret_cast<uint16_t *>(p);
    p += align256(cap * H * 2);
    b.dHU = reinterpret_cast<uint16_t *>(p);
    p += align256(cap * 2 * I * 2);
    b.wrow = reinterpret_cast<float *>(p);
    p += align256(cap * 4);
    b.part = reinterpret_cast<float *>(p);
    return b;
}

// The router weight of every dispatched row of one table.
int launch_row_weight(const moe_desc *d, int64_t tstride, const float *w, const moe_src *phi,
                      const int32_t *route_row, const int32_t *seg_off, float *wrow, hipStream_t s) {
    const int64_t cap = cap_rows(d);
    const int np_stride = tstride > d->Np ? (int)tstride : d->Np;
    TraceScope tr("bwd_row_weight", s);
    hipLaunchKernelGGL(k_row_weight, dim3((int)std::min<int64_t>((cap + 255) / 256, 4096)), dim3(256), 0, s, phi,
                       seg_off + d->L, route_row, w, wrow, np_stride, d->K, cap);
    return launch_status();
}

// The row weights and B1 of one table: the reverse-combine gather of the
// output gradient (dO_d) and its rows times w (dO_d w).
int bwd_gather(const moe_desc *d, int64_t tstride, const uint16_t *dOut, const float *w, const moe_src *phi,
               const int32_t *route_row, const int32_t *seg_off, const BwdBufs &bb, hipStream_t s) {
    const int64_t cap = cap_rows(d);
    const bool window = tstride > d->Np;
    const int32_t *npad = seg_off + d->L;
    const int np_stride = window ? (int)tstride : d->Np;
    if (launch_row_weight(d, tstride, w, phi, route_row, seg_off, bb.wrow, s) != MOE_OK) return MOE_EHIP;
    const int grid = (int)std::min<int64_t>((cap + 3) / 4, 16ll * device_cus());
    TraceScope tr("bwd_gather", s);
    hipLaunchKernelGGL(k_gather_scaled, dim3(grid), dim3(256), 0, s, dOut, phi, npad, bb.wrow, bb.dOd, bb.dOw,
                       np_stride, d->H, cap);
    return launch_status();
}

// The data gradients of one table's rows (B1, B2, dw, B3).  d describes the
// tokens the table covers (a window of tstride tokens per partition when
// tstride > d->Np: dOut, w, route_row and dw then point at the window's first
// token).
int bwd_dgrad(const moe_desc *d, int64_t tstride, const uint16_t *dOut, const float *w, const moe_src *phi,
              const int32_t *route_row, const int32_t *seg_off, const uint16_t *HU, const uint16_t *A,
              const uint16_t *W13, const uint16_t *W2, float *dw, const BwdBufs &bb, hipStream_t s) {
    const int64_t cap = cap_rows(d);
    const bool window = tstride > d->Np;
    BwdArgs a;
    a.dOd = bb.dOd;
    a.dXd = bb.dXd;
    a.dHU = bb.dHU;
    a.wrow = bb.wrow;
    a.part = bb.part;
    a.HU = HU;
    a.A = A;
    a.W13 = W13;
    a.W2 = W2;
    a.seg_off = seg_off;
    a.L = d->L;
    a.H = d->H;
    a.I = d->I;
    a.nparts = bwd_nparts(d);
    int rc = bwd_gather(d, tstride, dOut, w, phi, route_row, seg_off, bb, s);
    if (rc != MOE_OK) return rc;
    const int grid = gemm_grid();
    // B2: down-projection dgrad with the SwiGLU backward and dw partials
    {
        TraceScope tr("bwd_down", s);
        hipLaunchKernelGGL(k_bwd_down, dim3(grid), dim3(kFwdThreads), 0, s, a);
    }
    if (launch_status() != MOE_OK) return MOE_EHIP;
    const int64_t nslots = (int64_t)d->P * d->Np * d->K;
    {
        TraceScope tr("bwd_dw", s);
        hipLaunchKernelGGL(k_dw_finalize, dim3((int)std::min<int64_t>((nslots + 255) / 256, 4096)), dim3(256), 0, s,
                           route_row, bb.part, a.nparts, dw, nslots, window ? d->Np * d->K : 0,
                           window ? tstride * d->K : (int64_t)0);
    }
    if (launch_status() != MOE_OK) return MOE_EHIP;
    // B3: gate/up dgrad
    TraceScope tr("bwd_gateup", s);
    hipLaunchKernelGGL(k_bwd_gateup, dim3(grid), dim3(kFwdThreads), 0, s, a);
    return launch_status();
}

// B4 of one table: the reverse-dispatch sum of its tokens' row gradients.
WindowCombine reverse_dispatch(const moe_desc *d, int64_t tstride, const uint16_t *dXd, const int32_t *route_row,
                               uint16_t *dX) {
    const bool window = tstride > d->Np;
    WindowCombine rd{};
    rd.Y = dXd;
    rd.route_row = route_row;
    rd.w = nullptr;
    rd.out = dX;
    rd.K = d->K;
    rd.H = d->H;
    rd.tpp = window ? d->Np : 0;
    rd.ntok = (int64_t)d->P * d->Np;
    rd.tstride = window ? tstride : 0;
    return rd;
}

// B5 over the tables of `wa`, in one launch with the reverse dispatch `rd`
// (Y == nullptr: none).
int launch_wgrad(const WgradArgs &wa, const WindowCombine &rd, hipStream_t s) {
    TraceScope tr("bwd_wgrad_rdispatch", s);
    hipLaunchKernelGGL(k_wgrad, dim3(gemm_grid()), dim3(kFwdThreads), 0, s, wa, rd);
    return launch_status();
}

// B5 arguments for table 0 at the given buffers; more tables follow at
// `stride` elements (set by the caller).
WgradArgs wgrad_args(const moe_desc *d, const uint16_t *dOw, const uint16_t *A, const uint16_t *dHU,
                     const uint16_t *Xd, const int32_t *seg_off, float *dW13, float *dW2, bool accumulate) {
    WgradArgs wa{};
    wa.dOw = dOw;
    wa.A = A;
    wa.dHU = dHU;
    wa.Xd = Xd;
    wa.seg_off = seg_off;
    wa.stride = 0;
    wa.A_ring = nullptr;
    wa.slot_elems = 0;
    wa.ring_slots = 1;
    wa.m0 = 0;
    wa.M = 1;
    wa.a_in_ring = 0;
    wa.G = 1;
    wa.dW13 = dW13;
    wa.dW2 = dW2;
    wa.L = d->L;
    wa.H = d->H;
    wa.I = d->I;
    wa.accumulate = accumulate ? 1 : 0;
    return wa;
}

}  // namespace

extern "C" {

int moe_layer_fwd_shared(const moe_desc *d, int32_t Is, const int32_t *routes, const float *w, const uint16_t *X,
                         const uint16_t *W13, const uint16_t *W2, const uint16_t *W13s, const uint16_t *W2s,
                         int32_t *counts, int32_t *seg_off, moe_src *phi, int32_t *route_row, uint16_t *HU,
                         uint16_t *A, uint16_t *Y, uint16_t *HUs, uint16_t *As, uint16_t *Ys, uint16_t *out, void *ws,
                         size_t ws_bytes, void *stream) {
    int rc = check_desc(d, true);
    if (rc != MOE_OK) return rc;
    if (d->num_batches != 1 || Is < 1) return MOE_EINVAL;
    if (Is % 128) return MOE_EUNSUPPORTED;
    if (d->H > kZeroRowElems) return MOE_EUNSUPPORTED;  // padding rows read the static zero row
    if (((int64_t)d->P * d->Np / 256 + 1) * (Is / 128 + d->H / 256 + 1) >= (1ll << 30))
        return MOE_EUNSUPPORTED;  // 32-bit tile numbers
    const void *ptrs[] = {routes, w, X, W13, W2, W13s, W2s, counts, seg_off, phi, route_row, A, Y, As, Ys, out, ws};
    for (const void *p : ptrs)
        if (!p || !aligned16(p)) return MOE_EINVAL;
    if ((HU && !aligned16(HU)) || (HUs && !aligned16(HUs))) return MOE_EINVAL;
    if ((int64_t)ws_bytes < moe_workspace_bytes(d, MOE_OP_LAYER_FWD_SHARED)) return MOE_ENOSPC;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *wsb = static_cast<char *>(ws);
    uint32_t *bar = reinterpret_cast<uint32_t *>(wsb);
    moe_desc one = *d;
    one.num_batches = 1;
    char *sched_ws = wsb + kBarrierBytes;
    char *tbl = sched_ws + sched_ws_bytes(&one);
    int32_t *seg_s = reinterpret_cast<int32_t *>(tbl);
    moe_src *phi_s = reinterpret_cast<moe_src *>(tbl + 256);
    const int64_t ntok = (int64_t)d->P * d->Np, ntokp = shared_rows(d);
    {
        TraceScope tr("shared_table", s);
        hipLaunchKernelGGL(k_identity_table, dim3((int)std::min<int64_t>((ntokp + 255) / 256, 1024)), dim3(256), 0, s,
                           phi_s, seg_s, d->Np, ntok, ntokp);
    }
    if (launch_status() != MOE_OK) return MOE_EHIP;
    rc = launch_schedule(&one, routes, counts, seg_off, phi, route_row, sched_ws, s);
    if (rc != MOE_OK) return rc;
    FfnArgs fr = make_ffn_args(d, nullptr, W13, W2, seg_off, HU, A, Y, 0, bar, X, phi);
    moe_desc ds = *d;
    ds.L = 1;
    ds.I = Is;
    FfnArgs fs = make_ffn_args(&ds, nullptr, W13s, W2s, seg_s, HUs, As, Ys, 0, bar, X, phi_s);
    const int grid = gemm_grid();
    {
        TraceScope tr("shared_routed_gateup", s);
        hipLaunchKernelGGL(k_dual_gateup, dim3(grid), dim3(kFwdThreads), 0, s, fs, fr);
    }
    if (launch_status() != MOE_OK) return MOE_EHIP;
    {
        TraceScope tr("shared_routed_down", s);
        hipLaunchKernelGGL(k_dual_down, dim3(grid), dim3(kFwdThreads), 0, s, fs, fr);
    }
    if (launch_status() != MOE_OK) return MOE_EHIP;
    return launch_combine(d, Y, route_row, w, out, s, "combine_shared", 0, Ys);
}

int moe_layer_bwd(const moe_desc *d, const uint16_t *dOut, const int32_t *routes, const float *w, const moe_src *phi,
                  const int32_t *route_row, const int32_t *seg_off, const uint16_t *Xd, const uint16_t *HU,
                  const uint16_t *A, const uint16_t *W13, const uint16_t *W2, uint16_t *dX, float *dW13, float *dW2,
                  float *dw, void *ws, size_t ws_bytes, void *stream) {
    int rc = check_desc(d, true);
    if (rc != MOE_OK) return rc;
    if (!dOut || !routes || !w || !phi || !route_row || !seg_off || !Xd || !HU || !A || !W13 || !W2 || !dX || !dW13 ||
        !dW2 || !dw || !ws)
        return MOE_EINVAL;
    const void *ptrs[] = {dOut, phi, Xd, HU, A, W13, W2, dX, dW13, dW2, ws};
    for (const void *p : ptrs)
        if (!aligned16(p)) return MOE_EINVAL;
    if ((int64_t)ws_bytes < bwd_ws_bytes(d)) return MOE_ENOSPC;
    (void)routes;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const BwdBufs bb = carve_bwd(static_cast<char *>(ws), d);
    rc = bwd_dgrad(d, 0, dOut, w, phi, route_row, seg_off, HU, A, W13, W2, dw, bb, s);
    if (rc != MOE_OK) return rc;
    const WgradArgs wa = wgrad_args(d, bb.dOw, A, bb.dHU, Xd, seg_off, dW13, dW2, false);
    return launch_wgrad(wa, reverse_dispatch(d, 0, bb.dXd, route_row, dX), s);
}

int moe_quantize_mx(const uint16_t *src, int64_t rows, int32_t K, uint8_t *q, uint8_t *scales, void *stream) {
    if (rows < 0 || K <= 0 || K % 32) return MOE_EINVAL;
    if (rows == 0) return MOE_OK;
    if (!src || !q || !scales || !aligned16(src) || !aligned16(q)) return MOE_EINVAL;
    return launch_mx_quantize(src, rows, K, q, scales, static_cast<hipStream_t>(stream), "mx_quantize");
}

int moe_layer_fwd_mx(const moe_desc *d, const int32_t *routes, const float *w, const uint16_t *X,
                     const uint8_t *W13q, const uint8_t *W13s, const uint8_t *W2q, const uint8_t *W2s,
                     int32_t *counts, int32_t *seg_off, moe_src *phi, int32_t *route_row, uint8_t *Xq,
                     uint8_t *Xs, uint8_t *Aq, uint8_t *As, uint16_t *HU, uint16_t *Y, uint16_t *out, void *ws,
                     size_t ws_bytes, void *stream) {
    int rc = check_desc(d, true);
    if (rc != MOE_OK) return rc;
    if (d->num_batches != 1) return MOE_EINVAL;
    const void *a16[] = {routes, w, X, W13q, W2q, counts, seg_off, phi, route_row, Xq, Aq, Y, out, ws};
    for (const void *p : a16)
        if (!p || !aligned16(p)) return MOE_EINVAL;
    if (HU && !aligned16(HU)) return MOE_EINVAL;
    const void *a4[] = {W13s, W2s, Xs, As};
    for (const void *p : a4)
        if (!p || !aligned4(p)) return MOE_EINVAL;
    if (d->H % 128 || d->H > 2 * kZeroRowElems) return MOE_EUNSUPPORTED;
    if ((int64_t)ws_bytes < moe_workspace_bytes(d, MOE_OP_LAYER_FWD)) return MOE_ENOSPC;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *sched_ws = static_cast<char *>(ws) + kBarrierBytes;
    moe_desc one = *d;
    one.num_batches = 1;
    rc = launch_schedule(&one, routes, counts, seg_off, phi, route_row, sched_ws, s);
    if (rc != MOE_OK) return rc;
    rc = launch_mx_quantize(X, (int64_t)d->P * d->Np, d->H, Xq, Xs, s, "mx_quantize_x");
    if (rc != MOE_OK) return rc;
    MxFfnArgs a;
    a.Xq = Xq;
    a.Xs = Xs;
    a.phi = phi;
    a.Np = d->Np;
    a.W13q = W13q;
    a.W13s = W13s;
    a.W2q = W2q;
    a.W2s = W2s;
    a.seg_off = seg_off;
    a.Aq = Aq;
    a.As = As;
    a.HU = HU;
    a.Y = Y;
    a.L = d->L;
    a.H = d->H;
    a.I = d->I;
    // the MX down tiles write the outputs of the tokens with one local route
    rc = launch_single_route(d, route_row, phi, seg_off, w, out, sched_ws + sched_ws_bytes(&one), s, a.rc);
    if (rc != MOE_OK) return rc;
    const int grid = gemm_grid();
    {
        TraceScope tr("mx_gateup", s);
        // scale rows of H / 32 bytes: 16-byte scale DMAs when they are 16-byte aligned
        if (d->H % 512 == 0 && aligned16(Xs) && aligned16(W13s))
            hipLaunchKernelGGL(k_mx_gateup<4>, dim3(grid), dim3(kFwdThreads), 0, s, a);
        else
            hipLaunchKernelGGL(k_mx_gateup<1>, dim3(grid), dim3(kFwdThreads), 0, s, a);
    }
    if (launch_status() != MOE_OK) return MOE_EHIP;
    {
        TraceScope tr("mx_down", s);
        if (d->I % 512 == 0 && aligned16(As) && aligned16(W2s))
            hipLaunchKernelGGL(k_mx_down<4>, dim3(grid), dim3(kFwdThreads), 0, s, a);
        else
            hipLaunchKernelGGL(k_mx_down<1>, dim3(grid), dim3(kFwdThreads), 0, s, a);
    }
    if (launch_status() != MOE_OK) return MOE_EHIP;
    return launch_combine(d, Y, route_row, w, out, s, "combine", 0, nullptr, true);
}

}  // extern "C"

namespace {

int launch_colq(const ColQArgs &a, int64_t max_tiles, hipStream_t s, const char *name) {
    if (max_tiles <= 0) return MOE_OK;
    const int grid = (int)std::min<int64_t>(max_tiles, 8ll * device_cus());
    TraceScope tr(name, s);
    hipLaunchKernelGGL(k_mx_colq, dim3(grid), dim3(kColqThreads), 0, s, a);
    return launch_status();
}

int64_t colq_tiles(int64_t rows, int64_t cols, int64_t batch) {
    return (rows + kColqRows - 1) / kColqRows * ((cols + kColqCols - 1) / kColqCols) * batch;
}

// Column quantization of the dispatched rows [rows < *npad][C] of a table,
// segment-major: from bf16 rows (src, ld; gathered through phi when given)
// or from MX codes (q, s [cap][C]).
ColQArgs colq_rows(const uint16_t *src, int64_t ld, const moe_src *phi, int32_t Np, const uint8_t *srcq,
                   const uint8_t *srcs, const int32_t *seg_off, int L, int64_t cap, int C, uint8_t *q,
                   uint8_t *sc) {
    ColQArgs a{};
    a.src = src;
    a.ld = ld;
    a.in_bstride = 0;
    a.phi = phi;
    a.Np = Np;
    a.srcq = srcq;
    a.srcs = srcs;
    a.nrows = seg_off + L;
    a.seg_off = seg_off;
    a.L = L;
    a.R = cap;
    a.C = C;
    a.batch = 1;
    a.q = q;
    a.s = sc;
    a.ldq = 0;
    a.out_bstride = 0;
    return a;
}

}  // namespace

extern "C" {

int moe_quantize_mx_t(const uint16_t *src, int64_t batch, int32_t R, int32_t C, uint8_t *q, uint8_t *scales,
                      void *stream) {
    if (batch < 0 || R <= 0 || C <= 0 || R % 32 || C % 8) return MOE_EINVAL;
    if (batch == 0) return MOE_OK;
    if (!src || !q || !scales || !aligned16(src) || !aligned16(q)) return MOE_EINVAL;
    if (batch > (1ll << 30) / std::max<int64_t>(1, colq_tiles(R, C, 1))) return MOE_EUNSUPPORTED;
    ColQArgs a{};
    a.src = src;
    a.ld = C;
    a.in_bstride = (int64_t)R * C;
    a.R = R;
    a.C = C;
    a.batch = (int)batch;
    a.q = q;
    a.s = scales;
    a.ldq = R;
    a.out_bstride = (int64_t)R * C;
    return launch_colq(a, colq_tiles(R, C, batch), static_cast<hipStream_t>(stream), "mx_quantize_t");
}

int moe_layer_bwd_mx(const moe_desc *d, const uint16_t *dOut, const float *w, const uint16_t *X, const moe_src *phi,
                     const int32_t *route_row, const int32_t *seg_off, const uint16_t *HU, const uint8_t *Aq,
                     const uint8_t *As, const uint8_t *W13tq, const uint8_t *W13ts, const uint8_t *W2tq,
                     const uint8_t *W2ts, uint16_t *dX, float *dW13, float *dW2, float *dw, void *ws,
                     size_t ws_bytes, void *stream) {
    int rc = check_desc(d, true);
    if (rc != MOE_OK) return rc;
    if (d->num_batches != 1) return MOE_EINVAL;
    const void *a16[] = {dOut, X, phi, HU, Aq, W13tq, W2tq, dX, ws};
    for (const void *p : a16)
        if (!p || !aligned16(p)) return MOE_EINVAL;
    const void *a4[] = {w, route_row, seg_off, As, W13ts, W2ts, dW13, dW2, dw};
    for (const void *p : a4)
        if (!p || !aligned4(p)) return MOE_EINVAL;
    if ((int64_t)ws_bytes < mx_bwd_ws_bytes(d)) return MOE_ENOSPC;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t cap = cap_rows(d);
    const int H = d->H, I = d->I;
    char *wsb = static_cast<char *>(ws);
    BwdBufs bb{};
    bb.dXd = reinterpret_cast<uint16_t *>(wsb);
    bb.dHU = reinterpret_cast<uint16_t *>(wsb + mx_dhu_offset(d));
    bb.wrow = reinterpret_cast<float *>(wsb + mx_wrow_offset(d));
    bb.part = reinterpret_cast<float *>(wsb + mx_part_offset(d));
    const MxBwdBufs mx = carve_mx_bwd(wsb, d);
    uint8_t *const *mb = mx.b;
    rc = launch_row_weight(d, 0, w, phi, route_row, seg_off, bb.wrow, s);
    if (rc != MOE_OK) return rc;
    // B1 fused with both encodings of dO_d: the rows of dOut pulled through
    // phi, their row codes for the down dgrad and the column codes of
    // bf16(dO_d w) for dW2, in one read
    ColQArgs qo = colq_rows(dOut, H, phi, d->Np, nullptr, nullptr, seg_off, d->L, cap, H, mb[kDOwTq], mb[kDOwTs]);
    qo.wrow = bb.wrow;
    qo.rq = mb[kDOq];
    qo.rs = mb[kDOs];
    rc = launch_colq(qo, colq_tiles(cap, H, 1), s, "mx_bwd_gather_quantize_dO");
    if (rc != MOE_OK) return rc;
    MxBwdArgs a;
    a.dOq = mb[kDOq];
    a.dOs = mb[kDOs];
    a.W2tq = W2tq;
    a.W2ts = W2ts;
    a.Aq = Aq;
    a.As = As;
    a.HU = HU;
    a.wrow = bb.wrow;
    a.dHU = bb.dHU;
    a.part = bb.part;
    a.dHUq = mb[kDHUq];
    a.dHUs = mb[kDHUs];
    a.W13tq = W13tq;
    a.W13ts = W13ts;
    a.dXd = bb.dXd;
    a.seg_off = seg_off;
    a.L = d->L;
    a.H = H;
    a.I = I;
    a.nparts = bwd_nparts(d);
    const int grid = gemm_grid();
    {
        // B2; scale rows of H / 32 bytes: 16-byte scale DMAs when aligned
        TraceScope tr("mx_bwd_down", s);
        if (H % 512 == 0 && aligned16(W2ts))
            hipLaunchKernelGGL(k_mx_bwd_down<4>, dim3(grid), dim3(kFwdThreads), 0, s, a);
        else
            hipLaunchKernelGGL(k_mx_bwd_down<1>, dim3(grid), dim3(kFwdThreads), 0, s, a);
    }
    if (launch_status() != MOE_OK) return MOE_EHIP;
    const int64_t nslots = (int64_t)d->P * d->Np * d->K;
    {
        TraceScope tr("bwd_dw", s);
        hipLaunchKernelGGL(k_dw_finalize, dim3((int)std::min<int64_t>((nslots + 255) / 256, 4096)), dim3(256), 0, s,
                           route_row, bb.part, a.nparts, dw, nslots, 0, (int64_t)0);
    }
    if (launch_status() != MOE_OK) return MOE_EHIP;
    // dHU: row codes for the gate/up dgrad and column codes for dW13, one read
    ColQArgs qh = colq_rows(bb.dHU, 2 * I, nullptr, 0, nullptr, nullptr, seg_off, d->L, cap, 2 * I, mb[kDHUTq],
                            mb[kDHUTs]);
    qh.rq = mb[kDHUq];
    qh.rs = mb[kDHUs];
    rc = launch_colq(qh, colq_tiles(cap, 2 * I, 1), s, "mx_bwd_quantize_dHU");
    if (rc != MOE_OK) return rc;
    {
        TraceScope tr("mx_bwd_gateup", s);
        if ((2 * I) % 512 == 0 && aligned16(W13ts))
            hipLaunchKernelGGL(k_mx_bwd_gateup<4>, dim3(grid), dim3(kFwdThreads), 0, s, a);
        else
            hipLaunchKernelGGL(k_mx_bwd_gateup<1>, dim3(grid), dim3(kFwdThreads), 0, s, a);
    }
    if (launch_status() != MOE_OK) return MOE_EHIP;
    // the other two weight-gradient operands, quantized along the rows
    rc = launch_colq(colq_rows(nullptr, 0, nullptr, 0, Aq, As, seg_off, d->L, cap, I, mb[kATq], mb[kATs]),
                     colq_tiles(cap, I, 1), s, "mx_bwd_colq_a");
    if (rc != MOE_OK) return rc;
    rc = launch_colq(colq_rows(X, H, phi, d->Np, nullptr, nullptr, seg_off, d->L, cap, H, mb[kXdTq], mb[kXdTs]),
                     colq_tiles(cap, H, 1), s, "mx_bwd_colq_Xd");
    if (rc != MOE_OK) return rc;
    MxWgradArgs wa;
    wa.dOwTq = mb[kDOwTq];
    wa.dOwTs = mb[kDOwTs];
    wa.aTq = mb[kATq];
    wa.aTs = mb[kATs];
    wa.dHUTq = mb[kDHUTq];
    wa.dHUTs = mb[kDHUTs];
    wa.XdTq = mb[kXdTq];
    wa.XdTs = mb[kXdTs];
    wa.seg_off = seg_off;
    wa.dW13 = dW13;
    wa.dW2 = dW2;
    wa.L = d->L;
    wa.H = H;
    wa.I = I;
    TraceScope tr("mx_bwd_wgrad_rdispatch", s);
    hipLaunchKernelGGL(k_mx_wgrad, dim3(grid), dim3(kFwdThreads), 0, s, wa,
                       reverse_dispatch(d, 0, bb.dXd, route_row, dX));
    return launch_status();
}

}  // extern "C"

namespace {

// ---------------------------------------------------------------------------
// Macrobatch ring.
// ---------------------------------------------------------------------------

// Checks shared by the ring calls; dm describes one macrobatch (Np =
// mb_tokens) with num_batches = M macrobatches.
int ring_check(const moe_desc *d, int32_t mb_tokens, int32_t ring_slots, moe_desc &dm, int &M) {
    int rc = check_desc(d, true);
    if (rc != MOE_OK) return rc;
    if (d->num_batches != 1 || mb_tokens < 1 || d->Np % mb_tokens || ring_slots < 1) return MOE_EINVAL;
    if (d->H > kZeroRowElems) return MOE_EUNSUPPORTED;  // padding rows read the static zero row
    dm = *d;
    dm.Np = mb_tokens;
    M = d->Np / mb_tokens;
    dm.num_batches = M;
    return check_desc(&dm, true);
}

// Ring backward workspace: the per-table buffers (BwdBufs) of one macrobatch,
// whose dO_d * w and dHU are then kept for each of the G macrobatches of a
// weight-gradient group together with their X rows and replayed HU, A.
int64_t ring_group_slot_bytes(const moe_desc *d1) {
    const int64_t cap = cap_rows(d1), H = d1->H, I = d1->I;
    return align256(cap * H * 2) * 2 + align256(cap * 2 * I * 2) * 2 + align256(cap * I * 2);
}

int64_t ring_bwd_bytes(const moe_desc *d1, int G) { return bwd_ws_bytes(d1) + G * ring_group_slot_bytes(d1); }

}  // namespace

extern "C" {

int64_t moe_ring_capacity_rows(const moe_desc *d, int32_t mb_tokens) {
    moe_desc dm;
    int M;
    if (ring_check(d, mb_tokens, 1, dm, M) != MOE_OK) return -1;
    dm.num_batches = 1;
    return cap_rows(&dm);
}

int64_t moe_ring_workspace_bytes(const moe_desc *d, int32_t mb_tokens, int32_t wgrad_group, int op) {
    moe_desc dm;
    int M;
    if (ring_check(d, mb_tokens, 1, dm, M) != MOE_OK) return -1;
    moe_desc d1 = dm;
    d1.num_batches = 1;
    if (op == MOE_OP_LAYER_FWD) return kBarrierBytes + sched_ws_bytes(&dm) + single_route_bytes(&d1);
    if (op != MOE_OP_LAYER_BWD || wgrad_group < 1 || wgrad_group > kMaxWgradGroup) return -1;
    return ring_bwd_bytes(&d1, std::min(wgrad_group, M));
}

int moe_layer_fwd_ring(const moe_desc *d, int32_t mb_tokens, int32_t ring_slots, const int32_t *routes,
                       const float *w, const uint16_t *X, const uint16_t *W13, const uint16_t *W2, int32_t *counts,
                       int32_t *seg_off, moe_src *phi, int32_t *route_row, uint16_t *HU, uint16_t *A, uint16_t *Y,
                       uint16_t *out, void *ws, size_t ws_bytes, void *stream) {
    moe_desc dm;
    int M;
    int rc = ring_check(d, mb_tokens, ring_slots, dm, M);
    if (rc != MOE_OK) return rc;
    const void *ptrs[] = {routes, w, X, W13, W2, counts, seg_off, phi, route_row, HU, A, Y, out, ws};
    for (const void *p : ptrs)
        if (!p || !aligned16(p)) return MOE_EINVAL;
    if ((int64_t)ws_bytes < moe_ring_workspace_bytes(d, mb_tokens, 1, MOE_OP_LAYER_FWD)) return MOE_ENOSPC;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *wsb = static_cast<char *>(ws);
    uint32_t *bar = reinterpret_cast<uint32_t *>(wsb);
    const int64_t B = mb_tokens, K = d->K, H = d->H, I = d->I, L = d->L, Np = d->Np;
    // every macrobatch's table in one batched schedule: table m is token window m
    rc = launch_schedule(&dm, routes, counts, seg_off, phi, route_row, wsb + kBarrierBytes, s, Np * K, B * K);
    if (rc != MOE_OK) return rc;
    moe_desc d1 = dm;
    d1.num_batches = 1;
    const int64_t capm = cap_rows(&d1);
    char *tab = wsb + kBarrierBytes + sched_ws_bytes(&dm);  // the single-route table of one macrobatch
    const int grid = gemm_grid();
    // reversed ring: the last macrobatch first, so the first ones stay resident
    for (int i = 0; i < M; ++i) {
        const int m = M - 1 - i, slot = i % ring_slots;
        FfnArgs fa = make_ffn_args(&d1, nullptr, W13, W2, seg_off + (int64_t)m * (L + 1),
                                   HU + (int64_t)slot * capm * 2 * I, A + (int64_t)slot * capm * I, Y, 0, bar,
                                   X + (int64_t)m * B * H, phi + (int64_t)m * capm);
        fa.Np = d->Np;  // partition stride of X
        WindowCombine wc{};  // Y == nullptr: no combine in the first launch
        if (i > 0) {  // the combine of the macrobatch walked before this one
            const int64_t t0 = (int64_t)(m + 1) * B;
            wc.Y = Y;
            wc.route_row = route_row + t0 * K;
            wc.w = w + t0 * K;
            wc.out = out + t0 * H;
        }
        wc.K = d->K;
        wc.H = d->H;
        wc.tpp = (int)B;
        wc.ntok = (int64_t)d->P * B;
        wc.tstride = Np;
        wc.skip_single = 1;
        {
            TraceScope tr("ring_gateup_combine", s);
            hipLaunchKernelGGL(k_ring_gateup_combine, dim3(grid), dim3(kFwdThreads), 0, s, fa, wc);
        }
        if (launch_status() != MOE_OK) return MOE_EHIP;
        // the down tiles write the outputs of this macrobatch's single-route tokens
        const int64_t t0 = (int64_t)m * B;
        rc = launch_single_route(&d1, route_row + t0 * K, phi + (int64_t)m * capm, seg_off + (int64_t)m * (L + 1),
                                 w + t0 * K, out + t0 * H, tab, s, fa.rc, Np);
        if (rc != MOE_OK) return rc;
        {
            TraceScope tr("ring_down", s);
            hipLaunchKernelGGL(k_ffn_down_w, dim3(grid), dim3(kWideThreads), 0, s, fa);
        }
        if (launch_status() != MOE_OK) return MOE_EHIP;
    }
    return launch_combine(&d1, Y, route_row, w, out, s, "ring_combine", Np, nullptr, true);  // macrobatch 0
}

int moe_layer_bwd_ring(const moe_desc *d, int32_t mb_tokens, int32_t ring_slots, int32_t wgrad_group,
                       const uint16_t *dOut, const float *w, const uint16_t *X, const uint16_t *W13,
                       const uint16_t *W2, const moe_src *phi, const int32_t *route_row, const int32_t *seg_off,
                       const uint16_t *HU, const uint16_t *A, uint16_t *dX, float *dW13, float *dW2, float *dw,
                       void *ws, size_t ws_bytes, void *stream) {
    moe_desc dm;
    int M;
    int rc = ring_check(d, mb_tokens, ring_slots, dm, M);
    if (rc != MOE_OK) return rc;
    if (wgrad_group < 1 || wgrad_group > kMaxWgradGroup) return MOE_EINVAL;
    const void *ptrs[] = {dOut, w, X, W13, W2, phi, route_row, seg_off, HU, A, dX, dW13, dW2, dw, ws};
    for (const void *p : ptrs)
        if (!p || !aligned16(p)) return MOE_EINVAL;
    const int G = std::min<int>(wgrad_group, M);
    if ((int64_t)ws_bytes < moe_ring_workspace_bytes(d, mb_tokens, wgrad_group, MOE_OP_LAYER_BWD)) return MOE_ENOSPC;
    hipStream_t s = static_cast<hipStream_t>(stream);
    moe_desc d1 = dm;
    d1.num_batches = 1;
    const int64_t capm = cap_rows(&d1), B = mb_tokens, K = d->K, H = d->H, I = d->I, L = d->L, Np = d->Np;
    BwdBufs bb = carve_bwd(static_cast<char *>(ws), &d1);
    char *slots = static_cast<char *>(ws) + bwd_ws_bytes(&d1);
    struct Slot {
        uint16_t *dOw, *Xd, *dHU, *HUr, *Ar;
    };
    auto slot_of = [&](int j) {
        char *p = slots + j * ring_group_slot_bytes(&d1);
        Slot sl;
        sl.dOw = reinterpret_cast<uint16_t *>(p);
        p += align256(capm * H * 2);
        sl.Xd = reinterpret_cast<uint16_t *>(p);
        p += align256(capm * H * 2);
        sl.dHU = reinterpret_cast<uint16_t *>(p);
        p += align256(capm * 2 * I * 2);
        sl.HUr = reinterpret_cast<uint16_t *>(p);
        p += align256(capm * 2 * I * 2);
        sl.Ar = reinterpret_cast<uint16_t *>(p);
        return sl;
    };
    const Slot s0 = slot_of(0);
    const int64_t slot_stride = ring_group_slot_bytes(&d1) / 2;  // elements between two slots' buffers
    uint32_t a_in_ring = 0;
    for (int m = 0; m < M; ++m) {
        const int j = m % G;  // this macrobatch's place in its weight-gradient group
        const Slot sl = slot_of(j);
        const int64_t t0 = (int64_t)m * B;
        const int32_t *so = seg_off + (int64_t)m * (L + 1);
        const moe_src *ph = phi + (int64_t)m * capm;
        const uint16_t *hu, *aa;
        if (m < ring_slots) {  // still in the ring: walked among the forward's last ring_slots
            const int64_t slot = (M - 1 - m) % ring_slots;
            hu = HU + slot * capm * 2 * I;
            aa = A + slot * capm * I;
        } else {  // replay: the forward's gate/up of this macrobatch, from X through its table
            FfnArgs fa = make_ffn_args(&d1, nullptr, W13, W2, so, sl.HUr, sl.Ar, nullptr, 0, nullptr, X + t0 * H, ph);
            fa.Np = d->Np;
            {
                TraceScope tr("ring_replay_gateup", s);
                hipLaunchKernelGGL(k_ffn_gateup, dim3(gemm_grid()), dim3(kFwdThreads), 0, s, fa);
            }
            if (launch_status() != MOE_OK) return MOE_EHIP;
            hu = sl.HUr;
            aa = sl.Ar;
        }
        // the dispatched rows of X, for the gate/up weight gradient
        rc = launch_gather(&d1, X + t0 * H, ph, so, sl.Xd, s, "ring_bwd_gather_x", (int)Np);
        if (rc != MOE_OK) return rc;
        bb.dOw = sl.dOw;
        bb.dHU = sl.dHU;
        rc = bwd_dgrad(&d1, Np, dOut + t0 * H, w + t0 * K, ph, route_row + t0 * K, so, hu, aa, W13, W2, dw + t0 * K,
                       bb, s);
        if (rc != MOE_OK) return rc;
        if (m < ring_slots) a_in_ring |= 1u << j;
        const WindowCombine rd = reverse_dispatch(&d1, Np, bb.dXd, route_row + t0 * K, dX + t0 * H);
        if (j == G - 1 || m == M - 1) {
            // the group's weight gradients in one pass (added in ascending group
            // order), with this macrobatch's reverse dispatch
            const int m0 = m - j;
            WgradArgs wa = wgrad_args(&d1, s0.dOw, s0.Ar, s0.dHU, s0.Xd, seg_off + (int64_t)m0 * (L + 1), dW13, dW2,
                                      m0 > 0);
            wa.stride = slot_stride;
            wa.A_ring = A;
            wa.slot_elems = capm * I;
            wa.ring_slots = ring_slots;
            wa.m0 = m0;
            wa.M = M;
            wa.a_in_ring = a_in_ring;
            wa.G = j + 1;
            rc = launch_wgrad(wa, rd, s);
            if (rc != MOE_OK) return rc;
            a_in_ring = 0;
        } else {
            TraceScope tr("bwd_reverse_dispatch", s);
            const int64_t ntok = rd.ntok;
            const int grid = (int)std::min<int64_t>((ntok + 3) / 4, 16ll * device_cus());
            hipLaunchKernelGGL(k_combine, dim3(grid), dim3(256), 0, s, rd.Y, rd.route_row, rd.w, rd.out, rd.K, rd.H,
                               ntok, rd.tpp, rd.tstride, (const uint16_t *)nullptr, 0);
            if (launch_status() != MOE_OK) return MOE_EHIP;
        }
    }
    return MOE_OK;
}

int moe_trace_enable(int max_records) {
    std::lock_guard<std::mutex> g(g_trace_mu);
    for (auto &r : g_trace) {
        (void)hipEventDestroy(r.start);
        (void)hipEventDestroy(r.stop);
    }
    g_trace.clear();
    g_trace_cap = 0;
    g_trace_used = 0;
    if (max_records <= 0) return MOE_OK;
    g_trace.resize(max_records);
    // Timing events without the system-scope fence: the default release at
    // each record writes the L2s back for the host (about 10 us between two
    // traced launches); the host reads these events only through
    // hipEventElapsedTime, after synchronizing.
    constexpr unsigned flags = hipEventDefault | hipEventDisableSystemFence;
    for (auto &r : g_trace) {
        if (hipEventCreateWithFlags(&r.start, flags) != hipSuccess ||
            hipEventCreateWithFlags(&r.stop, flags) != hipSuccess)
            return MOE_EHIP;
        r.name[0] = 0;
    }
    g_trace_cap = max_records;
    return MOE_OK;
}

int moe_trace_read(char *kernel, float *ms, int max_records) {
    std::lock_guard<std::mutex> g(g_trace_mu);
    int n = std::min(g_trace_used, max_records);
    for (int i = 0; i < n; ++i) {
        float t = -1.f;
        if (hipEventElapsedTime(&t, g_trace[i].start, g_trace[i].stop) != hipSuccess) t = -1.f;
        if (kernel) memcpy(kernel + 32 * i, g_trace[i].name, 32);
        if (ms) ms[i] = t;
    }
    return n;
}

}  // extern "C"
