/*
 * moe.h — C ABI of one GPU's share of a Mixture-of-Experts layer on MI355X
 * (gfx950): an on-device counting-sort schedule, a row gather, a SwiGLU expert
 * FFN as a grouped bf16 GEMM, a fixed-order combine, and the backward pass
 * that reuses the same table.
 *
 * Sources:
 *   [MoK]  "Mixture-of-Kittens: A MoE Megakernel for GB300 NVL72" (reading notes)
 *   [SOSO] "Scan once, scatter once"
 *   [BPT]  "Beyond Peak TFLOPs: Why Communication-Compute Overlap Dictates ML
 *          Productivity Goodput"
 *
 * Conventions shared by every call
 *   - Every pointer is a DEVICE pointer owned by the caller unless the
 *     argument says "host".  The library allocates no device memory, never
 *     synchronises the device or the stream, and keeps no state between calls
 *     (apart from the optional launch trace below).  Calls are asynchronous on
 *     `stream` (a hipStream_t passed as void*, NULL = the null stream).
 *   - bf16 tensors are raw bfloat16 (uint16_t storage).  All tensors are dense,
 *     row-major, in the shapes given; device pointers must be 16-byte aligned.
 *   - Return value: MOE_OK or a negative MOE_E* code; moe_strerror() names it.
 *     Arguments are checked on the host before anything is launched; a failed
 *     check launches nothing and writes nothing.  Device data (route ids, the
 *     table) is not validated on the host: route ids outside
 *     [expert_base, expert_base + L) are simply not local (negative "dropped"
 *     ids included) and are skipped; those outside [0, E) are also counted on
 *     the device (MOE_WS_INVALID_IDS below).
 *   - Results are bitwise reproducible run to run: integer work is exact,
 *     and every floating-point reduction has a fixed order (no float atomics).
 *   - Calls that share buffers must be ordered by the caller (same stream or
 *     events).  Concurrent calls on different buffers are independent.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Error codes. */
enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,       /* bad dimension, NULL pointer or misaligned pointer */
    MOE_ENOSPC = -2,       /* workspace or capacity smaller than required       */
    MOE_EUNSUPPORTED = -3, /* valid but not supported (e.g. H % 64 != 0)        */
    MOE_EHIP = -4,         /* a HIP launch or runtime call failed                */
};

/* Problem description (host struct, read during the call only).
 *   P            source partitions (the "peers" of [MoK] section 2; here P slices
 *                of the routing tensor resident in local HBM)
 *   Np           tokens per partition
 *   K            top-k slots per token
 *   E            global experts
 *   L            local experts: ids [expert_base, expert_base + L)
 *   expert_base  first local expert id (ep_rank * L for contiguous ownership)
 *   pad_rows     every expert segment is padded to a multiple of this many rows
 *                ([SOSO]: 256)
 *   sched_threads logical scheduler threads per partition ([SOSO]: 1,024).  The
 *                table does not depend on it (logical threads own contiguous
 *                route chunks, so the order is the stable one); it is accepted
 *                for interface fidelity and must be >= 1.
 *   H, I         hidden size and expert intermediate size (SwiGLU: W13 holds
 *                gate rows [0, I) and up rows [I, 2I))
 *   num_batches  moe_schedule only: independent routing tensors per call (>= 1)
 */
typedef struct moe_desc {
    int32_t P, Np, K, E, L, expert_base, pad_rows, sched_threads, H, I, num_batches;
} moe_desc;

/* One row of the pull table Phi ([MoK] section 2; [BPT] section 2.A): the
 * partition and token a dispatched row is pulled from; (-1, -1) on padding. */
typedef struct moe_src {
    int32_t part;
    int32_t tok;
} moe_src;

const char *moe_strerror(int code);

/* Worst-case dispatched rows for `d`: P*Np*K + L*(pad_rows - 1).  Every
 * row-indexed buffer below (phi, Xd, HU, A, Y, dO_d, dHU, dXd) must hold this
 * many rows, so that no routing ever needs a host round trip or a dropped
 * token ([MoK] section 4; [BPT] section 2.B).  Returns -1 for an invalid d. */
int64_t moe_capacity_rows(const moe_desc *d);

/* Workspace bytes needed by an operation (MOE_OP_*); -1 for an invalid d.  The
 * workspace is caller-owned scratch: contents on entry are ignored except
 * where a call says otherwise, and it must not be shared by concurrent calls. */
enum {
    MOE_OP_SCHEDULE = 0,
    MOE_OP_DISPATCH = 1,
    MOE_OP_EXPERT_FFN = 2,
    MOE_OP_COMBINE = 3,
    MOE_OP_LAYER_FWD = 4,
    MOE_OP_LAYER_BWD = 5,
    MOE_OP_LAYER_FWD_SHARED = 6,
    MOE_OP_LAYER_BWD_MX = 7,
};
int64_t moe_workspace_bytes(const moe_desc *d, int op);

/*
 * Status words the library leaves in a caller's workspace.  Nothing is read
 * back to the host by the library (it never synchronises); a caller that
 * wants them copies the words after the call has finished.
 *
 *   MOE_WS_INVALID_IDS     int32 per routing table: the number of route ids
 *                          outside [0, E) the schedule saw (negative "dropped"
 *                          ids included).  Such ids are never local and are
 *                          skipped ([MoK] section 2 places only the local
 *                          routes); the count lets a caller detect a corrupt
 *                          routing tensor without a host round trip.  Written
 *                          by every call that runs the schedule: num_batches
 *                          words for moe_schedule, one for moe_layer_fwd,
 *                          moe_layer_fwd_mx and moe_layer_fwd_shared, and one
 *                          per macrobatch (M words) for moe_layer_fwd_ring.
 *   MOE_WS_BARRIER_STATUS  uint32: 0 after a call whose device-wide waits all
 *                          completed, 1 if one gave up.  Only the persistent
 *                          and chunked paths (moe_layer_fwd with
 *                          MOE_PERSISTENT or chunk_rows > 0, moe_expert_ffn
 *                          with chunk_rows > 0) wait across workgroups: they
 *                          clear the word, and every wait is bounded (about a
 *                          second of spinning) so that a grid whose workgroups
 *                          were not all resident ends instead of hanging.  When
 *                          the word is 1 the outputs of that call are
 *                          undefined.  Other calls leave it untouched.
 *
 * moe_workspace_field returns the byte offset of `field` in the workspace of
 * operation `op` (moe_workspace_bytes), or -1 if d is invalid or op has no
 * such field.  moe_layer_fwd_mx uses MOE_OP_LAYER_FWD's offsets, and so does
 * moe_layer_fwd_ring for the two status words (its single-route table sits
 * after its M tables' schedule workspace, so MOE_WS_SINGLE_ROUTE does not
 * apply to it).
 */
enum {
    MOE_WS_INVALID_IDS = 0,
    MOE_WS_BARRIER_STATUS = 1,
    /* inspection of moe_layer_bwd_mx (op MOE_OP_LAYER_BWD_MX); only the rows
     * below seg_off[L] are written by a call.  The column-code buffers are
     * segment-major: local expert l (rows [S, S + n), S = seg_off[l],
     * n = seg_off[l+1] - S) owns a [C][n] block of codes at byte C * S and a
     * [C][n/32] block of scale bytes at byte C * S / 32. */
    MOE_WS_MX_DHU = 2,     /* bf16 [cap][2I]: dHU (gate then up columns)       */
    MOE_WS_MX_DO_Q = 3,    /* [cap][H]:   dO_d row codes (along H)             */
    MOE_WS_MX_DO_S = 4,    /* [cap][H/32]                                      */
    MOE_WS_MX_DHU_Q = 5,   /* [cap][2I]:  dHU row codes (along 2I)             */
    MOE_WS_MX_DHU_S = 6,   /* [cap][2I/32]                                     */
    MOE_WS_MX_DOWT_Q = 7,  /* C = H:  (dO_d w) column codes (along the rows)   */
    MOE_WS_MX_DOWT_S = 8,  /*         their scale bytes                        */
    MOE_WS_MX_AT_Q = 9,    /* C = I:  a column codes                           */
    MOE_WS_MX_AT_S = 10,   /*                                                  */
    MOE_WS_MX_XDT_Q = 11,  /* C = H:  Xd column codes                          */
    MOE_WS_MX_XDT_S = 12,  /*                                                  */
    MOE_WS_MX_DHUT_Q = 13, /* C = 2I: dHU column codes                         */
    MOE_WS_MX_DHUT_S = 14, /*                                                  */
    /* inspection of moe_layer_fwd and moe_layer_fwd_mx (op MOE_OP_LAYER_FWD):
     * int32 pairs [cap][2], rows below seg_off[L] written by a call that
     * combines single-route tokens in its down GEMM (separate launches, no
     * chunks): (token p * Np + t, bits of its fp32 weight) for a row whose
     * token has exactly one local route, (-1, 0) for every other row and for
     * padding rows. */
    MOE_WS_SINGLE_ROUTE = 15,
};
int64_t moe_workspace_field(const moe_desc *d, int op, int field);

/*
 * moe_schedule — the counting-sort pull schedule of [MoK] section 2 built on
 * the device in the four stages of [SOSO] ("The fix is a counting sort"):
 * count routes per local expert, partition and logical thread; prefix the
 * counts; pad every expert segment to pad_rows and take its base row; scatter
 * every route once to Phi[S[l] + p] with
 *     p = sum_{r'} min(M[l][r'], o) + #{ r' < r : M[l][r'] > o },
 * o being the route's ordinal among partition r's routes to expert l in flat
 * (token-major, then slot) order.  Route ids are read once as int32; the count
 * stage leaves each route's local id as one byte in the workspace and the
 * scatter reads those (with more than 255 local experts it reads the int32 ids
 * again).
 *
 * For each batch b in [0, num_batches):
 *   routes     int32   [nb][P][Np][K]  in: expert id of every slot
 *   counts     int32   [nb][L][P]      out: M[l][r]
 *   seg_off    int32   [nb][L+1]       out: S; seg_off[L] = padded rows Npad
 *   phi        moe_src [nb][cap]       out: rows [0, Npad) written; rows past
 *                                      Npad are left untouched
 *   route_row  int32   [nb][P][Np][K]  out: row of each slot, -1 if not local
 *   ws         >= moe_workspace_bytes(d, MOE_OP_SCHEDULE) bytes
 * Bit-exact and deterministic.  Npad stays on the device.
 */
int moe_schedule(const moe_desc *d, const int32_t *routes, int32_t *counts, int32_t *seg_off,
                 moe_src *phi, int32_t *route_row, void *ws, size_t ws_bytes, void *stream);

/*
 * moe_dispatch — pull dispatch ([MoK] section 2; [BPT] section 2.A) as a local
 * gather: Xd[i] = X[phi[i].part][phi[i].tok] bit for bit for i < Npad =
 * seg_off[L]; padding rows are written as zeros.  Rows >= Npad untouched.
 *   X        bf16    [P][Np][H]
 *   phi      moe_src [cap], seg_off int32 [L+1] (from moe_schedule)
 *   Xd       bf16    [cap][H]
 * The same call is the backward's reverse-combine gather (dOut -> dO_d).
 */
int moe_dispatch(const moe_desc *d, const uint16_t *X, const moe_src *phi, const int32_t *seg_off,
                 uint16_t *Xd, void *stream);

/*
 * moe_expert_ffn — SwiGLU expert FFN as grouped GEMMs over the expert
 * segments ([MoK] sections 3 and 5): for every row i < Npad of segment l
 *     HU[i] = Xd[i] W13[l]^T            (fp32 accumulate; gate | up)
 *     A[i]  = silu(HU[i][:I]) * HU[i][I:]   (rounded to bf16)
 *     Y[i]  = A[i] W2[l]^T              (fp32 accumulate, rounded to bf16)
 *   Xd   bf16 [cap][H]     W13 bf16 [L][2I][H]     W2 bf16 [L][H][I]
 *   seg_off int32 [L+1]
 *   HU   bf16 [cap][2I] or NULL (saved pre-activations for the backward)
 *   A    bf16 [cap][I]     Y bf16 [cap][H]
 *   chunk_rows  0: one pass over all rows.  > 0: rows are processed in chunks
 *               of chunk_rows dispatched rows (a multiple of 256), the down
 *               projection of chunk c overlapping the gate/up projection of
 *               chunk c+1 inside one persistent launch (the minibatch T of
 *               [MoK] section 3).
 *   ws   >= moe_workspace_bytes(d, MOE_OP_EXPERT_FFN)
 * Requires H % 256 == 0 and I % 128 == 0 (else MOE_EUNSUPPORTED).  The
 * GEMM launches number their 256-row tiles with 32-bit integers: shapes whose
 * tile counts come near 2^30 (weights of petabytes) are MOE_EUNSUPPORTED for
 * every call that runs a GEMM.
 */
int moe_expert_ffn(const moe_desc *d, const uint16_t *Xd, const uint16_t *W13, const uint16_t *W2,
                   const int32_t *seg_off, uint16_t *HU, uint16_t *A, uint16_t *Y, int32_t chunk_rows,
                   void *ws, size_t ws_bytes, void *stream);

/*
 * moe_combine — push combine ([MoK] section 2) as a local fixed-order sum:
 *     out[r][t] = sum_{j = 0..K-1, route_row[r][t][j] >= 0} w[r][t][j] * Y[route_row[r][t][j]]
 * accumulated in fp32 in ascending j and rounded once to bf16; tokens with no
 * local slot get zeros.  w may be NULL (every weight 1): that is the
 * backward's reverse-dispatch sum (dXd -> dX).
 *   Y bf16 [cap][H]   route_row int32 [P][Np][K]   w float [P][Np][K] or NULL
 *   out bf16 [P][Np][H]
 */
int moe_combine(const moe_desc *d, const uint16_t *Y, const int32_t *route_row, const float *w,
                uint16_t *out, void *stream);

/* Flags of moe_layer_fwd. */
enum {
    MOE_PERSISTENT = 1, /* run every stage inside one persistent cooperative launch */
};

/*
 * moe_layer_fwd — the whole forward share: schedule, dispatch, expert FFN,
 * combine.  Outputs as in the four calls above (HU may be NULL).  With
 * MOE_PERSISTENT set, every stage runs inside one persistent launch whose
 * workgroups pass device-side barriers between stages ([MoK] section 5,
 * megakernel fusion); otherwise one launch per stage.  Both give bitwise the
 * same results.  chunk_rows as in moe_expert_ffn.
 * Without MOE_PERSISTENT and with chunk_rows == 0, a token with exactly one
 * local route has its output row written by the down GEMM's epilogue (the
 * combine's one-term sum, same fp32 product and bf16 rounding) and the
 * combine launch skips it; out is bitwise what the other paths write.  The
 * row of Y of such a route is then not written (nothing else reads it: the
 * backward takes HU and A), so Y holds the rows of tokens with two or more
 * local routes and the padding rows; the persistent and chunked paths write
 * every row.  The table of such rows (one int32 per row of capacity) is
 * rebuilt by every call, so nothing an earlier call left in ws is read.
 * Xd may be NULL: the dispatch is then fused into the gate/up GEMM, whose
 * operand loads pull each row from X through phi ([MoK] section 2, pull
 * dispatch hidden behind the GEMM), and no dispatched copy is written; every
 * other output is bitwise the same.  Needs H <= 32768 (else
 * MOE_EUNSUPPORTED).  moe_layer_bwd needs Xd: a caller that wants the
 * backward either passes Xd here or fills it later with moe_dispatch.
 *   ws >= moe_workspace_bytes(d, MOE_OP_LAYER_FWD)
 * Uses d->num_batches == 1.
 */
int moe_layer_fwd(const moe_desc *d, const int32_t *routes, const float *w, const uint16_t *X,
                  const uint16_t *W13, const uint16_t *W2, int32_t *counts, int32_t *seg_off,
                  moe_src *phi, int32_t *route_row, uint16_t *Xd, uint16_t *HU, uint16_t *A,
                  uint16_t *Y, uint16_t *out, int32_t flags, int32_t chunk_rows, void *ws,
                  size_t ws_bytes, void *stream);

/*
 * moe_layer_fwd_noalloc — moe_layer_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same call and the same results, without the
 * workspace argument.  Its workspace is a static device array inside the
 * library, MOE_NOALLOC_SCRATCH_BYTES per GPU, which every GPU the library runs
 * on holds until the process ends.  The call allocates and frees nothing
 * (its first call on a device looks up that device's copy of the array).
 *   status  nullable device int32[2] (4-byte aligned): on completion [0] the
 *           MOE_WS_INVALID_IDS count of this call, [1] its
 *           MOE_WS_BARRIER_STATUS word (0 when the call does not wait across
 *           workgroups)
 * Errors: those of moe_layer_fwd, and MOE_ENOSPC when
 * moe_workspace_bytes(d, MOE_OP_LAYER_FWD) exceeds MOE_NOALLOC_SCRATCH_BYTES
 * (nothing is launched then).  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (different streams, or different host
 * threads, not ordered by the caller) race and give undefined results.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (8 << 20)
int moe_layer_fwd_noalloc(const moe_desc *d, const int32_t *routes, const float *w, const uint16_t *X,
                          const uint16_t *W13, const uint16_t *W2, int32_t *counts, int32_t *seg_off, moe_src *phi,
                          int32_t *route_row, uint16_t *Xd, uint16_t *HU, uint16_t *A, uint16_t *Y, uint16_t *out,
                          int32_t flags, int32_t chunk_rows, int32_t *status, void *stream);

/*
 * moe_layer_fwd_shared — the layer forward with a shared expert: a dense
 * SwiGLU FFN over every token beside the routed experts ([BPT] section 2.C:
 * the shared expert computed while the first routed rows are pulled; [MoK]
 * section 5: the shared expert stays bf16).  Per token g,
 *   out[g] = bf16( sum_{j asc, local} w[g][j] * Y[route_row[g][j]] + S[g] ),
 *   S = W2s (silu(W1s x) * (W3s x))  rounded to bf16 once (Ys).
 *   Is     shared intermediate size, a multiple of 128
 *   W13s   bf16 [2 Is][H]   gate rows [0, Is), up rows [Is, 2 Is)
 *   W2s    bf16 [H][Is]
 *   HUs    bf16 [ntokp][2 Is] out, nullable: saved shared pre-activations
 *   As     bf16 [ntokp][Is]   out: shared activations
 *   Ys     bf16 [ntokp][H]    out: S; rows past P*Np are zero
 *   with ntokp = P*Np rounded up to a multiple of 256.  The routed arguments
 *   are those of moe_layer_fwd with Xd = NULL (the dispatch fused into the
 *   gate/up operand loads).
 *   ws >= moe_workspace_bytes(d, MOE_OP_LAYER_FWD_SHARED)
 * Launches: the schedule, one gate/up launch holding the shared and the
 * routed tiles, one down launch holding both, the combine adding S.  The
 * routed rows (HU, A, Y) are bitwise those of moe_layer_fwd.  Errors as
 * moe_layer_fwd, and MOE_EINVAL for Is < 1, MOE_EUNSUPPORTED for Is % 128,
 * H > 65536 or shared tile counts past 32-bit tile numbers.
 */
int moe_layer_fwd_shared(const moe_desc *d, int32_t Is, const int32_t *routes, const float *w, const uint16_t *X,
                         const uint16_t *W13, const uint16_t *W2, const uint16_t *W13s, const uint16_t *W2s,
                         int32_t *counts, int32_t *seg_off, moe_src *phi, int32_t *route_row, uint16_t *HU,
                         uint16_t *A, uint16_t *Y, uint16_t *HUs, uint16_t *As, uint16_t *Ys, uint16_t *out, void *ws,
                         size_t ws_bytes, void *stream);

/*
 * MXFP8 routed experts ([MoK] section 5, mixed precision).  Format (the OCP
 * Microscaling reading of "MXFP8"): blocks of 32 consecutive elements along
 * the reduction dimension share one E8M0 scale byte b (scale 2^(b - 127),
 * b = floor(log2 max|x|) - 8 + 127 clamped to [0, 254]; 0 for an all-zero
 * block); every element is the FP8 E4M3 code (1-4-3, bias 7) of x / scale,
 * rounded to nearest with ties to even and saturated at +-448.
 *
 * moe_quantize_mx — row-wise MX quantization of a bf16 matrix.
 *   src     bf16 [rows][K], K a multiple of 32, 16-byte aligned
 *   q       out: uint8 codes [rows][K], 16-byte aligned
 *   scales  out: uint8 scale bytes [rows][K/32]
 * Used for the weights (W13 [L][2I][H] as 2IL rows of H, W2 [L][H][I] as HL
 * rows of I) once per weight update, and inside moe_layer_fwd_mx for X.
 * Errors: MOE_EINVAL for a NULL or misaligned pointer, rows < 0 or K not a
 * positive multiple of 32.
 */
int moe_quantize_mx(const uint16_t *src, int64_t rows, int32_t K, uint8_t *q, uint8_t *scales,
                    void *stream);

/*
 * moe_layer_fwd_mx — the forward share with MXFP8 routed experts: schedule as
 * in moe_schedule; X quantized row-wise (codes Xq [P*Np][H], scales Xs
 * [P*Np][H/32]); the gate/up GEMM pulls each dispatched row's codes from Xq
 * through phi ([MoK] section 2, pull dispatch; padding rows read zeros),
 * accumulates in fp32 and in its epilogue computes a = silu(h) * u and
 * quantizes it (codes Aq [cap][I], scales As [cap][I/32]); the down GEMM
 * multiplies the MX codes of a and W2 into Y (bf16 [cap][H]); the combine is
 * moe_combine's, with the tokens that have one local route written by the
 * down GEMM's epilogue and their rows of Y not written (as in moe_layer_fwd).
 *   W13q, W13s  MX codes [L][2I][H] and scales [L][2I][H/32] of W13 (rows
 *               [0,I) gate, [I,2I) up), e.g. from moe_quantize_mx
 *   W2q, W2s    MX codes [L][H][I] and scales [L][H][I/32] of W2
 *   counts, seg_off, phi, route_row   out, as in moe_schedule
 *   Xq, Xs, Aq, As, Y, out            out (Xq, Aq, Y, out 16-byte aligned;
 *                                     Xs, As, W13s, W2s 4-byte aligned)
 *   HU          nullable out: bf16 [cap][2I], h then u rounded once from the
 *               fp32 accumulators (16-byte aligned), what moe_layer_bwd_mx
 *               needs besides Aq / As
 *   ws >= moe_workspace_bytes(d, MOE_OP_LAYER_FWD)
 * Needs H a multiple of 128 and H <= 65536 (MOE_EUNSUPPORTED otherwise),
 * d->num_batches == 1.  Every float reduction has a fixed order, so repeated
 * calls give bitwise the same outputs.
 */
int moe_layer_fwd_mx(const moe_desc *d, const int32_t *routes, const float *w, const uint16_t *X,
                     const uint8_t *W13q, const uint8_t *W13s, const uint8_t *W2q, const uint8_t *W2s,
                     int32_t *counts, int32_t *seg_off, moe_src *phi, int32_t *route_row, uint8_t *Xq,
                     uint8_t *Xs, uint8_t *Aq, uint8_t *As, uint16_t *HU, uint16_t *Y, uint16_t *out, void *ws,
                     size_t ws_bytes, void *stream);

/*
 * moe_quantize_mx_t — MX quantization of the columns of bf16 matrices:
 * src [batch][R][C] -> q [batch][C][R] codes, scales [batch][C][R/32], each
 * column of src in blocks of 32 consecutive rows (the format above, blocked
 * along R).  The backward's weights: W2 [L][H][I] (R = H) for the down dgrad,
 * W13 [L][2I][H] (R = 2I) for the gate/up dgrad, once per weight update.
 * Needs R a multiple of 32 and C of 8; src and q 16-byte aligned.
 * Errors: MOE_EINVAL for bad sizes or pointers.
 */
int moe_quantize_mx_t(const uint16_t *src, int64_t batch, int32_t R, int32_t C, uint8_t *q, uint8_t *scales,
                      void *stream);

/*
 * moe_layer_bwd_mx — backward of moe_layer_fwd_mx with MXFP8 products ([BPT]
 * section 3 and [MoK] section 6 report an MXFP8 backward; [MoK] section 5
 * fuses the quantization into the loads, the GEMMs and SwiGLU).  Reading:
 * every product takes MX operands blocked along its own reduction dimension,
 * quantized from the value the bf16 backward (moe_layer_bwd) uses there:
 *   dA' = dO_d . W2[l]    over H:  dO_d rows, W2 columns (W2tq);
 *   dXd = dHU . W13[l]    over 2I: dHU rows, W13 columns (W13tq);
 *   dW2[l]  = (w dO_d)^T a, dW13[l] = dHU^T Xd, over the expert's dispatched
 *   rows: both operands quantized along the rows in blocks of 32 rows.
 * a is the forward's Aq / As (dequantized exactly); h and u its saved HU;
 * dw = dA' . a, dA = w dA', dh = dA u silu'(h), du = dA silu(h) in fp32;
 * dHU, dO_d w, dXd and dX are rounded to bf16 once, dW13 / dW2 / dw are fp32.
 *   dOut  bf16 [P][Np][H]   in
 *   w, phi, route_row, seg_off   from the forward
 *   X     bf16 [P][Np][H]   the forward's input (its rows are pulled through
 *                           phi and quantized along the dispatched rows)
 *   HU    bf16 [cap][2I], Aq [cap][I], As [cap][I/32]   saved by the forward
 *   W13tq, W13ts  MX codes [L][H][2I] and scales [L][H][2I/32] (moe_quantize_mx_t
 *                 of W13 with R = 2I, C = H)
 *   W2tq, W2ts    MX codes [L][I][H] and scales [L][I][H/32] (R = H, C = I)
 *   dX, dW13, dW2, dw   out, as in moe_layer_bwd
 *   ws >= moe_workspace_bytes(d, MOE_OP_LAYER_BWD_MX): dXd and dHU (bf16), the
 *   row weights and dw partials, the row codes of dO_d and dHU, and the four
 *   row-blocked operands of the weight gradients stored transposed per expert
 *   segment (the MOE_WS_MX_* fields).  dO_d itself is never written: one pass
 *   pulls the rows of dOut through phi and writes both of its encodings.
 * Pointers: dOut, X, phi, HU, Aq, W13tq, W2tq, dX, ws 16-byte aligned; the
 * others 4-byte aligned.  d->num_batches == 1.  Every reduction has a fixed
 * order, so repeated calls give bitwise the same outputs.
 */
int moe_layer_bwd_mx(const moe_desc *d, const uint16_t *dOut, const float *w, const uint16_t *X, const moe_src *phi,
                     const int32_t *route_row, const int32_t *seg_off, const uint16_t *HU, const uint8_t *Aq,
                     const uint8_t *As, const uint8_t *W13tq, const uint8_t *W13ts, const uint8_t *W2tq,
                     const uint8_t *W2ts, uint16_t *dX, float *dW13, float *dW2, float *dw, void *ws,
                     size_t ws_bytes, void *stream);

/*
 * moe_layer_bwd — backward of the forward share, reusing the forward table
 * ([MoK] section 2: pull reverse-combine, push reverse-dispatch; section 5:
 * router-weight gradient from the SwiGLU activations and the down-projection
 * dgrad; [BPT] section 2.C: weight gradients after the data gradients, each
 * accumulated over the token dimension in one fixed-order pass).
 *   dOut  bf16 [P][Np][H]           in: gradient of the layer output
 *   routes, w, phi, route_row, seg_off   from the forward
 *   Xd bf16 [cap][H], HU bf16 [cap][2I], A bf16 [cap][I]   saved by the forward
 *   W13, W2                          the forward weights
 *   dX    bf16  [P][Np][H]   out: sum over local slots of the row gradients
 *   dW13  float [L][2I][H]   out
 *   dW2   float [L][H][I]    out
 *   dw    float [P][Np][K]   out: router-weight gradient, 0 on non-local slots
 *   ws >= moe_workspace_bytes(d, MOE_OP_LAYER_BWD)
 * The workspace holds dO_d, dO_d times the row's router weight, dXd, dHU
 * (bf16, cap rows each), the row weights and per-row partial sums; the weights
 * and the saved activations are read where they lie (no transposed copies).
 * Every reduction has a fixed order.
 */
int moe_layer_bwd(const moe_desc *d, const uint16_t *dOut, const int32_t *routes, const float *w,
                  const moe_src *phi, const int32_t *route_row, const int32_t *seg_off,
                  const uint16_t *Xd, const uint16_t *HU, const uint16_t *A, const uint16_t *W13,
                  const uint16_t *W2, uint16_t *dX, float *dW13, float *dW2, float *dw, void *ws,
                  size_t ws_bytes, void *stream);

/*
 * Macrobatch ring ([BPT] section 2.B and [MoK] section 4: a fixed ring of
 * token buffers through which macrobatches cycle with no host sync and no
 * dropped token; combine of one macrobatch interleaved with the dispatch of
 * the next; the forward walks the ring in reverse so the activations the
 * backward needs first are the ones still resident).
 *
 * The Np tokens of every partition are cut into M = Np / mb_tokens
 * macrobatches: macrobatch m is tokens [m*mb_tokens, (m+1)*mb_tokens) of each
 * of the P partitions.  Each macrobatch has its own pull table, its expert
 * segments padded to pad_rows, in a ring slot of
 *   capm = moe_ring_capacity_rows(d, mb_tokens) = P*mb_tokens*K + L*(pad_rows-1)
 * rows.  Both calls need mb_tokens to divide Np, ring_slots >= 1,
 * d->num_batches == 1 and H <= 65536 (padding rows read a static zero row);
 * otherwise MOE_EINVAL / MOE_EUNSUPPORTED.  -1 from the two size queries
 * means such an invalid d or mb_tokens.
 */
int64_t moe_ring_capacity_rows(const moe_desc *d, int32_t mb_tokens);
/* op = MOE_OP_LAYER_FWD or MOE_OP_LAYER_BWD (the two calls below);
 * wgrad_group (1..16) matters for the backward only. */
int64_t moe_ring_workspace_bytes(const moe_desc *d, int32_t mb_tokens, int32_t wgrad_group, int op);

/*
 * moe_layer_fwd_ring — the layer forward through the ring.
 *   routes, w, X, W13, W2   as moe_layer_fwd
 *   counts    out: int32 [M][L][P]      per-macrobatch counts
 *   seg_off   out: int32 [M][L+1]       per-macrobatch segment offsets (rows of its slot)
 *   phi       out: moe_src [M][capm]    per-macrobatch pull tables; tok is the
 *                                       token's index inside the macrobatch
 *   route_row out: int32 [P][Np][K]     row of each route inside its macrobatch's
 *                                       slot, -1 for non-local slots
 *   HU        out: bf16 [ring_slots][capm][2I]  the ring: saved pre-activations
 *   A         out: bf16 [ring_slots][capm][I]   and activations
 *   Y         scratch: bf16 [capm][H]   one macrobatch's expert outputs
 *   out       out: bf16 [P][Np][H]      bitwise equal to moe_layer_fwd's
 *   ws >= moe_ring_workspace_bytes(d, mb_tokens, MOE_OP_LAYER_FWD)
 * All M tables come from one batched schedule launch.  The walk is
 * m = M-1, ..., 0: macrobatch m uses slot (M-1-m) % ring_slots; each step is
 * one launch holding the gate/up tiles of m (the dispatch fused into their
 * operand loads) together with the combine of m+1, then the down GEMM of m;
 * a last launch combines macrobatch 0.  As in moe_layer_fwd, the down GEMM
 * writes the outputs of the tokens with one local route itself (from a
 * per-row table of the macrobatch, rebuilt before each down launch) and the
 * combines skip them.  On return slot (M-1-m) % ring_slots holds macrobatch m
 * for every m < min(ring_slots, M).
 */
int moe_layer_fwd_ring(const moe_desc *d, int32_t mb_tokens, int32_t ring_slots, const int32_t *routes,
                       const float *w, const uint16_t *X, const uint16_t *W13, const uint16_t *W2, int32_t *counts,
                       int32_t *seg_off, moe_src *phi, int32_t *route_row, uint16_t *HU, uint16_t *A, uint16_t *Y,
                       uint16_t *out, void *ws, size_t ws_bytes, void *stream);

/*
 * moe_layer_bwd_ring — the backward of moe_layer_fwd_ring, with the same
 * d, mb_tokens and ring_slots, and phi, route_row, seg_off, HU, A as that
 * call left them (X, W13, W2 unchanged since).
 *   wgrad_group           1..16: macrobatches whose weight gradients are
 *                         summed in one pass ([BPT] section 2.C: wgrads
 *                         deferred after the dgrads, accumulated over the
 *                         token dimension in one pass; wgrad_group >= M gives
 *                         a single pass over all macrobatches)
 *   dOut, w, X, W13, W2   as moe_layer_bwd (X replaces the saved Xd)
 *   dX, dW13, dW2, dw     out, as moe_layer_bwd
 *   ws >= moe_ring_workspace_bytes(d, mb_tokens, wgrad_group, MOE_OP_LAYER_BWD)
 *        (it keeps the weight-gradient rows of min(wgrad_group, M) macrobatches)
 * Macrobatches are taken in token order m = 0, 1, ...: those still in the
 * ring (m < ring_slots) use their slot; the others are replayed (their
 * gate/up GEMM recomputed from X into the workspace, bitwise the forward's
 * values).  dX and dw are bitwise equal to moe_layer_bwd's.  The weight
 * gradients of a group are one K loop per output tile over the group's
 * macrobatches in ascending m, and groups are added in ascending order (a
 * fixed order, so reproducible, but rounded differently from moe_layer_bwd's
 * single table).  Errors as moe_layer_fwd_ring, and MOE_EINVAL for a
 * wgrad_group outside 1..16.
 */
int moe_layer_bwd_ring(const moe_desc *d, int32_t mb_tokens, int32_t ring_slots, int32_t wgrad_group,
                       const uint16_t *dOut, const float *w, const uint16_t *X, const uint16_t *W13,
                       const uint16_t *W2, const moe_src *phi, const int32_t *route_row, const int32_t *seg_off,
                       const uint16_t *HU, const uint16_t *A, uint16_t *dX, float *dW13, float *dW2, float *dw,
                       void *ws, size_t ws_bytes, void *stream);

/*
 * Launch trace (optional, host side).  moe_trace_enable(n) records, for the
 * next n kernel launches made by this library on any stream, a start and stop
 * event on the launch's own stream; moe_trace_read copies the finished
 * records (after the caller has synchronised) into host arrays `kernel`
 * (a short name per record, each up to 31 characters plus NUL, 32 bytes per
 * record) and `ms` (elapsed milliseconds), returning the count.
 * moe_trace_enable(0) stops recording and frees the events.  Not thread safe.
 */
int moe_trace_enable(int max_records);
int moe_trace_read(char *kernel, float *ms, int max_records);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
