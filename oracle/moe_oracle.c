/*
 * CPU oracle for one GPU's share of a Mixture-of-Experts layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain, obviously-correct
 * definition that the HIP kernels are checked against.  Only the tests, the
 * smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product path never does.  It shares no code, header, table or helper with
 * the HIP library.
 *
 * Sources (the pages this follows):
 *  [MoK]  "Mixture-of-Kittens: A MoE Megakernel for GB300 NVL72" (reading
 *         notes), section 2 "Push vs. Pull", on-device schedule generation:
 *         counts M, per-expert totals T, offsets S, and the stable cross-rank
 *         position p placed at Phi[S[l] + p]; section 3 (minibatch floor);
 *         section 5 (SonicMoE router-weight gradient).
 *  [SOSO] "Scan once, scatter once", section "The fix is a counting sort":
 *         four stages (count per local expert / peer / logical thread,
 *         prefix, pad to 256 and base row, scatter once), 1,024 logical
 *         threads per peer, 2*P*R route reads and E*1024 counters; and the
 *         opening section's description of the older scheduler (one block
 *         per expert and peer, each rescanning the peer's routes).
 *  [BPT]  "Beyond Peak TFLOPs", section 2.A (one two-column pull table
 *         {src_rank, src_idx} serves all four forward/backward phases) and
 *         section 2.C (weight gradients accumulated over tokens in one pass).
 *  [MoK] section 5 also runs the routed experts in MXFP8 with the activation
 *         quantization fused into the dispatch loads, the grouped GEMMs and
 *         SwiGLU; the MX functions at the end of this file follow the OCP
 *         Microscaling format for that reading (see there).
 *
 * Readings taken where the pages leave a step open (each is listed in the
 * design notes of the repository):
 *  - routes are int32 [P][Np][K]; a partition's routes are flattened
 *    row-major, i = t*K + j;
 *  - o is the 0-based ordinal of a route among its partition's routes to the
 *    same local expert, in ascending flat index (logical threads own
 *    contiguous chunks of ceil(R/NT) routes, which makes the order stable);
 *  - the sum over r' in the position formula runs over all P partitions;
 *  - Phi's src_idx is the token index t; a separate inverse map route_row
 *    gives each route's row (-1 for routes to non-local experts);
 *  - an empty expert gets a zero-length segment; padding rows sit at the
 *    tail of each segment and hold (-1, -1);
 *  - local experts are [base, base + L), segments in ascending local id.
 *
 * Floating point: bf16 inputs are widened exactly; every dot product and
 * every intermediate is kept in double; nothing is rounded to bf16.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double widen_bf16(uint16_t v) {
    uint32_t u = (uint32_t)v << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double sigmoid(double h) { return 1.0 / (1.0 + exp(-h)); }
static double silu(double h) { return h * sigmoid(h); }
/* d/dh [h * sigmoid(h)] = sigmoid(h) * (1 + h * (1 - sigmoid(h))) */
static double silu_grad(double h) {
    double s = sigmoid(h);
    return s * (1.0 + h * (1.0 - s));
}

static int is_local(int32_t e, int base, int L) { return e >= base && e < base + L; }

/* ------------------------------------------------------------------------ */
/* Sizing.                                                                    */
/* ------------------------------------------------------------------------ */

/* Worst-case number of dispatched rows: one row per route (all P*Np*K routes
 * may be local, since ids may repeat inside a token) plus at most pad-1
 * padding rows per expert: sum_l ceil(T_l/pad)*pad <= sum_l (T_l + pad - 1). */
int64_t orc_capacity_rows(int P, int Np, int K, int L, int pad) {
    return (int64_t)P * Np * K + (int64_t)L * (pad - 1);
}

/* Minibatch floor of [MoK] section 3: the smallest T for which the
 * gate/up and down projections each produce at least two waves of
 * bm x bn output tiles on C compute units: T >= 2*C*bm*bn / min(2I, H). */
int64_t orc_minibatch_floor(int64_t C, int64_t bm, int64_t bn, int64_t H, int64_t I) {
    int64_t n = 2 * I < H ? 2 * I : H;
    int64_t num = 2 * C * bm * bn;
    return (num + n - 1) / n;
}

/* ------------------------------------------------------------------------ */
/* Schedule, plain definition ([MoK] section 2).                              */
/* ------------------------------------------------------------------------ */

/*
 * First pass: for every partition r and every route in ascending flat index,
 * a local route gets o = M[l][r]++ (its ordinal among r's routes to l).
 * Totals T[l] = sum_r M[l][r]; segment length = T[l] rounded up to a multiple
 * of pad; S = exclusive prefix of the segment lengths.
 * Second pass: p = sum_{r'} min(M[l][r'], o) + #{r' < r : M[l][r'] > o};
 * row = S[l] + p; Phi[row] = (r, t); route_row[r][t][j] = row.
 * Rows of [0, S[L]) that no route reaches are padding: Phi = (-1, -1).
 *
 * counts: int32 [L][P]; seg_off: int32 [L+1]; phi: int32 [phi_rows][2];
 * route_row: int32 [P][Np][K].  reads (nullable) receives the number of route
 * reads.  Returns S[L] (the padded row count) or -1 if phi_rows is too small.
 */
int64_t orc_schedule(int P, int Np, int K, int L, int base, int pad,
                     const int32_t *routes, int32_t *counts, int32_t *seg_off,
                     int32_t *phi, int64_t phi_rows, int32_t *route_row,
                     int64_t *reads) {
    const int64_t R = (int64_t)Np * K;
    int64_t nreads = 0;
    int32_t *M = (int32_t *)calloc((size_t)L * P, sizeof(int32_t));
    int32_t *ord = (int32_t *)malloc((size_t)(P * R) * sizeof(int32_t));

    /* pass 1: ordinals and counts */
    for (int r = 0; r < P; ++r) {
        for (int64_t i = 0; i < R; ++i) {
            int32_t e = routes[r * R + i];
            ++nreads;
            if (is_local(e, base, L)) {
                int l = e - base;
                ord[r * R + i] = M[l * P + r]++;
            } else {
                ord[r * R + i] = -1;
            }
        }
    }

    /* totals, padding, segment bases */
    seg_off[0] = 0;
    for (int l = 0; l < L; ++l) {
        int64_t T = 0;
        for (int r = 0; r < P; ++r) T += M[l * P + r];
        int64_t padded = (T + pad - 1) / pad * pad;
        seg_off[l + 1] = (int32_t)(seg_off[l] + padded);
    }
    const int64_t npad = seg_off[L];
    if (npad > phi_rows) {
        free(M);
        free(ord);
        return -1;
    }
    for (int l = 0; l < L; ++l)
        for (int r = 0; r < P; ++r) counts[l * P + r] = M[l * P + r];
    for (int64_t row = 0; row < npad; ++row) {
        phi[2 * row] = -1;
        phi[2 * row + 1] = -1;
    }

    /* pass 2: place every route once */
    for (int r = 0; r < P; ++r) {
        for (int64_t i = 0; i < R; ++i) {
            int32_t e = routes[r * R + i];
            ++nreads;
            if (!is_local(e, base, L)) {
                route_row[r * R + i] = -1;
                continue;
            }
            int l = e - base;
            int32_t o = ord[r * R + i];
            int64_t p = 0;
            for (int q = 0; q < P; ++q) {
                int32_t m = M[l * P + q];
                p += m < o ? m : o;
                if (q < r && m > o) p += 1;
            }
            int64_t row = seg_off[l] + p;
            phi[2 * row] = r;
            phi[2 * row + 1] = (int32_t)(i / K);
            route_row[r * R + i] = (int32_t)row;
        }
    }
    if (reads) *reads = nreads;
    free(M);
    free(ord);
    return npad;
}

/* ------------------------------------------------------------------------ */
/* Schedule as the four counting-sort stages of [SOSO], with NT logical       */
/* threads per partition and per-(expert, partition, thread) counters.        */
/* ------------------------------------------------------------------------ */

/*
 * Logical thread tau of partition r owns the contiguous routes
 * [tau*c, min((tau+1)*c, R)), c = ceil(R / NT).
 *  stage 1 (count):   cnt[l][r][tau] = routes of (r, tau) to local expert l;
 *  stage 2 (prefix):  off[l][r][tau] = exclusive prefix over tau, and
 *                     M[l][r] = the total;
 *  stage 3 (pad/base): segment length rounded up to pad, S = prefix;
 *  stage 4 (scatter): thread tau walks its routes again; the k-th route to l
 *                     inside the thread has o = off[l][r][tau] + k, and is
 *                     placed with the same position formula.
 * Same outputs as orc_schedule.  stats[0] = route reads, stats[1] = number of
 * counters allocated (L*P*NT).
 */
int64_t orc_schedule_counting(int P, int Np, int K, int L, int base, int pad, int NT,
                              const int32_t *routes, int32_t *counts, int32_t *seg_off,
                              int32_t *phi, int64_t phi_rows, int32_t *route_row,
                              int64_t *stats) {
    const int64_t R = (int64_t)Np * K;
    const int64_t c = (R + NT - 1) / NT;
    const size_t ncnt = (size_t)L * P * NT;
    int32_t *cnt = (int32_t *)calloc(ncnt, sizeof(int32_t));
    int32_t *off = (int32_t *)calloc(ncnt, sizeof(int32_t));
    int32_t *M = (int32_t *)calloc((size_t)L * P, sizeof(int32_t));
    int32_t *run = (int32_t *)calloc((size_t)L, sizeof(int32_t));
    int64_t nreads = 0;
#define CNT(l, r, t) cnt[((size_t)(l) * P + (r)) * NT + (t)]
#define OFF(l, r, t) off[((size_t)(l) * P + (r)) * NT + (t)]

    /* stage 1: count */
    for (int r = 0; r < P; ++r)
        for (int t = 0; t < NT; ++t) {
            int64_t lo = t * c, hi = (t + 1) * c < R ? (t + 1) * c : R;
            for (int64_t i = lo; i < hi; ++i) {
                int32_t e = routes[r * R + i];
                ++nreads;
                if (is_local(e, base, L)) CNT(e - base, r, t) += 1;
            }
        }
    /* stage 2: thread-major exclusive prefix */
    for (int l = 0; l < L; ++l)
        for (int r = 0; r < P; ++r) {
            int32_t acc = 0;
            for (int t = 0; t < NT; ++t) {
                OFF(l, r, t) = acc;
                acc += CNT(l, r, t);
            }
            M[l * P + r] = acc;
        }
    /* stage 3: pad and base */
    seg_off[0] = 0;
    for (int l = 0; l < L; ++l) {
        int64_t T = 0;
        for (int r = 0; r < P; ++r) T += M[l * P + r];
        seg_off[l + 1] = (int32_t)(seg_off[l] + (T + pad - 1) / pad * pad);
    }
    const int64_t npad = seg_off[L];
    if (npad > phi_rows) {
        free(cnt); free(off); free(M); free(run);
        return -1;
    }
    for (int l = 0; l < L; ++l)
        for (int r = 0; r < P; ++r) counts[l * P + r] = M[l * P + r];
    for (int64_t row = 0; row < npad; ++row) {
        phi[2 * row] = -1;
        phi[2 * row + 1] = -1;
    }
    /* stage 4: scatter */
    for (int r = 0; r < P; ++r)
        for (int t = 0; t < NT; ++t) {
            int64_t lo = t * c, hi = (t + 1) * c < R ? (t + 1) * c : R;
            for (int l = 0; l < L; ++l) run[l] = 0;
            for (int64_t i = lo; i < hi; ++i) {
                int32_t e = routes[r * R + i];
                ++nreads;
                if (!is_local(e, base, L)) {
                    route_row[r * R + i] = -1;
                    continue;
                }
                int l = e - base;
                int32_t o = OFF(l, r, t) + run[l]++;
                int64_t p = 0;
                for (int q = 0; q < P; ++q) {
                    int32_t m = M[l * P + q];
                    p += m < o ? m : o;
                    if (q < r && m > o) p += 1;
                }
                int64_t row = seg_off[l] + p;
                phi[2 * row] = r;
                phi[2 * row + 1] = (int32_t)(i / K);
                route_row[r * R + i] = (int32_t)row;
            }
        }
#undef CNT
#undef OFF
    if (stats) {
        stats[0] = nreads;
        stats[1] = (int64_t)ncnt;
    }
    free(cnt); free(off); free(M); free(run);
    return npad;
}

/* ------------------------------------------------------------------------ */
/* The older scheduler's shape ([SOSO], opening section): one (expert, peer)  */
/* job per pair, each scanning the peer's whole route list twice.  It builds  */
/* each (expert, peer) token list in scan order and merges the lists round-   */
/* robin (round o visits peers 0..P-1 and takes item o where it exists).      */
/* It never evaluates the position formula, so it is an independent check.   */
/* Route ids outside [0, E) in a routing tensor of n ids.  The schedule
 * places only local routes ([MoK] section 2); an id that names no expert at
 * all (a negative "dropped" slot, or one past the last expert) is counted so
 * a caller can tell a corrupt routing tensor from a merely non-local one. */
int64_t orc_invalid_ids(int64_t n, int E, const int32_t *routes) {
    int64_t bad = 0;
    for (int64_t i = 0; i < n; ++i)
        if (routes[i] < 0 || routes[i] >= E) ++bad;
    return bad;
}

/* ------------------------------------------------------------------------ */

int64_t orc_schedule_rescan(int P, int Np, int K, int L, int base, int pad,
                            const int32_t *routes, int32_t *counts, int32_t *seg_off,
                            int32_t *phi, int64_t phi_rows, int32_t *route_row,
                            int64_t *reads) {
    const int64_t R = (int64_t)Np * K;
    int64_t nreads = 0;
    int32_t *M = (int32_t *)calloc((size_t)L * P, sizeof(int32_t));
    /* list[l][r] of flat route indices; at most R each */
    int64_t **lists = (int64_t **)calloc((size_t)L * P, sizeof(int64_t *));

    /* one pass per peer to mark every route as unplaced */
    for (int r = 0; r < P; ++r)
        for (int64_t i = 0; i < R; ++i) {
            (void)routes[r * R + i];
            ++nreads;
            route_row[r * R + i] = -1;
        }
    for (int l = 0; l < L; ++l)
        for (int r = 0; r < P; ++r) {
            int32_t n = 0;
            for (int64_t i = 0; i < R; ++i) { /* scan 1: count */
                ++nreads;
                if (routes[r * R + i] == base + l) ++n;
            }
            M[l * P + r] = n;
            lists[l * P + r] = (int64_t *)malloc(sizeof(int64_t) * (n ? n : 1));
            int32_t k = 0;
            for (int64_t i = 0; i < R; ++i) { /* scan 2: collect in order */
                ++nreads;
                if (routes[r * R + i] == base + l) lists[l * P + r][k++] = i;
            }
        }
    int64_t row = 0;
    int64_t status = 0;
    for (int l = 0; l < L; ++l) {
        seg_off[l] = (int32_t)row;
        int32_t longest = 0, total = 0;
        for (int r = 0; r < P; ++r) {
            if (M[l * P + r] > longest) longest = M[l * P + r];
            total += M[l * P + r];
        }
        int64_t seg_end = row + ((int64_t)total + pad - 1) / pad * pad;
        if (seg_end > phi_rows) { status = -1; break; }
        for (int32_t o = 0; o < longest; ++o)
            for (int r = 0; r < P; ++r)
                if (o < M[l * P + r]) {
                    int64_t i = lists[l * P + r][o];
                    phi[2 * row] = r;
                    phi[2 * row + 1] = (int32_t)(i / K);
                    route_row[r * R + i] = (int32_t)row;
                    ++row;
                }
        for (; row < seg_end; ++row) {
            phi[2 * row] = -1;
            phi[2 * row + 1] = -1;
        }
    }
    if (status == 0) {
        seg_off[L] = (int32_t)row;
        for (int l = 0; l < L; ++l)
            for (int r = 0; r < P; ++r) counts[l * P + r] = M[l * P + r];
    }
    for (int q = 0; q < L * P; ++q) free(lists[q]);
    free(lists);
    free(M);
    if (reads) *reads = nreads;
    return status == 0 ? row : -1;
}

/* ------------------------------------------------------------------------ */
/* Dispatch ([BPT] 2.A: the destination pulls rows by the two-column table).  */
/* ------------------------------------------------------------------------ */

/* Xd[row] = X[phi.part][phi.tok] bit for bit; padding rows are zero.
 * X: bf16 bits [P][Np][H]; Xd: bf16 bits [npad][H]. */
void orc_dispatch(int Np, int H, const uint16_t *X, const int32_t *phi, int64_t npad,
                  uint16_t *Xd) {
    for (int64_t row = 0; row < npad; ++row) {
        int32_t part = phi[2 * row], tok = phi[2 * row + 1];
        if (part < 0) {
            memset(Xd + row * H, 0, sizeof(uint16_t) * H);
        } else {
            memcpy(Xd + row * H, X + ((int64_t)part * Np + tok) * H, sizeof(uint16_t) * H);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Expert FFN (SwiGLU) per dispatched row.                                    */
/* ------------------------------------------------------------------------ */

static int expert_of_row(const int32_t *seg_off, int L, int64_t row) {
    for (int l = 0; l < L; ++l)
        if (row >= seg_off[l] && row < seg_off[l + 1]) return l;
    return -1;
}

/*
 * For each listed dispatched row i of segment l:
 *   h = Xd[i] . W13[l][n]       for n in [0, I)      (gate)
 *   u = Xd[i] . W13[l][I + n]   for n in [0, I)      (up)
 *   a = silu(h) * u
 *   y = a . W2[l][m]            for m in [0, H)      (down)
 * Xd: bf16 bits [*][H]; W13: bf16 bits [L][2I][H]; W2: bf16 bits [L][H][I].
 * Outputs (nullable): HU [n][2I], A [n][I], Y [n][H], all double.
 */
void orc_expert_ffn_rows(int L, int H, int I, const int32_t *seg_off, const uint16_t *Xd,
                         const uint16_t *W13, const uint16_t *W2, const int64_t *rows,
                         int64_t nrows, double *HU, double *A, double *Y) {
#pragma omp parallel
    {
        double *x = (double *)malloc(sizeof(double) * H);
        double *hu = (double *)malloc(sizeof(double) * 2 * I);
        double *a = (double *)malloc(sizeof(double) * I);
#pragma omp for schedule(dynamic, 1)
        for (int64_t q = 0; q < nrows; ++q) {
            int64_t row = rows[q];
            int l = expert_of_row(seg_off, L, row);
            for (int k = 0; k < H; ++k) x[k] = widen_bf16(Xd[row * H + k]);
            if (l < 0) { /* outside every segment: nothing to compute */
                for (int n = 0; n < 2 * I; ++n) hu[n] = 0.0;
            } else {
                const uint16_t *w = W13 + (int64_t)l * 2 * I * H;
                for (int n = 0; n < 2 * I; ++n) {
                    double s = 0.0;
                    for (int k = 0; k < H; ++k) s += x[k] * widen_bf16(w[(int64_t)n * H + k]);
                    hu[n] = s;
                }
            }
            for (int n = 0; n < I; ++n) a[n] = silu(hu[n]) * hu[I + n];
            if (HU) memcpy(HU + q * 2 * I, hu, sizeof(double) * 2 * I);
            if (A) memcpy(A + q * I, a, sizeof(double) * I);
            if (Y) {
                for (int m = 0; m < H; ++m) {
                    double s = 0.0;
                    if (l >= 0) {
                        const uint16_t *w2 = W2 + ((int64_t)l * H + m) * I;
                        for (int n = 0; n < I; ++n) s += a[n] * widen_bf16(w2[n]);
                    }
                    Y[q * H + m] = s;
                }
            }
        }
        free(x);
        free(hu);
        free(a);
    }
}

/* ------------------------------------------------------------------------ */
/* Combine, from dispatched-row outputs.                                       */
/* ------------------------------------------------------------------------ */

/*
 * out[r][t] = sum over j = 0..K-1 with a local expert of
 *             w[r][t][j] * Y[route_row[r][t][j]], in ascending j.
 * Tokens with no local route get zero.  Y rows are looked up through
 * yrow_index: Y_rows[yrow_index[row]] is the output of dispatched row `row`
 * (so a caller may pass only the rows it computed).  tokens: flat r*Np + t.
 * out: double [ntok][H].
 */
void orc_combine_tokens(int Np, int K, int H, const int32_t *route_row, const float *w,
                        const double *Y_rows, const int64_t *yrow_index,
                        const int64_t *tokens, int64_t ntok, double *out) {
#pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < ntok; ++q) {
        int64_t g = tokens[q];
        double *o = out + q * H;
        for (int m = 0; m < H; ++m) o[m] = 0.0;
        for (int j = 0; j < K; ++j) {
            int32_t row = route_row[g * K + j];
            if (row < 0) continue;
            double wj = (double)w[g * K + j];
            const double *y = Y_rows + yrow_index[row] * H;
            for (int m = 0; m < H; ++m) o[m] += wj * y[m];
        }
    }
    (void)Np;
}

/* ------------------------------------------------------------------------ */
/* Whole forward layer per token, straight from the definition (no schedule). */
/* ------------------------------------------------------------------------ */

/*
 * For each listed token (flat g = r*Np + t):
 *   out[g] = sum_{j, e_j local} w[g][j] * W2[l] . (silu(W13[l][:I] x) * W13[l][I:] x)
 * with x = X[g], l = e_j - base.  out: double [ntok][H].
 */
void orc_layer_fwd_tokens(int K, int L, int base, int H, int I, const int32_t *routes,
                          const float *w, const uint16_t *X, const uint16_t *W13,
                          const uint16_t *W2, const int64_t *tokens, int64_t ntok,
                          double *out) {
#pragma omp parallel
    {
        double *x = (double *)malloc(sizeof(double) * H);
        double *a = (double *)malloc(sizeof(double) * I);
#pragma omp for schedule(dynamic, 1)
        for (int64_t q = 0; q < ntok; ++q) {
            int64_t g = tokens[q];
            double *o = out + q * H;
            for (int m = 0; m < H; ++m) o[m] = 0.0;
            for (int k = 0; k < H; ++k) x[k] = widen_bf16(X[g * H + k]);
            for (int j = 0; j < K; ++j) {
                int32_t e = routes[g * K + j];
                if (!is_local(e, base, L)) continue;
                int l = e - base;
                const uint16_t *w13 = W13 + (int64_t)l * 2 * I * H;
                for (int n = 0; n < I; ++n) {
                    double h = 0.0, u = 0.0;
                    for (int k = 0; k < H; ++k) {
                        h += x[k] * widen_bf16(w13[(int64_t)n * H + k]);
                        u += x[k] * widen_bf16(w13[(int64_t)(I + n) * H + k]);
                    }
                    a[n] = silu(h) * u;
                }
                double wj = (double)w[g * K + j];
                for (int m = 0; m < H; ++m) {
                    const uint16_t *w2 = W2 + ((int64_t)l * H + m) * I;
                    double s = 0.0;
                    for (int n = 0; n < I; ++n) s += a[n] * widen_bf16(w2[n]);
                    o[m] += wj * s;
                }
            }
        }
        free(x);
        free(a);
    }
}

/* ------------------------------------------------------------------------ */
/* Backward ([MoK] sections 2 and 5, [BPT] section 2.C).                      */
/* ------------------------------------------------------------------------ */

/*
 * Per route (token g, slot j, local expert l, weight w), with x = X[g],
 * g_out = dOut[g]:
 *   h, u, a as in the forward;  dA' = W2[l]^T g_out  (length I)
 *   dw[g][j]  = <dA', a>        (router-weight gradient from the SwiGLU
 *                                 activations and the down-projection dgrad)
 *   dA = w dA';  dh = dA * u * silu'(h);  du = dA * silu(h)
 *   dX[g]    += W13[l][:I]^T dh + W13[l][I:]^T du
 *   dW2[l]   += (w g_out) (x) a         (outer product, [H][I])
 *   dW13[l]  += [dh; du] (x) x           ([2I][H])
 * Non-local routes contribute nothing and get dw = 0.  The weight gradients
 * accumulate over routes in ascending (token, slot) order, one expert per
 * thread.  All outputs are double and fully overwritten.
 * dX: [P*Np][H]; dW13: [L][2I][H]; dW2: [L][H][I]; dw: [P*Np][K].
 */
void orc_layer_bwd(int64_t ntok, int K, int L, int base, int H, int I, const int32_t *routes,
                   const float *w, const uint16_t *X, const uint16_t *W13, const uint16_t *W2,
                   const uint16_t *dOut, double *dX, double *dW13, double *dW2, double *dw) {
    /* token-side quantities: dX and dw */
#pragma omp parallel
    {
        double *x = (double *)malloc(sizeof(double) * H);
        double *go = (double *)malloc(sizeof(double) * H);
        double *h = (double *)malloc(sizeof(double) * I);
        double *u = (double *)malloc(sizeof(double) * I);
        double *dap = (double *)malloc(sizeof(double) * I);
#pragma omp for schedule(dynamic, 1)
        for (int64_t g = 0; g < ntok; ++g) {
            double *dx = dX + g * H;
            for (int k = 0; k < H; ++k) {
                dx[k] = 0.0;
                x[k] = widen_bf16(X[g * H + k]);
                go[k] = widen_bf16(dOut[g * H + k]);
            }
            for (int j = 0; j < K; ++j) {
                int32_t e = routes[g * K + j];
                dw[g * K + j] = 0.0;
                if (!is_local(e, base, L)) continue;
                int l = e - base;
                const uint16_t *w13 = W13 + (int64_t)l * 2 * I * H;
                const uint16_t *w2 = W2 + (int64_t)l * H * I;
                double wj = (double)w[g * K + j];
                double dot = 0.0;
                for (int n = 0; n < I; ++n) {
                    double hh = 0.0, uu = 0.0, d = 0.0;
                    for (int k = 0; k < H; ++k) {
                        hh += x[k] * widen_bf16(w13[(int64_t)n * H + k]);
                        uu += x[k] * widen_bf16(w13[(int64_t)(I + n) * H + k]);
                        d += go[k] * widen_bf16(w2[(int64_t)k * I + n]);
                    }
                    h[n] = hh;
                    u[n] = uu;
                    dap[n] = d;
                    dot += d * silu(hh) * uu;
                }
                dw[g * K + j] = dot;
                for (int n = 0; n < I; ++n) {
                    double dA = wj * dap[n];
                    double dh = dA * u[n] * silu_grad(h[n]);
                    double du = dA * silu(h[n]);
                    for (int k = 0; k < H; ++k)
                        dx[k] += dh * widen_bf16(w13[(int64_t)n * H + k]) +
                                 du * widen_bf16(w13[(int64_t)(I + n) * H + k]);
                }
            }
        }
        free(x); free(go); free(h); free(u); free(dap);
    }
    /* expert-side quantities: weight gradients, one expert per thread */
#pragma omp parallel
    {
        double *x = (double *)malloc(sizeof(double) * H);
        double *go = (double *)malloc(sizeof(double) * H);
        double *h = (double *)malloc(sizeof(double) * I);
        double *u = (double *)malloc(sizeof(double) * I);
        double *a = (double *)malloc(sizeof(double) * I);
        double *dap = (double *)malloc(sizeof(double) * I);
#pragma omp for schedule(dynamic, 1)
        for (int l = 0; l < L; ++l) {
            double *gw13 = dW13 + (int64_t)l * 2 * I * H;
            double *gw2 = dW2 + (int64_t)l * H * I;
            memset(gw13, 0, sizeof(double) * 2 * I * H);
            memset(gw2, 0, sizeof(double) * H * I);
            const uint16_t *w13 = W13 + (int64_t)l * 2 * I * H;
            const uint16_t *w2 = W2 + (int64_t)l * H * I;
            for (int64_t g = 0; g < ntok; ++g)
                for (int j = 0; j < K; ++j) {
                    if (routes[g * K + j] != base + l) continue;
                    double wj = (double)w[g * K + j];
                    for (int k = 0; k < H; ++k) {
                        x[k] = widen_bf16(X[g * H + k]);
                        go[k] = widen_bf16(dOut[g * H + k]);
                    }
                    for (int n = 0; n < I; ++n) {
                        double hh = 0.0, uu = 0.0, d = 0.0;
                        for (int k = 0; k < H; ++k) {
                            hh += x[k] * widen_bf16(w13[(int64_t)n * H + k]);
                            uu += x[k] * widen_bf16(w13[(int64_t)(I + n) * H + k]);
                            d += go[k] * widen_bf16(w2[(int64_t)k * I + n]);
                        }
                        h[n] = hh; u[n] = uu; dap[n] = d;
                        a[n] = silu(hh) * uu;
                    }
                    for (int m = 0; m < H; ++m)
                        for (int n = 0; n < I; ++n) gw2[(int64_t)m * I + n] += wj * go[m] * a[n];
                    for (int n = 0; n < I; ++n) {
                        double dA = wj * dap[n];
                        double dh = dA * u[n] * silu_grad(h[n]);
                        double du = dA * silu(h[n]);
                        for (int k = 0; k < H; ++k) {
                            gw13[(int64_t)n * H + k] += dh * x[k];
                            gw13[(int64_t)(I + n) * H + k] += du * x[k];
                        }
                    }
                }
        }
        free(x); free(go); free(h); free(u); free(a); free(dap);
    }
}

/*
 * Sampled backward for shapes too large for orc_layer_bwd.
 * Token side: for each listed token, dX[g] and dw[g][*] exactly as above.
 * Expert side: for expert l, the listed elements of dW13[l] (pairs (n, k),
 * n in [0, 2I)) and of dW2[l] (pairs (m, n)), each a sum over all of l's
 * routes in ascending (token, slot) order.  Only the scalars each element
 * needs are formed, so a sample costs O(routes * H) per element.
 */
void orc_bwd_tokens(int K, int L, int base, int H, int I, const int32_t *routes,
                    const float *w, const uint16_t *X, const uint16_t *W13, const uint16_t *W2,
                    const uint16_t *dOut, const int64_t *tokens, int64_t ntok, double *dX,
                    double *dw) {
#pragma omp parallel
    {
        double *x = (double *)malloc(sizeof(double) * H);
        double *go = (double *)malloc(sizeof(double) * H);
        double *h = (double *)malloc(sizeof(double) * I);
        double *u = (double *)malloc(sizeof(double) * I);
        double *dap = (double *)malloc(sizeof(double) * I);
#pragma omp for schedule(dynamic, 1)
        for (int64_t q = 0; q < ntok; ++q) {
            int64_t g = tokens[q];
            double *dx = dX + q * H;
            for (int k = 0; k < H; ++k) {
                dx[k] = 0.0;
                x[k] = widen_bf16(X[g * H + k]);
                go[k] = widen_bf16(dOut[g * H + k]);
            }
            for (int j = 0; j < K; ++j) {
                int32_t e = routes[g * K + j];
                dw[q * K + j] = 0.0;
                if (!is_local(e, base, L)) continue;
                int l = e - base;
                const uint16_t *w13 = W13 + (int64_t)l * 2 * I * H;
                const uint16_t *w2 = W2 + (int64_t)l * H * I;
                double wj = (double)w[g * K + j];
                double dot = 0.0;
                for (int n = 0; n < I; ++n) {
                    double hh = 0.0, uu = 0.0, d = 0.0;
                    for (int k = 0; k < H; ++k) {
                        hh += x[k] * widen_bf16(w13[(int64_t)n * H + k]);
                        uu += x[k] * widen_bf16(w13[(int64_t)(I + n) * H + k]);
                        d += go[k] * widen_bf16(w2[(int64_t)k * I + n]);
                    }
                    h[n] = hh; u[n] = uu; dap[n] = d;
                    dot += d * silu(hh) * uu;
                }
                dw[q * K + j] = dot;
                for (int n = 0; n < I; ++n) {
                    double dA = wj * dap[n];
                    double dh = dA * u[n] * silu_grad(h[n]);
                    double du = dA * silu(h[n]);
                    for (int k = 0; k < H; ++k)
                        dx[k] += dh * widen_bf16(w13[(int64_t)n * H + k]) +
                                 du * widen_bf16(w13[(int64_t)(I + n) * H + k]);
                }
            }
        }
        free(x); free(go); free(h); free(u); free(dap);
    }
}

/* Selected elements of the weight gradients of local expert l ([BPT]
 * section 2.C: sums over the token dimension):
 *   dW13[l][nn][k] = sum over routes to l of d{h,u}[n] * x[k]   (n = nn mod I;
 *                    dh for gate rows nn < I, du for up rows),
 *   dW2[l][m][n]   = sum over routes to l of w * dOut[m] * a[n],
 * routes taken in ascending (token, slot) order.  The per-route quantities of
 * a column n (h, u and dA' = W2[:, n] . dOut) are computed once per route and
 * shared by every requested element of that column; each element's sum still
 * runs over the routes in that order.  a13 / a2 (nullable) receive the sums
 * of the terms' absolute values: a rounding of relative size e in every term
 * moves the sum by at most e times that, which bounds the error of a result
 * computed from rounded intermediates. */
void orc_wgrad_elems(int64_t ntok, int K, int L, int base, int H, int I, int l,
                     const int32_t *routes, const float *w, const uint16_t *X,
                     const uint16_t *W13, const uint16_t *W2, const uint16_t *dOut,
                     const int64_t *w13_elems, int64_t n13, double *g13,
                     const int64_t *w2_elems, int64_t n2, double *g2,
                     double *a13, double *a2) {
    const uint16_t *w13 = W13 + (int64_t)l * 2 * I * H;
    const uint16_t *w2 = W2 + (int64_t)l * H * I;
    (void)L;
    /* the distinct columns n and, per column, its requested elements */
    int *cnt = (int *)calloc((size_t)I + 1, sizeof(int));
    for (int64_t q = 0; q < n13; ++q) cnt[(w13_elems[2 * q] % I) + 1]++;
    for (int64_t q = 0; q < n2; ++q) cnt[w2_elems[2 * q + 1] + 1]++;
    for (int n = 0; n < I; ++n) cnt[n + 1] += cnt[n];
    int64_t *items = (int64_t *)malloc((size_t)(n13 + n2 + 1) * sizeof(int64_t));
    int *fill = (int *)calloc((size_t)I, sizeof(int));
    /* item >= 0: a dW13 element; item < 0: dW2 element -item - 1 */
    for (int64_t q = 0; q < n13; ++q) {
        int n = (int)(w13_elems[2 * q] % I);
        items[cnt[n] + fill[n]++] = q;
    }
    for (int64_t q = 0; q < n2; ++q) {
        int n = (int)w2_elems[2 * q + 1];
        items[cnt[n] + fill[n]++] = -q - 1;
    }
    for (int64_t q = 0; q < n13; ++q) g13[q] = 0.0;
    for (int64_t q = 0; q < n2; ++q) g2[q] = 0.0;
    if (a13)
        for (int64_t q = 0; q < n13; ++q) a13[q] = 0.0;
    if (a2)
        for (int64_t q = 0; q < n2; ++q) a2[q] = 0.0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int n = 0; n < I; ++n) {
        if (cnt[n + 1] == cnt[n]) continue;
        for (int64_t g = 0; g < ntok; ++g)
            for (int j = 0; j < K; ++j) {
                if (routes[g * K + j] != base + l) continue;
                double hh = 0.0, uu = 0.0, d = 0.0;
                for (int k = 0; k < H; ++k) {
                    double xk = widen_bf16(X[g * H + k]);
                    hh += xk * widen_bf16(w13[(int64_t)n * H + k]);
                    uu += xk * widen_bf16(w13[(int64_t)(I + n) * H + k]);
                    d += widen_bf16(dOut[g * H + k]) * widen_bf16(w2[(int64_t)k * I + n]);
                }
                double wr = (double)w[g * K + j];
                double dA = wr * d;
                for (int c = cnt[n]; c < cnt[n + 1]; ++c) {
                    int64_t it = items[c];
                    if (it >= 0) {
                        int64_t nn = w13_elems[2 * it], kk = w13_elems[2 * it + 1];
                        double grad = nn < I ? dA * uu * silu_grad(hh) : dA * silu(hh);
                        double t = grad * widen_bf16(X[g * H + kk]);
                        g13[it] += t;
                        if (a13) a13[it] += fabs(t);
                    } else {
                        int64_t q = -it - 1, m = w2_elems[2 * q];
                        double t = wr * widen_bf16(dOut[g * H + m]) * silu(hh) * uu;
                        g2[q] += t;
                        if (a2) a2[q] += fabs(t);
                    }
                }
            }
    }
    free(cnt); free(items); free(fill);
}

/* ------------------------------------------------------------------------ */
/* MXFP8 ([MoK] section 5, mixed precision: routed experts in MXFP8).        */
/* ------------------------------------------------------------------------ */
/*
 * Reading (the pages name MXFP8 and E4M3 for weights and activations but not
 * the block format): the OCP Microscaling format.  A block is 32 consecutive
 * elements along the reduction dimension; it shares one E8M0 scale
 * X = 2^(floor(log2(amax)) - 8) (8 = exponent of the largest E4M3 normal,
 * 448 = 1.75 * 2^8), stored as the byte e + 127 with e clamped to
 * [-127, 127]; every element is x / X rounded to FP8 E4M3 (1-4-3, bias 7,
 * subnormals, no infinities) to nearest, ties to even, saturating at +-448.
 * An all-zero block gets the byte 0 (X = 2^-127).  The scaling by a power of
 * two is exact, so the codes of a bf16 input are a fixed function of it.
 */

/* value of an E4M3 code (the NaN codes 0x7F / 0xFF return NAN) */
double orc_e4m3_value(int code) {
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    double v = e == 0 ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 10);
    return s ? -v : v;
}

/* nearest E4M3 code of a finite y, ties to even, saturating at +-448 */
int orc_e4m3_encode(double y) {
    int s = signbit(y) ? 1 : 0;
    double a = fabs(y);
    if (a >= 448.0) return (s << 7) | 0x7E;
    int ea;
    frexp(a, &ea); /* a = f * 2^ea, f in [0.5, 1): floor(log2 a) = ea - 1 */
    int qexp = a < ldexp(1.0, -6) ? -9 : (ea - 1) - 3; /* exponent of one quantum */
    double q = nearbyint(ldexp(a, -qexp));              /* default rounding: to nearest even */
    double mag = ldexp(q, qexp);
    if (mag >= 448.0) return (s << 7) | 0x7E;
    if (mag < ldexp(1.0, -6)) return (s << 7) | (int)ldexp(mag, 9); /* subnormal, m = 0..7 */
    int em;
    frexp(mag, &em);
    int E = em - 1;                                      /* mag in [2^E, 2^(E+1)) */
    int m = (int)(ldexp(mag, -E) * 8.0) - 8;
    return (s << 7) | ((E + 7) << 3) | m;
}

/* scale byte and codes of one block of 32 doubles */
static void mx_block(const double *x, uint8_t *q, uint8_t *sbyte) {
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs(x[i]));
    int se = -127;
    if (amax > 0.0) {
        int ea;
        frexp(amax, &ea);
        se = (ea - 1) - 8;
        if (se < -127) se = -127;
        if (se > 127) se = 127;
    }
    *sbyte = (uint8_t)(se + 127);
    for (int i = 0; i < 32; ++i) q[i] = (uint8_t)orc_e4m3_encode(ldexp(x[i], -se));
}

/* row-wise MX quantization of bf16 bits [rows][K] (K % 32 == 0):
 * q [rows][K] codes, s [rows][K/32] scale bytes */
void orc_mx_quantize(const uint16_t *src, int64_t rows, int K, uint8_t *q, uint8_t *s) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double x[32];
        for (int b = 0; b < K / 32; ++b) {
            for (int i = 0; i < 32; ++i) x[i] = widen_bf16(src[r * K + b * 32 + i]);
            mx_block(x, q + r * K + b * 32, s + r * (K / 32) + b);
        }
    }
}

/* the same for double input (the activations a of the SwiGLU) */
void orc_mx_quantize_f64(const double *src, int64_t rows, int K, uint8_t *q, uint8_t *s) {
    for (int64_t r = 0; r < rows; ++r)
        for (int b = 0; b < K / 32; ++b) mx_block(src + r * K + b * 32, q + r * K + b * 32, s + r * (K / 32) + b);
}

static double mx_value(const uint8_t *q, const uint8_t *s, int64_t i) {
    return ldexp(orc_e4m3_value(q[i]), (int)s[i / 32] - 127);
}

/*
 * MXFP8 expert FFN of listed dispatched rows: Xq/Xs are the MX codes and
 * scales of the dispatched rows [*][H]; W13q/W13s [L][2I][H] (blocks along
 * H); W2q/W2s [L][H][I] (blocks along I).  Per row of segment l:
 *   h, u = dequantized row . dequantized W13[l] rows (double);
 *   a = silu(h) * u (double, returned in A);
 *   a is MX-quantized along I (codes Aq [n][I], scales As [n][I/32]);
 *   y = dequantized a . dequantized W2[l] rows (returned in Y).
 * Outputs nullable except that Y needs the quantized a.
 */
void orc_mx_expert_ffn_rows(int L, int H, int I, const int32_t *seg_off, const uint8_t *Xq,
                            const uint8_t *Xs, const uint8_t *W13q, const uint8_t *W13s,
                            const uint8_t *W2q, const uint8_t *W2s, const int64_t *rows, int64_t nrows,
                            double *A, uint8_t *Aq, uint8_t *As, double *Y, double *HUv, double *HUabs) {
#pragma omp parallel
    {
        double *x = (double *)malloc(sizeof(double) * H);
        double *a = (double *)malloc(sizeof(double) * I);
        uint8_t *aq = (uint8_t *)malloc(I);
        uint8_t *as = (uint8_t *)malloc(I / 32);
#pragma omp for schedule(dynamic, 1)
        for (int64_t qi = 0; qi < nrows; ++qi) {
            int64_t row = rows[qi];
            int l = expert_of_row(seg_off, L, row);
            for (int k = 0; k < H; ++k) x[k] = mx_value(Xq + row * H, Xs + row * (H / 32), k);
            for (int n = 0; n < I; ++n) {
                double h = 0.0, u = 0.0, habs = 0.0, uabs = 0.0;
                if (l >= 0) {
                    const uint8_t *gq = W13q + ((int64_t)l * 2 * I + n) * H;
                    const uint8_t *gs = W13s + ((int64_t)l * 2 * I + n) * (H / 32);
                    const uint8_t *uq = W13q + ((int64_t)l * 2 * I + I + n) * H;
                    const uint8_t *us = W13s + ((int64_t)l * 2 * I + I + n) * (H / 32);
                    for (int k = 0; k < H; ++k) {
                        double th = x[k] * mx_value(gq, gs, k), tu = x[k] * mx_value(uq, us, k);
                        h += th;
                        u += tu;
                        habs += fabs(th);
                        uabs += fabs(tu);
                    }
                }
                a[n] = silu(h) * u;
                /* h, u and the sums of their terms' magnitudes (the scale of
                 * any accumulation error in h and u), gate then up */
                if (HUv) {
                    HUv[qi * 2 * I + n] = h;
                    HUv[qi * 2 * I + I + n] = u;
                }
                if (HUabs) {
                    HUabs[qi * 2 * I + n] = habs;
                    HUabs[qi * 2 * I + I + n] = uabs;
                }
            }
            orc_mx_quantize_f64(a, 1, I, aq, as);
            if (A) memcpy(A + qi * I, a, sizeof(double) * I);
            if (Aq) memcpy(Aq + qi * I, aq, I);
            if (As) memcpy(As + qi * (I / 32), as, I / 32);
            if (Y) {
                for (int m = 0; m < H; ++m) {
                    double y = 0.0;
                    if (l >= 0) {
                        const uint8_t *wq = W2q + ((int64_t)l * H + m) * I;
                        const uint8_t *ws = W2s + ((int64_t)l * H + m) * (I / 32);
                        for (int n = 0; n < I; ++n) y += mx_value(aq, as, n) * mx_value(wq, ws, n);
                    }
                    Y[qi * H + m] = y;
                }
            }
        }
        free(x);
        free(a);
        free(aq);
        free(as);
    }
}

/*
 * MXFP8 forward per token straight from the definition (no schedule): as
 * orc_layer_fwd_tokens with every product taken on MX-dequantized operands
 * and a MX-quantized before the down projection.  Xq/Xs: [P*Np][H].
 */
void orc_mx_layer_fwd_tokens(int K, int L, int base, int H, int I, const int32_t *routes,
                             const float *w, const uint8_t *Xq, const uint8_t *Xs,
                             const uint8_t *W13q, const uint8_t *W13s, const uint8_t *W2q,
                             const uint8_t *W2s, const int64_t *tokens, int64_t ntok, double *out) {
#pragma omp parallel
    {
        double *x = (double *)malloc(sizeof(double) * H);
        double *a = (double *)malloc(sizeof(double) * I);
        uint8_t *aq = (uint8_t *)malloc(I);
        uint8_t *as = (uint8_t *)malloc(I / 32);
#pragma omp for schedule(dynamic, 1)
        for (int64_t qi = 0; qi < ntok; ++qi) {
            int64_t g = tokens[qi];
            double *o = out + qi * H;
            for (int m = 0; m < H; ++m) o[m] = 0.0;
            for (int k = 0; k < H; ++k) x[k] = mx_value(Xq + g * H, Xs + g * (H / 32), k);
            for (int j = 0; j < K; ++j) {
                int32_t e = routes[g * K + j];
                if (!is_local(e, base, L)) continue;
                int l = e - base;
                for (int n = 0; n < I; ++n) {
                    double h = 0.0, u = 0.0;
                    const uint8_t *gq = W13q + ((int64_t)l * 2 * I + n) * H;
                    const uint8_t *gs = W13s + ((int64_t)l * 2 * I + n) * (H / 32);
                    const uint8_t *uq = W13q + ((int64_t)l * 2 * I + I + n) * H;
                    const uint8_t *us = W13s + ((int64_t)l * 2 * I + I + n) * (H / 32);
                    for (int k = 0; k < H; ++k) {
                        h += x[k] * mx_value(gq, gs, k);
                        u += x[k] * mx_value(uq, us, k);
                    }
                    a[n] = silu(h) * u;
                }
                orc_mx_quantize_f64(a, 1, I, aq, as);
                double wj = (double)w[g * K + j];
                for (int m = 0; m < H; ++m) {
                    const uint8_t *wq = W2q + ((int64_t)l * H + m) * I;
                    const uint8_t *ws = W2s + ((int64_t)l * H + m) * (I / 32);
                    double y = 0.0;
                    for (int n = 0; n < I; ++n) y += mx_value(aq, as, n) * mx_value(wq, ws, n);
                    o[m] += wj * y;
                }
            }
        }
        free(x);
        free(a);
        free(aq);
        free(as);
    }
}

/* ------------------------------------------------------------------------ */
/* MXFP8 backward ([BPT] section 3 and [MoK] section 6 report an MXFP8       */
/* backward; neither spells out its quantization).                           */
/* ------------------------------------------------------------------------ */
/*
 * Reading: every product of the backward takes MX operands, each blocked
 * along that product's own reduction dimension and quantized from the value
 * the bf16 backward uses at that point:
 *   down dgrad     dA'[i] = sum_k dO[k] W2[l][k][i]   (over H): the row of
 *                  dOut along H, the column i of W2[l] along H;
 *   gate/up dgrad  dXd[k] = sum_n dHU[n] W13[l][n][k] (over 2I): the dHU row
 *                  along 2I, the column k of W13[l] along 2I;
 *   dW2[l][m][i]   = sum_r (w dO)[r][m] a[r][i]      (over the expert's
 *                  dispatched rows): both columns along the rows;
 *   dW13[l][n][k]  = sum_r dHU[r][n] Xd[r][k]         (over the rows): both
 *                  columns along the rows.
 * Row blocks are 32 consecutive dispatched rows (segments start at multiples
 * of 256, so no block straddles two experts); padding rows are zero.  The
 * elementwise steps are those of the bf16 backward: a is what the forward's
 * down projection consumed (its MX codes, dequantized), dw = dA' . a,
 * dA = w dA', dh = dA u silu'(h), du = dA silu(h), with h and u as the
 * forward saves them (bf16).  Where a code depends on a value that the
 * kernels hold in bf16 (h and u, dHU, w dO), that value is rounded as they
 * round it (to float, then to bf16, ties to even) before it is used, so both
 * sides quantize the same number; everything else stays double.
 */

/* float rounding of v, then bf16 with ties to even (finite v) */
static double round_bf16_f32(double v) {
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* the 256 E4M3 values, so dequantizing a row costs one lookup per element */
static double e4m3_tab[256];
static int e4m3_tab_ready;
static void e4m3_tab_init(void) {
    if (e4m3_tab_ready) return;
    for (int c = 0; c < 256; ++c) e4m3_tab[c] = orc_e4m3_value(c);
    e4m3_tab_ready = 1;
}

/* dequantized MX row: out[k] = value(q[k]) * 2^(s[k/32] - 127) */
static void mx_row(const uint8_t *q, const uint8_t *s, int K, double *out) {
    for (int b = 0; b < K / 32; ++b) {
        double sc = ldexp(1.0, (int)s[b] - 127);
        for (int i = 0; i < 32; ++i) out[b * 32 + i] = e4m3_tab[q[b * 32 + i]] * sc;
    }
}

/* MX quantize-then-dequantize of n doubles (n % 32 == 0) in place */
static void mx_roundtrip(double *x, int64_t n) {
    uint8_t q[32], s;
    for (int64_t b = 0; b < n / 32; ++b) {
        mx_block(x + b * 32, q, &s);
        double sc = ldexp(1.0, (int)s - 127);
        for (int i = 0; i < 32; ++i) x[b * 32 + i] = e4m3_tab[q[i]] * sc;
    }
}

/*
 * Token side of the MX backward for the listed tokens: dX[q] (the sum over
 * the token's local slots j ascending of the gate/up dgrad row) and dw[q][j]
 * (0 for slots that are not local).  The forward quantities of each route are
 * recomputed as orc_mx_layer_fwd_tokens computes them.  Weights: W13q/W13s
 * [L][2I][H] (forward, blocks along H); W2tq/W2ts [L][I][H] (column i of W2[l],
 * blocks along H); W13tq/W13ts [L][H][2I] (column k of W13[l], blocks along
 * 2I).  dwabs (nullable) gets the sum of |dA'[i] a[i]| per slot.
 */
void orc_mx_bwd_tokens(int K, int L, int base, int H, int I, const int32_t *routes, const float *w,
                       const uint8_t *Xq, const uint8_t *Xs, const uint8_t *W13q, const uint8_t *W13s,
                       const uint8_t *W2tq, const uint8_t *W2ts, const uint8_t *W13tq, const uint8_t *W13ts,
                       const uint16_t *dOut, const int64_t *tokens, int64_t ntok, double *dX, double *dw,
                       double *dwabs) {
    e4m3_tab_init();
#pragma omp parallel
    {
        double *x = (double *)malloc(sizeof(double) * H);
        double *go = (double *)malloc(sizeof(double) * H);
        double *wr = (double *)malloc(sizeof(double) * (H > 2 * I ? H : 2 * I));
        double *h = (double *)malloc(sizeof(double) * I);
        double *u = (double *)malloc(sizeof(double) * I);
        double *a = (double *)malloc(sizeof(double) * I);
        double *dhu = (double *)malloc(sizeof(double) * 2 * I);
#pragma omp for schedule(dynamic, 1)
        for (int64_t q = 0; q < ntok; ++q) {
            int64_t g = tokens[q];
            double *dx = dX + q * H;
            for (int k = 0; k < H; ++k) {
                dx[k] = 0.0;
                go[k] = widen_bf16(dOut[g * H + k]);
            }
            mx_row(Xq + g * H, Xs + g * (H / 32), H, x);
            mx_roundtrip(go, H); /* dO along H */
            for (int j = 0; j < K; ++j) {
                int32_t e = routes[g * K + j];
                dw[q * K + j] = 0.0;
                if (dwabs) dwabs[q * K + j] = 0.0;
                if (!is_local(e, base, L)) continue;
                int l = e - base;
                /* forward of this route: h, u, a (MX codes, dequantized) */
                for (int n = 0; n < I; ++n) {
                    double hh = 0.0, uu = 0.0;
                    mx_row(W13q + ((int64_t)l * 2 * I + n) * H, W13s + ((int64_t)l * 2 * I + n) * (H / 32), H, wr);
                    for (int k = 0; k < H; ++k) hh += x[k] * wr[k];
                    mx_row(W13q + ((int64_t)l * 2 * I + I + n) * H, W13s + ((int64_t)l * 2 * I + I + n) * (H / 32),
                           H, wr);
                    for (int k = 0; k < H; ++k) uu += x[k] * wr[k];
                    a[n] = silu(hh) * uu;
                    h[n] = round_bf16_f32(hh); /* as saved */
                    u[n] = round_bf16_f32(uu);
                }
                mx_roundtrip(a, I);
                /* down dgrad, router-weight gradient, SwiGLU backward */
                double wj = (double)w[g * K + j], dot = 0.0, dabs = 0.0;
                for (int i = 0; i < I; ++i) {
                    double d = 0.0;
                    mx_row(W2tq + ((int64_t)l * I + i) * H, W2ts + ((int64_t)l * I + i) * (H / 32), H, wr);
                    for (int k = 0; k < H; ++k) d += go[k] * wr[k];
                    dot += d * a[i];
                    dabs += fabs(d * a[i]);
                    double dA = wj * d;
                    dhu[i] = round_bf16_f32(dA * u[i] * silu_grad(h[i]));
                    dhu[I + i] = round_bf16_f32(dA * silu(h[i]));
                }
                dw[q * K + j] = dot;
                if (dwabs) dwabs[q * K + j] = dabs;
                /* gate/up dgrad on dHU quantized along 2I */
                mx_roundtrip(dhu, 2 * I);
                for (int k = 0; k < H; ++k) {
                    double s = 0.0;
                    mx_row(W13tq + ((int64_t)l * H + k) * 2 * I, W13ts + ((int64_t)l * H + k) * (2 * I / 32), 2 * I,
                           wr);
                    for (int n = 0; n < 2 * I; ++n) s += dhu[n] * wr[n];
                    dx[k] += s;
                }
            }
        }
        free(x); free(go); free(wr); free(h); free(u); free(a); free(dhu);
    }
}

/*
 * Weight gradients of local expert l in the MX backward, listed elements:
 * dW13[l][nn][k] (pairs (nn, k), nn in [0, 2I)) and dW2[l][m][i] (pairs
 * (m, i)), each a sum over the segment's dispatched rows [seg_off[l],
 * seg_off[l+1]) in ascending order of the products of two columns quantized
 * along the rows (reading above).  Row r holds the route phi[r] = (part, tok)
 * of slot j with route_row[part*Np + tok][j] == r (padding rows: zero).  Each
 * distinct column is quantized once and shared by its elements.  a13 / a2
 * (nullable) get the sums of the terms' magnitudes.
 */
void orc_mx_wgrad_elems(int Np, int K, int L, int H, int I, int l, const int32_t *seg_off, const int32_t *phi,
                        const int32_t *route_row, const float *w, const uint16_t *X, const uint8_t *Xq,
                        const uint8_t *Xs, const uint8_t *W13q, const uint8_t *W13s, const uint8_t *W2tq,
                        const uint8_t *W2ts, const uint16_t *dOut, const int64_t *w13_elems, int64_t n13,
                        double *g13, const int64_t *w2_elems, int64_t n2, double *g2, double *a13, double *a2) {
    e4m3_tab_init();
    (void)L;
    const int64_t s0 = seg_off[l], nr = (int64_t)seg_off[l + 1] - s0;
    /* per row: token and router weight (-1 / 0 for padding) */
    int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (nr + 1));
    double *wrow = (double *)malloc(sizeof(double) * (nr + 1));
    for (int64_t r = 0; r < nr; ++r) {
        tok[r] = -1;
        wrow[r] = 0.0;
        int32_t p = phi[2 * (s0 + r)], t = phi[2 * (s0 + r) + 1];
        if (p < 0) continue;
        int64_t g = (int64_t)p * Np + t;
        tok[r] = g;
        for (int j = 0; j < K; ++j)
            if (route_row[g * K + j] == s0 + r) wrow[r] = (double)w[g * K + j];
    }
    /* which forward columns n (of I) each row needs: a's 32-blocks of the dW2
     * elements' i, and the i = nn mod I of the dW13 elements */
    char *need_a = (char *)calloc((size_t)I, 1), *need_d = (char *)calloc((size_t)I, 1);
    for (int64_t q = 0; q < n2; ++q) {
        int64_t b = w2_elems[2 * q + 1] / 32;
        for (int i = 0; i < 32; ++i) need_a[b * 32 + i] = 1;
    }
    for (int64_t q = 0; q < n13; ++q) need_d[w13_elems[2 * q] % I] = 1;
    /* per row and needed column: a (dequantized MX), dHU (gate, up) as bf16 */
    double *A = (double *)calloc((size_t)(nr * I + 1), sizeof(double));
    double *DH = (double *)calloc((size_t)(nr * 2 * I + 1), sizeof(double));
#pragma omp parallel
    {
        double *x = (double *)malloc(sizeof(double) * H);
        double *go = (double *)malloc(sizeof(double) * H);
        double *wr = (double *)malloc(sizeof(double) * H);
        double *a = (double *)malloc(sizeof(double) * I);
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < nr; ++r) {
            if (tok[r] < 0) continue;
            int64_t g = tok[r];
            mx_row(Xq + g * H, Xs + g * (H / 32), H, x);
            for (int k = 0; k < H; ++k) go[k] = widen_bf16(dOut[g * H + k]);
            mx_roundtrip(go, H);
            for (int n = 0; n < I; ++n) {
                a[n] = 0.0;
                if (!need_a[n] && !need_d[n]) continue;
                double hh = 0.0, uu = 0.0;
                mx_row(W13q + ((int64_t)l * 2 * I + n) * H, W13s + ((int64_t)l * 2 * I + n) * (H / 32), H, wr);
                for (int k = 0; k < H; ++k) hh += x[k] * wr[k];
                mx_row(W13q + ((int64_t)l * 2 * I + I + n) * H, W13s + ((int64_t)l * 2 * I + I + n) * (H / 32), H,
                       wr);
                for (int k = 0; k < H; ++k) uu += x[k] * wr[k];
                a[n] = silu(hh) * uu;
                if (need_d[n]) {
                    double d = 0.0;
                    mx_row(W2tq + ((int64_t)l * I + n) * H, W2ts + ((int64_t)l * I + n) * (H / 32), H, wr);
                    for (int k = 0; k < H; ++k) d += go[k] * wr[k];
                    double hb = round_bf16_f32(hh), ub = round_bf16_f32(uu), dA = wrow[r] * d;
                    DH[r * 2 * I + n] = round_bf16_f32(dA * ub * silu_grad(hb));
                    DH[r * 2 * I + I + n] = round_bf16_f32(dA * silu(hb));
                }
            }
            /* a's codes: only whole needed blocks are meaningful */
            for (int b = 0; b < I / 32; ++b) {
                if (!need_a[b * 32]) continue;
                mx_roundtrip(a + b * 32, 32);
                for (int i = 0; i < 32; ++i) A[r * I + b * 32 + i] = a[b * 32 + i];
            }
        }
        free(x); free(go); free(wr); free(a);
    }
    /* the elements: each pair of columns quantized along the rows */
#pragma omp parallel
    {
        double *c1 = (double *)malloc(sizeof(double) * (nr + 1));
        double *c2 = (double *)malloc(sizeof(double) * (nr + 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t q = 0; q < n13 + n2; ++q) {
            if (q < n13) {
                int64_t nn = w13_elems[2 * q], k = w13_elems[2 * q + 1];
                for (int64_t r = 0; r < nr; ++r) {
                    c1[r] = DH[r * 2 * I + nn];
                    c2[r] = tok[r] < 0 ? 0.0 : widen_bf16(X[tok[r] * H + k]);
                }
            } else {
                int64_t e = q - n13, m = w2_elems[2 * e], i = w2_elems[2 * e + 1];
                for (int64_t r = 0; r < nr; ++r) {
                    c1[r] = tok[r] < 0 ? 0.0 : round_bf16_f32(wrow[r] * widen_bf16(dOut[tok[r] * H + m]));
                    c2[r] = A[r * I + i];
                }
            }
            mx_roundtrip(c1, nr);
            mx_roundtrip(c2, nr);
            double s = 0.0, sa = 0.0;
            for (int64_t r = 0; r < nr; ++r) {
                s += c1[r] * c2[r];
                sa += fabs(c1[r] * c2[r]);
            }
            if (q < n13) {
                g13[q] = s;
                if (a13) a13[q] = sa;
            } else {
                g2[q - n13] = s;
                if (a2) a2[q - n13] = sa;
            }
        }
        free(c1); free(c2);
    }
    free(tok); free(wrow); free(need_a); free(need_d); free(A); free(DH);
}
