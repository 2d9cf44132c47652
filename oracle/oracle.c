/*
 * oracle.c -- plain, slow, single-threaded CPU oracle for the MoE token shuffle.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * bench's CPU-baseline leg load this library.  The product path (the HIP
 * library under moe_expert_token_amd/) never calls it, and the two share no
 * code: this file defines its own error values, its own bf16 conversions and
 * its own loops.
 *
 * What it computes (sources, cited by page title and section):
 *  - "FUSCO: High-Performance Distributed Data Shuffling via
 *    Transformation-Communication Fusion", abstract: MoE routes each token
 *    to its experts; the expert-major layout the experts need differs from
 *    the device-major layout the exchange needs; a light-weight planner
 *    removes redundant sends.
 *  - The FUSCO press summary, Groups 2-3: the exchange is described by
 *    logical segments, so rows land in place with no extra rearrangement.
 *  - The DySHARP write-up ("Accelerating MoE with Dynamic In-Switch
 *    Computing on Multi-GPUs"), section 2 / Fig. 1 (dispatch sends a token
 *    to every device holding one of its experts; combine sums the expert
 *    results back per token) and section 5 (a token keeps one logical
 *    position plus a list of targets; each destination maps it to its own
 *    local layout).
 *
 * Readings where the pages are silent:
 *  - experts sit on ranks in contiguous blocks: rank(e) = e / (E/R);
 *  - rows inside every rank and expert segment are in ascending token order;
 *  - a (token, rank) pair is sent once even when several of the token's
 *    experts share that rank;
 *  - no capacity limit, padding or dropping; every routed pair is placed;
 *  - combine accumulates in fp32, starting from +0, over the k slots in
 *    ascending slot order, one correctly rounded fused multiply-add per
 *    slot, then one round-to-nearest-even conversion to bf16.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fPIC -shared oracle.c -lm
 * (no fast-math, no OpenMP, no intrinsics).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Error values (the same numbers as the library's, written out here). */
#define OR_OK              0
#define OR_E_INVALID_ARG  (-1)
#define OR_E_ALIGN        (-2)
#define OR_E_BAD_INDEX    (-4)
#define OR_E_OVERFLOW     (-6)

typedef struct {
    int32_t num_tokens, hidden, num_experts, top_k, num_ranks;
} oracle_dims;

/* Every array is caller-allocated host memory.  Sizes, with
 * T tokens, k top-k, E experts, R ranks, Epr = E/R, KR = min(k,R),
 * D = min(k,Epr):
 *   expert_count[E], expert_offset[E+1], rank_count[R], rank_offset[R+1],
 *   send_token[T*KR], tok_rank_row[T*KR], fan_src[T*k], fan_dst[T*KR*D],
 *   comb_row[T*k], rank_segs[R*4], expert_segs[E*4], n_rank_rows[1]. */
typedef struct {
    int32_t *expert_count, *expert_offset, *rank_count, *rank_offset;
    int32_t *send_token, *tok_rank_row, *fan_src, *fan_dst, *comb_row;
    int32_t *rank_segs, *expert_segs, *n_rank_rows;
} oracle_plan_out;

static int imin(int a, int b) { return a < b ? a : b; }

/* Dimension checks (same conditions and codes as the library's). */
int oracle_check_dims(const oracle_dims* d)
{
    if (!d) return OR_E_INVALID_ARG;
    if (d->num_tokens < 0 || d->hidden <= 0 || d->num_experts <= 0 ||
        d->top_k <= 0 || d->num_ranks <= 0)
        return OR_E_INVALID_ARG;
    if (d->top_k > d->num_experts || d->num_experts % d->num_ranks != 0)
        return OR_E_INVALID_ARG;
    if (d->hidden % 8 != 0) return OR_E_ALIGN;
    if ((int64_t)d->num_tokens * d->top_k >= ((int64_t)1 << 31)) return OR_E_OVERFLOW;
    return OR_OK;
}

/* Top-k ids must lie in [0, E) and be distinct within a token's row: a
 * token picks k different experts. */
int oracle_check_index(const oracle_dims* d, const int32_t* idx)
{
    const int T = d->num_tokens, k = d->top_k, E = d->num_experts;
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int e = idx[(int64_t)t * k + j];
            if (e < 0 || e >= E) return OR_E_BAD_INDEX;
            for (int i = 0; i < j; ++i)
                if (idx[(int64_t)t * k + i] == e) return OR_E_BAD_INDEX;
        }
    return OR_OK;
}

/* Does token t route to rank r?  (some slot's expert lives on r) */
static int token_hits_rank(const int32_t* row, int k, int Epr, int r)
{
    for (int j = 0; j < k; ++j)
        if (row[j] / Epr == r) return 1;
    return 0;
}

/*
 * The plan: counts, offsets, and the placement of every (token, rank) row in
 * the rank-major buffer and of every (token, expert) row in the
 * expert-major buffer, plus the segment descriptors.
 */
int oracle_plan(const oracle_dims* d, const int32_t* idx, const oracle_plan_out* o)
{
    int rc = oracle_check_dims(d);
    if (rc) return rc;
    if (d->num_tokens > 0 && !idx) return OR_E_INVALID_ARG;
    rc = oracle_check_index(d, idx);
    if (rc) return rc;

    const int T = d->num_tokens, k = d->top_k, E = d->num_experts, R = d->num_ranks;
    const int Epr = E / R, KR = imin(k, R), D = imin(k, Epr);

    /* Count. expert_count[e]: routed (token, expert) pairs with expert e.
     * rank_count[r]: tokens with at least one expert on r (each token
     * counted once per rank -- the deduplicated sends). */
    for (int e = 0; e < E; ++e) o->expert_count[e] = 0;
    for (int r = 0; r < R; ++r) o->rank_count[r] = 0;
    for (int t = 0; t < T; ++t) {
        const int32_t* row = idx + (int64_t)t * k;
        for (int j = 0; j < k; ++j) o->expert_count[row[j]] += 1;
        for (int r = 0; r < R; ++r)
            if (token_hits_rank(row, k, Epr, r)) o->rank_count[r] += 1;
    }

    /* Offsets: exclusive prefix sums. */
    o->expert_offset[0] = 0;
    for (int e = 0; e < E; ++e) o->expert_offset[e + 1] = o->expert_offset[e] + o->expert_count[e];
    o->rank_offset[0] = 0;
    for (int r = 0; r < R; ++r) o->rank_offset[r + 1] = o->rank_offset[r] + o->rank_count[r];
    const int N = o->rank_offset[R];
    *o->n_rank_rows = N;

    /* Place, visiting tokens in ascending order with one cursor per segment.
     * row_of_rank[r] holds the rank row of the current token on rank r. */
    int32_t* cur_e = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    int32_t* cur_r = (int32_t*)malloc(sizeof(int32_t) * (size_t)R);
    int32_t* row_of_rank = (int32_t*)malloc(sizeof(int32_t) * (size_t)R);
    if (!cur_e || !cur_r || !row_of_rank) { free(cur_e); free(cur_r); free(row_of_rank); return OR_E_INVALID_ARG; }
    for (int e = 0; e < E; ++e) cur_e[e] = o->expert_offset[e];
    for (int r = 0; r < R; ++r) cur_r[r] = o->rank_offset[r];

    for (int t = 0; t < T; ++t) {
        const int32_t* row = idx + (int64_t)t * k;
        int slot = 0;
        /* (a) one rank row per distinct rank, ranks ascending */
        for (int r = 0; r < R; ++r) {
            row_of_rank[r] = -1;
            if (!token_hits_rank(row, k, Epr, r)) continue;
            int p = cur_r[r]++;
            o->send_token[p] = t;
            o->tok_rank_row[(int64_t)t * KR + slot] = p;
            row_of_rank[r] = p;
            ++slot;
        }
        for (; slot < KR; ++slot) o->tok_rank_row[(int64_t)t * KR + slot] = -1;
        /* (b) one expert row per slot */
        for (int j = 0; j < k; ++j) {
            int e = row[j];
            int q = cur_e[e]++;
            o->fan_src[q] = row_of_rank[e / Epr];
            o->comb_row[(int64_t)t * k + j] = q;
        }
    }
    free(cur_e); free(cur_r); free(row_of_rank);

    /* The receiver's local map: for each rank row, the expert rows it feeds,
     * ascending; -1 pads the unused tail. */
    int32_t* fill = (int32_t*)calloc((size_t)(N > 0 ? N : 1), sizeof(int32_t));
    if (!fill) return OR_E_INVALID_ARG;
    for (int64_t i = 0; i < (int64_t)N * D; ++i) o->fan_dst[i] = -1;
    for (int64_t q = 0; q < (int64_t)T * k; ++q) {
        int p = o->fan_src[q];
        o->fan_dst[(int64_t)p * D + fill[p]] = (int32_t)q;
        fill[p] += 1;
    }
    free(fill);

    /* Logical segment descriptors {rank, expert (-1 for a rank segment),
     * row_offset, row_count}. */
    for (int r = 0; r < R; ++r) {
        o->rank_segs[4 * r + 0] = r;
        o->rank_segs[4 * r + 1] = -1;
        o->rank_segs[4 * r + 2] = o->rank_offset[r];
        o->rank_segs[4 * r + 3] = o->rank_count[r];
    }
    for (int e = 0; e < E; ++e) {
        o->expert_segs[4 * e + 0] = e / Epr;
        o->expert_segs[4 * e + 1] = e;
        o->expert_segs[4 * e + 2] = o->expert_offset[e];
        o->expert_segs[4 * e + 3] = o->expert_count[e];
    }
    return OR_OK;
}

/*
 * Dispatch, as two row copies:
 *   send:    xr[p] = x[send_token[p]]     for p < N   (rank-major, deduplicated)
 *   fan-out: xe[q] = xr[fan_src[q]]       for q < T*k (expert-major, read from xr)
 * Rows are bf16 bit patterns, copied unchanged.
 */
int oracle_dispatch(const oracle_dims* d, const int32_t* send_token, const int32_t* fan_src,
                    int32_t n_rank_rows, const uint16_t* x, uint16_t* xr, uint16_t* xe)
{
    int rc = oracle_check_dims(d);
    if (rc) return rc;
    const int64_t H = d->hidden, Tk = (int64_t)d->num_tokens * d->top_k;
    const size_t row_bytes = (size_t)H * sizeof(uint16_t);
    for (int64_t p = 0; p < n_rank_rows; ++p)
        memcpy(xr + p * H, x + (int64_t)send_token[p] * H, row_bytes);
    for (int64_t q = 0; q < Tk; ++q)
        memcpy(xe + q * H, xr + (int64_t)fan_src[q] * H, row_bytes);
    return OR_OK;
}

/* bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 bits. */
static float bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* fp32 -> bf16, round to nearest, ties to even; NaN stays a (quiet) NaN of
 * the same sign; overflow rounds to infinity. */
static uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t keep = u >> 16;          /* the 16 bits that survive truncation */
    uint32_t rest = u & 0xffffu;      /* the 16 bits that are dropped */
    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;
    return (uint16_t)keep;
}

/* The rounding that ends every stored bf16 row, on its own, so that tests
 * can pin it on inputs no sum produces (signalling NaNs, values next to the
 * overflow threshold): out[i] = f32_to_bf16_rne(the fp32 value with bits
 * in[i]).  The bits are taken as integers so that nothing on the way changes
 * a NaN. */
void oracle_round_bf16(const uint32_t* in, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        float f;
        memcpy(&f, &in[i], sizeof f);
        out[i] = f32_to_bf16_rne(f);
    }
}

/*
 * Combine: out[t][h] = bf16( sum over j = 0..k-1 of w[t][j] * ye[comb_row[t][j]][h] ),
 * summed in fp32 from +0 in ascending j with one fused multiply-add per term.
 */
int oracle_combine(const oracle_dims* d, const int32_t* comb_row, const uint16_t* ye,
                   const float* w, uint16_t* out)
{
    int rc = oracle_check_dims(d);
    if (rc) return rc;
    const int T = d->num_tokens, k = d->top_k;
    const int64_t H = d->hidden;
    for (int t = 0; t < T; ++t)
        for (int64_t h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int j = 0; j < k; ++j) {
                int64_t q = comb_row[(int64_t)t * k + j];
                acc = fmaf(w[(int64_t)t * k + j], bf16_to_f32(ye[q * H + h]), acc);
            }
            out[(int64_t)t * H + h] = f32_to_bf16_rne(acc);
        }
    return OR_OK;
}

/* --------------------------------------------------------------------------
 * Training direction and the deduplicated return path.
 *
 * The FUSCO abstract reports end-to-end training latency, so the shuffle
 * runs backwards too.  The DySHARP write-up (section 2 / Fig. 1) notes that
 * the results two experts on one device produce for a token can be summed
 * before they travel back; applied on the return path this gives one row per
 * (token, rank) pair, exactly as dispatch sends one.  Readings (pages
 * silent): every sum accumulates in fp32 from +0 in the stated order; rows
 * that travel between ranks are bf16 (the payload format of the forward
 * direction); each stored row is rounded once to bf16 (nearest, ties even).
 * -------------------------------------------------------------------------- */

/* Backward of dispatch (the adjoint of the two copies):
 *   grad_xr[p] = bf16( sum over the expert rows q that rank row p fed, q
 *                      ascending, of grad_xe[q] )        -- on the receiver
 *   grad_x[t]  = bf16( sum over t's rank rows p, ranks ascending, of
 *                      grad_xr[p] )                       -- on the sender  */
int oracle_dispatch_backward(const oracle_dims* d, const int32_t* fan_dst, const int32_t* tok_rank_row,
                             int32_t n_rank_rows, const uint16_t* grad_xe, uint16_t* grad_xr, uint16_t* grad_x)
{
    int rc = oracle_check_dims(d);
    if (rc) return rc;
    const int T = d->num_tokens, k = d->top_k, R = d->num_ranks;
    const int Epr = d->num_experts / R, KR = imin(k, R), D = imin(k, Epr);
    const int64_t H = d->hidden;
    for (int64_t p = 0; p < n_rank_rows; ++p)
        for (int64_t h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int i = 0; i < D; ++i) {
                int64_t q = fan_dst[p * D + i];
                if (q < 0) break;
                acc = acc + bf16_to_f32(grad_xe[q * H + h]);
            }
            grad_xr[p * H + h] = f32_to_bf16_rne(acc);
        }
    for (int64_t t = 0; t < T; ++t)
        for (int64_t h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int i = 0; i < KR; ++i) {
                int64_t p = tok_rank_row[t * KR + i];
                if (p < 0) break;
                acc = acc + bf16_to_f32(grad_xr[p * H + h]);
            }
            grad_x[t * H + h] = f32_to_bf16_rne(acc);
        }
    return OR_OK;
}

/* Backward of combine, out[t] = sum_j w[t][j] * ye[comb_row[t][j]]:
 *   grad_ye[comb_row[t][j]] = bf16( w[t][j] * grad_out[t] )   (fp32 product)
 *   grad_w[t][j] = sum over h of grad_out[t][h] * ye[comb_row[t][j]][h]
 * The gate gradient is returned in fp64: each bf16 x bf16 product is exact
 * in fp64 and the sum keeps 53 bits, so it stands for the exact value. */
int oracle_combine_backward(const oracle_dims* d, const int32_t* comb_row, const uint16_t* grad_out,
                            const uint16_t* ye, const float* w, uint16_t* grad_ye, double* grad_w)
{
    int rc = oracle_check_dims(d);
    if (rc) return rc;
    const int T = d->num_tokens, k = d->top_k;
    const int64_t H = d->hidden;
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            const int64_t q = comb_row[t * k + j];
            const float wj = w[t * k + j];
            double dot = 0.0;
            for (int64_t h = 0; h < H; ++h) {
                const float g = bf16_to_f32(grad_out[t * H + h]);
                const float prod = wj * g;
                grad_ye[q * H + h] = f32_to_bf16_rne(prod);
                dot += (double)g * (double)bf16_to_f32(ye[q * H + h]);
            }
            grad_w[t * k + j] = dot;
        }
    return OR_OK;
}

/* Combine with one row per (token, rank) on the way back:
 *   partial[p] = bf16( sum over the expert rows q fed by rank row p, q
 *                      ascending, of gate(q) * ye[q] )   (fp32 fma chain)
 *   out[t]     = bf16( sum over t's rank rows p, ranks ascending, of partial[p] )
 * gate(q) is w[t][j] for the (t, j) with comb_row[t][j] = q. */
int oracle_combine_rank_partial(const oracle_dims* d, const int32_t* fan_dst, const int32_t* tok_rank_row,
                                const int32_t* comb_row, int32_t n_rank_rows, const uint16_t* ye, const float* w,
                                uint16_t* partial, uint16_t* out)
{
    int rc = oracle_check_dims(d);
    if (rc) return rc;
    const int T = d->num_tokens, k = d->top_k, R = d->num_ranks;
    const int Epr = d->num_experts / R, KR = imin(k, R), D = imin(k, Epr);
    const int64_t H = d->hidden, Tk = (int64_t)T * k;
    float* gate = (float*)malloc(sizeof(float) * (size_t)(Tk > 0 ? Tk : 1));
    if (!gate) return OR_E_INVALID_ARG;
    for (int64_t i = 0; i < Tk; ++i) gate[comb_row[i]] = w[i];
    for (int64_t p = 0; p < n_rank_rows; ++p)
        for (int64_t h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int i = 0; i < D; ++i) {
                int64_t q = fan_dst[p * D + i];
                if (q < 0) break;
                acc = fmaf(gate[q], bf16_to_f32(ye[q * H + h]), acc);
            }
            partial[p * H + h] = f32_to_bf16_rne(acc);
        }
    free(gate);
    for (int64_t t = 0; t < T; ++t)
        for (int64_t h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int i = 0; i < KR; ++i) {
                int64_t p = tok_rank_row[t * KR + i];
                if (p < 0) break;
                acc = acc + bf16_to_f32(partial[p * H + h]);
            }
            out[t * H + h] = f32_to_bf16_rne(acc);
        }
    return OR_OK;
}

/*
 * The same return path with the per-(token, rank) partials kept in fp32
 * (DySHARP write-up, section 2 / Fig. 1: a device sums its experts' results
 * for a token before they travel back).  partial[p] = the fp32 fused
 * multiply-add chain of gate * ye over rank row p's expert rows in ascending
 * expert row, not rounded; out[t] = bf16 of the fp32 sum, from +0, of
 * token t's partials in ascending rank.  The only rounding to bf16 is the
 * last one.
 */
int oracle_combine_rank_partial_f32(const oracle_dims* d, const int32_t* fan_dst, const int32_t* tok_rank_row,
                                    const int32_t* comb_row, int32_t n_rank_rows, const uint16_t* ye,
                                    const float* w, float* partial, uint16_t* out)
{
    int rc = oracle_check_dims(d);
    if (rc) return rc;
    const int T = d->num_tokens, k = d->top_k, R = d->num_ranks;
    const int Epr = d->num_experts / R, KR = imin(k, R), D = imin(k, Epr);
    const int64_t H = d->hidden, Tk = (int64_t)T * k;
    float* g = (float*)malloc(sizeof(float) * (size_t)(Tk > 0 ? Tk : 1));
    if (!g) return OR_E_INVALID_ARG;
    for (int64_t s = 0; s < Tk; ++s) g[comb_row[s]] = w[s];   /* the gate each expert row carries */
    for (int64_t p = 0; p < n_rank_rows; ++p)
        for (int64_t h = 0; h < H; ++h) {
            float sum = 0.0f;
            for (int e = 0; e < D; ++e) {
                const int64_t q = fan_dst[p * D + e];
                if (q < 0) break;
                sum = fmaf(g[q], bf16_to_f32(ye[q * H + h]), sum);
            }
            partial[p * H + h] = sum;
        }
    free(g);
    for (int64_t t = 0; t < T; ++t)
        for (int64_t h = 0; h < H; ++h) {
            float sum = 0.0f;
            for (int r = 0; r < KR; ++r) {
                const int64_t p = tok_rank_row[t * KR + r];
                if (p < 0) break;
                sum = sum + partial[p * H + h];
            }
            out[t * H + h] = f32_to_bf16_rne(sum);
        }
    return OR_OK;
}
