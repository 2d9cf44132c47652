/*
 * moe_shuffle.h -- C ABI of the MoE token shuffle for AMD MI355X (gfx950).
 *
 * The shuffle moves token activations to experts and back on one GPU, with
 * expert-parallel ranks as logical partitions of one HBM buffer:
 *
 *   plan      routing -> counts, offsets, row maps and segment descriptors
 *   dispatch  token-major x -> rank-major xr (one row per (token, rank) pair)
 *             -> expert-major xe (receiver fan-out, read from xr)
 *   combine   expert outputs ye -> gate-weighted top-k sum in token order
 *
 * Sources (cited by page and section):
 *  - FUSCO abstract ("FUSCO: High-Performance Distributed Data Shuffling via
 *    Transformation-Communication Fusion"): the experts need an expert-major
 *    layout, the exchange a device-major one; the layout is captured once
 *    and the reshaping is done on the way; light-weight planning removes
 *    redundant sends.
 *  - FUSCO press summary, Groups 2-3: the interface is a set of logical
 *    segments that say exactly where each row is read and placed, with no
 *    staging buffer and no rearrangement afterwards.
 *  - DySHARP write-up ("Accelerating MoE with Dynamic In-Switch Computing on
 *    Multi-GPUs"), section 2 / Fig. 1 (dispatch and combine, and the
 *    duplicate payloads they carry) and section 5 / Fig. 5, Fig. 9 (a token
 *    keeps one logical index plus a target list; each destination keeps its
 *    own map from that index to its local rows).
 *
 * Conventions for every call:
 *  - Dimensions: T tokens, H hidden size, E experts, k top-k, R ranks,
 *    Epr = E / R experts per rank; expert e lives on rank e / Epr.
 *    KR = min(k, R) (ranks one token can reach), D = min(k, Epr) (experts of
 *    one rank one token can use).  N = number of deduplicated (token, rank)
 *    rows, known on the device after plan (host: moe_shuffle_plan_query).
 *  - Activations are bf16, passed as raw 16-bit patterns; rows are
 *    contiguous and row-major, H elements each.  Gates are fp32 [T, k].
 *    topk_idx is int32 [T, k]; its k ids must be distinct and in [0, E).
 *  - Every pointer argument named as device memory is caller-owned device
 *    memory (e.g. a torch tensor).  The library allocates no device memory.
 *  - H % 8 == 0 and all activation pointers 16-byte aligned (rows move as
 *    16-byte vectors); the workspace must be 256-byte aligned.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    All calls are asynchronous and stream-ordered except
 *    moe_shuffle_plan_query, which synchronises the stream.
 *  - Every function returns an int status (MOE_SHUFFLE_OK or a negative
 *    code below); nothing is thrown across the ABI.  A failing call writes
 *    no output.
 *  - Implementation limits: E + R <= 1024, k <= 64, T * k < 2^31 and
 *    T * k * ceil(H / 512) < 2^31 - 64 (otherwise MOE_SHUFFLE_E_OVERFLOW).
 */
#ifndef MOE_SHUFFLE_H
#define MOE_SHUFFLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
    MOE_SHUFFLE_OK = 0,
    MOE_SHUFFLE_E_INVALID_ARG = -1, /* null pointer, dims <= 0 (T may be 0), k > E, E % R != 0,
                                       overlapping buffers, too small xr */
    MOE_SHUFFLE_E_ALIGN = -2,       /* H % 8 != 0, or a pointer not 16 B (workspace: 256 B) aligned */
    MOE_SHUFFLE_E_WORKSPACE = -3,   /* workspace smaller than moe_shuffle_workspace_size() */
    MOE_SHUFFLE_E_BAD_INDEX = -4,   /* a top-k id out of [0, E) or repeated within a token;
                                       detected on the device, reported by plan_query */
    MOE_SHUFFLE_E_HIP = -5,         /* a HIP launch or runtime call failed (see
                                       moe_shuffle_last_hip_error) */
    MOE_SHUFFLE_E_OVERFLOW = -6     /* sizes beyond the implementation limits */
};

/* Opaque host-side plan handle: the dims plus the workspace it lives in. */
typedef struct moe_shuffle_plan_s* moe_shuffle_plan_t;

typedef struct {
    int32_t num_tokens;  /* T >= 0 */
    int32_t hidden;      /* H > 0, multiple of 8 */
    int32_t num_experts; /* E > 0 */
    int32_t top_k;       /* 0 < k <= E */
    int32_t num_ranks;   /* R > 0, E % R == 0 */
} moe_shuffle_dims;

/* A logical segment: rows [row_offset, row_offset + row_count) of the
 * rank-major buffer (expert == -1) or of the expert-major buffer. */
typedef struct {
    int32_t rank, expert, row_offset, row_count;
} moe_segment;

typedef struct {
    int32_t n_rank_rows;   /* N */
    int32_t n_expert_rows; /* T * k */
    int32_t status;        /* MOE_SHUFFLE_OK or MOE_SHUFFLE_E_BAD_INDEX */
    int32_t max_rank_rows; /* T * KR, the bound usable without a query */
} moe_shuffle_plan_info;

/* Device pointers into the workspace, valid after the plan's kernels ran. */
typedef struct {
    int32_t* expert_count;  /* [E]   routed (token, expert) pairs per expert */
    int32_t* expert_offset; /* [E+1] exclusive prefix sum of expert_count */
    int32_t* rank_count;    /* [R]   distinct tokens per rank */
    int32_t* rank_offset;   /* [R+1] exclusive prefix sum of rank_count; [R] = N */
    int32_t* send_token;    /* [N]   rank row p -> its token */
    int32_t* tok_rank_row;  /* [T][KR] token -> its rank rows, ranks ascending, -1 padded */
    int32_t* fan_src;       /* [T*k] expert row q -> the rank row it is copied from */
    int32_t* fan_dst;       /* [N][D] rank row -> the expert rows it feeds, ascending, -1 padded */
    int32_t* comb_row;      /* [T][k] (token, slot) -> its expert row */
    moe_segment* rank_segs;   /* [R] */
    moe_segment* expert_segs; /* [E] */
    int32_t* status;        /* [1] */
    int32_t* n_rank_rows;   /* [1] N */
    int32_t tok_rank_width; /* KR */
    int32_t fan_dst_width;  /* D */
} moe_shuffle_plan_arrays;

/* Boundary helper, not a step of the method: the bytes of caller-owned
 * device workspace a plan with these dims needs.  The workspace holds the
 * plan's logical segments and row maps (FUSCO press summary, Group 3) and
 * the scratch of the later calls.  Host only, no device work.  Errors:
 * INVALID_ARG, ALIGN, OVERFLOW for bad dims. */
int moe_shuffle_workspace_size(const moe_shuffle_dims* dims, size_t* bytes);

/*
 * Plan the routing (FUSCO abstract: the planner; press summary, Group 3:
 * the logical segments).  Counts experts and distinct (token, rank) pairs
 * per token tile, scans them into offsets, and places every row in
 * ascending token order inside its segment.
 *   topk_idx   device int32 [T, k]; must stay alive until the plan's
 *              kernels have run on `stream`.
 *   workspace  device, >= moe_shuffle_workspace_size() bytes, 256 B
 *              aligned; holds every plan array; must stay alive and
 *              unmodified while the plan is used.
 *   plan       out: a new host handle (free with moe_shuffle_plan_destroy).
 * Bad top-k ids are found on the device: the status word is set, the
 * place step and every later dispatch/combine on this plan write nothing,
 * and moe_shuffle_plan_query returns MOE_SHUFFLE_E_BAD_INDEX.
 */
int moe_shuffle_plan(const moe_shuffle_dims* dims, const int32_t* topk_idx, void* workspace,
                     size_t workspace_bytes, void* stream, moe_shuffle_plan_t* plan);

/*
 * Dispatch = send, then fan-out (FUSCO abstract: token-major to
 * device-major without a separate rearrangement pass; DySHARP section 2:
 * a token bound for a rank is sent there once).
 *   x        device bf16 [T, H], read only.
 *   xr       device bf16 [xr_rows, H]; rows [0, N) are written.  xr_rows
 *            must be >= T*KR, or >= N once moe_shuffle_plan_query has run.
 *   xe       device bf16 [T*k, H]; every row is written.
 * x, xr and xe must not overlap.
 */
int moe_shuffle_dispatch(moe_shuffle_plan_t plan, const void* x, void* xr, int64_t xr_rows,
                         void* xe, void* stream);

/* The send half alone: xr[p] = x[send_token[p]] for p < N.  Each x row is
 * read once and written to its <= KR rank rows. */
int moe_shuffle_dispatch_send(moe_shuffle_plan_t plan, const void* x, void* xr, int64_t xr_rows,
                              void* stream);

/* The receiver half alone (DySHARP section 5: each destination maps the
 * arriving row to its own local rows): xe[q] = xr[fan_src[q]] for q < T*k,
 * done by reading each rank row once and writing its <= D expert rows. */
int moe_shuffle_dispatch_fanout(moe_shuffle_plan_t plan, const void* xr, int64_t xr_rows, void* xe,
                                void* stream);

/*
 * Combine (DySHARP section 2 / Fig. 1: the expert results of a token are
 * summed back into its row):
 *   out[t, h] = bf16_rne( acc ),  acc = +0.0f, then for j = 0 .. k-1:
 *               acc = fmaf(topk_w[t, j], float(ye[comb_row[t, j], h]), acc)
 *   ye      device bf16 [T*k, H] (expert-major, as dispatch laid out xe; it
 *           may be the xe buffer itself).
 *   topk_w  device fp32 [T, k].
 *   out     device bf16 [T, H]; must not overlap ye.
 */
int moe_shuffle_combine(moe_shuffle_plan_t plan, const void* ye, const float* topk_w, void* out,
                        void* stream);

/*
 * Token ranges (DySHARP write-up, section 6 / Fig. 12: the shuffle runs per
 * group of tokens, so the dispatch of one group overlaps later stages of the
 * previous one).  Both calls act on the tokens [t0, t1) of the plan: t0 a
 * multiple of 64 (the plan's token tile), t1 a multiple of 64 or T.
 * Rows land exactly where the whole-batch calls put them: the rank rows of
 * the range are a contiguous sub-range of every rank segment, its expert
 * rows a contiguous sub-range of every expert segment.  Buffers are the
 * whole-batch ones (x [T,H], xr, xe [T*k,H], ye, topk_w [T,k], out [T,H]);
 * calls on disjoint ranges may run concurrently on different streams, and
 * combine of a range may start once that range's dispatch (and expert work)
 * is complete.  Errors as for moe_shuffle_dispatch / moe_shuffle_combine,
 * plus MOE_SHUFFLE_E_INVALID_ARG for a range off those boundaries.
 */
int moe_shuffle_dispatch_range(moe_shuffle_plan_t plan, const void* x, void* xr, int64_t xr_rows, void* xe,
                               int32_t t0, int32_t t1, void* stream);
int moe_shuffle_combine_range(moe_shuffle_plan_t plan, const void* ye, const float* topk_w, void* out, int32_t t0,
                              int32_t t1, void* stream);

/*
 * The return path with one row per (token, rank) pair, and the training
 * direction.  The FUSCO abstract reports training latency, so the shuffle
 * also runs backwards; the DySHARP write-up (section 2 / Fig. 1) notes that
 * the results of a token's experts on one device can be summed before they
 * travel back, which is the send-once rule applied to the return path.
 * Arithmetic: fp32 accumulator from +0, terms in the stated order, one
 * round-to-nearest-even to bf16 per stored row; rows exchanged between ranks
 * are bf16.
 */

/* Receiver side:  rank_rows[p] = bf16( sum over the expert rows q that rank
 * row p fed (fan_dst[p], ascending q) of g(q) * expert_rows[q] ), p < N, with
 * g(q) = topk_w[t][j] for comb_row[t][j] = q, or g = 1 when topk_w is NULL.
 *   expert_rows  device bf16 [T*k, H] (expert-major)
 *   topk_w       device fp32 [T, k] or NULL
 *   rank_rows    device bf16 [rank_rows_cap, H]; rows [0, N) are written;
 *                rank_rows_cap as for xr in moe_shuffle_dispatch.
 * Uses the plan workspace for the gates of the expert rows. */
int moe_shuffle_sum_expert_rows(moe_shuffle_plan_t plan, const void* expert_rows, const float* topk_w,
                                void* rank_rows, int64_t rank_rows_cap, void* stream);

/* Sender side:  out[t] = bf16( sum over t's rank rows p (tok_rank_row[t],
 * ranks ascending) of rank_rows[p] ), t < T.
 *   rank_rows  device bf16 [rank_rows_cap, H] (rows [0, N) are read)
 *   out        device bf16 [T, H]; must not overlap rank_rows. */
int moe_shuffle_sum_rank_rows(moe_shuffle_plan_t plan, const void* rank_rows, int64_t rank_rows_cap, void* out,
                              void* stream);

/* Backward of dispatch (the adjoint of the two copies): grad_xr = the
 * receiver's unweighted sum of grad_xe, then grad_x = the sender's sum of
 * grad_xr.  grad_xe [T*k, H], grad_xr [grad_xr_rows, H], grad_x [T, H],
 * all bf16, pairwise disjoint. */
int moe_shuffle_dispatch_backward(moe_shuffle_plan_t plan, const void* grad_xe, void* grad_xr,
                                  int64_t grad_xr_rows, void* grad_x, void* stream);

/* Combine through per-(token, rank) partial rows: partial = the receiver's
 * gate-weighted sum of ye, out = the sender's sum of partial.  The return
 * path carries N rows instead of T*k.  ye [T*k, H], partial [partial_rows, H],
 * out [T, H] bf16, pairwise disjoint; topk_w fp32 [T, k]. */
int moe_shuffle_combine_rank_partial(moe_shuffle_plan_t plan, const void* ye, const float* topk_w, void* partial,
                                     int64_t partial_rows, void* out, void* stream);

/* The same return path with the per-(token, rank) partials kept in fp32
 * (twice the wire bytes of the bf16 partials, one rounding fewer):
 *   partial[p] = fp32 fma chain of gate * ye over rank row p's expert rows
 *                (ascending), not rounded;
 *   out[t]     = bf16( fp32 sum from +0 of t's partials, ascending rank ).
 * ye [T*k, H] bf16, partial fp32 [partial_rows, H] (partial_rows as for xr
 * in moe_shuffle_dispatch), out [T, H] bf16, pairwise disjoint; topk_w fp32
 * [T, k]. */
int moe_shuffle_combine_rank_partial_f32(moe_shuffle_plan_t plan, const void* ye, const float* topk_w,
                                         float* partial, int64_t partial_rows, void* out, void* stream);

/* Backward of combine, out[t] = sum_j w[t][j] * ye[comb_row[t][j]]:
 *   grad_ye[comb_row[t][j]] = bf16( fp32(w[t][j] * grad_out[t]) )
 *   grad_w[t][j] = sum over h of grad_out[t][h] * ye[comb_row[t][j]][h] in fp32:
 *     each lane sums its elements in ascending h, a fixed 6-level tree adds
 *     the 64 lanes, then the chunks of the row (512 or 1024 elements) are
 *     added in order.
 *   grad_out [T, H], ye [T*k, H], grad_ye [T*k, H] bf16; topk_w, grad_w fp32
 *   [T, k].  grad_ye must not overlap ye or grad_out.  Uses the plan
 *   workspace for the per-chunk partial sums. */
int moe_shuffle_combine_backward(moe_shuffle_plan_t plan, const void* grad_out, const void* ye, const float* topk_w,
                                 void* grad_ye, float* grad_w, void* stream);

/* ---- allocation-free planning ----
 * For callers that cannot allocate memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  The same plan as
 * moe_shuffle_plan, with two differences:
 *  - the workspace is a static device buffer of
 *    MOE_SHUFFLE_STATIC_WORKSPACE_BYTES that the library holds on every GPU
 *    it runs on, until the process ends;
 *  - the host handle is built in the caller's `storage`.
 * The call allocates nothing: no hipMalloc or hipFree, no host heap, no
 * library routine that allocates.  Its first call on a device looks up the
 * buffer's address on that device, once: make that call before capturing
 * later ones into a HIP graph.
 *   dims, topk_idx  as for moe_shuffle_plan.
 *   stream  a stream of the current device (NULL: its null stream).
 *   storage caller-owned host memory for the handle; it must outlive every
 *           use of the plan.
 *   plan    out: the handle, which points into storage.  Every other call
 *           takes it like any plan.  moe_shuffle_plan_destroy on it frees
 *           nothing.
 * There is one buffer per GPU, shared by every call:
 *  - each moe_shuffle_plan_static on a GPU overwrites it, so an earlier
 *    static plan on that GPU is invalid from then on;
 *  - calls on one GPU that overlap in time (other streams, other threads)
 *    race on it.
 * Nothing in it needs clearing between calls: every word a call reads was
 * written earlier by its plan or by the call itself.
 * Errors: as for moe_shuffle_plan, plus:
 *  - MOE_SHUFFLE_E_WORKSPACE when these dims need more than
 *    MOE_SHUFFLE_STATIC_WORKSPACE_BYTES (moe_shuffle_workspace_size tells);
 *    nothing is launched and the buffer keeps its contents;
 *  - MOE_SHUFFLE_E_INVALID_ARG for a stream of another device. */
#define MOE_SHUFFLE_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)

typedef struct {
    uint64_t opaque[64];
} moe_shuffle_plan_storage;

int moe_shuffle_plan_static(const moe_shuffle_dims* dims, const int32_t* topk_idx, void* stream,
                            moe_shuffle_plan_storage* storage, moe_shuffle_plan_t* plan);

/* Boundary helper, not a step of the method.  Synchronises `stream` and
 * reads back N, the size of the rank-major (device-major) buffer of the
 * exchange (FUSCO abstract), and the status word.  Returns the plan's
 * status (MOE_SHUFFLE_OK or MOE_SHUFFLE_E_BAD_INDEX); after it, xr may be
 * sized at exactly N rows. */
int moe_shuffle_plan_query(moe_shuffle_plan_t plan, void* stream, moe_shuffle_plan_info* info);

/* Boundary helper, not a step of the method: the device pointers of the
 * plan arrays, i.e. the logical segment descriptors (FUSCO press summary,
 * Group 3) and the row maps.  No device work, no sync. */
int moe_shuffle_plan_arrays_get(moe_shuffle_plan_t plan, moe_shuffle_plan_arrays* arrays);

/* ---- measurement helper (not a step of the shuffle) ----
 * The reference streaming copy: dst[0 .. bytes) = src[0 .. bytes), 16-byte
 * vectors with the non-temporal hint, one per lane.  It gives the HBM
 * ceiling of a plain copy on the device at hand, against which the row
 * kernels' bandwidth is read.
 *   src, dst  device, 16 B aligned, not overlapping; caller-owned
 *   bytes     a multiple of 16 (0 launches nothing)
 * Returns MOE_SHUFFLE_E_ALIGN for a misaligned pointer or size,
 * MOE_SHUFFLE_E_INVALID_ARG for NULL or overlapping buffers,
 * MOE_SHUFFLE_E_OVERFLOW past 2^31 - 1 blocks of 4 KiB.  Asynchronous on
 * `stream`. */
int moe_shuffle_copy_reference(const void* src, void* dst, size_t bytes, void* stream);

/* Boundary helper, not a step of the method: frees the host handle of
 * moe_shuffle_plan (not the workspace).  NULL and handles of
 * moe_shuffle_plan_static are ignored. */
void moe_shuffle_plan_destroy(moe_shuffle_plan_t plan);

/* Boundary helper, not a step of the method: static text for a status
 * code. */
const char* moe_shuffle_strerror(int code);

/* Boundary helper, not a step of the method: the hipError_t of the
 * calling thread's last MOE_SHUFFLE_E_HIP. */
int moe_shuffle_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_SHUFFLE_H */
