// abi.hip -- the extern "C" boundary: argument checks, workspace layout,
// launches and error mapping.  Everything that touches data runs in the
// kernels (plan.hip, rows.hip, reduce.hip, combine_bwd.hip); this file only
// validates and launches.
#include <hip/hip_runtime.h>

#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>

#include "internal.h"
#include "moe_shuffle.h"

struct moe_shuffle_plan_s {
    moe_shuffle_dims dims;
    ms::Layout L;
    char* ws;
    int64_t n_known;  // N after moe_shuffle_plan_query, else -1
    int owned;        // 1: allocated by moe_shuffle_plan (destroy frees it); 0: in caller storage
};

static_assert(sizeof(moe_shuffle_plan_s) <= sizeof(moe_shuffle_plan_storage),
              "the plan handle must fit the caller's storage");
static_assert(alignof(moe_shuffle_plan_s) <= alignof(moe_shuffle_plan_storage),
              "the caller's storage must be aligned for the plan handle");

// The workspace of moe_shuffle_plan_static: one per GPU, held until the
// process ends.  In host code this name is only a stand-in, not a device
// address: host code never passes it to a kernel or a copy; it uses the
// address that hipGetSymbolAddress gives on each device (static_scratch).
static __device__ __align__(256) unsigned char scratch[MOE_SHUFFLE_STATIC_WORKSPACE_BYTES];

namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e)
{
    g_last_hip_error = (int)e;
    return MOE_SHUFFLE_E_HIP;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int check_dims(const moe_shuffle_dims* d)
{
    if (!d) return MOE_SHUFFLE_E_INVALID_ARG;
    if (d->num_tokens < 0 || d->hidden <= 0 || d->num_experts <= 0 || d->top_k <= 0 || d->num_ranks <= 0)
        return MOE_SHUFFLE_E_INVALID_ARG;
    if (d->top_k > d->num_experts || d->num_experts % d->num_ranks != 0) return MOE_SHUFFLE_E_INVALID_ARG;
    if (d->hidden % 8 != 0) return MOE_SHUFFLE_E_ALIGN;
    if ((int64_t)d->num_tokens * d->top_k >= ((int64_t)1 << 31)) return MOE_SHUFFLE_E_OVERFLOW;
    if (d->top_k > ms::kMaxTopK || d->num_experts + d->num_ranks > ms::kMaxCols) return MOE_SHUFFLE_E_OVERFLOW;
    // kernels index 512-element pieces of rows with int: every row count
    // (at most T*k) times the pieces per row must stay below 2^31
    const int64_t pieces = ((int64_t)d->hidden / 8 + ms::kWave - 1) / ms::kWave;
    if ((int64_t)d->num_tokens * d->top_k * pieces + 64 >= ((int64_t)1 << 31)) return MOE_SHUFFLE_E_OVERFLOW;
    return MOE_SHUFFLE_OK;
}

bool misaligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) != 0; }

bool overlap(const void* a, size_t an, const void* b, size_t bn)
{
    if (an == 0 || bn == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bn && b0 < a0 + an;
}

int check_plan(const moe_shuffle_plan_s* p)
{
    return (p && p->ws) ? MOE_SHUFFLE_OK : MOE_SHUFFLE_E_INVALID_ARG;
}

template <class T>
T* at(const moe_shuffle_plan_s* p, size_t off) { return (T*)(p->ws + off); }

int64_t rank_rows_needed(const moe_shuffle_plan_s* p)
{
    return p->n_known >= 0 ? p->n_known : (int64_t)p->L.T * p->L.KR;
}

}  // namespace

namespace ms {

void make_layout(const moe_shuffle_dims& d, Layout& L)
{
    L.T = d.num_tokens; L.H = d.hidden; L.E = d.num_experts; L.k = d.top_k; L.R = d.num_ranks;
    L.Epr = L.E / L.R;
    L.KR = L.k < L.R ? L.k : L.R;
    L.D = L.k < L.Epr ? L.k : L.Epr;
    L.C = L.E + L.R;
    L.ntiles = L.T > 0 ? (L.T + kPlanTile - 1) / kPlanTile : 1;
    const size_t T = (size_t)L.T, k = (size_t)L.k, KR = (size_t)L.KR, D = (size_t)L.D, i4 = sizeof(int32_t);
    size_t o = 0;
    auto take = [&](size_t bytes) { const size_t at = o; o = align256(o + bytes); return at; };
    L.status = take(i4);
    L.n_rank_rows = take(i4);
    L.expert_count = take(i4 * L.E);
    L.expert_offset = take(i4 * (L.E + 1));
    L.rank_count = take(i4 * L.R);
    L.rank_offset = take(i4 * (L.R + 1));
    L.send_token = take(i4 * T * KR);
    L.tok_rank_row = take(i4 * T * KR);
    L.fan_src = take(i4 * T * k);
    L.fan_dst = take(i4 * T * KR * D);
    L.comb_row = take(i4 * T * k);
    L.rank_segs = take(4 * i4 * L.R);
    L.expert_segs = take(4 * i4 * L.E);
    L.tile_hist = take(i4 * (size_t)(L.C + 1) * L.ntiles);
    L.tile_base = take(i4 * (size_t)L.C * L.ntiles);
    L.col_total = take(i4 * L.C);
    L.gate_of_row = take(i4 * T * k);
    L.bwd_dots = take(i4 * T * (size_t)((L.H / 8 + kWave - 1) / kWave) * k);
    L.total = o;
}

}  // namespace ms

extern "C" {

int moe_shuffle_workspace_size(const moe_shuffle_dims* dims, size_t* bytes)
{
    const int rc = check_dims(dims);
    if (rc) return rc;
    if (!bytes) return MOE_SHUFFLE_E_INVALID_ARG;
    ms::Layout L;
    ms::make_layout(*dims, L);
    *bytes = L.total;
    return MOE_SHUFFLE_OK;
}

}  // extern "C"

namespace {

// Fills the handle and launches the plan's kernels into its workspace.
hipError_t launch_plan_into(moe_shuffle_plan_s* p, const moe_shuffle_dims* dims, const ms::Layout& L,
                            const int32_t* topk_idx, char* workspace, void* stream)
{
    p->dims = *dims;
    p->L = L;
    p->ws = workspace;
    p->n_known = -1;
    ms::PlanPtrs P;
    P.idx = topk_idx;
    P.status = at<int32_t>(p, L.status);
    P.n_rank_rows = at<int32_t>(p, L.n_rank_rows);
    P.expert_count = at<int32_t>(p, L.expert_count);
    P.expert_offset = at<int32_t>(p, L.expert_offset);
    P.rank_count = at<int32_t>(p, L.rank_count);
    P.rank_offset = at<int32_t>(p, L.rank_offset);
    P.send_token = at<int32_t>(p, L.send_token);
    P.tok_rank_row = at<int32_t>(p, L.tok_rank_row);
    P.fan_src = at<int32_t>(p, L.fan_src);
    P.fan_dst = at<int32_t>(p, L.fan_dst);
    P.comb_row = at<int32_t>(p, L.comb_row);
    P.rank_segs = at<int32_t>(p, L.rank_segs);
    P.expert_segs = at<int32_t>(p, L.expert_segs);
    P.tile_hist = at<int32_t>(p, L.tile_hist);
    P.tile_base = at<int32_t>(p, L.tile_base);
    P.col_total = at<int32_t>(p, L.col_total);
    return ms::launch_plan(L, P, (hipStream_t)stream);
}

// Checks shared by both plan entry points; fills L.
int check_plan_args(const moe_shuffle_dims* dims, const int32_t* topk_idx, const moe_shuffle_plan_t* plan,
                    ms::Layout* L)
{
    const int rc = check_dims(dims);
    if (rc) return rc;
    if (!plan || (dims->num_tokens > 0 && !topk_idx)) return MOE_SHUFFLE_E_INVALID_ARG;
    if (misaligned(topk_idx, 4)) return MOE_SHUFFLE_E_ALIGN;
    ms::make_layout(*dims, *L);
    return MOE_SHUFFLE_OK;
}

// The address of `scratch` on each device, looked up once per device (with
// that device current) by static_scratch.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// The static workspace on the device of `stream` (which must be the current
// device).
int static_scratch(void* stream, char** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= kMaxDevices) return MOE_SHUFFLE_E_INVALID_ARG;
    if (stream) {
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice((hipStream_t)stream, &sdev);
        if (e != hipSuccess) return hip_fail(e);
        if (sdev != dev) return MOE_SHUFFLE_E_INVALID_ARG;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e);
        if (!ptr || misaligned(ptr, 256)) return MOE_SHUFFLE_E_ALIGN;
        g_scratch[dev] = ptr;
    }
    *out = (char*)g_scratch[dev];
    return MOE_SHUFFLE_OK;
}

}  // namespace

extern "C" {

int moe_shuffle_plan(const moe_shuffle_dims* dims, const int32_t* topk_idx, void* workspace, size_t workspace_bytes,
                     void* stream, moe_shuffle_plan_t* plan)
{
    ms::Layout L;
    int rc = check_plan_args(dims, topk_idx, plan, &L);
    if (rc) return rc;
    if (!workspace) return MOE_SHUFFLE_E_INVALID_ARG;
    if (misaligned(workspace, 256)) return MOE_SHUFFLE_E_ALIGN;
    if (workspace_bytes < L.total) return MOE_SHUFFLE_E_WORKSPACE;

    moe_shuffle_plan_s* p = (moe_shuffle_plan_s*)calloc(1, sizeof(moe_shuffle_plan_s));
    if (!p) return MOE_SHUFFLE_E_INVALID_ARG;
    p->owned = 1;
    const hipError_t e = launch_plan_into(p, dims, L, topk_idx, (char*)workspace, stream);
    if (e != hipSuccess) {
        free(p);
        return hip_fail(e);
    }
    *plan = p;
    return MOE_SHUFFLE_OK;
}

int moe_shuffle_plan_static(const moe_shuffle_dims* dims, const int32_t* topk_idx, void* stream,
                            moe_shuffle_plan_storage* storage, moe_shuffle_plan_t* plan)
{
    ms::Layout L;
    int rc = check_plan_args(dims, topk_idx, plan, &L);
    if (rc) return rc;
    if (!storage) return MOE_SHUFFLE_E_INVALID_ARG;
    if (L.total > MOE_SHUFFLE_STATIC_WORKSPACE_BYTES) return MOE_SHUFFLE_E_WORKSPACE;
    char* ws = nullptr;
    rc = static_scratch(stream, &ws);
    if (rc) return rc;
    // the handle lives in the caller's storage (placement new: no allocation)
    moe_shuffle_plan_s* p = new (static_cast<void*>(storage)) moe_shuffle_plan_s{};
    p->owned = 0;
    const hipError_t e = launch_plan_into(p, dims, L, topk_idx, ws, stream);
    if (e != hipSuccess) return hip_fail(e);
    *plan = p;
    return MOE_SHUFFLE_OK;
}

}  // extern "C"

namespace {

int check_send(const moe_shuffle_plan_s* plan, const void* x, const void* xr, int64_t xr_rows)
{
    const ms::Layout& L = plan->L;
    if (!x || !xr) return MOE_SHUFFLE_E_INVALID_ARG;
    if (misaligned(x, 16) || misaligned(xr, 16)) return MOE_SHUFFLE_E_ALIGN;
    if (xr_rows < rank_rows_needed(plan)) return MOE_SHUFFLE_E_INVALID_ARG;
    const size_t row = (size_t)L.H * 2;
    if (overlap(x, row * L.T, xr, row * (size_t)xr_rows)) return MOE_SHUFFLE_E_INVALID_ARG;
    return MOE_SHUFFLE_OK;
}

int check_fanout(const moe_shuffle_plan_s* plan, const void* xr, int64_t xr_rows, const void* xe)
{
    const ms::Layout& L = plan->L;
    if (!xr || !xe) return MOE_SHUFFLE_E_INVALID_ARG;
    if (misaligned(xe, 16) || misaligned(xr, 16)) return MOE_SHUFFLE_E_ALIGN;
    if (xr_rows < rank_rows_needed(plan)) return MOE_SHUFFLE_E_INVALID_ARG;
    const size_t row = (size_t)L.H * 2;
    if (overlap(xe, row * (size_t)L.T * L.k, xr, row * (size_t)xr_rows)) return MOE_SHUFFLE_E_INVALID_ARG;
    return MOE_SHUFFLE_OK;
}

hipError_t launch_send(const moe_shuffle_plan_s* plan, const void* x, void* xr, void* stream)
{
    const ms::Layout& L = plan->L;
    return ms::launch_fanout_rows(true, x, xr, at<int32_t>(plan, L.tok_rank_row), L.KR, L.T, nullptr, L.H,
                                  at<int32_t>(plan, L.status), (hipStream_t)stream);
}

hipError_t launch_fanout(const moe_shuffle_plan_s* plan, const void* xr, void* xe, void* stream)
{
    const ms::Layout& L = plan->L;
    return ms::launch_fanout_rows(false, xr, xe, at<int32_t>(plan, L.fan_dst), L.D, rank_rows_needed(plan),
                                  at<int32_t>(plan, L.n_rank_rows), L.H, at<int32_t>(plan, L.status),
                                  (hipStream_t)stream);
}

}  // namespace

extern "C" {

int moe_shuffle_dispatch_send(moe_shuffle_plan_t plan, const void* x, void* xr, int64_t xr_rows, void* stream)
{
    int rc = check_plan(plan);
    if (rc) return rc;
    if (plan->L.T == 0) return MOE_SHUFFLE_OK;
    rc = check_send(plan, x, xr, xr_rows);
    if (rc) return rc;
    const hipError_t e = launch_send(plan, x, xr, stream);
    return e == hipSuccess ? MOE_SHUFFLE_OK : hip_fail(e);
}

int moe_shuffle_dispatch_fanout(moe_shuffle_plan_t plan, const void* xr, int64_t xr_rows, void* xe, void* stream)
{
    int rc = check_plan(plan);
    if (rc) return rc;
    if (plan->L.T == 0) return MOE_SHUFFLE_OK;
    rc = check_fanout(plan, xr, xr_rows, xe);
    if (rc) return rc;
    const hipError_t e = launch_fanout(plan, xr, xe, stream);
    return e == hipSuccess ? MOE_SHUFFLE_OK : hip_fail(e);
}

int moe_shuffle_dispatch(moe_shuffle_plan_t plan, const void* x, void* xr, int64_t xr_rows, void* xe, void* stream)
{
    int rc = check_plan(plan);
    if (rc) return rc;
    const ms::Layout& L = plan->L;
    if (L.T == 0) return MOE_SHUFFLE_OK;
    // every check before the first launch, so a failing call writes nothing
    rc = check_send(plan, x, xr, xr_rows);
    if (rc) return rc;
    rc = check_fanout(plan, xr, xr_rows, xe);
    if (rc) return rc;
    const size_t row = (size_t)L.H * 2;
    if (overlap(x, row * L.T, xe, row * (size_t)L.T * L.k)) return MOE_SHUFFLE_E_INVALID_ARG;
    hipError_t e = launch_send(plan, x, xr, stream);
    if (e == hipSuccess) e = launch_fanout(plan, xr, xe, stream);
    return e == hipSuccess ? MOE_SHUFFLE_OK : hip_fail(e);
}

int moe_shuffle_combine(moe_shuffle_plan_t plan, const void* ye, const float* topk_w, void* out, void* stream)
{
    int rc = check_plan(plan);
    if (rc) return rc;
    const ms::Layout& L = plan->L;
    if (L.T == 0) return MOE_SHUFFLE_OK;
    if (!ye || !topk_w || !out) return MOE_SHUFFLE_E_INVALID_ARG;
    if (misaligned(ye, 16) || misaligned(out, 16) || misaligned(topk_w, 4)) return MOE_SHUFFLE_E_ALIGN;
    const size_t row = (size_t)L.H * 2;
    if (overlap(ye, row * (size_t)L.T * L.k, out, row * L.T)) return MOE_SHUFFLE_E_INVALID_ARG;
    const hipError_t e = ms::launch_combine_rows(ye, topk_w, at<int32_t>(plan, L.comb_row), out, L.T, L.k, L.H,
                                                 at<int32_t>(plan, L.status), (hipStream_t)stream);
    return e == hipSuccess ? MOE_SHUFFLE_OK : hip_fail(e);
}

int moe_shuffle_sum_expert_rows(moe_shuffle_plan_t plan, const void* expert_rows, const float* topk_w,
                                void* rank_rows, int64_t rank_rows_cap, void* stream)
{
    int rc = check_plan(plan);
    if (rc) return rc;
    const ms::Layout& L = plan->L;
    if (L.T == 0) return MOE_SHUFFLE_OK;
    if (!expert_rows || !rank_rows) return MOE_SHUFFLE_E_INVALID_ARG;
    if (misaligned(expert_rows, 16) || misaligned(rank_rows, 16) || misaligned(topk_w, 4)) return MOE_SHUFFLE_E_ALIGN;
    const int64_t need = rank_rows_needed(plan);
    if (rank_rows_cap < need) return MOE_SHUFFLE_E_INVALID_ARG;
    const size_t row = (size_t)L.H * 2;
    if (overlap(expert_rows, row * (size_t)L.T * L.k, rank_rows, row * (size_t)rank_rows_cap))
        return MOE_SHUFFLE_E_INVALID_ARG;
    const hipError_t e = ms::launch_sum_expert_rows(
        expert_rows, (int64_t)L.T * L.k, topk_w, at<int32_t>(plan, L.comb_row), at<float>(plan, L.gate_of_row),
        at<int32_t>(plan, L.fan_dst), L.D, rank_rows, need, at<int32_t>(plan, L.n_rank_rows), L.H,
        at<int32_t>(plan, L.status), (hipStream_t)stream);
    return e == hipSuccess ? MOE_SHUFFLE_OK : hip_fail(e);
}

int moe_shuffle_sum_rank_rows(moe_shuffle_plan_t plan, const void* rank_rows, int64_t rank_rows_cap, void* out,
                              void* stream)
{
    int rc = check_plan(plan);
    if (rc) return rc;
    const ms::Layout& L = plan->L;
    if (L.T == 0) return MOE_SHUFFLE_OK;
    if (!rank_rows || !out) return MOE_SHUFFLE_E_INVALID_ARG;
    if (misaligned(rank_rows, 16) || misaligned(out, 16)) return MOE_SHUFFLE_E_ALIGN;
    if (rank_rows_cap < rank_rows_needed(plan)) return MOE_SHUFFLE_E_INVALID_ARG;
    const size_t row = (size_t)L.H * 2;
    if (overlap(rank_rows, row * (size_t)rank_rows_cap, out, row * L.T)) return MOE_SHUFFLE_E_INVALID_ARG;
    const hipError_t e = ms::launch_sum_rank_rows(rank_rows, rank_rows_cap, at<int32_t>(plan, L.tok_rank_row), L.KR,
                                                  out, L.T, L.H, at<int32_t>(plan, L.status), (hipStream_t)stream);
    return e == hipSuccess ? MOE_SHUFFLE_OK : hip_fail(e);
}

int moe_shuffle_dispatch_backward(moe_shuffle_plan_t plan, const void* grad_xe, void* grad_xr, int64_t grad_xr_rows,
                                  void* grad_x, void* stream)
{
    int rc = check_plan(plan);
    if (rc) return rc;
    const ms::Layout& L = plan->L;
    if (L.T == 0) return MOE_SHUFFLE_OK;
    if (!grad_xe || !grad_xr || !grad_x) return MOE_SHUFFLE_E_INVALID_ARG;
    const size_t row = (size_t)L.H * 2;
    if (overlap(grad_xe, row * (size_t)L.T * L.k, grad_x, row * L.T)) return MOE_SHUFFLE_E_INVALID_ARG;
    if (misaligned(grad_x, 16) || misaligned(grad_xr, 16) || misaligned(grad_xe, 16)) return MOE_SHUFFLE_E_ALIGN;
    if (grad_xr_rows < rank_rows_needed(plan)) return MOE_SHUFFLE_E_INVALID_ARG;
    if (overlap(grad_xr, row * (size_t)grad_xr_rows, grad_x, row * L.T) ||
        overlap(grad_xe, row * (size_t)L.T * L.k, grad_xr, row * (size_t)grad_xr_rows))
        return MOE_SHUFFLE_E_INVALID_ARG;
    rc = moe_shuffle_sum_expert_rows(plan, grad_xe, nullptr, grad_xr, grad_xr_rows, stream);
    if (rc) return rc;
    return moe_shuffle_sum_rank_rows(plan, grad_xr, grad_xr_rows, grad_x, stream);
}

int moe_shuffle_combine_rank_partial(moe_shuffle_plan_t plan, const void* ye, const float* topk_w, void* partial,
                                     int64_t partial_rows, void* out, void* stream)
{
    int rc = check_plan(plan);
    if (rc) return rc;
    const ms::Layout& L = plan->L;
    if (L.T == 0) return MOE_SHUFFLE_OK;
    if (!ye || !topk_w || !partial || !out) return MOE_SHUFFLE_E_INVALID_ARG;
    if (misaligned(ye, 16) || misaligned(partial, 16) || misaligned(out, 16) || misaligned(topk_w, 4))
        return MOE_SHUFFLE_E_ALIGN;
    if (partial_rows < rank_rows_needed(plan)) return MOE_SHUFFLE_E_INVALID_ARG;
    const size_t row = (size_t)L.H * 2;
    if (overlap(ye, row * (size_t)L.T * L.k, out, row * L.T) ||
        overlap(ye, row * (size_t)L.T * L.k, partial, row * (size_t)partial_rows) ||
        overlap(partial, row * (size_t)partial_rows, out, row * L.T))
        return MOE_SHUFFLE_E_INVALID_ARG;
    rc = moe_shuffle_sum_expert_rows(plan, ye, topk_w, partial, partial_rows, stream);
    if (rc) return rc;
    return moe_shuffle_sum_rank_rows(plan, partial, partial_rows, out, stream);
}

int moe_shuffle_combine_rank_partial_f32(moe_shuffle_plan_t plan, const void* ye, const float* topk_w,
                                         float* partial, int64_t partial_rows, void* out, void* stream)
{
    int rc = check_plan(plan);
    if (rc) return rc;
    const ms::Layout& L = plan->L;
    if (L.T == 0) return MOE_SHUFFLE_OK;
    if (!ye || !topk_w || !partial || !out) return MOE_SHUFFLE_E_INVALID_ARG;
    if (misaligned(ye, 16) || misaligned(partial, 16) || misaligned(out, 16) || misaligned(topk_w, 4))
        return MOE_SHUFFLE_E_ALIGN;
    const int64_t need = rank_rows_needed(plan);
    if (partial_rows < need) return MOE_SHUFFLE_E_INVALID_ARG;
    const size_t row = (size_t)L.H * 2, prow = (size_t)L.H * 4;
    if (overlap(ye, row * (size_t)L.T * L.k, out, row * L.T) ||
        overlap(ye, row * (size_t)L.T * L.k, partial, prow * (size_t)partial_rows) ||
        overlap(partial, prow * (size_t)partial_rows, out, row * L.T))
        return MOE_SHUFFLE_E_INVALID_ARG;
    hipError_t e = ms::launch_sum_expert_rows(ye, (int64_t)L.T * L.k, topk_w, at<int32_t>(plan, L.comb_row),
                                              at<float>(plan, L.gate_of_row), at<int32_t>(plan, L.fan_dst), L.D,
                                              partial, need, at<int32_t>(plan, L.n_rank_rows), L.H,
                                              at<int32_t>(plan, L.status), (hipStream_t)stream, true);
    if (e != hipSuccess) return hip_fail(e);
    e = ms::launch_sum_rank_rows(partial, partial_rows, at<int32_t>(plan, L.tok_rank_row), L.KR, out, L.T, L.H,
                                 at<int32_t>(plan, L.status), (hipStream_t)stream, true);
    return e == hipSuccess ? MOE_SHUFFLE_OK : hip_fail(e);
}

int moe_shuffle_combine_backward(moe_shuffle_plan_t plan, const void* grad_out, const void* ye, const float* topk_w,
                                 void* grad_ye, float* grad_w, void* stream)
{
    int rc = check_plan(plan);
    if (rc) return rc;
    const ms::Layout& L = plan->L;
    if (L.T == 0) return MOE_SHUFFLE_OK;
    if (!grad_out || !ye || !topk_w || !grad_ye || !grad_w) return MOE_SHUFFLE_E_INVALID_ARG;
    if (misaligned(grad_out, 16) || misaligned(ye, 16) || misaligned(grad_ye, 16) || misaligned(topk_w, 4) ||
        misaligned(grad_w, 4))
        return MOE_SHUFFLE_E_ALIGN;
    const size_t row = (size_t)L.H * 2, erows = row * (size_t)L.T * L.k;
    if (overlap(grad_ye, erows, ye, erows) || overlap(grad_ye, erows, grad_out, row * L.T) ||
        overlap(grad_w, sizeof(float) * (size_t)L.T * L.k, grad_ye, erows))
        return MOE_SHUFFLE_E_INVALID_ARG;
    const hipError_t e = ms::launch_combine_backward(grad_out, ye, topk_w, at<int32_t>(plan, L.comb_row), grad_ye,
                                                     grad_w, at<float>(plan, L.bwd_dots), L.T, L.k, L.H,
                                                     at<int32_t>(plan, L.status), (hipStream_t)stream);
    return e == hipSuccess ? MOE_SHUFFLE_OK : hip_fail(e);
}

int moe_shuffle_dispatch_range(moe_shuffle_plan_t plan, const void* x, void* xr, int64_t xr_rows, void* xe,
                               int32_t t0, int32_t t1, void* stream)
{
    int rc = check_plan(plan);
    if (rc) return rc;
    const ms::Layout& L = plan->L;
    if (t0 < 0 || t1 < t0 || t1 > L.T || t0 % ms::kPlanTile != 0 || (t1 % ms::kPlanTile != 0 && t1 != L.T))
        return MOE_SHUFFLE_E_INVALID_ARG;
    if (t1 == t0) return MOE_SHUFFLE_OK;
    rc = check_send(plan, x, xr, xr_rows);
    if (rc) return rc;
    rc = check_fanout(plan, xr, xr_rows, xe);
    if (rc) return rc;
    const size_t row = (size_t)L.H * 2;
    if (overlap(x, row * L.T, xe, row * (size_t)L.T * L.k)) return MOE_SHUFFLE_E_INVALID_ARG;
    const int32_t* status = at<int32_t>(plan, L.status);
    hipError_t e = ms::launch_fanout_rows(true, (const char*)x + row * (size_t)t0, xr,
                                          at<int32_t>(plan, L.tok_rank_row) + (size_t)t0 * L.KR, L.KR, t1 - t0,
                                          nullptr, L.H, status, (hipStream_t)stream);
    if (e == hipSuccess)
        e = ms::launch_fanout_range(xr, xe, at<int32_t>(plan, L.fan_dst), L.D, at<int32_t>(plan, L.rank_offset),
                                    at<int32_t>(plan, L.tile_base), at<int32_t>(plan, L.col_total), L.E, L.R, L.ntiles,
                                    t0, t1, L.T, L.KR, L.H, status, (hipStream_t)stream);
    return e == hipSuccess ? MOE_SHUFFLE_OK : hip_fail(e);
}

int moe_shuffle_combine_range(moe_shuffle_plan_t plan, const void* ye, const float* topk_w, void* out, int32_t t0,
                              int32_t t1, void* stream)
{
    int rc = check_plan(plan);
    if (rc) return rc;
    const ms::Layout& L = plan->L;
    if (t0 < 0 || t1 < t0 || t1 > L.T || t0 % ms::kPlanTile != 0 || (t1 % ms::kPlanTile != 0 && t1 != L.T))
        return MOE_SHUFFLE_E_INVALID_ARG;
    if (t1 == t0) return MOE_SHUFFLE_OK;
    if (!ye || !topk_w || !out) return MOE_SHUFFLE_E_INVALID_ARG;
    if (misaligned(ye, 16) || misaligned(out, 16) || misaligned(topk_w, 4)) return MOE_SHUFFLE_E_ALIGN;
    const size_t row = (size_t)L.H * 2;
    if (overlap(ye, row * (size_t)L.T * L.k, out, row * L.T)) return MOE_SHUFFLE_E_INVALID_ARG;
    const hipError_t e = ms::launch_combine_rows(ye, topk_w + (size_t)t0 * L.k,
                                                 at<int32_t>(plan, L.comb_row) + (size_t)t0 * L.k,
                                                 (char*)out + row * (size_t)t0, t1 - t0, L.k, L.H,
                                                 at<int32_t>(plan, L.status), (hipStream_t)stream);
    return e == hipSuccess ? MOE_SHUFFLE_OK : hip_fail(e);
}

int moe_shuffle_plan_query(moe_shuffle_plan_t plan, void* stream, moe_shuffle_plan_info* info)
{
    int rc = check_plan(plan);
    if (rc) return rc;
    if (!info) return MOE_SHUFFLE_E_INVALID_ARG;
    int32_t st = 0, n = 0;
    hipError_t e = hipMemcpyAsync(&st, at<int32_t>(plan, plan->L.status), sizeof st, hipMemcpyDeviceToHost,
                                  (hipStream_t)stream);
    if (e == hipSuccess)
        e = hipMemcpyAsync(&n, at<int32_t>(plan, plan->L.n_rank_rows), sizeof n, hipMemcpyDeviceToHost,
                           (hipStream_t)stream);
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    info->status = st;
    info->n_rank_rows = st == MOE_SHUFFLE_OK ? n : 0;
    info->n_expert_rows = plan->L.T * plan->L.k;
    info->max_rank_rows = plan->L.T * plan->L.KR;
    if (st == MOE_SHUFFLE_OK) plan->n_known = n;
    return st;
}

int moe_shuffle_plan_arrays_get(moe_shuffle_plan_t plan, moe_shuffle_plan_arrays* a)
{
    int rc = check_plan(plan);
    if (rc) return rc;
    if (!a) return MOE_SHUFFLE_E_INVALID_ARG;
    const ms::Layout& L = plan->L;
    a->expert_count = at<int32_t>(plan, L.expert_count);
    a->expert_offset = at<int32_t>(plan, L.expert_offset);
    a->rank_count = at<int32_t>(plan, L.rank_count);
    a->rank_offset = at<int32_t>(plan, L.rank_offset);
    a->send_token = at<int32_t>(plan, L.send_token);
    a->tok_rank_row = at<int32_t>(plan, L.tok_rank_row);
    a->fan_src = at<int32_t>(plan, L.fan_src);
    a->fan_dst = at<int32_t>(plan, L.fan_dst);
    a->comb_row = at<int32_t>(plan, L.comb_row);
    a->rank_segs = at<moe_segment>(plan, L.rank_segs);
    a->expert_segs = at<moe_segment>(plan, L.expert_segs);
    a->status = at<int32_t>(plan, L.status);
    a->n_rank_rows = at<int32_t>(plan, L.n_rank_rows);
    a->tok_rank_width = L.KR;
    a->fan_dst_width = L.D;
    return MOE_SHUFFLE_OK;
}

int moe_shuffle_copy_reference(const void* src, void* dst, size_t bytes, void* stream)
{
    if (bytes == 0) return MOE_SHUFFLE_OK;
    if (!src || !dst) return MOE_SHUFFLE_E_INVALID_ARG;
    if (bytes % 16 || misaligned(src, 16) || misaligned(dst, 16)) return MOE_SHUFFLE_E_ALIGN;
    if (overlap(src, bytes, dst, bytes)) return MOE_SHUFFLE_E_INVALID_ARG;
    if (bytes / 16 > (size_t)0x7fffffff * ms::kBlock) return MOE_SHUFFLE_E_OVERFLOW;
    const hipError_t e = ms::launch_copy_reference(src, dst, (int64_t)(bytes / 16), (hipStream_t)stream);
    return e == hipSuccess ? MOE_SHUFFLE_OK : hip_fail(e);
}

void moe_shuffle_plan_destroy(moe_shuffle_plan_t plan)
{
    if (plan && plan->owned) free(plan);
}

const char* moe_shuffle_strerror(int code)
{
    switch (code) {
        case MOE_SHUFFLE_OK: return "ok";
        case MOE_SHUFFLE_E_INVALID_ARG: return "invalid argument";
        case MOE_SHUFFLE_E_ALIGN: return "misaligned size or pointer";
        case MOE_SHUFFLE_E_WORKSPACE: return "workspace too small";
        case MOE_SHUFFLE_E_BAD_INDEX: return "top-k id out of range or repeated within a token";
        case MOE_SHUFFLE_E_HIP: return "HIP runtime error";
        case MOE_SHUFFLE_E_OVERFLOW: return "size beyond implementation limits";
        default: return "unknown status";
    }
}

int moe_shuffle_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
