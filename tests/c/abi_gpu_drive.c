/* Drives the library from C on the GPU, with plain HIP allocations and the
 * default stream (no Python, no PyTorch): plan, query, dispatch and combine
 * of one small batch read from stdin, then every plan array and row buffer
 * printed to stdout for the caller to compare.
 *
 * stdin:  T H E k R, then T*k expert ids, T*H values of x, T*k gates, and a
 *         flag: 0 = the identity expert (ye = xe), 1 = T*k*H values of ye.
 *         Every value must be exact in bf16 (it is stored by truncation).
 * stdout: one line per array, "name v0 v1 ...", rows as float values.
 * Exit status 0 on success; 2 for bad input; 3 for a library or HIP error,
 * printed with its code. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "moe_shuffle.h"

static int die(const char* what, int code)
{
    printf("ERROR %s %d\n", what, code);
    return 3;
}

#define HIP_OK(call)                                        \
    do {                                                    \
        hipError_t e_ = (call);                             \
        if (e_ != hipSuccess) return die(#call, (int)e_);   \
    } while (0)
#define MS_OK(call)                                         \
    do {                                                    \
        int rc_ = (call);                                   \
        if (rc_ != MOE_SHUFFLE_OK) return die(#call, rc_);  \
    } while (0)

static uint16_t to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

static float from_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static int read_floats(float* v, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        if (scanf("%f", &v[i]) != 1) return 0;
    return 1;
}

static void print_ints(const char* name, const int32_t* v, size_t n)
{
    printf("%s", name);
    for (size_t i = 0; i < n; ++i) printf(" %d", v[i]);
    printf("\n");
}

static void print_rows(const char* name, const uint16_t* v, size_t n)
{
    printf("%s", name);
    for (size_t i = 0; i < n; ++i) printf(" %.9g", (double)from_bf16(v[i]));
    printf("\n");
}

/* Copies n int32 of device array `src` to the host and prints them. */
static int dump(const char* name, const int32_t* src, size_t n)
{
    int32_t* h = (int32_t*)malloc(n * sizeof(int32_t) + 1);
    if (!h) return 0;
    if (n && hipMemcpy(h, src, n * sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess) {
        free(h);
        return 0;
    }
    print_ints(name, h, n);
    free(h);
    return 1;
}

int main(void)
{
    moe_shuffle_dims d;
    if (scanf("%d %d %d %d %d", &d.num_tokens, &d.hidden, &d.num_experts, &d.top_k, &d.num_ranks) != 5) return 2;
    const size_t T = (size_t)d.num_tokens, H = (size_t)d.hidden, k = (size_t)d.top_k;
    const size_t R = (size_t)d.num_ranks, E = (size_t)d.num_experts;
    const size_t KR = k < R ? k : R;
    int32_t* idx = (int32_t*)malloc(T * k * sizeof(int32_t) + 1);
    float* xf = (float*)malloc(T * H * sizeof(float) + 1);
    float* w = (float*)malloc(T * k * sizeof(float) + 1);
    float* yef = (float*)malloc(T * k * H * sizeof(float) + 1);
    uint16_t* x16 = (uint16_t*)malloc(T * H * 2 + 1);
    uint16_t* rows16 = (uint16_t*)malloc(T * k * H * 2 + 1);
    if (!idx || !xf || !w || !yef || !x16 || !rows16) return 2;
    for (size_t i = 0; i < T * k; ++i)
        if (scanf("%d", &idx[i]) != 1) return 2;
    if (!read_floats(xf, T * H) || !read_floats(w, T * k)) return 2;
    int own_ye = 0;
    if (scanf("%d", &own_ye) != 1) return 2;
    if (own_ye && !read_floats(yef, T * k * H)) return 2;
    for (size_t i = 0; i < T * H; ++i) x16[i] = to_bf16(xf[i]);

    size_t ws_bytes = 0;
    MS_OK(moe_shuffle_workspace_size(&d, &ws_bytes));
    void *ws, *d_idx, *d_x, *d_w, *d_xr, *d_xe, *d_ye, *d_out;
    HIP_OK(hipMalloc(&ws, ws_bytes));
    HIP_OK(hipMalloc(&d_idx, T * k * sizeof(int32_t) + 4));
    HIP_OK(hipMalloc(&d_x, T * H * 2 + 16));
    HIP_OK(hipMalloc(&d_w, T * k * sizeof(float) + 4));
    HIP_OK(hipMalloc(&d_xr, T * KR * H * 2 + 16));
    HIP_OK(hipMalloc(&d_xe, T * k * H * 2 + 16));
    HIP_OK(hipMalloc(&d_ye, T * k * H * 2 + 16));
    HIP_OK(hipMalloc(&d_out, T * H * 2 + 16));
    HIP_OK(hipMemcpy(d_idx, idx, T * k * sizeof(int32_t), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_x, x16, T * H * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_w, w, T * k * sizeof(float), hipMemcpyHostToDevice));

    moe_shuffle_plan_t plan = NULL;
    MS_OK(moe_shuffle_plan(&d, (const int32_t*)d_idx, ws, ws_bytes, NULL, &plan));
    moe_shuffle_plan_info info;
    MS_OK(moe_shuffle_plan_query(plan, NULL, &info));
    printf("status %d\nN %d\n", info.status, info.n_rank_rows);
    moe_shuffle_plan_arrays a;
    MS_OK(moe_shuffle_plan_arrays_get(plan, &a));
    const size_t N = (size_t)info.n_rank_rows, D = (size_t)a.fan_dst_width;
    if (!dump("expert_count", a.expert_count, E) || !dump("expert_offset", a.expert_offset, E + 1) ||
        !dump("rank_count", a.rank_count, R) || !dump("rank_offset", a.rank_offset, R + 1) ||
        !dump("send_token", a.send_token, N) || !dump("tok_rank_row", a.tok_rank_row, T * (size_t)a.tok_rank_width) ||
        !dump("fan_src", a.fan_src, T * k) || !dump("fan_dst", a.fan_dst, N * D) ||
        !dump("comb_row", a.comb_row, T * k) || !dump("rank_segs", (const int32_t*)a.rank_segs, 4 * R) ||
        !dump("expert_segs", (const int32_t*)a.expert_segs, 4 * E))
        return die("copy of a plan array", 0);

    MS_OK(moe_shuffle_dispatch(plan, d_x, d_xr, (int64_t)(T * KR), d_xe, NULL));
    if (own_ye) {
        for (size_t i = 0; i < T * k * H; ++i) rows16[i] = to_bf16(yef[i]);
        HIP_OK(hipMemcpy(d_ye, rows16, T * k * H * 2, hipMemcpyHostToDevice));
    } else {
        HIP_OK(hipMemcpy(d_ye, d_xe, T * k * H * 2, hipMemcpyDeviceToDevice));
    }
    MS_OK(moe_shuffle_combine(plan, d_ye, (const float*)d_w, d_out, NULL));
    HIP_OK(hipDeviceSynchronize());

    HIP_OK(hipMemcpy(rows16, d_xr, N * H * 2, hipMemcpyDeviceToHost));
    print_rows("xr", rows16, N * H);
    HIP_OK(hipMemcpy(rows16, d_xe, T * k * H * 2, hipMemcpyDeviceToHost));
    print_rows("xe", rows16, T * k * H);
    HIP_OK(hipMemcpy(rows16, d_out, T * H * 2, hipMemcpyDeviceToHost));
    print_rows("out", rows16, T * H);

    moe_shuffle_plan_destroy(plan);
    hipFree(ws); hipFree(d_idx); hipFree(d_x); hipFree(d_w);
    hipFree(d_xr); hipFree(d_xe); hipFree(d_ye); hipFree(d_out);
    free(idx); free(xf); free(w); free(yef); free(x16); free(rows16);
    return 0;
}
