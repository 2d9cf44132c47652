// combine_bwd.hip -- backward of the combine: grad_ye rows and the gate
// gradient, in two passes.
#include "device_common.h"

namespace ms {

// Sum of p[s] over the 64 lanes for the 8 slots s, scattered: lane l ends
// with the total of slot s(l) = 4*bit5(l) + 2*bit4(l) + bit3(l).  Each step
// halves the values a lane carries (10 shuffles in all instead of 48); every
// slot's total is the same fixed 6-level pairwise tree in every lane.
__device__ __forceinline__ float reduce_scatter8(const float p[8], int lane)
{
    const bool h5 = (lane & 32) != 0, h4 = (lane & 16) != 0, h3 = (lane & 8) != 0;
    float a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float keep = h5 ? p[i + 4] : p[i];
        const float send = h5 ? p[i] : p[i + 4];
        a[i] = keep + __shfl_xor(send, 32, kWave);
    }
    float b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float keep = h4 ? a[i + 2] : a[i];
        const float send = h4 ? a[i] : a[i + 2];
        b[i] = keep + __shfl_xor(send, 16, kWave);
    }
    float c = (h3 ? b[1] : b[0]) + __shfl_xor(h3 ? b[0] : b[1], 8, kWave);
    c += __shfl_xor(c, 4, kWave);
    c += __shfl_xor(c, 2, kWave);
    c += __shfl_xor(c, 1, kWave);
    return c;
}

// ---------------------------------------------------------------- combine backward
//
// For out[t] = sum_j w[t][j] * ye[q(t,j)]:
//   grad_ye[q(t,j)] = bf16( w[t][j] * grad_out[t] )        (one fp32 product)
//   grad_w[t][j]    = sum_h grad_out[t][h] * ye[q(t,j)][h]
// One wave per 64*U-vector chunk of a token's row: the chunk of grad_out is
// loaded once and reused for all k slots.  The gate gradient is summed in a
// fixed order: each lane over its 8U elements (ascending h), a 6-level tree
// over the 64 lanes, then (gate_grad_kernel) the chunks of a row in
// ascending order.  Each bf16 x bf16 product is exact in fp32.

// PART selects the work: 1 = the grad_ye rows, 2 = the gate-gradient
// partials.  Two passes, a write-heavy one (read grad_out, write k rows)
// and a read-only one (read grad_out and k rows), against one pass doing
// both, whose mix of k row reads and k row writes per token keeps HBM from
// streaming: backward step 3.655 ms against 3.815 ms (one pass, U = 2; long
// prefill) and 0.831 against 0.841 ms (DeepSeek-V3-like) on the MI355X.
template <int U, bool FULL, int PART>
__device__ __forceinline__ void combine_bwd_rows(int* s_tile, const u32x4* __restrict__ grad_out,
                                                 const u32x4* __restrict__ ye, const float* __restrict__ w,
                                                 const int32_t* __restrict__ comb_row, u32x4* __restrict__ grad_ye,
                                                 float* __restrict__ dots, int T, int k, RowSplit rs, GridSpan gs,
                                                 const int32_t* __restrict__ status)
{
    if (status[0] != MOE_SHUFFLE_OK) return;
    const int b = span_block(gs);
    int first, count;
    block_rows<kWavesPerBlock>(b * kWavesPerBlock, T, rs, &first, &count);
    if (count <= 0) return;
    int* s_rows = s_tile;
    int* s_w = s_tile + kWavesPerBlock * k;
    for (int i = threadIdx.x; i < count * k; i += kBlock) {
        s_rows[i] = comb_row[(int64_t)first * k + i];
        s_w[i] = __float_as_int(w[(int64_t)first * k + i]);
    }
    __syncthreads();

    const int wave = wave_id(), lane = lane_id();
    const int u = b * kWavesPerBlock + wave;
    const int t = fdiv(u, rs.div);
    if (t >= T) return;
    const int V = rs.V;
    const int chunk = u - t * rs.cpr;
    const int c0 = chunk * (kWave * U);
    const int* trow = s_rows + (t - first) * k;
    const int* tw = s_w + (t - first) * k;

    float g_[U][8];  // this chunk of grad_out
    const u32x4* gp = grad_out + (int64_t)t * V + c0;
#pragma unroll
    for (int i = 0; i < U; ++i) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (FULL || c0 + i * kWave + lane < V) v = load_row16<MS_CBWD_NT_LOAD>(gp + i * kWave + lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            g_[i][2 * e] = __uint_as_float(v[e] << 16);
            g_[i][2 * e + 1] = __uint_as_float(v[e] & 0xffff0000u);
        }
    }
    constexpr int G = 8;  // slots per group: one reduce-scatter per group
    for (int j0 = 0; j0 < k; j0 += G) {
        // the group's ye loads back to back, then products and gate-gradient partials
        int q[G];
        float wj[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            q[g] = (j0 + g < k) ? __builtin_amdgcn_readfirstlane(trow[j0 + g]) : -1;
            wj[g] = (j0 + g < k) ? __int_as_float(__builtin_amdgcn_readfirstlane(tw[j0 + g])) : 0.0f;
        }
        u32x4 v[G][U];
#pragma unroll
        for (int g = 0; g < G; ++g)
            if ((PART & 2) && q[g] >= 0) {
                const u32x4* y = ye + (int64_t)q[g] * V + c0;
#pragma unroll
                for (int i = 0; i < U; ++i)
                    if (FULL || c0 + i * kWave + lane < V) v[g][i] = load_row16<MS_CBWD_NT_LOAD>(y + i * kWave + lane);
            }
        float part[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            part[g] = 0.0f;
            if (q[g] < 0) continue;
            u32x4* gy = grad_ye + (int64_t)q[g] * V + c0;
#pragma unroll
            for (int i = 0; i < U; ++i) {
                if (FULL || c0 + i * kWave + lane < V) {
                    if constexpr ((PART & 2) != 0) {
                        const u32x4 vv = v[g][i];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            part[g] = __builtin_fmaf(g_[i][2 * e], __uint_as_float(vv[e] << 16), part[g]);
                            part[g] = __builtin_fmaf(g_[i][2 * e + 1], __uint_as_float(vv[e] & 0xffff0000u), part[g]);
                        }
                    }
                    if constexpr ((PART & 1) != 0) {
                        u32x4 pk;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            pk[e] = bf16_rne(__fmul_rn(wj[g], g_[i][2 * e])) |
                                    (bf16_rne(__fmul_rn(wj[g], g_[i][2 * e + 1])) << 16);
                        store_row16<MS_CBWD_NT_STORE>(pk, gy + i * kWave + lane);
                    }
                }
            }
        }
        if constexpr ((PART & 2) != 0) {
            const float total = reduce_scatter8(part, lane);
            const int slot = j0 + 4 * ((lane >> 5) & 1) + 2 * ((lane >> 4) & 1) + ((lane >> 3) & 1);
            if ((lane & 7) == 0 && slot < k) dots[((int64_t)t * rs.cpr + chunk) * k + slot] = total;
        }
    }
}

#define MS_CBWD_KERNEL(NAME, PART)                                                                               \
    template <int U, bool FULL>                                                                                   \
    __global__ __launch_bounds__(kBlock) void NAME(const u32x4* __restrict__ grad_out,                            \
                                                   const u32x4* __restrict__ ye, const float* __restrict__ w,     \
                                                   const int32_t* __restrict__ comb_row,                          \
                                                   u32x4* __restrict__ grad_ye, float* __restrict__ dots, int T,  \
                                                   int k, RowSplit rs, GridSpan gs,                               \
                                                   const int32_t* __restrict__ status)                            \
    {                                                                                                             \
        extern __shared__ int s_tile[];                                                                           \
        combine_bwd_rows<U, FULL, PART>(s_tile, grad_out, ye, w, comb_row, grad_ye, dots, T, k, rs, gs, status);  \
    }
// grad_ye[comb_row[t][j]] = bf16(w[t][j] * grad_out[t]).
MS_CBWD_KERNEL(combine_bwd_grad_kernel, 1)
// dots[t][chunk][j] = the chunk's share of <grad_out[t], ye[comb_row[t][j]]>.
MS_CBWD_KERNEL(combine_bwd_dot_kernel, 2)
#undef MS_CBWD_KERNEL

// grad_w[t][j] = sum over chunks c (ascending) of dots[t][c][j].
__global__ __launch_bounds__(kBlock) void gate_grad_kernel(const float* __restrict__ dots, int T, int k, int cpr,
                                                           float* __restrict__ grad_w,
                                                           const int32_t* __restrict__ status)
{
    if (status[0] != MOE_SHUFFLE_OK) return;
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= (int64_t)T * k) return;
    const int64_t t = i / k, j = i - t * k;
    const float* d = dots + t * cpr * k + j;
    float acc = 0.0f;
    for (int c = 0; c < cpr; ++c) acc += d[(int64_t)c * k];
    grad_w[i] = acc;
}

// Vectors per lane of a unit in the two passes, chosen on whole backward
// steps on the MI355X: grad_ye at U = 1 with the partials at U = 2 ran
// 3.633 ms (long prefill) against 3.690 ms with the partials at U = 1 and
// 3.723 ms with grad_ye at U = 2.
#ifndef MS_CBWD_GRAD_UNIT
#define MS_CBWD_GRAD_UNIT 1
#endif
#ifndef MS_CBWD_DOT_UNIT
#define MS_CBWD_DOT_UNIT 2
#endif
// The gate gradient's summation order (8U products per lane, the lane tree,
// then the 512U-element chunks) is part of the stated arithmetic, and the
// tolerance it is tested against assumes U = 1 or 2.
static_assert(MS_CBWD_DOT_UNIT == 1 || MS_CBWD_DOT_UNIT == 2, "the gate-gradient pass sums at U = 1 or 2");
// Pass order: grad_ye first.  With plain loads the partials first measured
// 0.900 against 0.878 ms per backward step (DeepSeek-V3-like); with
// non-temporal loads the order makes no difference (0.833 against 0.831).
#ifndef MS_CBWD_DOT_FIRST
#define MS_CBWD_DOT_FIRST 0
#endif

template <int U>
static hipError_t launch_cbwd_pass(bool grad, const void* grad_out, const void* ye, const float* w,
                                   const int32_t* comb_row, void* grad_ye, float* dots, int T, int k, int V,
                                   const int32_t* status, hipStream_t s, int* cpr)
{
    RowSplit rs;
    if (!make_split(V, U, T, &rs)) return hipErrorInvalidValue;
    *cpr = rs.cpr;
    const int64_t blocks = ((int64_t)T * rs.cpr + kWavesPerBlock - 1) / kWavesPerBlock;
    const size_t lds = tile_lds_bytes(k, 2, kWavesPerBlock);
    const u32x4* gp = (const u32x4*)grad_out;
    const u32x4* yp = (const u32x4*)ye;
    u32x4* gyp = (u32x4*)grad_ye;
    const bool full = V % (kWave * U) == 0;
    return launch_spans(blocks, kBlock, [&](dim3 grid, GridSpan gs) {
        if (grad && full)
            hipLaunchKernelGGL((combine_bwd_grad_kernel<U, true>), grid, dim3(kBlock), lds, s, gp, yp, w, comb_row,
                               gyp, dots, T, k, rs, gs, status);
        else if (grad)
            hipLaunchKernelGGL((combine_bwd_grad_kernel<U, false>), grid, dim3(kBlock), lds, s, gp, yp, w, comb_row,
                               gyp, dots, T, k, rs, gs, status);
        else if (full)
            hipLaunchKernelGGL((combine_bwd_dot_kernel<U, true>), grid, dim3(kBlock), lds, s, gp, yp, w, comb_row,
                               gyp, dots, T, k, rs, gs, status);
        else
            hipLaunchKernelGGL((combine_bwd_dot_kernel<U, false>), grid, dim3(kBlock), lds, s, gp, yp, w, comb_row,
                               gyp, dots, T, k, rs, gs, status);
    });
}

static hipError_t launch_cbwd(bool grad, int U, const void* grad_out, const void* ye, const float* w,
                              const int32_t* comb_row, void* grad_ye, float* dots, int T, int k, int V,
                              const int32_t* status, hipStream_t s, int* cpr)
{
    switch (U) {
        case 1: return launch_cbwd_pass<1>(grad, grad_out, ye, w, comb_row, grad_ye, dots, T, k, V, status, s, cpr);
        case 2: return launch_cbwd_pass<2>(grad, grad_out, ye, w, comb_row, grad_ye, dots, T, k, V, status, s, cpr);
        case 4: return launch_cbwd_pass<4>(grad, grad_out, ye, w, comb_row, grad_ye, dots, T, k, V, status, s, cpr);
        default: return launch_cbwd_pass<8>(grad, grad_out, ye, w, comb_row, grad_ye, dots, T, k, V, status, s, cpr);
    }
}

hipError_t launch_combine_backward(const void* grad_out, const void* ye, const float* w, const int32_t* comb_row,
                                   void* grad_ye, float* grad_w, float* dots, int T, int k, int H,
                                   const int32_t* status, hipStream_t s)
{
    if (T <= 0) return hipSuccess;
    const int V = H / 8;
    int cpr = 0, unused = 0;
    for (int pass = 0; pass < 2; ++pass) {
        const bool grad = (pass == 0) != (MS_CBWD_DOT_FIRST != 0);
        const hipError_t e = launch_cbwd(grad, fit_unit(V, grad ? MS_CBWD_GRAD_UNIT : MS_CBWD_DOT_UNIT), grad_out, ye,
                                         w, comb_row, grad_ye, dots, T, k, V, status, s, grad ? &unused : &cpr);
        if (e != hipSuccess) return e;
    }
    const int64_t n = (int64_t)T * k;
    hipLaunchKernelGGL(gate_grad_kernel, dim3((unsigned)((n + kBlock - 1) / kBlock)), dim3(kBlock), 0, s, dots, T, k,
                       cpr, grad_w, status);
    return hipGetLastError();
}

}  // namespace ms
