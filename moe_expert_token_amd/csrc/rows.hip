// rows.hip -- the two halves of dispatch and their token-range forms (HBM
// bound, no MFMA: nothing here is a contraction).
//   fanout_rows  each source row is read once, 16 bytes per lane, and
//                written to every row its target list names.  It serves
//                both halves of dispatch: x -> xr (targets: the token's rank
//                rows) and xr -> xe (targets: the receiver's expert rows;
//                DySHARP write-up, section 5: target list plus a
//                destination-local map).
//   token ranges the same for the tokens [t0, t1) alone, for pipelining.
#include "device_common.h"

namespace ms {

// ---------------------------------------------------------------- send and fan-out

// Body shared by the send and fan-out kernels (two names, so that traces and
// counters tell the two halves of dispatch apart).  WPB waves per block.
// With the row count on the device and L > 1, each block takes L rounds of
// WPB units, round i at unit block i * (blocks of the grid) + this block,
// so the grid sized by the bound has L times fewer blocks and the rounds
// past the true count end the block at once.
template <int U, bool FULL, bool NTL, bool NTS, int WPB, int L>
__device__ __forceinline__ void fanout_rows(int* s_tile, const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                            const int32_t* __restrict__ map, int width, int64_t n_bound,
                                            const int32_t* __restrict__ n_dev, RowSplit rs, GridSpan gs,
                                            const int32_t* __restrict__ status)
{
    if (status[0] != MOE_SHUFFLE_OK) return;
    const int64_t n = n_dev ? (int64_t)n_dev[0] : n_bound;
    const int wave = wave_id(), lane = lane_id();
    const int V = rs.V;
#pragma unroll 1
    for (int round = 0; round < L; ++round) {
        const int u0 = L == 1 ? block_first_unit<WPB>(n_dev != nullptr, gs)
                              : (round * gs.total + span_block(gs)) * WPB;
        if (L > 1 && (int64_t)u0 >= n * rs.cpr) return;  // uniform: every later round is empty too
        int first, count;
        block_rows<WPB>(u0, n, rs, &first, &count);
        if (count <= 0) return;  // the whole block is past the last row
        if (round > 0) __syncthreads();  // the previous round's targets are no longer read
        for (int i = threadIdx.x; i < count * width; i += WPB * kWave) s_tile[i] = map[(int64_t)first * width + i];
        __syncthreads();

        const int u = u0 + wave;
        const int row = fdiv(u, rs.div);
        if (row < n) {
            const int c0 = (u - row * rs.cpr) * (kWave * U);
            const u32x4* s = src + (int64_t)row * V + c0;
            u32x4 v[U];
#pragma unroll
            for (int i = 0; i < U; ++i)
                if (FULL || c0 + i * kWave + lane < V) v[i] = load_row16<NTL>(s + i * kWave + lane);
            const int* targets = s_tile + (row - first) * width;
            for (int d = 0; d < width; ++d) {
                const int p = __builtin_amdgcn_readfirstlane(targets[d]);
                if (p < 0) break;
                u32x4* o = dst + (int64_t)p * V + c0;
#pragma unroll
                for (int i = 0; i < U; ++i)
                    if (FULL || c0 + i * kWave + lane < V) store_row16<NTS>(v[i], o + i * kWave + lane);
            }
        }
    }
}

#define MS_FANOUT_KERNEL(NAME, NTL, NTS)                                                                        \
    template <int U, bool FULL, int WPB, int L>                                                                  \
    __global__ __launch_bounds__(WPB * kWave) void NAME(const u32x4* __restrict__ src, u32x4* __restrict__ dst,  \
                                                        const int32_t* __restrict__ map, int width,             \
                                                        int64_t n_bound, const int32_t* __restrict__ n_dev,     \
                                                        RowSplit rs, GridSpan gs,                               \
                                                        const int32_t* __restrict__ status)                     \
    {                                                                                                            \
        extern __shared__ int s_tile[]; /* [rows of this block][width] */                                        \
        fanout_rows<U, FULL, NTL, NTS, WPB, L>(s_tile, src, dst, map, width, n_bound, n_dev, rs, gs, status);    \
    }
// x -> xr: source rows are tokens, targets their rank rows.
MS_FANOUT_KERNEL(dispatch_send_kernel, MS_SEND_NT_LOAD, MS_SEND_NT_STORE)
// xr -> xe: source rows are rank rows, targets the receiver's expert rows.
MS_FANOUT_KERNEL(dispatch_fanout_kernel, MS_FANOUT_NT_LOAD, MS_FANOUT_NT_STORE)
#undef MS_FANOUT_KERNEL

// Vectors per lane of a unit (a unit is 64*U vectors of one row).
#ifndef MS_SEND_UNIT
#define MS_SEND_UNIT 1
#endif
#ifndef MS_FANOUT_UNIT
#define MS_FANOUT_UNIT 1
#endif

// Rounds per block of the fan-out when the row count is on the device.
// Measured on the MI355X (fan-out, grid sized by T*min(k,R)): two rounds
// 302 -> 294 us (DeepSeek-V3-like) and 515 -> 470 us (skewed, where the
// bound is twice the true count); four and eight rounds were slower.
#ifndef MS_FANOUT_ROUNDS
#define MS_FANOUT_ROUNDS 2
#endif

template <int U, int WPB, int L>
static hipError_t launch_fanout_uwl(bool send, const void* src, void* dst, const int32_t* map, int width,
                                    int64_t n_bound, const int32_t* n_dev, int V, const int32_t* status,
                                    hipStream_t s)
{
    RowSplit rs;
    if (!make_split(V, U, n_bound, &rs)) return hipErrorInvalidValue;
    const int64_t ublocks = (n_bound * rs.cpr + WPB - 1) / WPB;
    const dim3 block(WPB * kWave);
    const size_t lds = tile_lds_bytes(width, 1, WPB);
    const u32x4* sp = (const u32x4*)src;
    u32x4* dp = (u32x4*)dst;
    const bool full = V % (kWave * U) == 0;
    return launch_spans((ublocks + L - 1) / L, WPB * kWave, [&](dim3 grid, GridSpan gs) {
        if (send && full)
            hipLaunchKernelGGL((dispatch_send_kernel<U, true, WPB, L>), grid, block, lds, s, sp, dp, map, width,
                               n_bound, n_dev, rs, gs, status);
        else if (send)
            hipLaunchKernelGGL((dispatch_send_kernel<U, false, WPB, L>), grid, block, lds, s, sp, dp, map, width,
                               n_bound, n_dev, rs, gs, status);
        else if (full)
            hipLaunchKernelGGL((dispatch_fanout_kernel<U, true, WPB, L>), grid, block, lds, s, sp, dp, map, width,
                               n_bound, n_dev, rs, gs, status);
        else
            hipLaunchKernelGGL((dispatch_fanout_kernel<U, false, WPB, L>), grid, block, lds, s, sp, dp, map, width,
                               n_bound, n_dev, rs, gs, status);
    });
}

template <int U, int WPB>
static hipError_t launch_fanout_uw(bool send, const void* src, void* dst, const int32_t* map, int width,
                                   int64_t n_bound, const int32_t* n_dev, int V, const int32_t* status, hipStream_t s)
{
    if (n_dev && MS_FANOUT_ROUNDS > 1)
        return launch_fanout_uwl<U, WPB, MS_FANOUT_ROUNDS>(send, src, dst, map, width, n_bound, n_dev, V, status, s);
    return launch_fanout_uwl<U, WPB, 1>(send, src, dst, map, width, n_bound, n_dev, V, status, s);
}

// Waves per block of the send (its row count is known on the host): 2
// against 4, measured on the MI355X (DeepSeek-V3-like / skewed / long
// prefill): 146 / 200 / 669 us against 153 / 206 / 715 us; 1, 8 and 16
// waves were slower.
#ifndef MS_SEND_WAVES
#define MS_SEND_WAVES 2
#endif

template <int U>
static hipError_t launch_fanout_u(bool send, const void* src, void* dst, const int32_t* map, int width,
                                  int64_t n_bound, const int32_t* n_dev, int V, const int32_t* status, hipStream_t s)
{
    if constexpr (U <= 2) {  // big blocks only with small units (no register pressure)
        if (n_dev) return launch_fanout_uw<U, kWavesBig>(send, src, dst, map, width, n_bound, n_dev, V, status, s);
    }
    if (send) return launch_fanout_uw<U, MS_SEND_WAVES>(send, src, dst, map, width, n_bound, n_dev, V, status, s);
    return launch_fanout_uw<U, kWavesPerBlock>(send, src, dst, map, width, n_bound, n_dev, V, status, s);
}

hipError_t launch_fanout_rows(bool send, const void* src, void* dst, const int32_t* map, int width, int64_t n_bound,
                              const int32_t* n_dev, int H, const int32_t* status, hipStream_t s)
{
    if (n_bound <= 0) return hipSuccess;
    const int V = H / 8;
    switch (fit_unit(V, send ? MS_SEND_UNIT : MS_FANOUT_UNIT)) {
        case 1: return launch_fanout_u<1>(send, src, dst, map, width, n_bound, n_dev, V, status, s);
        case 2: return launch_fanout_u<2>(send, src, dst, map, width, n_bound, n_dev, V, status, s);
        case 4: return launch_fanout_u<4>(send, src, dst, map, width, n_bound, n_dev, V, status, s);
        default: return launch_fanout_u<8>(send, src, dst, map, width, n_bound, n_dev, V, status, s);
    }
}

// ---------------------------------------------------------------- token ranges
//
// Dispatch and combine of the tokens [t0, t1) alone, so a caller can
// pipeline token chunks (DySHARP write-up, section 6 / Fig. 12: dispatch of
// one group of tokens proceeds while later stages work on the previous one).
// Rows follow token order inside every segment, so the rank rows of the
// range are, in each rank segment r, the contiguous rows
//   [rank_offset[r] + P_r(t0), rank_offset[r] + P_r(t1)),
// P_r(t) = tokens before t that reach rank r, read from the plan's tile
// bases (t a multiple of the 64-token plan tile) or, at t = T, the rank's
// count.  Each block rebuilds that table for itself (no shared scratch, so
// ranges on different streams never race) and each wave finds its segment
// by binary search.

struct RangeArgs {
    const int32_t* rank_offset;
    const int32_t* tile_base;  // column-major [C][ntiles]
    const int32_t* col_total;  // [C]
    int E, R, ntiles;
    int tile0, tile1;          // tile index of t0; of t1, or -1 for t1 = T
};

__device__ __forceinline__ int range_prefix(const RangeArgs& g, int r, int tile)
{
    return tile < 0 ? g.col_total[g.E + r] : g.tile_base[(int64_t)(g.E + r) * g.ntiles + tile];
}

template <int U, bool FULL, int L>
__global__ __launch_bounds__(kBlock) void dispatch_fanout_range_kernel(const u32x4* __restrict__ src,
                                                                       u32x4* __restrict__ dst,
                                                                       const int32_t* __restrict__ fan_dst, int D,
                                                                       RangeArgs g, RowSplit rs, GridSpan gs,
                                                                       const int32_t* __restrict__ status)
{
    extern __shared__ int s_tab[];  // start[R] then exclusive prefix of lengths [R + 1]
    __shared__ int s_wsum[kWavesPerBlock];
    if (status[0] != MOE_SHUFFLE_OK) return;
    const int R = g.R;
    int* s_start = s_tab;
    int* s_pre = s_tab + R;
    int carry = 0;
    for (int r0 = 0; r0 < R; r0 += kBlock) {
        const int r = r0 + (int)threadIdx.x;
        int len = 0;
        if (r < R) {
            const int a = range_prefix(g, r, g.tile0);
            const int b = range_prefix(g, r, g.tile1);
            s_start[r] = g.rank_offset[r] + a;
            len = b - a;
        }
        int total;
        const int incl = block_inclusive_scan(len, s_wsum, &total);
        if (r < R) s_pre[r] = carry + incl - len;
        carry += total;
    }
    if (threadIdx.x == 0) s_pre[R] = carry;
    __syncthreads();

    // L rounds of units per block share the table; a row's target list is
    // one vector load (lane d holds target d), read back with readlane.
    const int wave = wave_id(), lane = lane_id();
    const int V = rs.V;
#pragma unroll 1
    for (int round = 0; round < L; ++round) {
        const int u = (round * gs.total + span_block(gs)) * kWavesPerBlock + wave;
        const int l = fdiv(u, rs.div);
        if (l >= carry) return;  // later rounds only go further
        int lo = 0, hi = R - 1;  // largest r with s_pre[r] <= l
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_pre[mid] <= l) lo = mid;
            else hi = mid - 1;
        }
        const int p = __builtin_amdgcn_readfirstlane(s_start[lo] + (l - s_pre[lo]));
        const int c0 = (u - l * rs.cpr) * (kWave * U);
        const u32x4* sp = src + (int64_t)p * V + c0;
        u32x4 v[U];
#pragma unroll
        for (int i = 0; i < U; ++i)
            if (FULL || c0 + i * kWave + lane < V) v[i] = load_row16<MS_FANOUT_NT_LOAD>(sp + i * kWave + lane);
        const int tv = lane < D ? fan_dst[(int64_t)p * D + lane] : -1;
        for (int d = 0; d < D; ++d) {
            const int q = __builtin_amdgcn_readlane(tv, d);
            if (q < 0) break;
            u32x4* o = dst + (int64_t)q * V + c0;
#pragma unroll
            for (int i = 0; i < U; ++i)
                if (FULL || c0 + i * kWave + lane < V) store_row16<MS_FANOUT_NT_STORE>(v[i], o + i * kWave + lane);
        }
    }
}

// Rounds per block of the range fan-out: the per-block rank table is built
// once for L rounds of units.  Measured on the MI355X (dispatch of a batch
// in 4 token chunks, DeepSeek-V3-like): 550 us at one round, 476 us at four,
// against 440 us for the whole batch in one call.
#ifndef MS_RANGE_ROUNDS
#define MS_RANGE_ROUNDS 4
#endif

hipError_t launch_fanout_range(const void* xr, void* xe, const int32_t* fan_dst, int D, const int32_t* rank_offset,
                               const int32_t* tile_base, const int32_t* col_total, int E, int R, int ntiles, int t0,
                               int t1, int T, int KR, int H, const int32_t* status, hipStream_t s)
{
    if (t1 <= t0) return hipSuccess;
    const int V = H / 8;
    RowSplit rs;
    const int64_t bound = (int64_t)(t1 - t0) * KR;  // each token reaches at most KR ranks
    if (!make_split(V, 1, bound, &rs)) return hipErrorInvalidValue;
    RangeArgs g;
    g.rank_offset = rank_offset; g.tile_base = tile_base; g.col_total = col_total;
    g.E = E; g.R = R; g.ntiles = ntiles;
    g.tile0 = t0 / kPlanTile;
    g.tile1 = t1 == T ? -1 : t1 / kPlanTile;
    constexpr int L = MS_RANGE_ROUNDS;
    const int64_t ublocks = (bound * rs.cpr + kWavesPerBlock - 1) / kWavesPerBlock;
    const size_t lds = sizeof(int) * (2 * (size_t)R + 1);
    const u32x4* sp = (const u32x4*)xr;
    u32x4* dp = (u32x4*)xe;
    return launch_spans((ublocks + L - 1) / L, kBlock, [&](dim3 grid, GridSpan gs) {
        if (V % kWave == 0)
            hipLaunchKernelGGL((dispatch_fanout_range_kernel<1, true, L>), grid, dim3(kBlock), lds, s, sp, dp,
                               fan_dst, D, g, rs, gs, status);
        else
            hipLaunchKernelGGL((dispatch_fanout_range_kernel<1, false, L>), grid, dim3(kBlock), lds, s, sp, dp,
                               fan_dst, D, g, rs, gs, status);
    });
}

}  // namespace ms
