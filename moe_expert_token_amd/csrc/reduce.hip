// reduce.hip -- "k rows in, one row out": the combine (DySHARP write-up,
// section 2 / Fig. 1) and, with the same body, the receiver's and the
// sender's sums of the training direction and the rank-partial combine.
#include "device_common.h"

namespace ms {

// ---------------------------------------------------------------- reductions
//
// One gather-reduce body serves every "k rows in, one row out" step:
//   combine                 out[t]  = sum_j  w[t][j] * ye[comb_row[t][j]]
//   sum of expert rows      rr[p]   = sum_q  (gate(q) *) src[q], q in fan_dst[p]
//                           (receiver side: dispatch backward, rank-partial combine)
//   sum of rank rows        out[t]  = sum_p  src[p], p in tok_rank_row[t]
//                           (sender side of the same two)
// fp32 accumulator from +0, one fused multiply-add per term in map order
// (weight 1 for an unweighted sum, where fma(1, x, acc) is exactly x + acc),
// one round-to-nearest-even to bf16.  A -1 entry ends a map row.

#ifndef MS_COMBINE_UNIT
#define MS_COMBINE_UNIT 1
#endif

enum WeightMode { kUnweighted = 0, kPerSlot = 1, kPerSourceRow = 2 };

// One wave's unit: chunk c0 of output row `row`, its map row and gates in LDS.
// Row formats of a reduction: IO_BF16 bf16 rows in and out; IO_F32_OUT bf16
// rows in, fp32 rows out (not rounded); IO_F32_IN fp32 rows in, bf16 out.
// A wave's piece of a row is 64 element groups of 8 (one per lane): 1 KiB
// of bf16, 2 KiB of fp32.  fp32 pieces move as two 1 KiB instructions, each
// contiguous across the wave (lane l holds floats 4l .. 4l+3 of its half),
// and are regrouped between lanes with shuffles, so that every memory
// instruction covers whole cache lines.
enum RowIO { IO_BF16 = 0, IO_F32_OUT = 1, IO_F32_IN = 2 };

template <int IO>
struct Term {
    u32x4 a, b;  // fp32 pieces: the two contiguous 1 KiB halves as loaded
};

// The piece of a source row starting at element group cb; lanes past the
// row's V groups load zeros.
template <int IO, bool FULL, bool NTL>
__device__ __forceinline__ Term<IO> load_term(const u32x4* row, int cb, int V, int lane)
{
    Term<IO> t;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    if constexpr (IO == IO_F32_IN) {
        const int va = 2 * cb + lane, vb = 2 * cb + kWave + lane;  // 16-byte vectors of the fp32 row
        t.a = (FULL || va < 2 * V) ? load_row16<NTL>(row + va) : zero;
        t.b = (FULL || vb < 2 * V) ? load_row16<NTL>(row + vb) : zero;
    } else {
        t.a = (FULL || cb + lane < V) ? load_row16<NTL>(row + cb + lane) : zero;
    }
    return t;
}

// acc (this lane's 8 elements, group cb + lane) += wj * the term.  Called by
// every lane of the wave (the fp32 form shuffles).
template <int IO>
__device__ __forceinline__ void fma_term(float acc[8], float wj, const Term<IO>& t, int lane)
{
    if constexpr (IO == IO_F32_IN) {
        // group l sits in half A (l < 32) or B (l >= 32), lanes 2(l & 31) and 2(l & 31) + 1
        const int src = 2 * (lane & (kWave / 2 - 1));
        const bool in_b = lane >= kWave / 2;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float lo_a = __shfl(__uint_as_float(t.a[e]), src, kWave);
            const float lo_b = __shfl(__uint_as_float(t.b[e]), src, kWave);
            const float hi_a = __shfl(__uint_as_float(t.a[e]), src + 1, kWave);
            const float hi_b = __shfl(__uint_as_float(t.b[e]), src + 1, kWave);
            acc[e] = __builtin_fmaf(wj, in_b ? lo_b : lo_a, acc[e]);
            acc[4 + e] = __builtin_fmaf(wj, in_b ? hi_b : hi_a, acc[4 + e]);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] = __builtin_fmaf(wj, __uint_as_float(t.a[e] << 16), acc[2 * e]);
            acc[2 * e + 1] = __builtin_fmaf(wj, __uint_as_float(t.a[e] & 0xffff0000u), acc[2 * e + 1]);
        }
    }
}

// One wave's unit: element groups c0 .. c0 + 64U - 1 of output row `row`
// (lane l of piece i holds group c0 + 64i + l), its map row and gates in LDS.
template <int U, bool FULL, int WMODE, bool NTL, bool NTS, int MAXW, int IO>
__device__ __forceinline__ void reduce_unit_row(const u32x4* __restrict__ src, const int* trow, const int* tw,
                                                int width, const float* __restrict__ w, u32x4* __restrict__ out,
                                                int row, int c0, int V, int lane)
{
    const int src_stride = IO == IO_F32_IN ? 2 * V : V;  // 16-byte vectors per source row
    float acc[U][8];
#pragma unroll
    for (int i = 0; i < U; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i][e] = 0.0f;
    // Terms in groups of G: the group's row indices first, then all its
    // loads back to back (G KiB in flight per wave instead of one), then the
    // fused multiply-adds in ascending term order.  A -1 ends the map row.
    // With MAXW <= G the term loop is one straight-line group (no back edge),
    // which lets every load of the group be in flight at once.  Whole-row
    // units (U = 8) already carry 8 KiB per term and keep a plain loop: an
    // unrolled one hoists the next term's loads and the extra registers cost
    // more occupancy than they buy.  Lanes past the row's end accumulate
    // zeros and store nothing.
    constexpr int G = U >= 8 ? 1 : 8 / U;
    if constexpr (G == 1) {
#pragma unroll 1
        for (int j = 0; j < width; ++j) {
            const int q = __builtin_amdgcn_readfirstlane(trow[j]);
            if (q < 0) break;
            float wj = 1.0f;
            if (WMODE == kPerSlot) wj = __int_as_float(__builtin_amdgcn_readfirstlane(tw[j]));
            if (WMODE == kPerSourceRow) wj = w[q];
            const u32x4* y = src + (int64_t)q * src_stride;
#pragma unroll
            for (int i = 0; i < U; ++i) {
                fma_term<IO>(acc[i], wj, load_term<IO, FULL, NTL>(y, c0 + i * kWave, V, lane), lane);
                // one 1 KiB piece at a time keeps registers (and occupancy) at
                // their best for whole-row units
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    bool ended = G == 1;
#pragma unroll
    for (int j0 = 0; j0 < (MAXW <= G ? G : MAXW); j0 += G) {
        if (!ended && j0 < width) {
            int q[G];
#pragma unroll
            for (int g = 0; g < G; ++g)
                q[g] = (j0 + g < width) ? __builtin_amdgcn_readfirstlane(trow[j0 + g]) : -1;
            Term<IO> v[G][U];
#pragma unroll
            for (int g = 0; g < G; ++g)
                if (q[g] >= 0) {
                    const u32x4* y = src + (int64_t)q[g] * src_stride;
#pragma unroll
                    for (int i = 0; i < U; ++i) v[g][i] = load_term<IO, FULL, NTL>(y, c0 + i * kWave, V, lane);
                }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                if (q[g] >= 0) {
                    float wj = 1.0f;
                    if (WMODE == kPerSlot) wj = __int_as_float(__builtin_amdgcn_readfirstlane(tw[j0 + g]));
                    if (WMODE == kPerSourceRow) wj = w[q[g]];
#pragma unroll
                    for (int i = 0; i < U; ++i) fma_term<IO>(acc[i], wj, v[g][i], lane);
                }
            }
            ended = q[G - 1] < 0;  // a -1 ends the map row; all later entries are -1 too
        }
    }
    if constexpr (IO == IO_F32_OUT) {
        // lane l stores floats 4l .. 4l+3 of each contiguous 1 KiB half: half A
        // holds groups c0 + 64i + (l >> 1), half B groups c0 + 64i + 32 + (l >> 1)
        u32x4* o = out + (int64_t)row * (2 * V);
        const int src_a = lane >> 1, src_b = kWave / 2 + (lane >> 1);
        const bool upper = lane & 1;
#pragma unroll
        for (int i = 0; i < U; ++i) {
            u32x4 pa, pb;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a_lo = __shfl(acc[i][e], src_a, kWave), a_hi = __shfl(acc[i][4 + e], src_a, kWave);
                const float b_lo = __shfl(acc[i][e], src_b, kWave), b_hi = __shfl(acc[i][4 + e], src_b, kWave);
                pa[e] = __float_as_uint(upper ? a_hi : a_lo);
                pb[e] = __float_as_uint(upper ? b_hi : b_lo);
            }
            const int va = 2 * (c0 + i * kWave) + lane, vb = va + kWave;
            if (FULL || va < 2 * V) store_row16<NTS>(pa, o + va);
            if (FULL || vb < 2 * V) store_row16<NTS>(pb, o + vb);
        }
    } else {
        u32x4* o = out + (int64_t)row * V + c0;
#pragma unroll
        for (int i = 0; i < U; ++i) {
            if (FULL || c0 + i * kWave + lane < V) {
                u32x4 pk;
#pragma unroll
                for (int e = 0; e < 4; ++e) pk[e] = bf16_rne(acc[i][2 * e]) | (bf16_rne(acc[i][2 * e + 1]) << 16);
                store_row16<NTS>(pk, o + i * kWave + lane);
            }
        }
    }
}

// Stages the map rows (and per-slot gates) of the block's units in LDS, then
// one unit per wave.  With the row count on the device and L > 1, each
// block takes L rounds of WPB units (as fanout_rows does).
template <int U, bool FULL, int WMODE, bool NTL, bool NTS, int WPB, int MAXW, int L, int IO>
__device__ __forceinline__ void reduce_rows(int* s_tile, const u32x4* __restrict__ src,
                                            const int32_t* __restrict__ map, int width,
                                            const float* __restrict__ w, u32x4* __restrict__ out, int64_t n_bound,
                                            const int32_t* __restrict__ n_dev, RowSplit rs, GridSpan gs,
                                            const int32_t* __restrict__ status)
{
    if (status[0] != MOE_SHUFFLE_OK) return;
    const int64_t n = n_dev ? (int64_t)n_dev[0] : n_bound;
    const int wave = wave_id(), lane = lane_id();
    int* s_rows = s_tile;             // [rows of this block][width]
    int* s_w = s_tile + WPB * width;  // per-slot gates, same shape
#pragma unroll 1
    for (int round = 0; round < L; ++round) {
        const int u0 = L == 1 ? block_first_unit<WPB>(n_dev != nullptr, gs)
                              : (round * gs.total + span_block(gs)) * WPB;
        if (L > 1 && (int64_t)u0 >= n * rs.cpr) return;  // uniform: every later round is empty too
        int first, count;
        block_rows<WPB>(u0, n, rs, &first, &count);
        if (count <= 0) return;
        if (round > 0) __syncthreads();  // the previous round's map rows are no longer read
        for (int i = threadIdx.x; i < count * width; i += WPB * kWave) {
            s_rows[i] = map[(int64_t)first * width + i];
            if (WMODE == kPerSlot) s_w[i] = __float_as_int(w[(int64_t)first * width + i]);
        }
        __syncthreads();
        const int u = u0 + wave;
        const int row = fdiv(u, rs.div);
        if (row < n)
            reduce_unit_row<U, FULL, WMODE, NTL, NTS, MAXW, IO>(src, s_rows + (row - first) * width,
                                                            s_w + (row - first) * width, width, w, out, row,
                                                            (u - row * rs.cpr) * (kWave * U), rs.V, lane);
    }
}

#define MS_REDUCE_KERNEL(NAME, NTL, NTS)                                                                         \
    template <int U, bool FULL, int WMODE, int WPB, int MAXW, int L, int IO>                                     \
    __global__ __launch_bounds__(WPB * kWave) void NAME(const u32x4* __restrict__ src,                           \
                                                        const int32_t* __restrict__ map, int width,             \
                                                        const float* __restrict__ w, u32x4* __restrict__ out,   \
                                                        int64_t n_bound, const int32_t* __restrict__ n_dev,     \
                                                        RowSplit rs, GridSpan gs,                               \
                                                        const int32_t* __restrict__ status)                     \
    {                                                                                                            \
        extern __shared__ int s_tile[];                                                                          \
        reduce_rows<U, FULL, WMODE, NTL, NTS, WPB, MAXW, L, IO>(s_tile, src, map, width, w, out, n_bound, n_dev, \
                                                                rs, gs, status);                                 \
    }
// ye (expert-major) -> out (token-major): the forward combine.
MS_REDUCE_KERNEL(combine_rows_kernel, MS_COMBINE_NT_LOAD, MS_COMBINE_NT_STORE)
// expert-major rows -> one row per (token, rank): the receiver's sum.
MS_REDUCE_KERNEL(sum_expert_rows_kernel, MS_SUMX_NT_LOAD, MS_SUMX_NT_STORE)
// rank-major rows -> one row per token: the sender's sum.
MS_REDUCE_KERNEL(sum_rank_rows_kernel, MS_SUMR_NT_LOAD, MS_SUMR_NT_STORE)
#undef MS_REDUCE_KERNEL

// Gathers from a large buffer use whole-row units: past a few GiB of
// source rows, 8 KiB units measured faster than 1 KiB units on the MI355X
// (65536 tokens x 8 x 8 KiB combine: 0.80 ms against 0.94 ms); below it 1 KiB
// units were as fast or faster.
#ifndef MS_COMBINE_UNIT_LARGE
#define MS_COMBINE_UNIT_LARGE 8
#endif
#ifndef MS_COMBINE_LARGE_BYTES
#define MS_COMBINE_LARGE_BYTES (2ll << 30)
#endif

#ifndef MS_SUMX_UNIT
#define MS_SUMX_UNIT 2  // measured: 279 us against 338 us at U = 1 (DeepSeek-V3-like)
#endif
// The sender's sum gathers a token's rank rows at 2 KiB units.  At 1 KiB it
// is faster only while the memory system still holds the state its own
// previous call left (155 against 162 us, DeepSeek-V3-like): after the
// combine backward, or a 1 GiB copy, in between, 1 KiB units take 187 and
// 168 us, while 2 KiB units take 162-164 us whatever ran before.  In the
// training direction the combine backward (and, in a model, the expert
// GEMMs) runs before it, so the 2 KiB unit is the faster one there too.
#ifndef MS_SUMR_UNIT
#define MS_SUMR_UNIT 2
#endif

// The receiver's sum keeps 2 KiB units over large sources too: 1306 us
// against 1399 us with whole rows (65536 tokens x 8 x 8 KiB); the sender's
// sum was within 3 % at every unit size and keeps whole rows.
#ifndef MS_SUMX_UNIT_LARGE
#define MS_SUMX_UNIT_LARGE 2
#endif
#ifndef MS_SUMR_UNIT_LARGE
#define MS_SUMR_UNIT_LARGE MS_COMBINE_UNIT_LARGE
#endif

// fp32 partial rows: the receiver's sum that writes them takes 1 KiB units
// and the sender's sum that reads them 2 KiB units (4 KiB of fp32 per
// term).  Where a token reaches about 4 ranks, a group of 8 slots at U = 1
// holds about 4 live terms; at U = 2 all of them go out in one group of 4
// with twice the bytes each, so a wave keeps twice the loads in flight.
// Measured per rank-partial combine with fp32 partials: skewed 1.169 ->
// 1.024 ms, long prefill 3.406 -> 3.192 ms.
#ifndef MS_SUMX_F32_UNIT
#define MS_SUMX_F32_UNIT 1
#endif
#ifndef MS_SUMR_F32_UNIT
#define MS_SUMR_F32_UNIT 2
#endif

static int reduce_unit(int kind, int io, int V, int64_t src_bytes)
{
    if (io == IO_F32_OUT) return fit_unit(V, MS_SUMX_F32_UNIT);
    if (io == IO_F32_IN) return fit_unit(V, MS_SUMR_F32_UNIT);
    const bool large = src_bytes > (int64_t)MS_COMBINE_LARGE_BYTES;
    const int small_unit = kind == 1 ? MS_SUMX_UNIT : kind == 2 ? MS_SUMR_UNIT : MS_COMBINE_UNIT;
    const int large_unit = kind == 1 ? MS_SUMX_UNIT_LARGE : kind == 2 ? MS_SUMR_UNIT_LARGE : MS_COMBINE_UNIT_LARGE;
    return fit_unit(V, large ? large_unit : small_unit);
}

enum ReduceKind { kCombine = 0, kSumExpertRows = 1, kSumRankRows = 2 };

// Rounds per block of the receiver's sum: two rounds measured slower there
// (280 -> 297 us, DeepSeek-V3-like), so one.
#ifndef MS_SUMX_ROUNDS
#define MS_SUMX_ROUNDS 1
#endif

template <int KIND, int U, bool FULL, int WMODE, int WPB, int MAXW, int L, int IO>
static hipError_t launch_reduce_kernel(int64_t blocks, size_t lds, hipStream_t s, const u32x4* src,
                                       const int32_t* map, int width, const float* w, u32x4* out, int64_t n_bound,
                                       const int32_t* n_dev, RowSplit rs, const int32_t* status)
{
    const dim3 block(WPB * kWave);
    return launch_spans(blocks, WPB * kWave, [&](dim3 grid, GridSpan gs) {
        if constexpr (KIND == kCombine)
            hipLaunchKernelGGL((combine_rows_kernel<U, FULL, WMODE, WPB, MAXW, 1, IO_BF16>), grid, block, lds, s, src,
                               map, width, w, out, n_bound, n_dev, rs, gs, status);
        else if constexpr (KIND == kSumExpertRows && L > 1) {
            if (n_dev)
                hipLaunchKernelGGL((sum_expert_rows_kernel<U, FULL, WMODE, WPB, MAXW, L, IO>), grid, block, lds, s,
                                   src, map, width, w, out, n_bound, n_dev, rs, gs, status);
            else
                hipLaunchKernelGGL((sum_expert_rows_kernel<U, FULL, WMODE, WPB, MAXW, 1, IO>), grid, block, lds, s,
                                   src, map, width, w, out, n_bound, n_dev, rs, gs, status);
        } else if constexpr (KIND == kSumExpertRows)
            hipLaunchKernelGGL((sum_expert_rows_kernel<U, FULL, WMODE, WPB, MAXW, 1, IO>), grid, block, lds, s, src,
                               map, width, w, out, n_bound, n_dev, rs, gs, status);
        else
            hipLaunchKernelGGL((sum_rank_rows_kernel<U, FULL, WMODE, WPB, MAXW, 1, IO>), grid, block, lds, s, src,
                               map, width, w, out, n_bound, n_dev, rs, gs, status);
    });
}

template <int KIND, int WMODE, int U, int WPB, int IO>
static hipError_t launch_reduce_uw(const void* src, const int32_t* map, int width, const float* w, void* out,
                                   int64_t n_bound, const int32_t* n_dev, int V, const int32_t* status, hipStream_t s)
{
    RowSplit rs;
    if (!make_split(V, U, n_bound, &rs)) return hipErrorInvalidValue;
    // rounds only where the row count is on the device (the receiver's sum)
    constexpr int L = KIND == kSumExpertRows ? MS_SUMX_ROUNDS : 1;
    const int64_t ublocks = (n_bound * rs.cpr + WPB - 1) / WPB;
    const int rounds = n_dev ? L : 1;
    const int64_t blocks = (ublocks + rounds - 1) / rounds;
    const size_t lds = tile_lds_bytes(width, 2, WPB);
    const u32x4* sp = (const u32x4*)src;
    u32x4* op = (u32x4*)out;
    const bool full = V % (kWave * U) == 0;
    if (width <= 8 && full)
        return launch_reduce_kernel<KIND, U, true, WMODE, WPB, 8, L, IO>(blocks, lds, s, sp, map, width, w, op,
                                                                         n_bound, n_dev, rs, status);
    if (width <= 8)
        return launch_reduce_kernel<KIND, U, false, WMODE, WPB, 8, L, IO>(blocks, lds, s, sp, map, width, w, op,
                                                                          n_bound, n_dev, rs, status);
    if (full)
        return launch_reduce_kernel<KIND, U, true, WMODE, WPB, kMaxTopK, L, IO>(blocks, lds, s, sp, map, width, w, op,
                                                                                n_bound, n_dev, rs, status);
    return launch_reduce_kernel<KIND, U, false, WMODE, WPB, kMaxTopK, L, IO>(blocks, lds, s, sp, map, width, w, op,
                                                                             n_bound, n_dev, rs, status);
}

// Waves per block of the receiver's sum (its row count is on the device):
// 2 against 4, measured on whole steps on the MI355X, DeepSeek-V3-like /
// skewed / long prefill: backward 0.803 / 1.364 / 3.630 against 0.808 /
// 1.367 / 3.656 ms, rank-partial 0.440 / 0.669 / 2.011 against 0.445 /
// 0.670 / 2.025 ms (fp32 partials within 0.3 % either way).
#ifndef MS_SUMX_WAVES
#define MS_SUMX_WAVES 2
#endif
// Waves per block of the sender's sum: 4.  Measured on whole steps on the
// MI355X, 2 waves were as fast or slower everywhere; 8 waves gained 0.5 %
// on the DeepSeek-V3-like and skewed workloads and lost 1-2 % on the long
// prefill.
#ifndef MS_SUMR_WAVES
#define MS_SUMR_WAVES kWavesPerBlock
#endif

template <int KIND, int WMODE, int U, int IO>
static hipError_t launch_reduce_u(const void* src, const int32_t* map, int width, const float* w, void* out,
                                  int64_t n_bound, const int32_t* n_dev, int V, const int32_t* status, hipStream_t s)
{
    if constexpr (U <= 2) {
        if (n_dev)
            return launch_reduce_uw<KIND, WMODE, U, MS_SUMX_WAVES, IO>(src, map, width, w, out, n_bound, n_dev, V,
                                                                       status, s);
    }
    if constexpr (KIND == kSumRankRows)
        return launch_reduce_uw<KIND, WMODE, U, MS_SUMR_WAVES, IO>(src, map, width, w, out, n_bound, n_dev, V, status,
                                                                   s);
    return launch_reduce_uw<KIND, WMODE, U, kWavesPerBlock, IO>(src, map, width, w, out, n_bound, n_dev, V, status, s);
}

template <int KIND, int WMODE, int IO = IO_BF16>
static hipError_t launch_reduce(const void* src, int64_t src_rows, const int32_t* map, int width, const float* w,
                                void* out, int64_t n_bound, const int32_t* n_dev, int H, const int32_t* status,
                                hipStream_t s)
{
    if (n_bound <= 0) return hipSuccess;
    const int V = H / 8;
    const int64_t src_bytes = src_rows * (int64_t)H * (IO == IO_F32_IN ? 4 : 2);
    switch (reduce_unit(KIND, IO, V, src_bytes)) {
        case 1: return launch_reduce_u<KIND, WMODE, 1, IO>(src, map, width, w, out, n_bound, n_dev, V, status, s);
        case 2: return launch_reduce_u<KIND, WMODE, 2, IO>(src, map, width, w, out, n_bound, n_dev, V, status, s);
        case 4: return launch_reduce_u<KIND, WMODE, 4, IO>(src, map, width, w, out, n_bound, n_dev, V, status, s);
        default: return launch_reduce_u<KIND, WMODE, 8, IO>(src, map, width, w, out, n_bound, n_dev, V, status, s);
    }
}

hipError_t launch_combine_rows(const void* ye, const float* w, const int32_t* rows, void* out, int T, int k, int H,
                               const int32_t* status, hipStream_t s)
{
    return launch_reduce<kCombine, kPerSlot>(ye, (int64_t)T * k, rows, k, w, out, T, nullptr, H, status, s);
}

// gate_of_row[comb_row[t][j]] = w[t][j]: the gate each expert row carries.
__global__ __launch_bounds__(kBlock) void gate_of_row_kernel(const float* __restrict__ w,
                                                             const int32_t* __restrict__ comb_row, int64_t n,
                                                             float* __restrict__ gate_of_row,
                                                             const int32_t* __restrict__ status)
{
    if (status[0] != MOE_SHUFFLE_OK) return;
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i < n) gate_of_row[comb_row[i]] = w[i];
}

hipError_t launch_sum_expert_rows(const void* src, int64_t src_rows, const float* w, const int32_t* comb_row,
                                  float* gate_of_row, const int32_t* fan_dst, int D, void* out, int64_t n_bound,
                                  const int32_t* n_dev, int H, const int32_t* status, hipStream_t s, bool f32_out)
{
    if (n_bound <= 0) return hipSuccess;
    if (!w && !f32_out)
        return launch_reduce<kSumExpertRows, kUnweighted>(src, src_rows, fan_dst, D, nullptr, out, n_bound, n_dev, H,
                                                          status, s);
    if (!w) return hipErrorInvalidValue;  // fp32 partials are only made for the weighted return path
    hipLaunchKernelGGL(gate_of_row_kernel, dim3((unsigned)((src_rows + kBlock - 1) / kBlock)), dim3(kBlock), 0, s, w,
                       comb_row, src_rows, gate_of_row, status);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (f32_out)
        return launch_reduce<kSumExpertRows, kPerSourceRow, IO_F32_OUT>(src, src_rows, fan_dst, D, gate_of_row, out,
                                                                        n_bound, n_dev, H, status, s);
    return launch_reduce<kSumExpertRows, kPerSourceRow>(src, src_rows, fan_dst, D, gate_of_row, out, n_bound, n_dev,
                                                        H, status, s);
}

hipError_t launch_sum_rank_rows(const void* src, int64_t src_rows, const int32_t* tok_rank_row, int KR, void* out,
                                int T, int H, const int32_t* status, hipStream_t s, bool f32_in)
{
    if (f32_in)
        return launch_reduce<kSumRankRows, kUnweighted, IO_F32_IN>(src, src_rows, tok_rank_row, KR, nullptr, out, T,
                                                                   nullptr, H, status, s);
    return launch_reduce<kSumRankRows, kUnweighted>(src, src_rows, tok_rank_row, KR, nullptr, out, T, nullptr, H,
                                                    status, s);
}

}  // namespace ms
