// shuffle_kernels.hip -- gfx950 kernels of the MoE token shuffle.
//
// Plan (FUSCO abstract: the light-weight planner that drops redundant
// sends; press summary, Group 3: logical segments):
//   plan_count  one block per 256-token tile; every wave ORs its lanes'
//               bits into one 64-bit LDS mask per expert and per rank, so a
//               token with several experts on one rank sets that rank's bit
//               once (the send-once rule) and no result depends on the
//               order of the atomics.  Counts are popcounts of the masks.
//   plan_scan   one block per histogram column: wavefront-level exclusive
//               scan over the tiles.
//   plan_place  recomputes the masks, scans the column totals into
//               offsets, and gives every (token, rank) and (token, expert)
//               pair its row: tile base + earlier waves + mbcnt(mask).  Rows
//               come out in ascending token order inside every segment.
// Data movement (HBM bound, no MFMA: nothing here is a contraction):
//   fanout_rows   each source row is read once, 16 bytes per lane, and
//                 written to every row its target list names.  It serves
//                 both halves of dispatch: x -> xr (targets: the token's
//                 rank rows) and xr -> xe (targets: the receiver's expert
//                 rows; DySHARP write-up, section 5: target list plus a
//                 destination-local map).
//   combine_rows  k rows in, one row out: fp32 fused multiply-add in
//                 ascending slot order, one round-to-nearest-even to bf16
//                 (DySHARP write-up, section 2 / Fig. 1: combine).
// Index tiles (target lists, combine rows and gates) are staged per wave in
// LDS with one coalesced load and broadcast from there as scalars.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace ms {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Number of set bits of `m` in lanes below this one.
__device__ __forceinline__ int mbcnt(unsigned long long m)
{
    return __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
}

// Inclusive scan over a 256-thread block; s_wsum holds 4 ints.  Returns the
// inclusive prefix of `v`; *total receives the block sum.  Contains barriers:
// call from every thread.
__device__ __forceinline__ int block_inclusive_scan(int v, int* s_wsum, int* total)
{
    const int lane = lane_id(), wave = threadIdx.x >> 6;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        int n = __shfl_up(v, d, kWave);
        if (lane >= d) v += n;
    }
    if (lane == kWave - 1) s_wsum[wave] = v;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) {
        int x = s_wsum[w];
        before += (w < wave) ? x : 0;
        all += x;
    }
    __syncthreads();
    *total = all;
    return v + before;
}

// Exclusive scan of src[0..n) into dst[0..n] (dst[n] = sum), block-wide.
__device__ void block_exclusive_scan_array(const int32_t* src, int n, int* dst, int* s_wsum)
{
    int carry = 0;
    for (int base = 0; base < n; base += kBlock) {
        const int i = base + (int)threadIdx.x;
        const int v = i < n ? src[i] : 0;
        int total;
        const int incl = block_inclusive_scan(v, s_wsum, &total);
        if (i < n) dst[i] = carry + incl - v;
        carry += total;
    }
    if (threadIdx.x == 0) dst[n] = carry;
    __syncthreads();
}

// ---------------------------------------------------------------- plan_count

// hist is column-major [(C+1)][ntiles]; column C holds the tile's error flag.
__global__ __launch_bounds__(kBlock) void plan_count_kernel(const int32_t* __restrict__ idx, int T, int k,
                                                            int E, int Epr, int C, int ntiles,
                                                            int32_t* __restrict__ hist)
{
    extern __shared__ unsigned long long s_mask[];  // [4][C]
    __shared__ int s_slots, s_ecount;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int tile = blockIdx.x;
    if (tid == 0) { s_slots = 0; s_ecount = 0; }
    for (int i = tid; i < kWavesPerBlock * C; i += kBlock) s_mask[i] = 0ull;
    __syncthreads();

    const int t = tile * kPlanTile + tid;
    int bad = 0, nslots = 0;
    if (t < T) {
        const int32_t* row = idx + (int64_t)t * k;
        const unsigned long long bit = 1ull << lane;
        unsigned long long* m = s_mask + wave * C;
        for (int j = 0; j < k; ++j) {
            const int e = row[j];
            if ((unsigned)e >= (unsigned)E) { bad = 1; continue; }
            ++nslots;
            atomicOr(&m[e], bit);
            atomicOr(&m[E + e / Epr], bit);
        }
    }
    if (nslots) atomicAdd(&s_slots, nslots);
    bad = __syncthreads_or(bad);

    int ecount = 0;
    for (int c = tid; c < C; c += kBlock) {
        int cnt = 0;
#pragma unroll
        for (int w = 0; w < kWavesPerBlock; ++w) cnt += __popcll(s_mask[w * C + c]);
        hist[(int64_t)c * ntiles + tile] = cnt;
        if (c < E) ecount += cnt;
    }
    if (ecount) atomicAdd(&s_ecount, ecount);
    __syncthreads();
    // A token that names one expert twice sets that expert's bit once, so
    // the expert popcounts fall short of the in-range slots.
    if (tid == 0) hist[(int64_t)C * ntiles + tile] = (bad || s_ecount != s_slots) ? 1 : 0;
}

// ---------------------------------------------------------------- plan_scan

// Block c < C: exclusive scan of column c over the tiles.  Block C: status.
__global__ __launch_bounds__(kBlock) void plan_scan_kernel(const int32_t* __restrict__ hist, int ntiles, int C,
                                                           int32_t* __restrict__ tile_base,
                                                           int32_t* __restrict__ col_total,
                                                           int32_t* __restrict__ status)
{
    __shared__ int s_wsum[kWavesPerBlock];
    const int c = blockIdx.x;
    const int tid = threadIdx.x;
    if (c == C) {
        int bad = 0;
        for (int i = tid; i < ntiles; i += kBlock) bad |= hist[(int64_t)C * ntiles + i];
        bad = __syncthreads_or(bad);
        if (tid == 0) status[0] = bad ? MOE_SHUFFLE_E_BAD_INDEX : MOE_SHUFFLE_OK;
        return;
    }
    const int32_t* col = hist + (int64_t)c * ntiles;
    int32_t* out = tile_base + (int64_t)c * ntiles;
    int carry = 0;
    for (int base = 0; base < ntiles; base += kBlock) {
        const int i = base + tid;
        const int v = i < ntiles ? col[i] : 0;
        int total;
        const int incl = block_inclusive_scan(v, s_wsum, &total);
        if (i < ntiles) out[i] = carry + incl - v;
        carry += total;
    }
    if (tid == 0) col_total[c] = carry;
}

// ---------------------------------------------------------------- plan_place

struct PlaceArgs {
    const int32_t* idx;
    int T, k, E, R, Epr, KR, D, C, ntiles;
    const int32_t* tile_base;
    const int32_t* col_total;
    const int32_t* status;
    int32_t *expert_count, *expert_offset, *rank_count, *rank_offset;
    int32_t *send_token, *tok_rank_row, *fan_src, *fan_dst, *comb_row;
    int32_t *rank_segs, *expert_segs, *n_rank_rows;
};

__global__ __launch_bounds__(kBlock) void plan_place_kernel(PlaceArgs a)
{
    if (a.status[0] != MOE_SHUFFLE_OK) return;
    extern __shared__ unsigned long long s_dyn[];
    const int C = a.C, E = a.E, R = a.R;
    unsigned long long* s_mask = s_dyn;                        // [4][C]
    int* s_wbase = (int*)(s_mask + kWavesPerBlock * C);        // [4][C]
    int* s_off = s_wbase + kWavesPerBlock * C;                 // [E+1] then [R+1]
    __shared__ int s_wsum[kWavesPerBlock];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int tile = blockIdx.x;

    // Segment offsets from the column totals (every block, redundantly).
    block_exclusive_scan_array(a.col_total, E, s_off, s_wsum);
    block_exclusive_scan_array(a.col_total + E, R, s_off + E + 1, s_wsum);

    if (tile == 0) {
        for (int e = tid; e < E; e += kBlock) {
            const int cnt = a.col_total[e];
            a.expert_count[e] = cnt;
            a.expert_offset[e] = s_off[e];
            int32_t* seg = a.expert_segs + 4 * e;
            seg[0] = e / a.Epr; seg[1] = e; seg[2] = s_off[e]; seg[3] = cnt;
        }
        for (int r = tid; r < R; r += kBlock) {
            const int cnt = a.col_total[E + r];
            a.rank_count[r] = cnt;
            a.rank_offset[r] = s_off[E + 1 + r];
            int32_t* seg = a.rank_segs + 4 * r;
            seg[0] = r; seg[1] = -1; seg[2] = s_off[E + 1 + r]; seg[3] = cnt;
        }
        if (tid == 0) {
            a.expert_offset[E] = s_off[E];
            a.rank_offset[R] = s_off[E + 1 + R];
            a.n_rank_rows[0] = s_off[E + 1 + R];
        }
    }

    // Rebuild this tile's masks.
    for (int i = tid; i < kWavesPerBlock * C; i += kBlock) s_mask[i] = 0ull;
    __syncthreads();
    const int t = tile * kPlanTile + tid;
    const int k = a.k;
    const int32_t* row = a.idx + (int64_t)t * k;
    if (t < a.T) {
        const unsigned long long bit = 1ull << lane;
        unsigned long long* m = s_mask + wave * C;
        for (int j = 0; j < k; ++j) {
            const int e = row[j];
            atomicOr(&m[e], bit);
            atomicOr(&m[E + e / a.Epr], bit);
        }
    }
    __syncthreads();

    // First row of every column for each wave of this tile.
    for (int c = tid; c < C; c += kBlock) {
        int run = (c < E ? s_off[c] : s_off[E + 1 + (c - E)]) + a.tile_base[(int64_t)c * a.ntiles + tile];
#pragma unroll
        for (int w = 0; w < kWavesPerBlock; ++w) {
            s_wbase[w * C + c] = run;
            run += __popcll(s_mask[w * C + c]);
        }
    }
    __syncthreads();
    if (t >= a.T) return;

    const unsigned long long* m = s_mask + wave * C;
    const int* wb = s_wbase + wave * C;
    const int Epr = a.Epr, KR = a.KR, D = a.D;

    for (int j = 0; j < k; ++j) {
        const int e = row[j];
        a.comb_row[(int64_t)t * k + j] = wb[e] + mbcnt(m[e]);
    }
    // Distinct ranks of the token in ascending order; for each, its experts
    // on that rank in ascending order.
    int slot = 0, prev_r = -1;
    for (;;) {
        int r = 0x7fffffff;
        for (int j = 0; j < k; ++j) {
            const int rr = row[j] / Epr;
            if (rr > prev_r && rr < r) r = rr;
        }
        if (r == 0x7fffffff) break;
        const int p = wb[E + r] + mbcnt(m[E + r]);
        a.tok_rank_row[(int64_t)t * KR + slot] = p;
        a.send_token[p] = t;
        ++slot;
        int nd = 0, prev_e = -1;
        for (;;) {
            int e = 0x7fffffff;
            for (int j = 0; j < k; ++j) {
                const int ee = row[j];
                if (ee / Epr == r && ee > prev_e && ee < e) e = ee;
            }
            if (e == 0x7fffffff) break;
            const int q = wb[e] + mbcnt(m[e]);
            a.fan_src[q] = p;
            a.fan_dst[(int64_t)p * D + nd] = q;
            ++nd;
            prev_e = e;
        }
        for (; nd < D; ++nd) a.fan_dst[(int64_t)p * D + nd] = -1;
        prev_r = r;
    }
    for (; slot < KR; ++slot) a.tok_rank_row[(int64_t)t * KR + slot] = -1;
}

hipError_t launch_plan(const Layout& L, const PlanPtrs& P, hipStream_t s)
{
    const int ntiles = L.ntiles;
    const size_t lds_count = sizeof(unsigned long long) * kWavesPerBlock * L.C;
    hipLaunchKernelGGL(plan_count_kernel, dim3(ntiles), dim3(kBlock), lds_count, s, P.idx, L.T, L.k, L.E,
                       L.Epr, L.C, ntiles, P.tile_hist);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(plan_scan_kernel, dim3(L.C + 1), dim3(kBlock), 0, s, P.tile_hist, ntiles, L.C,
                       P.tile_base, P.col_total, P.status);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    PlaceArgs a;
    a.idx = P.idx;
    a.T = L.T; a.k = L.k; a.E = L.E; a.R = L.R; a.Epr = L.Epr; a.KR = L.KR; a.D = L.D; a.C = L.C;
    a.ntiles = ntiles;
    a.tile_base = P.tile_base; a.col_total = P.col_total; a.status = P.status;
    a.expert_count = P.expert_count; a.expert_offset = P.expert_offset;
    a.rank_count = P.rank_count; a.rank_offset = P.rank_offset;
    a.send_token = P.send_token; a.tok_rank_row = P.tok_rank_row; a.fan_src = P.fan_src;
    a.fan_dst = P.fan_dst; a.comb_row = P.comb_row;
    a.rank_segs = P.rank_segs; a.expert_segs = P.expert_segs; a.n_rank_rows = P.n_rank_rows;
    const size_t lds_place = lds_count + sizeof(int) * (kWavesPerBlock * L.C + L.E + L.R + 2);
    hipLaunchKernelGGL(plan_place_kernel, dim3(ntiles), dim3(kBlock), lds_place, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------- row movement

// Rows handled by one wave per index tile.
constexpr int kRowsPerWave = 4;

// How a row of V 16-byte vectors is cut: chunks of 64*U vectors, U <= umax.
static inline void pick_unroll(int V, int umax, int* U, int* nchunks)
{
    const int v64 = (V + kWave - 1) / kWave;
    const int nch = (v64 + umax - 1) / umax;
    *nchunks = nch;
    *U = (v64 + nch - 1) / nch;
}

template <int U, bool FULL>
__global__ __launch_bounds__(kBlock) void fanout_rows_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                             const int32_t* __restrict__ map, int width,
                                                             int64_t n_bound, const int32_t* __restrict__ n_dev,
                                                             int V, const int32_t* __restrict__ status)
{
    extern __shared__ int s_tile[];  // [4][kRowsPerWave * width]
    if (status[0] != MOE_SHUFFLE_OK) return;
    const int wave = wave_id(), lane = lane_id();
    const int64_t n = n_dev ? (int64_t)n_dev[0] : n_bound;
    const int64_t row0 = ((int64_t)blockIdx.x * kWavesPerBlock + wave) * kRowsPerWave;
    if (row0 >= n) return;
    const int rows = (int)((n - row0) < kRowsPerWave ? (n - row0) : kRowsPerWave);

    // Stage this wave's target lists (one coalesced load) in its LDS slot.
    int* tile = s_tile + wave * kRowsPerWave * width;
    const int32_t* msrc = map + row0 * width;
    for (int i = lane; i < rows * width; i += kWave) tile[i] = msrc[i];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    for (int r = 0; r < rows; ++r) {
        const u32x4* s = src + (row0 + r) * (int64_t)V;
        for (int c0 = 0; c0 < V; c0 += kWave * U) {
            u32x4 v[U];
#pragma unroll
            for (int i = 0; i < U; ++i) {
                const int x = c0 + i * kWave + lane;
                if (FULL || x < V) v[i] = __builtin_nontemporal_load(s + x);
            }
            for (int d = 0; d < width; ++d) {
                const int p = __builtin_amdgcn_readfirstlane(tile[r * width + d]);
                if (p < 0) break;
                u32x4* o = dst + (int64_t)p * V;
#pragma unroll
                for (int i = 0; i < U; ++i) {
                    const int x = c0 + i * kWave + lane;
                    if (FULL || x < V) __builtin_nontemporal_store(v[i], o + x);
                }
            }
        }
    }
}

template <int U>
static void launch_fanout_u(dim3 grid, size_t lds, hipStream_t s, const u32x4* src, u32x4* dst,
                            const int32_t* map, int width, int64_t n_bound, const int32_t* n_dev, int V,
                            const int32_t* status)
{
    if (V % (kWave * U) == 0)
        hipLaunchKernelGGL((fanout_rows_kernel<U, true>), grid, dim3(kBlock), lds, s, src, dst, map, width, n_bound,
                           n_dev, V, status);
    else
        hipLaunchKernelGGL((fanout_rows_kernel<U, false>), grid, dim3(kBlock), lds, s, src, dst, map, width, n_bound,
                           n_dev, V, status);
}

hipError_t launch_fanout_rows(const void* src, void* dst, const int32_t* map, int width, int64_t n_bound,
                              const int32_t* n_dev, int H, const int32_t* status, hipStream_t s)
{
    if (n_bound <= 0) return hipSuccess;
    const int V = H / 8;
    int U, nch;
    pick_unroll(V, 16, &U, &nch);
    const int64_t rows_per_block = (int64_t)kWavesPerBlock * kRowsPerWave;
    const dim3 grid((unsigned)((n_bound + rows_per_block - 1) / rows_per_block));
    const size_t lds = sizeof(int) * kWavesPerBlock * kRowsPerWave * width;
    const u32x4* sp = (const u32x4*)src;
    u32x4* dp = (u32x4*)dst;
    switch (U) {
#define MS_CASE(u) case u: launch_fanout_u<u>(grid, lds, s, sp, dp, map, width, n_bound, n_dev, V, status); break;
        MS_CASE(1) MS_CASE(2) MS_CASE(3) MS_CASE(4) MS_CASE(5) MS_CASE(6) MS_CASE(7) MS_CASE(8)
        MS_CASE(9) MS_CASE(10) MS_CASE(11) MS_CASE(12) MS_CASE(13) MS_CASE(14) MS_CASE(15) MS_CASE(16)
#undef MS_CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------- combine

// fp32 -> bf16 bits, round to nearest even; NaN -> quiet NaN of the same sign.
__device__ __forceinline__ unsigned bf16_rne(float f)
{
    const unsigned u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <int U, bool FULL>
__global__ __launch_bounds__(kBlock) void combine_rows_kernel(const u32x4* __restrict__ ye, const float* __restrict__ w,
                                                              const int32_t* __restrict__ rows_map,
                                                              u32x4* __restrict__ out, int T, int k, int V,
                                                              const int32_t* __restrict__ status)
{
    extern __shared__ int s_tile[];  // [4][kRowsPerWave * k] rows, then [4][kRowsPerWave * k] gates
    if (status[0] != MOE_SHUFFLE_OK) return;
    const int wave = wave_id(), lane = lane_id();
    const int64_t t0 = ((int64_t)blockIdx.x * kWavesPerBlock + wave) * kRowsPerWave;
    if (t0 >= T) return;
    const int nt = (int)((T - t0) < kRowsPerWave ? (T - t0) : kRowsPerWave);

    int* trow = s_tile + wave * kRowsPerWave * k;
    int* tw = s_tile + kWavesPerBlock * kRowsPerWave * k + wave * kRowsPerWave * k;
    for (int i = lane; i < nt * k; i += kWave) {
        trow[i] = rows_map[t0 * k + i];
        tw[i] = __float_as_int(w[t0 * k + i]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    for (int r = 0; r < nt; ++r) {
        u32x4* o = out + (t0 + r) * (int64_t)V;
        for (int c0 = 0; c0 < V; c0 += kWave * U) {
            float acc[U][8];
#pragma unroll
            for (int i = 0; i < U; ++i)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[i][e] = 0.0f;
            for (int j = 0; j < k; ++j) {
                const int q = __builtin_amdgcn_readfirstlane(trow[r * k + j]);
                const float wj = __int_as_float(__builtin_amdgcn_readfirstlane(tw[r * k + j]));
                const u32x4* y = ye + (int64_t)q * V;
#pragma unroll
                for (int i = 0; i < U; ++i) {
                    const int x = c0 + i * kWave + lane;
                    if (FULL || x < V) {
                        const u32x4 v = __builtin_nontemporal_load(y + x);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            acc[i][2 * e] = __builtin_fmaf(wj, __uint_as_float(v[e] << 16), acc[i][2 * e]);
                            acc[i][2 * e + 1] = __builtin_fmaf(wj, __uint_as_float(v[e] & 0xffff0000u), acc[i][2 * e + 1]);
                        }
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < U; ++i) {
                const int x = c0 + i * kWave + lane;
                if (FULL || x < V) {
                    u32x4 pk;
#pragma unroll
                    for (int e = 0; e < 4; ++e) pk[e] = bf16_rne(acc[i][2 * e]) | (bf16_rne(acc[i][2 * e + 1]) << 16);
                    __builtin_nontemporal_store(pk, o + x);
                }
            }
        }
    }
}

template <int U>
static void launch_combine_u(dim3 grid, size_t lds, hipStream_t s, const u32x4* ye, const float* w,
                             const int32_t* rows, u32x4* out, int T, int k, int V, const int32_t* status)
{
    if (V % (kWave * U) == 0)
        hipLaunchKernelGGL((combine_rows_kernel<U, true>), grid, dim3(kBlock), lds, s, ye, w, rows, out, T, k, V,
                           status);
    else
        hipLaunchKernelGGL((combine_rows_kernel<U, false>), grid, dim3(kBlock), lds, s, ye, w, rows, out, T, k, V,
                           status);
}

hipError_t launch_combine_rows(const void* ye, const float* w, const int32_t* rows, void* out, int T, int k, int H,
                               const int32_t* status, hipStream_t s)
{
    if (T <= 0) return hipSuccess;
    const int V = H / 8;
    int U, nch;
    pick_unroll(V, 8, &U, &nch);
    const int64_t rows_per_block = (int64_t)kWavesPerBlock * kRowsPerWave;
    const dim3 grid((unsigned)((T + rows_per_block - 1) / rows_per_block));
    const size_t lds = sizeof(int) * 2 * kWavesPerBlock * kRowsPerWave * k;
    const u32x4* yp = (const u32x4*)ye;
    u32x4* op = (u32x4*)out;
    switch (U) {
#define MS_CASE(u) case u: launch_combine_u<u>(grid, lds, s, yp, w, rows, op, T, k, V, status); break;
        MS_CASE(1) MS_CASE(2) MS_CASE(3) MS_CASE(4) MS_CASE(5) MS_CASE(6) MS_CASE(7) MS_CASE(8)
#undef MS_CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ms
