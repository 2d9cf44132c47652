// shuffle_kernels.hip -- gfx950 kernels of the MoE token shuffle.
//
// Plan (FUSCO abstract: the light-weight planner that drops redundant
// sends; press summary, Group 3: logical segments):
//   plan_count  one wave per 64-token tile; the wave ORs its lanes' bits
//               into one 64-bit LDS mask per expert and per rank, so a token
//               with several experts on one rank sets that rank's bit once
//               (the send-once rule) and no result depends on the order of
//               the atomics.  Counts are popcounts of the masks.
//   plan_scan   one block per histogram column: wavefront-level exclusive
//               scan over the tiles.
//   plan_place  recomputes the masks, scans the column totals into
//               offsets, and gives every (token, rank) and (token, expert)
//               pair its row: tile base + mbcnt(mask).  Rows
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
//                 (DySHARP write-up, section 2 / Fig. 1: combine).  The same
//                 body sums expert rows per rank row (receiver) and rank rows
//                 per token (sender) for the training direction and the
//                 rank-partial combine.
//   token ranges  dispatch and combine of a token range, for pipelining.
//   combine backward  grad_ye rows and the gate-gradient partials, in two
//                 passes.
// Index tiles (target lists, combine rows and gates) are staged per block in
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

// n / d for 0 <= n < 2^31 with a host-computed multiplier (round-up method).
struct FastDiv {
    unsigned mul;
    int shift;
};

__device__ __forceinline__ int fdiv(int n, FastDiv f)
{
    return (int)((__umulhi((unsigned)n, f.mul) + (unsigned)n) >> f.shift);
}

static FastDiv make_fastdiv(int d)
{
    int l = 0;
    while ((1ll << l) < d) ++l;
    const unsigned long long m = ((1ull << 32) * ((1ull << l) - (unsigned long long)d)) / (unsigned long long)d + 1;
    FastDiv f;
    f.mul = (unsigned)m;
    f.shift = l;
    return f;
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

// ---------------------------------------------------------------- plan_count

// Sum over the wave (every lane gets it).
__device__ __forceinline__ int wave_sum(int v)
{
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) v += __shfl_xor(v, d, kWave);
    return v;
}

// Inclusive scan over the wave.
__device__ __forceinline__ int wave_inclusive_scan(int v)
{
    const int lane = lane_id();
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int n = __shfl_up(v, d, kWave);
        if (lane >= d) v += n;
    }
    return v;
}

// One wave per 64-token tile.  hist is column-major [(C+1)][ntiles];
// column C holds the tile's error flag.
template <int KMAX>
__global__ __launch_bounds__(kWave) void plan_count_kernel(const int32_t* __restrict__ idx, int T, int k,
                                                           int E, FastDiv epr, int C, int ntiles,
                                                           int32_t* __restrict__ hist)
{
    extern __shared__ unsigned long long s_mask[];  // [C]
    const int lane = threadIdx.x;
    const int tile = blockIdx.x;
    const int t = tile * kPlanTile + lane;

    // The ids first (their load overlaps the clearing of the masks).
    int ev[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) ev[j] = -1;
    if (t < T) {
        const int32_t* row = idx + (int64_t)t * k;
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if (j < k) ev[j] = row[j];
    }
    for (int i = lane; i < C; i += kWave) s_mask[i] = 0ull;
    __syncthreads();

    int bad = 0, nslots = 0;
    if (t < T) {
        const unsigned long long bit = 1ull << lane;
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            if (j < k) {
                const int e = ev[j];
                if ((unsigned)e >= (unsigned)E) {
                    bad = 1;
                } else {
                    ++nslots;
                    atomicOr(&s_mask[e], bit);
                    atomicOr(&s_mask[E + fdiv(e, epr)], bit);
                }
            }
        }
    }
    __syncthreads();

    int ecount = 0;
    for (int c = lane; c < C; c += kWave) {
        const int cnt = __popcll(s_mask[c]);
        hist[(int64_t)c * ntiles + tile] = cnt;
        if (c < E) ecount += cnt;
    }
    // A token that names one expert twice sets that expert's bit once, so
    // the expert popcounts fall short of the in-range slots.
    const bool any_bad = __ballot(bad) != 0ull;
    const int slots = wave_sum(nslots), placed = wave_sum(ecount);
    if (lane == 0) hist[(int64_t)C * ntiles + tile] = (any_bad || placed != slots) ? 1 : 0;
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
    FastDiv epr;
    const int32_t* tile_base;
    const int32_t* col_total;
    const int32_t* status;
    int32_t *expert_count, *expert_offset, *rank_count, *rank_offset;
    int32_t *send_token, *tok_rank_row, *fan_src, *fan_dst, *comb_row;
    int32_t *rank_segs, *expert_segs, *n_rank_rows;
};

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Writes one lane's index row of `width` entries, -1 padded: with width a
// multiple of 4, in 16-byte groups (the row start is 16-byte aligned);
// otherwise one entry at a time.
struct RowWriter {
    int32_t* row;
    int width, n;
    bool vec;
    i32x4 pend;

    __device__ RowWriter(int32_t* r, int w) : row(r), width(w), n(0), vec((w & 3) == 0), pend{-1, -1, -1, -1} {}
    __device__ void start(int32_t* r)
    {
        row = r;
        n = 0;
        pend = i32x4{-1, -1, -1, -1};
    }
    __device__ void put(int v)
    {
        if (vec) {
            const int i = n & 3;
            pend.x = i == 0 ? v : pend.x;
            pend.y = i == 1 ? v : pend.y;
            pend.z = i == 2 ? v : pend.z;
            pend.w = i == 3 ? v : pend.w;
            if (i == 3) {
                *(i32x4*)(row + (n & ~3)) = pend;
                pend = i32x4{-1, -1, -1, -1};
            }
        } else {
            row[n] = v;
        }
        ++n;
    }
    __device__ void finish()
    {
        if (vec) {
            int g = n & ~3;
            if (n & 3) {
                *(i32x4*)(row + g) = pend;
                g += 4;
            }
            for (; g < width; g += 4) *(i32x4*)(row + g) = i32x4{-1, -1, -1, -1};
        } else {
            for (int i = n; i < width; ++i) row[i] = -1;
        }
    }
};

template <int KMAX>
__global__ __launch_bounds__(kWave) void plan_place_kernel(PlaceArgs a)
{
    extern __shared__ unsigned long long s_dyn[];
    const int C = a.C, E = a.E, R = a.R;
    unsigned long long* s_mask = s_dyn;     // [C]
    int* s_wbase = (int*)(s_mask + C);      // [C]

    const int lane = threadIdx.x;
    const int tile = blockIdx.x;
    const int t = tile * kPlanTile + lane;
    const int k = a.k;
    constexpr int kCols = kMaxCols / kWave;  // histogram columns per lane

    // Every global load first, so their latencies overlap: the status word,
    // this lane's top-k ids, and for each column it owns the column total
    // and this tile's base within the column.
    const int status = a.status[0];
    int ev[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) ev[j] = 0x7fffffff;
    if (t < a.T) {
        const int32_t* row = a.idx + (int64_t)t * k;
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if (j < k) ev[j] = row[j];
    }
    int ct[kCols], tb[kCols];
#pragma unroll
    for (int i = 0; i < kCols; ++i) {
        const int c = lane + i * kWave;
        ct[i] = c < C ? a.col_total[c] : 0;
        tb[i] = c < C ? a.tile_base[(int64_t)c * a.ntiles + tile] : 0;
    }

    for (int i = lane; i < C; i += kWave) s_mask[i] = 0ull;
    __syncthreads();
    if (status != MOE_SHUFFLE_OK) return;

    // This tile's masks.
    if (t < a.T) {
        const unsigned long long bit = 1ull << lane;
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if (j < k) {
                atomicOr(&s_mask[ev[j]], bit);
                atomicOr(&s_mask[E + fdiv(ev[j], a.epr)], bit);
            }
    }

    // One exclusive scan over all columns, experts first then ranks; a rank
    // column's segment offset is its prefix minus the expert total.
    int excl[kCols];
    int carry = 0, etot = 0;
#pragma unroll
    for (int i = 0; i < kCols; ++i) {
        excl[i] = 0;
        if (i * kWave < C) {  // uniform
            const int incl = wave_inclusive_scan(ct[i]);
            excl[i] = carry + incl - ct[i];
            carry += __shfl(incl, kWave - 1, kWave);
            if (i == (E >> 6)) etot = __shfl(excl[i], E & (kWave - 1), kWave);  // uniform
        }
    }
    __syncthreads();  // the masks are complete

    // Segment offsets (tile 0 publishes them) and the first row of every
    // column for this tile.
#pragma unroll
    for (int i = 0; i < kCols; ++i) {
        const int c = lane + i * kWave;
        if (i * kWave < C && c < C) {
            const int off = c < E ? excl[i] : excl[i] - etot;
            if (tile == 0) {
                if (c < E) {
                    a.expert_count[c] = ct[i];
                    a.expert_offset[c] = off;
                    int32_t* seg = a.expert_segs + 4 * c;
                    seg[0] = fdiv(c, a.epr); seg[1] = c; seg[2] = off; seg[3] = ct[i];
                } else {
                    const int r = c - E;
                    a.rank_count[r] = ct[i];
                    a.rank_offset[r] = off;
                    int32_t* seg = a.rank_segs + 4 * r;
                    seg[0] = r; seg[1] = -1; seg[2] = off; seg[3] = ct[i];
                }
            }
            s_wbase[c] = off + tb[i];
        }
    }
    if (tile == 0 && lane == 0) {
        a.expert_offset[E] = etot;
        a.rank_offset[R] = carry - etot;
        a.n_rank_rows[0] = carry - etot;
    }
    __syncthreads();
    if (t >= a.T) return;

    const unsigned long long* m = s_mask;
    const int* wb = s_wbase;
    const int KR = a.KR, D = a.D;

    // Expert row of every slot, in slot order.  Index rows whose width is a
    // multiple of 4 go out as 16-byte stores (a lane's row is contiguous).
    int qv[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) qv[j] = j < k ? wb[ev[j]] + mbcnt(m[ev[j]]) : 0;
    if ((k & 3) == 0) {
#pragma unroll
        for (int j = 0; j < KMAX; j += 4)
            if (j < k) {
                const i32x4 v = {qv[j], qv[j + 1], qv[j + 2], qv[j + 3]};
                *(i32x4*)(a.comb_row + (int64_t)t * k + j) = v;
            }
    } else {
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if (j < k) a.comb_row[(int64_t)t * k + j] = qv[j];
    }
    // Sort the (expert, row) pairs by expert id.  rank = expert / Epr is
    // monotone in the id, so the sorted list visits the token's ranks in
    // ascending order and, inside a rank, its experts in ascending order.
#pragma unroll
    for (int i = 1; i < KMAX; ++i)
#pragma unroll
        for (int j = i; j > 0; --j) {
            const bool sw = ev[j] < ev[j - 1];
            const int e0 = ev[j - 1], e1 = ev[j], q0 = qv[j - 1], q1 = qv[j];
            ev[j - 1] = sw ? e1 : e0;
            ev[j] = sw ? e0 : e1;
            qv[j - 1] = sw ? q1 : q0;
            qv[j] = sw ? q0 : q1;
        }
    // The rank rows of the token and each one's expert rows (-1 padded to D
    // and KR).  Rows of width 4n are written a 16-byte group at a time from
    // a pending group in registers.
    RowWriter rank_rows(a.tok_rank_row + (int64_t)t * KR, KR);
    RowWriter targets(a.fan_dst, D);
    int prev_r = -1, p = 0;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        if (j < k) {
            const int r = fdiv(ev[j], a.epr);
            if (r != prev_r) {
                if (prev_r >= 0) targets.finish();
                p = wb[E + r] + mbcnt(m[E + r]);
                rank_rows.put(p);
                a.send_token[p] = t;
                targets.start(a.fan_dst + (int64_t)p * D);
                prev_r = r;
            }
            a.fan_src[qv[j]] = p;
            targets.put(qv[j]);
        }
    }
    targets.finish();
    rank_rows.finish();
}

hipError_t launch_plan(const Layout& L, const PlanPtrs& P, hipStream_t s)
{
    const int ntiles = L.ntiles;
    const size_t lds_count = sizeof(unsigned long long) * L.C;
    const FastDiv epr = make_fastdiv(L.Epr);
    if (L.k <= 8)
        hipLaunchKernelGGL(plan_count_kernel<8>, dim3(ntiles), dim3(kWave), lds_count, s, P.idx, L.T, L.k, L.E,
                           epr, L.C, ntiles, P.tile_hist);
    else if (L.k <= 16)
        hipLaunchKernelGGL(plan_count_kernel<16>, dim3(ntiles), dim3(kWave), lds_count, s, P.idx, L.T, L.k, L.E,
                           epr, L.C, ntiles, P.tile_hist);
    else if (L.k <= 32)
        hipLaunchKernelGGL(plan_count_kernel<32>, dim3(ntiles), dim3(kWave), lds_count, s, P.idx, L.T, L.k, L.E,
                           epr, L.C, ntiles, P.tile_hist);
    else
        hipLaunchKernelGGL(plan_count_kernel<64>, dim3(ntiles), dim3(kWave), lds_count, s, P.idx, L.T, L.k, L.E,
                           epr, L.C, ntiles, P.tile_hist);
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
    a.epr = epr;
    a.tile_base = P.tile_base; a.col_total = P.col_total; a.status = P.status;
    a.expert_count = P.expert_count; a.expert_offset = P.expert_offset;
    a.rank_count = P.rank_count; a.rank_offset = P.rank_offset;
    a.send_token = P.send_token; a.tok_rank_row = P.tok_rank_row; a.fan_src = P.fan_src;
    a.fan_dst = P.fan_dst; a.comb_row = P.comb_row;
    a.rank_segs = P.rank_segs; a.expert_segs = P.expert_segs; a.n_rank_rows = P.n_rank_rows;
    const size_t lds_place = lds_count + sizeof(int) * L.C;
    if (L.k <= 8)
        hipLaunchKernelGGL(plan_place_kernel<8>, dim3(ntiles), dim3(kWave), lds_place, s, a);
    else if (L.k <= 16)
        hipLaunchKernelGGL(plan_place_kernel<16>, dim3(ntiles), dim3(kWave), lds_place, s, a);
    else if (L.k <= 32)
        hipLaunchKernelGGL(plan_place_kernel<32>, dim3(ntiles), dim3(kWave), lds_place, s, a);
    else
        hipLaunchKernelGGL(plan_place_kernel<64>, dim3(ntiles), dim3(kWave), lds_place, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------- row movement

// Work unit: one chunk of 64*U 16-byte vectors (1 KiB at U = 1) of one row,
// one wave per unit, the chunks of a row on consecutive waves.  Small units
// keep many independent 1 KiB requests in flight per CU and spread every row
// over several waves; measured on the MI355X, a random 14 KiB-row gather
// runs at ~6.0 TB/s this way against ~5.4 TB/s with one wave per row.
//
// A block (4 waves) first stages the target lists of the rows it touches in
// LDS with one coalesced load; each wave then broadcasts its targets as
// scalars.

// 16-byte row traffic, with or without the non-temporal hint.  Which side of
// which kernel carries the hint was chosen by measurement on the MI355X (the
// hint changes how lines are kept in L2 and the memory-side cache):
//   send              plain loads, plain stores (its scattered row writes go
//                     through L2)
//   fan-out           non-temporal loads and stores
//   combine           non-temporal loads and stores
//   receiver, sender  non-temporal loads and stores
//   combine backward  plain loads, non-temporal stores
// (DeepSeek-V3-like workload: send 153 us with plain stores against 178 us
// with non-temporal ones; fan-out 303 us against 324 us with plain loads.)
#ifndef MS_SEND_NT_LOAD
#define MS_SEND_NT_LOAD 0
#endif
#ifndef MS_SEND_NT_STORE
#define MS_SEND_NT_STORE 0
#endif
#ifndef MS_FANOUT_NT_LOAD
#define MS_FANOUT_NT_LOAD 1
#endif
#ifndef MS_FANOUT_NT_STORE
#define MS_FANOUT_NT_STORE 1
#endif
#ifndef MS_COMBINE_NT_LOAD
#define MS_COMBINE_NT_LOAD 1
#endif
#ifndef MS_COMBINE_NT_STORE
#define MS_COMBINE_NT_STORE 1
#endif
#ifndef MS_SUMX_NT_LOAD
#define MS_SUMX_NT_LOAD 1
#endif
#ifndef MS_SUMX_NT_STORE
#define MS_SUMX_NT_STORE 1
#endif
#ifndef MS_SUMR_NT_LOAD
#define MS_SUMR_NT_LOAD 1
#endif
#ifndef MS_SUMR_NT_STORE
#define MS_SUMR_NT_STORE 1
#endif
#ifndef MS_CBWD_NT_LOAD
#define MS_CBWD_NT_LOAD 0
#endif
#ifndef MS_CBWD_NT_STORE
#define MS_CBWD_NT_STORE 1
#endif

template <bool NT>
__device__ __forceinline__ u32x4 load_row16(const u32x4* p)
{
    if (NT) return __builtin_nontemporal_load(p);
    return *p;
}

template <bool NT>
__device__ __forceinline__ void store_row16(u32x4 v, u32x4* p)
{
    if (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

struct RowSplit {
    int V;        // 16-byte vectors per row
    int cpr;      // chunks per row
    FastDiv div;  // unit -> row
};

// First unit of this block.  When the row count is known only on the device
// the grid is sized by a bound and the blocks past the count have nothing to
// do; those kernels take the units in reverse block order, so the empty
// blocks are dispatched first and exit while the real work fills the
// machine, instead of trailing it (measured on the MI355X, fan-out: skewed
// workload 537 -> 526 us, long prefill 1383 -> 1328 us; a grid sized by the
// exact count would be 479 and 1295 us, which needs a host sync).
template <int WPB>
__device__ __forceinline__ int block_first_unit(bool reversed)
{
    const int b = reversed ? (int)(gridDim.x - 1 - blockIdx.x) : (int)blockIdx.x;
    return b * WPB;
}

// Rows touched by units [u0, u0 + WPB): [*first, *first + *count), clipped to n.
template <int WPB>
__device__ __forceinline__ void block_rows(int u0, int64_t n, const RowSplit& rs, int* first, int* count)
{
    const int r0 = fdiv(u0, rs.div);
    int r1 = fdiv(u0 + WPB - 1, rs.div);
    if ((int64_t)r1 >= n) r1 = (int)(n - 1);
    *first = r0;
    *count = r1 - r0 + 1;
}

// Body shared by the send and fan-out kernels (two names, so that traces and
// counters tell the two halves of dispatch apart).  WPB waves per block.
// With the row count on the device and L > 1, each block takes L rounds of
// WPB units, round i at unit block i * gridDim.x + blockIdx.x, so the grid
// sized by the bound has L times fewer blocks and the rounds past the true
// count end the block at once.
template <int U, bool FULL, bool NTL, bool NTS, int WPB, int L>
__device__ __forceinline__ void fanout_rows(int* s_tile, const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                            const int32_t* __restrict__ map, int width, int64_t n_bound,
                                            const int32_t* __restrict__ n_dev, RowSplit rs,
                                            const int32_t* __restrict__ status)
{
    if (status[0] != MOE_SHUFFLE_OK) return;
    const int64_t n = n_dev ? (int64_t)n_dev[0] : n_bound;
    const int wave = wave_id(), lane = lane_id();
    const int V = rs.V;
#pragma unroll 1
    for (int round = 0; round < L; ++round) {
        const int u0 = L == 1 ? block_first_unit<WPB>(n_dev != nullptr)
                              : (round * (int)gridDim.x + (int)blockIdx.x) * WPB;
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
                                                        RowSplit rs, const int32_t* __restrict__ status)        \
    {                                                                                                            \
        extern __shared__ int s_tile[]; /* [rows of this block][width] */                                        \
        fanout_rows<U, FULL, NTL, NTS, WPB, L>(s_tile, src, dst, map, width, n_bound, n_dev, rs, status);        \
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
#ifndef MS_COMBINE_UNIT
#define MS_COMBINE_UNIT 1
#endif

// Splits rows of V vectors into chunks of 64*U; false if rows * chunks overflows int.
static bool make_split(int V, int U, int64_t rows, RowSplit* rs)
{
    rs->V = V;
    rs->cpr = (V + kWave * U - 1) / (kWave * U);
    rs->div = make_fastdiv(rs->cpr);
    return rows * rs->cpr + 64 < ((int64_t)1 << 31);  // units of the last block stay below 2^31
}

// Kernels whose row count is known only on the device (fan-out, receiver
// sums) are sized by the host-side bound T*min(k,R); blocks past the true
// count exit at once (see block_first_unit).  Waves per block for them:
#ifndef MS_BIG_WAVES
#define MS_BIG_WAVES 4
#endif
constexpr int kWavesBig = MS_BIG_WAVES;

static unsigned grid_for(int64_t units, int wpb) { return (unsigned)((units + wpb - 1) / wpb); }

static size_t tile_lds_bytes(int width, int arrays, int wpb)
{
    return sizeof(int) * (size_t)arrays * wpb * width;  // at most one row per wave
}

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
    const dim3 grid((unsigned)((ublocks + L - 1) / L)), block(WPB * kWave);
    const size_t lds = tile_lds_bytes(width, 1, WPB);
    const u32x4* sp = (const u32x4*)src;
    u32x4* dp = (u32x4*)dst;
    const bool full = V % (kWave * U) == 0;
    if (send && full)
        hipLaunchKernelGGL((dispatch_send_kernel<U, true, WPB, L>), grid, block, lds, s, sp, dp, map, width, n_bound,
                           n_dev, rs, status);
    else if (send)
        hipLaunchKernelGGL((dispatch_send_kernel<U, false, WPB, L>), grid, block, lds, s, sp, dp, map, width,
                           n_bound, n_dev, rs, status);
    else if (full)
        hipLaunchKernelGGL((dispatch_fanout_kernel<U, true, WPB, L>), grid, block, lds, s, sp, dp, map, width,
                           n_bound, n_dev, rs, status);
    else
        hipLaunchKernelGGL((dispatch_fanout_kernel<U, false, WPB, L>), grid, block, lds, s, sp, dp, map, width,
                           n_bound, n_dev, rs, status);
    return hipGetLastError();
}

template <int U, int WPB>
static hipError_t launch_fanout_uw(bool send, const void* src, void* dst, const int32_t* map, int width,
                                   int64_t n_bound, const int32_t* n_dev, int V, const int32_t* status, hipStream_t s)
{
    if (n_dev && MS_FANOUT_ROUNDS > 1)
        return launch_fanout_uwl<U, WPB, MS_FANOUT_ROUNDS>(send, src, dst, map, width, n_bound, n_dev, V, status, s);
    return launch_fanout_uwl<U, WPB, 1>(send, src, dst, map, width, n_bound, n_dev, V, status, s);
}

template <int U>
static hipError_t launch_fanout_u(bool send, const void* src, void* dst, const int32_t* map, int width,
                                  int64_t n_bound, const int32_t* n_dev, int V, const int32_t* status, hipStream_t s)
{
    if constexpr (U <= 2) {  // big blocks only with small units (no register pressure)
        if (n_dev) return launch_fanout_uw<U, kWavesBig>(send, src, dst, map, width, n_bound, n_dev, V, status, s);
    }
    return launch_fanout_uw<U, kWavesPerBlock>(send, src, dst, map, width, n_bound, n_dev, V, status, s);
}

// Largest of {1, 2, 4, 8} not above `want` whose chunk does not exceed the row.
static int fit_unit(int V, int want)
{
    int u = want;
    while (u > 1 && kWave * u > V) u >>= 1;
    return u;
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
                                                                       RangeArgs g, RowSplit rs,
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
        const int u = (round * (int)gridDim.x + (int)blockIdx.x) * kWavesPerBlock + wave;
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
    const dim3 grid((unsigned)((ublocks + L - 1) / L));
    const size_t lds = sizeof(int) * (2 * (size_t)R + 1);
    const u32x4* sp = (const u32x4*)xr;
    u32x4* dp = (u32x4*)xe;
    if (V % kWave == 0)
        hipLaunchKernelGGL((dispatch_fanout_range_kernel<1, true, L>), grid, dim3(kBlock), lds, s, sp, dp, fan_dst, D,
                           g, rs, status);
    else
        hipLaunchKernelGGL((dispatch_fanout_range_kernel<1, false, L>), grid, dim3(kBlock), lds, s, sp, dp, fan_dst,
                           D, g, rs, status);
    return hipGetLastError();
}

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

// fp32 -> bf16 bits, round to nearest even; NaN -> quiet NaN of the same sign.
__device__ __forceinline__ unsigned bf16_rne(float f)
{
    const unsigned u = __float_as_uint(f);
    const unsigned rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    const unsigned quiet_nan = (u >> 16) | 0x40u;
    return (u & 0x7fffffffu) > 0x7f800000u ? quiet_nan : rounded;  // a select, not a branch
}

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

enum WeightMode { kUnweighted = 0, kPerSlot = 1, kPerSourceRow = 2 };

// One wave's unit: chunk c0 of output row `row`, its map row and gates in LDS.
template <int U, bool FULL, int WMODE, bool NTL, bool NTS, int MAXW>
__device__ __forceinline__ void reduce_unit_row(const u32x4* __restrict__ src, const int* trow, const int* tw,
                                                int width, const float* __restrict__ w, u32x4* __restrict__ out,
                                                int row, int c0, int V, int lane)
{
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
    // more occupancy than they buy.
    constexpr int G = U >= 8 ? 1 : 8 / U;
    if constexpr (G == 1) {
#pragma unroll 1
        for (int j = 0; j < width; ++j) {
            const int q = __builtin_amdgcn_readfirstlane(trow[j]);
            if (q < 0) break;
            float wj = 1.0f;
            if (WMODE == kPerSlot) wj = __int_as_float(__builtin_amdgcn_readfirstlane(tw[j]));
            if (WMODE == kPerSourceRow) wj = w[q];
            const u32x4* y = src + (int64_t)q * V + c0;
#pragma unroll
            for (int i = 0; i < U; ++i) {
                if (FULL || c0 + i * kWave + lane < V) {
                    const u32x4 vv = load_row16<NTL>(y + i * kWave + lane);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc[i][2 * e] = __builtin_fmaf(wj, __uint_as_float(vv[e] << 16), acc[i][2 * e]);
                        acc[i][2 * e + 1] =
                            __builtin_fmaf(wj, __uint_as_float(vv[e] & 0xffff0000u), acc[i][2 * e + 1]);
                    }
                }
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
            u32x4 v[G][U];
#pragma unroll
            for (int g = 0; g < G; ++g)
                if (q[g] >= 0) {
                    const u32x4* y = src + (int64_t)q[g] * V + c0;
#pragma unroll
                    for (int i = 0; i < U; ++i)
                        if (FULL || c0 + i * kWave + lane < V) v[g][i] = load_row16<NTL>(y + i * kWave + lane);
                }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                if (q[g] >= 0) {
                    float wj = 1.0f;
                    if (WMODE == kPerSlot) wj = __int_as_float(__builtin_amdgcn_readfirstlane(tw[j0 + g]));
                    if (WMODE == kPerSourceRow) wj = w[q[g]];
#pragma unroll
                    for (int i = 0; i < U; ++i) {
                        if (FULL || c0 + i * kWave + lane < V) {
                            const u32x4 vv = v[g][i];
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                acc[i][2 * e] = __builtin_fmaf(wj, __uint_as_float(vv[e] << 16), acc[i][2 * e]);
                                acc[i][2 * e + 1] =
                                    __builtin_fmaf(wj, __uint_as_float(vv[e] & 0xffff0000u), acc[i][2 * e + 1]);
                            }
                        }
                    }
                }
            }
            ended = q[G - 1] < 0;  // a -1 ends the map row; all later entries are -1 too
        }
    }
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

// Stages the map rows (and per-slot gates) of the block's units in LDS, then
// one unit per wave.  With the row count on the device and L > 1, each
// block takes L rounds of WPB units (as fanout_rows does).
template <int U, bool FULL, int WMODE, bool NTL, bool NTS, int WPB, int MAXW, int L>
__device__ __forceinline__ void reduce_rows(int* s_tile, const u32x4* __restrict__ src,
                                            const int32_t* __restrict__ map, int width,
                                            const float* __restrict__ w, u32x4* __restrict__ out, int64_t n_bound,
                                            const int32_t* __restrict__ n_dev, RowSplit rs,
                                            const int32_t* __restrict__ status)
{
    if (status[0] != MOE_SHUFFLE_OK) return;
    const int64_t n = n_dev ? (int64_t)n_dev[0] : n_bound;
    const int wave = wave_id(), lane = lane_id();
    int* s_rows = s_tile;             // [rows of this block][width]
    int* s_w = s_tile + WPB * width;  // per-slot gates, same shape
#pragma unroll 1
    for (int round = 0; round < L; ++round) {
        const int u0 = L == 1 ? block_first_unit<WPB>(n_dev != nullptr)
                              : (round * (int)gridDim.x + (int)blockIdx.x) * WPB;
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
            reduce_unit_row<U, FULL, WMODE, NTL, NTS, MAXW>(src, s_rows + (row - first) * width,
                                                            s_w + (row - first) * width, width, w, out, row,
                                                            (u - row * rs.cpr) * (kWave * U), rs.V, lane);
    }
}

#define MS_REDUCE_KERNEL(NAME, NTL, NTS)                                                                         \
    template <int U, bool FULL, int WMODE, int WPB, int MAXW, int L>                                             \
    __global__ __launch_bounds__(WPB * kWave) void NAME(const u32x4* __restrict__ src,                           \
                                                        const int32_t* __restrict__ map, int width,             \
                                                        const float* __restrict__ w, u32x4* __restrict__ out,   \
                                                        int64_t n_bound, const int32_t* __restrict__ n_dev,     \
                                                        RowSplit rs, const int32_t* __restrict__ status)        \
    {                                                                                                            \
        extern __shared__ int s_tile[];                                                                          \
        reduce_rows<U, FULL, WMODE, NTL, NTS, WPB, MAXW, L>(s_tile, src, map, width, w, out, n_bound, n_dev, rs, \
                                                            status);                                             \
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
#ifndef MS_SUMR_UNIT
#define MS_SUMR_UNIT 1
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

static int reduce_unit(int kind, int V, int64_t src_bytes)
{
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

template <int KIND, int U, bool FULL, int WMODE, int WPB, int MAXW, int L>
static void launch_reduce_kernel(dim3 grid, size_t lds, hipStream_t s, const u32x4* src, const int32_t* map,
                                 int width, const float* w, u32x4* out, int64_t n_bound, const int32_t* n_dev,
                                 RowSplit rs, const int32_t* status)
{
    const dim3 block(WPB * kWave);
    if constexpr (KIND == kCombine)
        hipLaunchKernelGGL((combine_rows_kernel<U, FULL, WMODE, WPB, MAXW, 1>), grid, block, lds, s, src, map, width,
                           w, out, n_bound, n_dev, rs, status);
    else if constexpr (KIND == kSumExpertRows && L > 1) {
        if (n_dev)
            hipLaunchKernelGGL((sum_expert_rows_kernel<U, FULL, WMODE, WPB, MAXW, L>), grid, block, lds, s, src, map,
                               width, w, out, n_bound, n_dev, rs, status);
        else
            hipLaunchKernelGGL((sum_expert_rows_kernel<U, FULL, WMODE, WPB, MAXW, 1>), grid, block, lds, s, src, map,
                               width, w, out, n_bound, n_dev, rs, status);
    } else if constexpr (KIND == kSumExpertRows)
        hipLaunchKernelGGL((sum_expert_rows_kernel<U, FULL, WMODE, WPB, MAXW, 1>), grid, block, lds, s, src, map,
                           width, w, out, n_bound, n_dev, rs, status);
    else
        hipLaunchKernelGGL((sum_rank_rows_kernel<U, FULL, WMODE, WPB, MAXW, 1>), grid, block, lds, s, src, map, width,
                           w, out, n_bound, n_dev, rs, status);
}

template <int KIND, int WMODE, int U, int WPB>
static hipError_t launch_reduce_uw(const void* src, const int32_t* map, int width, const float* w, void* out,
                                   int64_t n_bound, const int32_t* n_dev, int V, const int32_t* status, hipStream_t s)
{
    RowSplit rs;
    if (!make_split(V, U, n_bound, &rs)) return hipErrorInvalidValue;
    // rounds only where the row count is on the device (the receiver's sum)
    constexpr int L = KIND == kSumExpertRows ? MS_SUMX_ROUNDS : 1;
    const int64_t ublocks = (n_bound * rs.cpr + WPB - 1) / WPB;
    const int rounds = n_dev ? L : 1;
    const dim3 grid((unsigned)((ublocks + rounds - 1) / rounds));
    const size_t lds = tile_lds_bytes(width, 2, WPB);
    const u32x4* sp = (const u32x4*)src;
    u32x4* op = (u32x4*)out;
    const bool full = V % (kWave * U) == 0;
    if (width <= 8 && full)
        launch_reduce_kernel<KIND, U, true, WMODE, WPB, 8, L>(grid, lds, s, sp, map, width, w, op, n_bound, n_dev, rs,
                                                           status);
    else if (width <= 8)
        launch_reduce_kernel<KIND, U, false, WMODE, WPB, 8, L>(grid, lds, s, sp, map, width, w, op, n_bound, n_dev, rs,
                                                            status);
    else if (full)
        launch_reduce_kernel<KIND, U, true, WMODE, WPB, kMaxTopK, L>(grid, lds, s, sp, map, width, w, op, n_bound,
                                                                  n_dev, rs, status);
    else
        launch_reduce_kernel<KIND, U, false, WMODE, WPB, kMaxTopK, L>(grid, lds, s, sp, map, width, w, op, n_bound,
                                                                   n_dev, rs, status);
    return hipGetLastError();
}

template <int KIND, int WMODE, int U>
static hipError_t launch_reduce_u(const void* src, const int32_t* map, int width, const float* w, void* out,
                                  int64_t n_bound, const int32_t* n_dev, int V, const int32_t* status, hipStream_t s)
{
    if constexpr (U <= 2) {
        if (n_dev)
            return launch_reduce_uw<KIND, WMODE, U, kWavesBig>(src, map, width, w, out, n_bound, n_dev, V, status, s);
    }
    return launch_reduce_uw<KIND, WMODE, U, kWavesPerBlock>(src, map, width, w, out, n_bound, n_dev, V, status, s);
}

template <int KIND, int WMODE>
static hipError_t launch_reduce(const void* src, int64_t src_rows, const int32_t* map, int width, const float* w,
                                void* out, int64_t n_bound, const int32_t* n_dev, int H, const int32_t* status,
                                hipStream_t s)
{
    if (n_bound <= 0) return hipSuccess;
    const int V = H / 8;
    switch (reduce_unit(KIND, V, src_rows * (int64_t)H * 2)) {
        case 1: return launch_reduce_u<KIND, WMODE, 1>(src, map, width, w, out, n_bound, n_dev, V, status, s);
        case 2: return launch_reduce_u<KIND, WMODE, 2>(src, map, width, w, out, n_bound, n_dev, V, status, s);
        case 4: return launch_reduce_u<KIND, WMODE, 4>(src, map, width, w, out, n_bound, n_dev, V, status, s);
        default: return launch_reduce_u<KIND, WMODE, 8>(src, map, width, w, out, n_bound, n_dev, V, status, s);
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
                                  const int32_t* n_dev, int H, const int32_t* status, hipStream_t s)
{
    if (n_bound <= 0) return hipSuccess;
    if (!w) return launch_reduce<kSumExpertRows, kUnweighted>(src, src_rows, fan_dst, D, nullptr, out, n_bound,
                                                              n_dev, H, status, s);
    hipLaunchKernelGGL(gate_of_row_kernel, dim3((unsigned)((src_rows + kBlock - 1) / kBlock)), dim3(kBlock), 0, s, w,
                       comb_row, src_rows, gate_of_row, status);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_reduce<kSumExpertRows, kPerSourceRow>(src, src_rows, fan_dst, D, gate_of_row, out, n_bound, n_dev,
                                                        H, status, s);
}

hipError_t launch_sum_rank_rows(const void* src, int64_t src_rows, const int32_t* tok_rank_row, int KR, void* out,
                                int T, int H, const int32_t* status, hipStream_t s)
{
    return launch_reduce<kSumRankRows, kUnweighted>(src, src_rows, tok_rank_row, KR, nullptr, out, T, nullptr, H,
                                                    status, s);
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
// streaming: 1717 us against 1841 us (long prefill), 775 against 792 us
// (skewed), 436 us either way (DeepSeek-V3-like), on the MI355X.
template <int U, bool FULL, int PART>
__device__ __forceinline__ void combine_bwd_rows(int* s_tile, const u32x4* __restrict__ grad_out,
                                                 const u32x4* __restrict__ ye, const float* __restrict__ w,
                                                 const int32_t* __restrict__ comb_row, u32x4* __restrict__ grad_ye,
                                                 float* __restrict__ dots, int T, int k, RowSplit rs,
                                                 const int32_t* __restrict__ status)
{
    if (status[0] != MOE_SHUFFLE_OK) return;
    int first, count;
    block_rows<kWavesPerBlock>((int)blockIdx.x * kWavesPerBlock, T, rs, &first, &count);
    if (count <= 0) return;
    int* s_rows = s_tile;
    int* s_w = s_tile + kWavesPerBlock * k;
    for (int i = threadIdx.x; i < count * k; i += kBlock) {
        s_rows[i] = comb_row[(int64_t)first * k + i];
        s_w[i] = __float_as_int(w[(int64_t)first * k + i]);
    }
    __syncthreads();

    const int wave = wave_id(), lane = lane_id();
    const int u = (int)blockIdx.x * kWavesPerBlock + wave;
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
                                                   int k, RowSplit rs, const int32_t* __restrict__ status)        \
    {                                                                                                             \
        extern __shared__ int s_tile[];                                                                           \
        combine_bwd_rows<U, FULL, PART>(s_tile, grad_out, ye, w, comb_row, grad_ye, dots, T, k, rs, status);      \
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
// 1.444 ms (skewed) and 3.840 ms (long prefill) against 1.472 and 3.898 ms
// with U = 2 for both, and 1.48 and 3.96 ms for one fused pass at U = 1.
#ifndef MS_CBWD_GRAD_UNIT
#define MS_CBWD_GRAD_UNIT 1
#endif
#ifndef MS_CBWD_DOT_UNIT
#define MS_CBWD_DOT_UNIT 2
#endif
// Pass order: grad_ye first.  The partials first measured 0.900 against
// 0.878 ms per backward step (DeepSeek-V3-like).
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
    const dim3 grid(grid_for((int64_t)T * rs.cpr, kWavesPerBlock));
    const size_t lds = tile_lds_bytes(k, 2, kWavesPerBlock);
    const u32x4* gp = (const u32x4*)grad_out;
    const u32x4* yp = (const u32x4*)ye;
    u32x4* gyp = (u32x4*)grad_ye;
    const bool full = V % (kWave * U) == 0;
    if (grad && full)
        hipLaunchKernelGGL((combine_bwd_grad_kernel<U, true>), grid, dim3(kBlock), lds, s, gp, yp, w, comb_row, gyp,
                           dots, T, k, rs, status);
    else if (grad)
        hipLaunchKernelGGL((combine_bwd_grad_kernel<U, false>), grid, dim3(kBlock), lds, s, gp, yp, w, comb_row, gyp,
                           dots, T, k, rs, status);
    else if (full)
        hipLaunchKernelGGL((combine_bwd_dot_kernel<U, true>), grid, dim3(kBlock), lds, s, gp, yp, w, comb_row, gyp,
                           dots, T, k, rs, status);
    else
        hipLaunchKernelGGL((combine_bwd_dot_kernel<U, false>), grid, dim3(kBlock), lds, s, gp, yp, w, comb_row, gyp,
                           dots, T, k, rs, status);
    return hipGetLastError();
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
