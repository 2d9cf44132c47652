// plan.hip -- the routing plan (FUSCO abstract: the light-weight planner
// that drops redundant sends; press summary, Group 3: logical segments).
//   plan_count  one wave per 64-token tile; the wave ORs its lanes' bits
//               into one 64-bit LDS mask per expert and per rank, so a token
//               with several experts on one rank sets that rank's bit once
//               (the send-once rule) and no result depends on the order of
//               the atomics.  Counts are popcounts of the masks.
//   plan_scan   one block per histogram column: exclusive scan over the
//               tiles.
//   plan_place  recomputes the masks, scans the column totals into
//               offsets, and gives every (token, rank) and (token, expert)
//               pair its row: tile base + mbcnt(mask).  Rows come out in
//               ascending token order inside every segment.
//   plan_recount  up to 48 tiles with E + R <= 64 (while the recount
//               stays small): one launch of one block per tile, each block
//               counting every tile again (ballots over per-lane column
//               masks), so no block waits on another; then one wave places
//               the block's tile.
//   plan_small  up to 16 tiles (and 32 tile-slots): the three steps in one
//               block of one wave per tile.
// Each form loads a token's ids once, for both its count and place steps.
#include "device_common.h"

namespace ms {

// ---------------------------------------------------------------- plan_count

// The top-k ids of token t; slots past k, and every slot of a token past T,
// hold 0x7fffffff (they sort after every real id).  A row of 4n ids (2n)
// starting on a 16-byte (8-byte) boundary is read 16 (8) bytes at a time:
// a wave's rows are contiguous, so each instruction covers whole lines
// instead of one id per lane every 4k bytes.
template <int KMAX>
__device__ __forceinline__ void load_ids(const int32_t* __restrict__ idx, int T, int k, int t, int (&ev)[KMAX])
{
    typedef int i32x2 __attribute__((ext_vector_type(2)));
    typedef int i32x4v __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int j = 0; j < KMAX; ++j) ev[j] = 0x7fffffff;
    if (t < T) {
        const int32_t* row = idx + (int64_t)t * k;
        const unsigned long long base = (unsigned long long)idx;
        if ((k & 3) == 0 && (base & 15) == 0) {  // uniform
#pragma unroll
            for (int j = 0; j < KMAX; j += 4)
                if (j < k) {
                    const i32x4v v = *(const i32x4v*)(row + j);
                    ev[j] = v.x;
                    if (j + 1 < KMAX) ev[j + 1] = v.y;
                    if (j + 2 < KMAX) ev[j + 2] = v.z;
                    if (j + 3 < KMAX) ev[j + 3] = v.w;
                }
        } else if ((k & 1) == 0 && (base & 7) == 0) {  // uniform
#pragma unroll
            for (int j = 0; j < KMAX; j += 2)
                if (j < k) {
                    const i32x2 v = *(const i32x2*)(row + j);
                    ev[j] = v.x;
                    if (j + 1 < KMAX) ev[j + 1] = v.y;
                }
        } else {
#pragma unroll
            for (int j = 0; j < KMAX; ++j)
                if (j < k) ev[j] = row[j];
        }
    }
}

// One wave per 64-token tile, its ids already loaded.  hist is column-major
// [(C+1)][ntiles]; column C holds the tile's error flag.
template <int KMAX>
__device__ __forceinline__ void count_tile(const int (&ev)[KMAX], int T, int k, int E, FastDiv epr, int C,
                                           int ntiles, int32_t* __restrict__ hist, int tile, int lane,
                                           unsigned long long* s_mask /* [C], this wave's */)
{
    const int t = tile * kPlanTile + lane;
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

template <int KMAX>
__global__ __launch_bounds__(kWave) void plan_count_kernel(const int32_t* __restrict__ idx, int T, int k,
                                                           int E, FastDiv epr, int C, int ntiles,
                                                           int32_t* __restrict__ hist)
{
    extern __shared__ unsigned long long s_mask[];  // [C]
    const int tile = blockIdx.x, lane = threadIdx.x;
    int ev[KMAX];
    load_ids<KMAX>(idx, T, k, tile * kPlanTile + lane, ev);
    count_tile<KMAX>(ev, T, k, E, epr, C, ntiles, hist, tile, lane, s_mask);
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

// ev: this lane's top-k ids (load_ids); ct_src[c]: column totals;
// tb_src[c * tb_stride]: this tile's base in column c; status_src[0]: the
// plan status (global arrays, or their copies in LDS when the whole plan
// runs in one block).  NCOLS * 64 >= C.  A tile at or past ntiles only
// takes part in the barriers.
template <int KMAX, int NCOLS = kMaxCols / kWave>
__device__ __forceinline__ void place_tile(const PlaceArgs& a, int (&ev)[KMAX], int tile, int lane,
                                           unsigned long long* s_mask /* [C] */, int* s_wbase /* [C] */,
                                           const int32_t* ct_src, const int32_t* tb_src, int tb_stride,
                                           const int32_t* status_src)
{
    const int C = a.C, E = a.E, R = a.R;
    const int t = tile * kPlanTile + lane;
    const int k = a.k;
    constexpr int kCols = NCOLS;  // histogram columns per lane

    // Every load before the first use, so their latencies overlap: the
    // status word, and for each column this lane owns the column total and
    // this tile's base within the column.
    const int status = status_src[0];
    int ct[kCols], tb[kCols];
#pragma unroll
    for (int i = 0; i < kCols; ++i) {
        const int c = lane + i * kWave;
        ct[i] = c < C ? ct_src[c] : 0;
        tb[i] = c < C ? tb_src[(int64_t)c * tb_stride] : 0;
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

template <int KMAX>
__global__ __launch_bounds__(kWave) void plan_place_kernel(PlaceArgs a)
{
    extern __shared__ unsigned long long s_dyn[];
    const int tile = blockIdx.x, lane = threadIdx.x;
    int ev[KMAX];
    load_ids<KMAX>(a.idx, a.T, a.k, tile * kPlanTile + lane, ev);
    place_tile<KMAX>(a, ev, tile, lane, s_dyn, (int*)(s_dyn + a.C), a.col_total, a.tile_base + tile, a.ntiles,
                     a.status);
}

// ---------------------------------------------------------------- small batches
//
// Up to kSmallTiles tiles, the three steps run in one block of one wave per
// tile, separated by block barriers instead of kernel boundaries, with the
// tile histograms (scanned in place into the tile bases), the column totals
// and the status in LDS: one launch instead of three and no global round
// trip between the steps, which is most of the plan's time on a small
// batch.  Each lane loads its token's ids once, for both the count and the
// place step.  The count and place steps are the functions above; the scan
// is one wave per column.  The scan results also go to the workspace for the
// later kernels.  (One block is one CU: a block that loops its waves over
// more tiles measured slower than three launches from 17 tiles on, the
// CU's memory pipeline taking every tile's scattered index stores.)
constexpr int kSmallTiles = 16;
constexpr size_t kSmallLds = 48 * 1024;
constexpr int kSmallMaxTopK = 16;  // wider rows keep the three launches (registers at 16 waves per block)
constexpr int kSmallMaxSlots = 32; // tiles x top-k: one CU takes every index store, slower than three launches beyond

// LDS of the one-block plan: per wave its masks and row bases, then the
// shared histograms (plus the error column), the totals and the status.
static size_t small_plan_lds(int ntiles, int C)
{
    return (size_t)ntiles * C * (sizeof(unsigned long long) + sizeof(int)) +
           sizeof(int) * ((size_t)(C + 1) * ntiles + C + 1);
}

template <int KMAX>
__global__ __launch_bounds__(kSmallTiles * kWave) void plan_small_kernel(PlaceArgs a, int32_t* __restrict__ tile_base,
                                                                         int32_t* __restrict__ col_total,
                                                                         int32_t* __restrict__ status)
{
    extern __shared__ unsigned long long s_dyn[];
    const int C = a.C, ntiles = a.ntiles;
    const int wave = wave_id(), lane = lane_id();  // one wave per tile: blockDim.x = 64 * ntiles
    unsigned long long* s_mask = s_dyn + (size_t)wave * C;
    int* s_ints = (int*)(s_dyn + (size_t)ntiles * C);
    int* s_wbase = s_ints + (size_t)wave * C;
    int* s_tb = s_ints + (size_t)ntiles * C;      // [(C+1)][ntiles]: histograms, then tile bases
    int* s_ct = s_tb + (size_t)(C + 1) * ntiles;  // [C]
    int* s_status = s_ct + C;                     // [1]

    int ev[KMAX];
    load_ids<KMAX>(a.idx, a.T, a.k, wave * kPlanTile + lane, ev);
    count_tile<KMAX>(ev, a.T, a.k, a.E, a.epr, C, ntiles, s_tb, wave, lane, s_mask);
    __syncthreads();  // every tile's histogram is in LDS

    // Exclusive scan of each column over the tiles (at most 16: one lane per
    // tile), in place; column C holds the error flags.
    for (int c = wave; c <= C; c += ntiles) {
        int* col = s_tb + (size_t)c * ntiles;
        const int v = lane < ntiles ? col[lane] : 0;
        if (c == C) {
            const bool bad = __ballot(v != 0) != 0ull;
            const int st = bad ? MOE_SHUFFLE_E_BAD_INDEX : MOE_SHUFFLE_OK;
            if (lane == 0) {
                s_status[0] = st;
                status[0] = st;
            }
        } else {
            const int incl = wave_inclusive_scan(v);
            if (lane < ntiles) {
                col[lane] = incl - v;
                tile_base[(int64_t)c * ntiles + lane] = incl - v;
            }
            if (lane == kWave - 1) {
                s_ct[c] = incl;
                col_total[c] = incl;
            }
        }
    }
    __syncthreads();  // offsets and status are in LDS
    place_tile<KMAX>(a, ev, wave, lane, s_mask, s_wbase, s_ct, s_tb + wave, ntiles, s_status);
}

// ---------------------------------------------------------------- small batches, narrow histograms
//
// Up to 48 tiles with at most 64 histogram columns (E + R <= 64): one launch
// of one block per tile.  Every block counts every tile again -- wave w of
// the min(tiles, 16) waves counts tiles w, w + 16, w + 32 (the same number
// of trips in every wave), a lane's columns fit one 64-bit mask, and a
// column's count over a tile is the popcount of one ballot -- which gives it
// the column totals and its own tile's bases without waiting on any other
// block.  Then the wave that counted the block's tile places it with the
// functions above, from the ids it holds (the other waves pass through the
// same barriers with a tile past the end).  Block 0 publishes the status and
// the column totals, block b column b of the tile bases.  The recount grows
// with trips x (E + R + 3k) (ballots per column, id work per slot), so it is
// used only while that stays small; larger batches take the other forms.
constexpr int kRecountMaxCols = kWave;  // one lane per column
constexpr int kRecountWaves = 16;
constexpr int kRecountMaxTrips = 3;     // tiles per wave
constexpr int kRecountMaxTiles = kRecountWaves * kRecountMaxTrips;
constexpr int kRecountMaxWork = 66;     // trips x (E + R + 3k): measured faster than the other forms up to here

template <int KMAX, int TRIPS>
__global__ __launch_bounds__(kRecountWaves * kWave) void plan_recount_kernel(PlaceArgs a,
                                                                            int32_t* __restrict__ tile_base,
                                                                            int32_t* __restrict__ col_total,
                                                                            int32_t* __restrict__ status)
{
    __shared__ unsigned long long s_mask[kRecountWaves][kRecountMaxCols];
    __shared__ int s_wbase[kRecountWaves][kRecountMaxCols];
    __shared__ int s_ct[kRecountMaxCols], s_pre[kRecountMaxCols], s_bad, s_status;
    const int C = a.C, E = a.E, T = a.T, k = a.k, ntiles = a.ntiles;
    const int nwaves = blockDim.x / kWave;             // min(ntiles, 16)
    const int trips = (ntiles + nwaves - 1) / nwaves;  // <= TRIPS
    const int wave = wave_id(), lane = lane_id();
    const int b = blockIdx.x;  // this block's tile

    int ev[TRIPS][KMAX];
#pragma unroll
    for (int it = 0; it < TRIPS; ++it) load_ids<KMAX>(a.idx, T, k, (wave + it * nwaves) * kPlanTile + lane, ev[it]);
    if (threadIdx.x < C) {
        s_ct[threadIdx.x] = 0;
        s_pre[threadIdx.x] = 0;
    }
    if (threadIdx.x == 0) s_bad = 0;
    __syncthreads();

    // The column totals, and the counts of the tiles before b.
    const unsigned long long emask = (1ull << E) - 1;  // E < C <= 64
#pragma unroll
    for (int it = 0; it < TRIPS; ++it) {
        if (it >= trips) break;  // uniform
        const int tile = wave + it * nwaves;
        const int t = tile * kPlanTile + lane;
        unsigned long long m = 0ull;
        int bad = 0;
        if (t < T) {
            int nslots = 0;
#pragma unroll
            for (int j = 0; j < KMAX; ++j)
                if (j < k) {
                    const int e = ev[it][j];
                    if ((unsigned)e >= (unsigned)E) {
                        bad = 1;
                    } else {
                        ++nslots;
                        m |= 1ull << e;
                        m |= 1ull << (E + fdiv(e, a.epr));
                    }
                }
            // a repeated expert sets its bit once: fewer expert bits than slots
            if (__popcll(m & emask) != nslots) bad = 1;
        }
        int cnt = 0;
        for (int c = 0; c < C; ++c) {
            const int n = __popcll(__ballot((m >> c) & 1ull));
            cnt = lane == c ? n : cnt;
        }
        if (lane < C) {
            atomicAdd(&s_ct[lane], cnt);
            if (tile < b) atomicAdd(&s_pre[lane], cnt);
        }
        if (__ballot(bad) != 0ull && lane == 0) atomicOr(&s_bad, 1);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        s_status = s_bad ? MOE_SHUFFLE_E_BAD_INDEX : MOE_SHUFFLE_OK;
        if (b == 0) status[0] = s_status;
    }
    if (threadIdx.x < C) {
        tile_base[(int64_t)threadIdx.x * ntiles + b] = s_pre[threadIdx.x];
        if (b == 0) col_total[threadIdx.x] = s_ct[threadIdx.x];
    }
    __syncthreads();

    // The wave that counted tile b places it.
    const int owner = b % nwaves, it_b = b / nwaves;
    int evb[KMAX];
#pragma unroll
    for (int it = 0; it < TRIPS; ++it)
        if (it == it_b)  // uniform
#pragma unroll
            for (int j = 0; j < KMAX; ++j) evb[j] = ev[it][j];
    place_tile<KMAX, 1>(a, evb, wave == owner ? b : ntiles, lane, s_mask[wave], s_wbase[wave], s_ct, s_pre, 1,
                        &s_status);
}

static PlaceArgs place_args(const Layout& L, const PlanPtrs& P, FastDiv epr)
{
    PlaceArgs a;
    a.idx = P.idx;
    a.T = L.T; a.k = L.k; a.E = L.E; a.R = L.R; a.Epr = L.Epr; a.KR = L.KR; a.D = L.D; a.C = L.C;
    a.ntiles = L.ntiles;
    a.epr = epr;
    a.tile_base = P.tile_base; a.col_total = P.col_total; a.status = P.status;
    a.expert_count = P.expert_count; a.expert_offset = P.expert_offset;
    a.rank_count = P.rank_count; a.rank_offset = P.rank_offset;
    a.send_token = P.send_token; a.tok_rank_row = P.tok_rank_row; a.fan_src = P.fan_src;
    a.fan_dst = P.fan_dst; a.comb_row = P.comb_row;
    a.rank_segs = P.rank_segs; a.expert_segs = P.expert_segs; a.n_rank_rows = P.n_rank_rows;
    return a;
}

hipError_t launch_plan(const Layout& L, const PlanPtrs& P, hipStream_t s)
{
    // one 64-lane wave per tile: ntiles * 64 < T + 64 <= 2^31 work-items,
    // always one dispatch
    const int ntiles = L.ntiles;
    const size_t lds_count = sizeof(unsigned long long) * L.C;
    const FastDiv epr = make_fastdiv(L.Epr);
    const int rwaves = ntiles < kRecountWaves ? ntiles : kRecountWaves;
    const int rtrips = (ntiles + rwaves - 1) / rwaves;
    if (ntiles <= kRecountMaxTiles && L.C <= kRecountMaxCols && L.k <= (rtrips == 1 ? 16 : 8) &&
        rtrips * (L.C + 3 * L.k) <= kRecountMaxWork) {
        const PlaceArgs a = place_args(L, P, epr);
        const dim3 grid(ntiles), block(rwaves * kWave);
        if (rtrips == 1 && L.k <= 8)
            hipLaunchKernelGGL((plan_recount_kernel<8, 1>), grid, block, 0, s, a, P.tile_base, P.col_total, P.status);
        else if (rtrips == 1)
            hipLaunchKernelGGL((plan_recount_kernel<16, 1>), grid, block, 0, s, a, P.tile_base, P.col_total,
                               P.status);
        else
            hipLaunchKernelGGL((plan_recount_kernel<8, kRecountMaxTrips>), grid, block, 0, s, a, P.tile_base,
                               P.col_total, P.status);
        return hipGetLastError();
    }
    const size_t lds_small = small_plan_lds(ntiles, L.C);
    if (ntiles <= kSmallTiles && lds_small <= kSmallLds && L.k <= kSmallMaxTopK &&
        ntiles * L.k <= kSmallMaxSlots) {
        const PlaceArgs a = place_args(L, P, epr);
        const dim3 grid(1), block(ntiles * kWave);
        if (L.k <= 8)
            hipLaunchKernelGGL(plan_small_kernel<8>, grid, block, lds_small, s, a, P.tile_base, P.col_total,
                               P.status);
        else
            hipLaunchKernelGGL(plan_small_kernel<16>, grid, block, lds_small, s, a, P.tile_base, P.col_total,
                               P.status);
        return hipGetLastError();
    }
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
    const PlaceArgs a = place_args(L, P, epr);
    hipLaunchKernelGGL(plan_scan_kernel, dim3(L.C + 1), dim3(kBlock), 0, s, P.tile_hist, ntiles, L.C,
                       P.tile_base, P.col_total, P.status);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
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

}  // namespace ms
