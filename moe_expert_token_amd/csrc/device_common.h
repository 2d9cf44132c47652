// device_common.h -- helpers shared by the kernel files of the MoE token
// shuffle (library-internal): wave and lane ids, fast division, scans, the
// 16-byte row loads and stores with their per-kernel cache hints, the split
// of rows into per-wave work units, and the bf16 rounding.
#pragma once

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

static inline FastDiv make_fastdiv(int d)
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

// fp32 -> bf16 bits, round to nearest even; NaN -> quiet NaN of the same sign.
__device__ __forceinline__ unsigned bf16_rne(float f)
{
    const unsigned u = __float_as_uint(f);
    const unsigned rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    const unsigned quiet_nan = (u >> 16) | 0x40u;
    return (u & 0x7fffffffu) > 0x7f800000u ? quiet_nan : rounded;  // a select, not a branch
}

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
//   combine backward  non-temporal loads and stores
// (DeepSeek-V3-like workload: send 153 us with plain stores against 178 us
// with non-temporal ones; fan-out 303 us against 324 us with plain loads;
// backward step 0.827 ms with non-temporal combine-backward loads against
// 0.865 ms with plain ones.)
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
#define MS_CBWD_NT_LOAD 1
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

// A grid larger than one dispatch can carry (at most 2^32 - 1 work-items
// per dimension) goes out as several launches over consecutive pieces of
// it: block base + blockIdx.x of `total` is the block a kernel works as.
struct GridSpan {
    int base, total;
};

__device__ __forceinline__ int span_block(const GridSpan& g) { return g.base + (int)blockIdx.x; }

// Calls launch(grid, span) for consecutive pieces of `total` blocks of
// `threads` work-items each, none above 2^32 - 1 work-items; stops at the
// first launch error.
template <class F>
static hipError_t launch_spans(int64_t total, int threads, F&& launch)
{
    const int64_t cap = (int64_t)0xFFFFFFFFu / threads;
    for (int64_t base = 0; base < total; base += cap) {
        const int64_t n = total - base < cap ? total - base : cap;
        launch(dim3((unsigned)n), GridSpan{(int)base, (int)total});
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// First unit of this block.  When the row count is known only on the device
// the grid is sized by a bound and the blocks past the count have nothing to
// do; those kernels take the units in reverse block order, so the empty
// blocks are dispatched first and exit while the real work fills the
// machine, instead of trailing it (measured on the MI355X, fan-out: skewed
// workload 537 -> 526 us, long prefill 1383 -> 1328 us; a grid sized by the
// exact count would be 479 and 1295 us, which needs a host sync).
template <int WPB>
__device__ __forceinline__ int block_first_unit(bool reversed, const GridSpan& g)
{
    const int b = reversed ? g.total - 1 - span_block(g) : span_block(g);
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

// Splits rows of V vectors into chunks of 64*U; false if rows * chunks overflows int.
static inline bool make_split(int V, int U, int64_t rows, RowSplit* rs)
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

static inline size_t tile_lds_bytes(int width, int arrays, int wpb)
{
    return sizeof(int) * (size_t)arrays * wpb * width;  // at most one row per wave
}

// Largest of {1, 2, 4, 8} not above `want` whose chunk does not exceed the row.
static inline int fit_unit(int V, int want)
{
    int u = want;
    while (u > 1 && kWave * u > V) u >>= 1;
    return u;
}

}  // namespace ms
