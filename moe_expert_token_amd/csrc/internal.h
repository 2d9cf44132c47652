// internal.h -- workspace layout and kernel launchers shared by abi.hip and
// the kernel files (library-internal; not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_shuffle.h"

namespace ms {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kBlock = 256;        // threads per block (the plan kernels run one wave per block)
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kPlanTile = kWave;   // tokens per plan tile: one wave, one lane per token
constexpr int kMaxTopK = 64;
constexpr int kMaxCols = 1024;     // E + R: histogram columns per token tile

// Byte offsets of every array inside the caller's workspace.  Each array
// starts on a 256-byte boundary.
struct Layout {
    int T, H, E, k, R, Epr, KR, D, C, ntiles;
    size_t status, n_rank_rows;
    size_t expert_count, expert_offset, rank_count, rank_offset;
    size_t send_token, tok_rank_row, fan_src, fan_dst, comb_row;
    size_t rank_segs, expert_segs;
    size_t tile_hist, tile_base, col_total;
    size_t gate_of_row;  // fp32 [T*k]: the gate of every expert row (rank-partial combine)
    size_t bwd_dots;     // fp32 [T][ceil(H/512)][k]: gate-gradient partial sums
    size_t total;
};

// Fills `L` from validated dims.
void make_layout(const moe_shuffle_dims& d, Layout& L);

struct PlanPtrs {
    const int32_t* idx;
    int32_t *status, *n_rank_rows;
    int32_t *expert_count, *expert_offset, *rank_count, *rank_offset;
    int32_t *send_token, *tok_rank_row, *fan_src, *fan_dst, *comb_row;
    int32_t *rank_segs, *expert_segs;
    int32_t *tile_hist, *tile_base, *col_total;
};

// Each launcher returns the hipError_t of its launch(es).
hipError_t launch_plan(const Layout& L, const PlanPtrs& P, hipStream_t s);

// dst[map[u][d]] = src[u] for every source row u < n and every map entry
// d < width that is not -1.  n is read from n_dev when it is non-null (then
// n_bound bounds it); otherwise n = n_bound.  `send` picks the kernel name
// (send: x -> xr; otherwise fan-out: xr -> xe).
hipError_t launch_fanout_rows(bool send, const void* src, void* dst, const int32_t* map, int width,
                              int64_t n_bound, const int32_t* n_dev, int H,
                              const int32_t* status, hipStream_t s);

// out[t] = bf16( fp32 fma chain over j of w[t][j] * ye[rows[t][j]] ).
hipError_t launch_combine_rows(const void* ye, const float* w, const int32_t* rows, void* out,
                               int T, int k, int H, const int32_t* status, hipStream_t s);

// out[p] = bf16( sum over q in fan_dst[p] of (gate(q) *) src[q] ) for p < n;
// gate(q) is scattered from w through comb_row first when w is non-null.
// With f32_out (w non-null only) out holds the fp32 sums, not rounded.
hipError_t launch_sum_expert_rows(const void* src, int64_t src_rows, const float* w, const int32_t* comb_row,
                                  float* gate_of_row, const int32_t* fan_dst, int D, void* out, int64_t n_bound,
                                  const int32_t* n_dev, int H, const int32_t* status, hipStream_t s,
                                  bool f32_out = false);

// out[t] = bf16( sum over p in tok_rank_row[t] of src[p] ) for t < T; with
// f32_in the src rows are fp32.
hipError_t launch_sum_rank_rows(const void* src, int64_t src_rows, const int32_t* tok_rank_row, int KR, void* out,
                                int T, int H, const int32_t* status, hipStream_t s, bool f32_in = false);

// The fan-out of the rank rows that belong to tokens [t0, t1) (t0, t1
// multiples of kPlanTile, or t1 = T).
hipError_t launch_fanout_range(const void* xr, void* xe, const int32_t* fan_dst, int D, const int32_t* rank_offset,
                               const int32_t* tile_base, const int32_t* col_total, int E, int R, int ntiles, int t0,
                               int t1, int T, int KR, int H, const int32_t* status, hipStream_t s);

// grad_ye[q(t,j)] = bf16(w[t][j] * grad_out[t]); grad_w[t][j] = <grad_out[t], ye[q(t,j)]>.
hipError_t launch_combine_backward(const void* grad_out, const void* ye, const float* w, const int32_t* comb_row,
                                   void* grad_ye, float* grad_w, float* dots, int T, int k, int H,
                                   const int32_t* status, hipStream_t s);

// dst[i] = src[i] for the n_vectors 16-byte vectors (the reference copy).
hipError_t launch_copy_reference(const void* src, void* dst, int64_t n_vectors, hipStream_t s);

}  // namespace ms
