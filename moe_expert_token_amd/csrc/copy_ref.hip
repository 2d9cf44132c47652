// copy_ref.hip -- the reference streaming copy: the HBM ceiling that the
// row kernels are measured against (not a step of the shuffle).  One
// 16-byte vector per lane, 256 lanes per block, consecutive blocks on
// consecutive 4 KiB, non-temporal loads and stores: on the MI355X this
// simple form measured 6.49 TB/s (read + write) over 2 GiB, against 5.4 to
// 5.9 TB/s with 2 to 8 vectors per lane and 6.11 TB/s without the hint.
#include "device_common.h"

namespace ms {

__global__ __launch_bounds__(kBlock) void copy_reference_kernel(const u32x4* __restrict__ src,
                                                                u32x4* __restrict__ dst, int64_t n, GridSpan gs)
{
    const int64_t i = (int64_t)span_block(gs) * kBlock + threadIdx.x;
    if (i < n) store_row16<true>(load_row16<true>(src + i), dst + i);
}

hipError_t launch_copy_reference(const void* src, void* dst, int64_t n_vectors, hipStream_t s)
{
    if (n_vectors <= 0) return hipSuccess;
    const int64_t blocks = (n_vectors + kBlock - 1) / kBlock;
    if (blocks > 0x7fffffffll) return hipErrorInvalidValue;
    return launch_spans(blocks, kBlock, [&](dim3 grid, GridSpan gs) {
        hipLaunchKernelGGL(copy_reference_kernel, grid, dim3(kBlock), 0, s, (const u32x4*)src, (u32x4*)dst,
                           n_vectors, gs);
    });
}

}  // namespace ms
