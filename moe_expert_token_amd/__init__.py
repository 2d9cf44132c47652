"""MoE token shuffle for AMD MI355X (gfx950): plan, dispatch, combine.

A thin Python face of the C ABI in include/moe_shuffle.h; every step runs in
the HIP kernels of libmoe_shuffle.so.  Tensors are torch tensors on the GPU;
bf16 activations may be torch.bfloat16 or any 16-bit view of the same bits.
"""

from ._lib import (  # noqa: F401
    E_ALIGN, E_BAD_INDEX, E_HIP, E_INVALID_ARG, E_OVERFLOW, E_WORKSPACE, EXPORTS, LIB_PATH, OK, Dims,
    MoeShuffleError, Plan, dims_of, load, moe_shuffle_combine, moe_shuffle_dispatch, moe_shuffle_dispatch_fanout,
    moe_shuffle_dispatch_send, moe_shuffle_last_hip_error, moe_shuffle_plan, moe_shuffle_plan_arrays_get,
    moe_shuffle_plan_destroy, moe_shuffle_plan_query, moe_shuffle_strerror, moe_shuffle_workspace_size,
    plan_array_views, moe_shuffle_sum_expert_rows, moe_shuffle_sum_rank_rows, moe_shuffle_dispatch_backward,
    moe_shuffle_combine_rank_partial, moe_shuffle_combine_backward, moe_shuffle_dispatch_range,
    moe_shuffle_combine_range, moe_shuffle_combine_rank_partial_f32, moe_shuffle_copy_reference,
    moe_shuffle_plan_static, PlanStorage, STATIC_WORKSPACE_BYTES,
)
