"""MI355X-native MoE expert hot path: token permute, rank-major -> expert-major
reorder, grouped SwiGLU GEMM (bf16 MFMA) and its backward, weighted unpermute-combine with
special experts, the backward of the permute and of the combine, and the
deredundency dispatch indices and whiteboard combine.

The computation lives in libmoeperm.so (hand-written HIP for gfx950, C ABI in
include/libmoeperm.h); this package only binds it. Build it with
``python -c "import __graft_entry__ as g; g.build()"``.
"""
from .binding import (  # noqa: F401
    EXPORTS, LIB_PATH, MoeError, MoeSpecialExperts, combine_alloc, combine_grad_alloc,
    grouped_gemm_alloc, load,
    make_special, moe_grouped_gemm_swiglu, moe_grouped_gemm_swiglu_workspace_size, moe_permute,
    moe_permute_noalloc, moe_permute_rows, moe_permute_workspace_size, moe_rank_to_expert_reorder,
    moe_rank_to_expert_reorder_workspace_size, moe_unpermute_combine, moe_unpermute_grad,
    moe_unpermute_combine_grad, moe_unpermute_combine_grad_workspace_size,
    moe_deredundency_dispatch_indices, moe_deredundency_dispatch_indices_workspace_size,
    moe_deredundency_combine, moe_deredundency_combine_workspace_size, dered_indices_alloc,
    dered_combine_alloc, moe_grouped_gemm_swiglu_grad, moe_grouped_gemm_swiglu_grad_workspace_size,
    grouped_gemm_grad_alloc,
    moe_permute_grad, permute_alloc, permute_grad_alloc, reorder_alloc, status_str,
    unpermute_grad_alloc, workspace,
)
