"""Paged tree attention for AMD Instinct MI355X (gfx950).

The compute path is libpta.so (hand-written HIP kernels behind a C ABI, see
include/pta.h); this package is its thin Python binding.  PyTorch supplies
device memory and streams only.
"""
from ._lib import (  # noqa: F401
    PATHS,
    LookaheadCache,
    PreparedCall,
    prepare_kv_append,
    prepare_paged_tree_attn,
    PtaDims,
    PtaError,
    declared_functions,
    load,
    make_dims,
    taco_accept_commit,
    taco_gemm_w4a16,
    taco_gemm_w4a16_pack,
    taco_gemm_w8a8,
    taco_gemm_w8a16,
    taco_gemm_w8a16_pack,
    taco_gemm_w4a8,
    taco_kv_append,
    taco_la_tree_mask,
    NOALLOC_SCRATCH_BYTES,
    taco_paged_tree_attn_balanced,
    taco_paged_tree_attn_balanced_append,
    taco_paged_tree_attn_balanced_noalloc,
    taco_paged_tree_attn_balanced_workspace_size,
    taco_paged_tree_attn,
    taco_paged_tree_attn_append,
    taco_paged_tree_attn_shared_prefix,
    taco_paged_tree_attn_splitk,
    taco_paged_tree_attn_splitk_workspace_size,
    taco_pta_calib_mfma_bf16,
    taco_pta_calib_stream_read,
    taco_pta_status_string,
    taco_pta_validate,
    taco_pta_version,
)
