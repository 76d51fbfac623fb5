"""Fused W4A16 Mixture-of-Experts layer for MI355X (gfx950).

Thin Python binding over the C-ABI library libmoe_w4a16.so (declared in
include/moe_w4a16.h).  The binding only marshals arguments: torch tensors
provide device memory and the current HIP stream; every step of the layer
runs in the library's HIP kernels.  There is no fallback: if the library is
missing, every call raises.
"""
from ._binding import (  # noqa: F401
    ACT, FMT, KERNEL, ROUTE, QuantWeights, MoeError, lib, library_path,
    moe_align, moe_align_capacity, moe_align_large, moe_forward, moe_forward_block_m,
    moe_forward_workspace_bytes, moe_gptq_act_order_sort, moe_permute_slots,
    moe_forward_mxfp8, moe_forward_mxfp8_workspace_bytes, moe_mx_gemm1, moe_mx_gemm2,
    moe_mxfp8_quantize, mxfp8_lda, mxfp8_lds, moe_nvfp4_codes_by_chunk, moe_nvfp4_scales_by_chunk, moe_mxfp4_codes_by_chunk, moe_mxfp4_scales_by_chunk,
    moe_route, moe_route_align, moe_w4a16_gemm1, moe_w4a16_gemm2,
    NOALLOC_SCRATCH_BYTES, moe_forward_noalloc,
)
