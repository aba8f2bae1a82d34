"""MI355X (gfx950) W8A8 FP8 block-scaled MoE expert path (and its MXFP8, MXFP4 and bf16 variants).

The computation lives in libfp8moe.so (hand-written HIP kernels behind the C
ABI of include/fp8moe.h); this package only loads it and marshals torch
tensors into it.
"""

from ._lib import lib, Fp8MoeError, LIB_PATH  # noqa: F401
from .ops import (  # noqa: F401
    route_capacity, route_permute, fused_workspace_size, alloc_workspace, moe_fused_fp8,
    gemm1_swiglu_quant, gemm2_weighted, combine, gated_act_fp8_quant, select_tile, auto_tiles,
    select_tile_classes, pack_weights, WEIGHTS_ROW_MAJOR, WEIGHTS_MFMA_TILED,
    fused_mx_workspace_size, alloc_workspace_mx, moe_fused_mxfp8, pack_mx_scales, grouped_gemm_fp8,
    fused_mxfp4_workspace_size, alloc_workspace_mxfp4, moe_fused_mxfp4, pack_mxfp4_scales,
    gemm1_swiglu_quant_mxfp4, gemm2_weighted_mxfp4, gemm1_swiglu_quant_mx, gemm2_weighted_mx,
    fused_bf16_workspace_size, alloc_workspace_bf16, moe_fused_bf16, gemm1_swiglu_bf16, gemm2_weighted_bf16,
    tune_tiles_fp8, moe_fused_fp8_small, fused_small_workspace_size, small_layer_flag,
    moe_fused_fp8_noalloc, NOALLOC_SCRATCH_BYTES,
)
