"""Fused Mixture-of-Experts layer for AMD Instinct MI355X (gfx950).

The compute lives in the HIP library ``libmoe_mi355x.so`` (C ABI in
``include/moe.h``); this package is its Python binding.  See ``moe.py``.
"""
from .moe import (ACT_GELU, ACT_SILU, DTYPE_BF16, DTYPE_F32, DTYPE_FP8_BLOCK, DTYPE_FP8_E4M3,
                  DTYPE_MXFP4, QUANT_FP8, QUANT_FP8_BLOCK, QUANT_FP8X2, QUANT_NONE, SIGMOID, SOFTMAX, MoeError, Weights, moe_finalize,
                  moe_finalize_add_rmsnorm, moe_fused_experts, moe_fused_experts_unfinalized,
                  moe_fused_experts_unfinalized_noalloc,
                  moe_grouped_gemm1_act, moe_grouped_gemm1_act_batched,
                  moe_grouped_gemm1_act_gathered,
                  moe_grouped_gemm1_act_fp8, moe_grouped_gemm1_act_fp8_blockwise,
                  moe_grouped_gemm1_act_fp8_gathered,
                  moe_grouped_gemm1_act_fp8x2, moe_grouped_gemm2, moe_grouped_gemm2_fp8_blockwise,
                  moe_permute_fp8_blockwise, moe_quantize_fp8_blockwise,
                  moe_grouped_gemm2_batched, moe_grouped_gemm2_fp8, moe_grouped_gemm2_fp8x2,
                  moe_grouped_gemm_workspace_size, moe_permute,
                  moe_permute_batched, moe_permute_fp8, moe_permuted_rows, moe_quantize_fp8,
                  moe_quantize_fp8x2, moe_route_permute, moe_route_permute_gemm1_act, moe_route_topk,
                  moe_shared_workspace_size,
                  moe_workspace_size)

__all__ = [
    "ACT_GELU", "ACT_SILU", "DTYPE_BF16", "DTYPE_F32", "DTYPE_FP8_BLOCK", "DTYPE_FP8_E4M3",
    "DTYPE_MXFP4", "QUANT_FP8", "QUANT_FP8_BLOCK", "QUANT_FP8X2", "QUANT_NONE",
    "moe_grouped_gemm1_act_fp8_blockwise", "moe_grouped_gemm2_fp8_blockwise",
    "moe_grouped_gemm1_act_fp8_gathered",
    "moe_permute_fp8_blockwise", "moe_quantize_fp8_blockwise", "SIGMOID", "SOFTMAX", "MoeError", "Weights", "moe_finalize",
    "moe_finalize_add_rmsnorm", "moe_fused_experts", "moe_fused_experts_unfinalized",
    "moe_fused_experts_unfinalized_noalloc",
    "moe_grouped_gemm1_act", "moe_grouped_gemm1_act_batched",
    "moe_grouped_gemm1_act_gathered", "moe_grouped_gemm1_act_fp8",
    "moe_grouped_gemm1_act_fp8x2", "moe_grouped_gemm2", "moe_grouped_gemm2_batched", "moe_grouped_gemm2_fp8",
    "moe_grouped_gemm2_fp8x2", "moe_grouped_gemm_workspace_size", "moe_permute", "moe_permute_batched", "moe_permute_fp8",
    "moe_permuted_rows", "moe_quantize_fp8", "moe_quantize_fp8x2", "moe_route_permute", "moe_route_permute_gemm1_act", "moe_route_topk", "moe_shared_workspace_size",
    "moe_workspace_size",
]
