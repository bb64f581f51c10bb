"""FP8 block-scaled and 2:4-sparse FP8 linear layers for AMD MI355X (gfx950).

Python face of the C-ABI library ``libfp8lin.so`` (declared in
``include/fp8lin.h``): the calls of the quantized linear layer under their C
names.  torch supplies device memory and the stream; the arithmetic runs in
the library's HIP kernels.
"""
from ._binding import (EXPORTS, FP8L_ERR_ALIAS, FP8L_ERR_ALIGN, FP8L_ERR_DEVICE, FP8L_ERR_LAUNCH, FP8L_ERR_MEMORY,
                       FP8L_ERR_NULL, FP8L_ERR_SCRATCH, FP8L_ERR_SHAPE, FP8L_OK, GROUP, LIB_PATH, MAX_LINEAR_M,
                       Fp8LinError, fp8_block_gemm, fp8_block_gemm_noalloc, fp8_block_gemm_swiglu,
                       fp8_block_gemm_ue8m0, fp8_block_linear, fp8_grouped_gemm,
                       fp8_quant_act, fp8_quant_act_static, fp8_quant_act_tensor, fp8_quant_act_ue8m0,
                       fp8_quant_weight_block, fp8_quant_weight_block_ue8m0, fp8_quant_weight_tensor,
                       fp8_sparse24_gemm, fp8_sparse24_linear, fp8lin_release_graph_scratch, load_library,
                       prune24_compress, prune24_compress_tensor, status_str)

__all__ = [
    "fp8_quant_act", "fp8_quant_weight_block", "prune24_compress", "fp8_block_gemm", "fp8_sparse24_gemm",
    "fp8_quant_act_ue8m0", "fp8_quant_weight_block_ue8m0", "fp8_block_gemm_ue8m0", "fp8_grouped_gemm",
    "fp8_block_gemm_swiglu", "fp8_block_linear", "fp8_sparse24_linear", "fp8_quant_act_tensor",
    "fp8_quant_act_static", "fp8_quant_weight_tensor", "prune24_compress_tensor", "fp8_block_gemm_noalloc",
    "fp8lin_release_graph_scratch",
    "MAX_LINEAR_M", "load_library", "status_str", "Fp8LinError", "EXPORTS", "GROUP", "LIB_PATH",
    "FP8L_OK", "FP8L_ERR_NULL", "FP8L_ERR_SHAPE", "FP8L_ERR_ALIGN", "FP8L_ERR_ALIAS", "FP8L_ERR_DEVICE",
    "FP8L_ERR_LAUNCH", "FP8L_ERR_MEMORY", "FP8L_ERR_SCRATCH",
]
