"""MI355X-native ConvRot / ConvLinear4bit (rotated W4A4 linear) for gfx950.

The compute path is libconvrot.so (hand-written HIP kernels behind a C ABI, declared in
include/convrot.h); this package is its thin Python binding plus the ConvLinear4bit module.
"""
from ._lib import (  # noqa: F401
    CONVROT_BF16, CONVROT_F32, CONVROT_MAX_KP, ConvRotError, LIB_PATH, SIGNATURES,
    convrot_is_power_of_4, convrot_make_rht, convrot_padded_k, convrot_quant_weight,
    convrot_rotate_quant_act, convrot_status_string, convrot_version, convrot_w4a4_gemm,
    convrot_w4a4_linear, convrot_w4a4_workspace_bytes, load_library,
    convrot_quant_weight_i8, convrot_rotate_quant_act_i8, convrot_w8a8_gemm,
    convrot_w8a8_linear, convrot_w8a8_workspace_bytes,
    convrot_rotate_quant_act_mxfp4, convrot_quant_weight_mxfp4, convrot_mxfp4_gemm,
    convrot_mxfp4_workspace_bytes, convrot_mxfp4_linear, mx_scale_stride,
    convrot_w4a4_linear_noalloc, CONVROT_NOALLOC_SCRATCH_BYTES, convrot_w4a4_linear_fused,
    convrot_quant_rows_int4, convrot_dequant_int4,
)
from .linear import ConvLinear4bit, ConvLinear8bit, ConvLinearFP4  # noqa: F401

__all__ = [
    "ConvLinear4bit", "ConvLinear8bit", "ConvLinearFP4", "ConvRotError", "load_library", "convrot_status_string", "convrot_version",
    "convrot_padded_k", "convrot_is_power_of_4", "convrot_make_rht", "convrot_rotate_quant_act",
    "convrot_quant_weight", "convrot_w4a4_gemm", "convrot_w4a4_workspace_bytes",
    "convrot_w4a4_linear", "convrot_rotate_quant_act_i8", "convrot_quant_weight_i8",
    "convrot_w8a8_gemm", "convrot_w8a8_workspace_bytes", "convrot_w8a8_linear",
    "convrot_rotate_quant_act_mxfp4", "convrot_quant_weight_mxfp4", "convrot_mxfp4_gemm",
    "convrot_mxfp4_workspace_bytes", "convrot_mxfp4_linear", "convrot_w4a4_linear_noalloc",
    "convrot_w4a4_linear_fused", "convrot_quant_rows_int4", "convrot_dequant_int4",
]
