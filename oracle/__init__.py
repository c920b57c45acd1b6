"""CPU oracle for the ConvLinear4bit hot path -- test infrastructure only.

Importable from tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg;
never from the product package.
"""
from .convrot_oracle import *  # noqa: F401,F403
from .convrot_oracle import (  # noqa: F401
    INT4_QMAX, INT4_QMIN, base_regular_hadamard, bf16_bits_to_f32, check_group_size,
    convlinear4bit, dequantize, f32_to_bf16_bits, int_gemm, is_power_of_four, log4,
    pack_int4, padded_k, quantize, quantize_weight,
    regular_hadamard, rotate_groups, rotate_quantize, row_scales, to_f32, unpack_int4,
    w4a4_linear_from_codes, zero_pad_columns,
    INT8_QMAX, INT8_QMIN, rotate_quantize_int8, quantize_weight_int8, w8a8_linear_from_codes,
    convlinear8bit,
    MX_BLOCK, E2M1_EMAX, E8M0_BIAS, E2M1_GRID, e2m1_decode, e2m1_encode, mx_block_exponents,
    quantize_mxfp4, mxfp4_values, rotate_quantize_mxfp4, quantize_weight_mxfp4,
    mxfp4_linear_from_codes, convlinear_fp4,
)
