"""CPU oracle for the LLM.int8() linear layer (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU baseline leg import
this package. The product path (the HIP library and its binding) never does.
"""
from .oracle import (  # noqa: F401
    half_to_float,
    quantize_colwise,
    find_outliers,
    quantize_rowwise,
    gemm_i8,
    merge,
    merge_int8w,
    add_bias,
    quantize_tensorwise,
    linear_tensorwise,
    linear,
    linear_rows,
    e4m3_encode,
    e4m3_value,
    quantize_colwise_fp8,
    quantize_rowwise_fp8,
    gemm_fp8,
    merge_fp8,
    linear_fp8,
)
