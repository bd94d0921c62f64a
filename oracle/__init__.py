"""CPU oracle for block-scaled FP4 quantization -- test infrastructure only.

This package wraps ``fp4_oracle.c`` (plain scalar C, fp64 internally) with
numpy.  Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import it; the GPU library never does, and the two share no
code.  See the header of ``fp4_oracle.c`` for the pages each function follows.
"""
from .oracle import (  # noqa: F401
    build, build_sanitized, load, e2m1_value, e8m0_value, e4m3_value, e4m3_encode, e2m1_round,
    int4_round, mx_exponent, philox4x32_10, sr_draw, rht_sign_negative, quantize_mx,
    quantize_nv, tensor_amax, fwht, silu_mul, mx_gemm, dequantize, MX, NV, IF4, F32, BF16,
)
