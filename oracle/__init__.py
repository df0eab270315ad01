"""CPU oracle for 4-bit weight-only dequantize-and-multiply.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package entry's smoke check
and the benchmark's CPU-baseline leg may import this package.  The product path
(the HIP library and its Python binding) never calls it, and this package never
imports the product path: the two share no code, tables or constants.

What it computes, in plain NumPy:
  * bit-field decoders for fp16, bf16, float8_e4m3fn and E2M1;
  * int4 "g128 min/max" dequantization to fp32
    (rumik-oss-1-int4 card, section "Format");
  * NVFP4 weight-only dequantization to fp32
    (VoxCPM2-NVFP4 card, section "What was quantized");
  * BF16 weights to fp32;
  * y = x . W^T with x widened from BF16 and the fp32 weights widened to fp64,
    via an fp64 matrix product;
  * the fused neighbours of the product: RN_bf16 from fp64, the SiLU-gated
    activation h = RN_bf16(silu(g) * u), and the product plus a residual;
  * sampling from the head: top-k, softmax at a temperature, inverse-CDF draw
    with a caller-supplied uniform.

Every function is pinned by tests against values fixed outside this module
(hand-worked examples, closed forms, exhaustive comparison with numpy/torch
conversion routines, exact rational brute force).  No function here is
"parity unpinned".
"""
from .reference import (  # noqa: F401
    unpack_nibbles,
    fp16_value,
    bf16_value,
    e4m3fn_value,
    e2m1_value,
    q4g128_dequant_f32,
    nvfp4g16_dequant_f32,
    bf16_dequant_f32,
    gemv_f64,
    q4g128_gemv,
    nvfp4g16_gemv,
    bf16_gemv,
    bf16_round_bits,
    silu_mul_bf16,
    gemv_residual_f64,
    sample_topk,
    GROUP_Q4,
    GROUP_NVFP4,
)
