"""CPU oracle for the fused residual-add + RMSNorm + FP8/NVFP4 tail and the
Q/K norm + RoPE + FP8 store.

TEST INFRASTRUCTURE. This package is the plain, slow, obviously-correct
reference the HIP kernels are compared against. Only the tests, the smoke
check and the CPU-baseline leg of the benchmark may import it; the product
path (the C-ABI library and its Python binding) never does, and shares no code
with it. Arithmetic is numpy float32 (one IEEE rounding per operation, as the
method fixes binary32 for the norm) and float64 where exactness is needed
(sums of squares, code-table searches).

Every function is pinned by tests/test_oracle_*.py against something other
than itself: closed-form code tables, torch's own E4M3 and fp16/bf16
conversions, brute-force enumeration on tiny inputs, exact rational
arithmetic, hand-worked rows and invariants.
"""
from .codecs import (E2M1_VALUES, E4M3_MAX, e2m1_decode, e2m1_encode, e4m3_decode,
                     e4m3_encode, t_decode, t_encode)
from .tail import (add_rmsnorm_quant_fp8, add_rmsnorm_quant_nvfp4, exact_sum_to_f32,
                   exp_neg_rn32, gated_rmsnorm_quant_nvfp4, silu_gate,
                   mixed_kv_row_bytes, normalize, nvfp4_global_scale, qk_norm_rope_fp8,
                   qk_norm_rope_fp8_kv_store, qk_norm_rope_kv_store_mixed,
                   quant_fp8, quant_nvfp4,
                   residual_add, rmsnorm_f32, rope_neox, row_scale, sum_of_squares,
                   swizzle_block_scales)

__all__ = [
    "E2M1_VALUES", "E4M3_MAX", "e2m1_decode", "e2m1_encode", "e4m3_decode", "e4m3_encode",
    "t_decode", "t_encode", "add_rmsnorm_quant_fp8", "add_rmsnorm_quant_nvfp4",
    "exact_sum_to_f32", "normalize", "nvfp4_global_scale", "qk_norm_rope_fp8",
    "qk_norm_rope_fp8_kv_store", "qk_norm_rope_kv_store_mixed", "mixed_kv_row_bytes", "quant_fp8",
    "quant_nvfp4", "residual_add", "rmsnorm_f32", "rope_neox", "row_scale", "sum_of_squares",
    "swizzle_block_scales", "exp_neg_rn32", "gated_rmsnorm_quant_nvfp4", "silu_gate",
]
