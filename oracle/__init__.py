"""CPU oracle for the fused AWQ W4A16 linear (test infrastructure only).

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The HIP library and its Python binding never do.
"""
from .awq_ref import (  # noqa: F401
    AWQ_ORDER, AWQ_REVERSE, AwqFormatError, resolve_groups, validate_pack,
    pack_awq, unpack_awq, unpack_awq_gather, dequant_ref, dequant_ref_T,
    gemm_ref, gemm_ref_entries, fp16_rne, quantize_rtn,
    bf16_to_f64, f32_to_bf16_rne, gemm_ref_bf16, moe_align_ref, moe_gemm_ref,
)
