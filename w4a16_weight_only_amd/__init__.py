"""MI355X-native fused AWQ W4A16 linear: y = x . dequant(W) + bias.

The compute lives in libawq_w4a16.so (hand-written HIP for gfx950, C ABI in
include/awq_w4a16.h).  This package only marshals torch tensors into that ABI.
"""
from ._lib import (  # noqa: F401
    AWQ_OK, AWQ_ERR_NULL, AWQ_ERR_SHAPE, AWQ_ERR_GROUP, AWQ_ERR_ALIGN, AWQ_ERR_UNSUPPORTED,
    AWQ_ERR_HIP, AwqError, LIB_PATH, load as load_library, status_string,
)
from .linear import (  # noqa: F401
    AwqLinear, awq_dequant, awq_gemm, awq_moe_align, awq_moe_gemm, awq_quantize_rtn, group_size_from_config, plan, validate,
)
