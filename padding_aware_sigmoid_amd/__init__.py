"""Padding-aware, non-causal sigmoid attention for AMD Instinct MI355X (gfx950),
and softmax attention with the same padding design.

The compute lives in libsigattn.so: hand-written HIP kernels behind the C ABI
in include/sigattn.h. This package is its Python binding.
"""

from ._lib import (  # noqa: F401
    BF16,
    BIAS_CONSTANT,
    BIAS_NEG_LOG_NK,
    FP32,
    KERNEL_DKDV,
    KERNEL_DQ,
    KERNEL_FWD,
    LAYOUT_PACKED,
    LAYOUT_PADDED,
    NOALLOC_ROWS,
    SigattnError,
    lib_path,
    load,
    version,
)
from .ops import (  # noqa: F401
    SigmoidAttention,
    SigmoidAttentionVarlen,
    SoftmaxAttention,
    sigattn_bwd,
    sigattn_bwd_dk,
    sigattn_bwd_dkdv,
    sigattn_bwd_dq,
    sigattn_bwd_dv,
    sigattn_bwd_varlen,
    sigattn_fwd,
    sigattn_fwd_fp8,
    sigattn_fwd_varlen,
    sigattn_quantize_fp8,
    sigattn_softmax_bwd,
    sigattn_softmax_bwd_noalloc,
    sigattn_softmax_fwd,
    sigattn_tile_config,
    sigmoid_attention,
    sigmoid_attention_varlen,
    softmax_attention,
)
from .accounting import attention_flops  # noqa: F401
