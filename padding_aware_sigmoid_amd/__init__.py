"""Padding-aware, non-causal sigmoid attention for AMD Instinct MI355X (gfx950).

The compute lives in libsigattn.so: hand-written HIP kernels behind the C ABI
in include/sigattn.h. This package is its Python binding.
"""

from ._lib import BF16, FP32, KERNEL_DKDV, KERNEL_DQ, KERNEL_FWD, SigattnError, lib_path, load, version  # noqa: F401
from .ops import (  # noqa: F401
    SigmoidAttention,
    sigattn_bwd,
    sigattn_bwd_dk,
    sigattn_bwd_dkdv,
    sigattn_bwd_dq,
    sigattn_bwd_dv,
    sigattn_fwd,
    sigattn_tile_config,
    sigmoid_attention,
)
from .accounting import attention_flops  # noqa: F401
