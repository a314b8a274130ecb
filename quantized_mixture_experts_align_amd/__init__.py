"""MI355X (gfx950) W4A16 mixture-of-experts expert layer.

The computation runs in libmoe_w4a16.so (hand-written HIP, C ABI in include/moe_w4a16.h);
this package only marshals torch tensors into it.  Importing the package does not load the
library; the first call does, and fails loudly if it has not been built.
"""
from . import _lib
from .ops import (align_capacity, choose_block_m, gemm_choose, gemm_occupancy, gemm_config, moe_act, moe_align,
                  moe_combine, moe_norm_weight, moe_w4a16_gemm, moe_w4a16_gemm_act,
                  moe_w4a16_gemm_act_routed, moe_w4a16_prepare, prepared_size,
                  PreparedWeights, moe_fp8_requant, requant_choose, requant_config, moe_permute_cols,
                  moe_w4a16_gemm_combine, combine_counters,
                  moe_w4a16_gemm_combine_noalloc)
from .layer import MoELayer, Workspace

__all__ = [
    "align_capacity", "choose_block_m", "gemm_choose", "gemm_occupancy", "gemm_config", "moe_act", "moe_align",
    "moe_combine", "moe_norm_weight", "moe_w4a16_gemm", "moe_w4a16_gemm_act",
    "moe_w4a16_gemm_act_routed", "moe_w4a16_prepare", "prepared_size",
    "PreparedWeights", "MoELayer", "Workspace", "moe_fp8_requant", "requant_choose",
    "requant_config", "moe_permute_cols", "moe_w4a16_gemm_combine", "combine_counters",
    "moe_w4a16_gemm_combine_noalloc",
]
