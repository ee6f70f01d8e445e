"""MI355X (gfx950) fused MoE expert pipeline: count -> permute -> fp8 grouped
GEMM (w13) -> SiLU-and-mul + fp8 requant -> fp8 grouped GEMM (w2) -> unpermute
with topk weight and reduce, chunked over tokens.

The compute lives in libmoe_hip.so (C ABI in include/moe.h); this package is
its ctypes binding plus a small device-resident layer wrapper.
"""
from ._lib import (MOE_ACT_IDENTITY, MOE_ACT_SILU_MUL, MoeError, MoeProblem, load,  # noqa: F401
                   moe_act_quant, moe_count, moe_forward_chunked, moe_forward_workspace_size, moe_forward_workspace_slices,
                   moe_grouped_gemm_fp8, moe_grouped_gemm_tile_rows, moe_max_rows, moe_permute, moe_permute_workspace_size,
                   moe_quant_permute, moe_grouped_gemm_fp8_small, moe_act_quant_partials, moe_unpermute_partials,
                   moe_forward_plan_info, moe_unpermute_weight_reduce, problem)
from .layer import MoeLayer  # noqa: F401
