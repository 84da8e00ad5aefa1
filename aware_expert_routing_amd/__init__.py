"""MI355X-native decode MoE layer with Opportunistic Expert Activation routing.

The compute path is libmoe.so (hand-written HIP for gfx950, C ABI in
include/moe.h); this package is its thin Python binding plus a layer helper.
"""
from ._lib import (  # noqa: F401
    EXPORTED, HANDLE_BYTES, MOE_ROUTE_OEA, MOE_ROUTE_PRUNED, MOE_ROUTE_TOPK, MOE_DT_BF16, MOE_DT_F32, MOE_W_BF16, MOE_W_F32, MOE_W_INT4_G128,
    ExpertHandle, MoeError, dispatch, expert_ffn, ffn_workspace_bytes, handle_publish, hotness_ema,
    lib, pack_weights, quantize_int4_g128, route_dispatch, route_oea, route_topk, router_logits, status_str,
)
from .layer import ExpertTensors, MoELayer  # noqa: F401
