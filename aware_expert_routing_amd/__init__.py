"""MI355X-native decode MoE layer with Opportunistic Expert Activation routing.

The compute path is libmoe.so (hand-written HIP for gfx950, C ABI in
include/moe.h and include/moe_residency.h); this package is its thin Python
binding plus layer and residency helpers.
"""
from ._lib import (  # noqa: F401
    EXPORTED, HANDLE_BYTES, MOE_ROUTE_OEA, MOE_ROUTE_PRUNED, MOE_ROUTE_TOPK, MOE_DT_BF16, MOE_DT_F32, MOE_W_BF16, MOE_W_F32, MOE_W_INT4_G128,
    ExpertHandle, MoeError, NOALLOC_WORKSPACE_BYTES, dispatch, expert_ffn, expert_ffn_noalloc, expert_ffn_phase_events,
    ffn_workspace_bytes, handle_publish, hotness_ema,
    lib, pack_weights, quantize_int4_g128, stream_read, route_dispatch, route_oea, route_topk, router_logits, router_route_dispatch, status_str,
    MOE_EFULL, MOE_RES_EVICTING, MOE_RES_HI, MOE_RES_LO, MOE_RES_PROMOTING, ResidencyConfig, ResidencyStats,
    budget_create, budget_release, budget_try_reserve, pool_alloc, pool_create, pool_free, residency_create,
    residency_select, residency_stats, residency_step,
)
from .layer import ExpertTensors, MoELayer, capture_layers, k0_schedule  # noqa: F401
from .residency import Residency, ema_hot_set, pinned_hi_version  # noqa: F401
