"""MI355X-native Hy3-style sparse MoE FFN layer: HIP kernels behind a C ABI
(include/hy3moe.h) and this thin ctypes binding."""
from .binding import (EXPORTED_SYMBOLS, HY3MOE_BF16, HY3MOE_F32,
                      HY3MOE_N_STAGES, HY3MOE_ROUTE_SIGMOID_BIAS, HY3MOE_ROUTE_SOFTMAX,
                      STAGE_NAMES, HY3MOE_ERR_SCRATCH, hy3moe_forward_static,
                      hy3moe_route_planes, router_split,
                      hy3moe_forward_timed,
                      HY3MOE_ROUTER_FP32, HY3MOE_ROUTER_SPLIT2_BF16, Hy3MoEError,
                      alloc_workspace, forward, hy3moe_config, hy3moe_forward,
                      hy3moe_quantize_e4m3, hy3moe_route, hy3moe_weights,
                      hy3moe_workspace_bytes,
                      hy3moe_workspace_layout, hy3moe_ws_layout, load, make_config,
                      route, strerror)
from .binding import ATTN_EXPORTED_SYMBOLS, ATTN_TILE, AttnPlan, attn_decode, attn_plan

__all__ = [
    "EXPORTED_SYMBOLS", "HY3MOE_BF16", "HY3MOE_F32", "HY3MOE_N_STAGES", "STAGE_NAMES",
    "hy3moe_forward_timed", "HY3MOE_ERR_SCRATCH", "hy3moe_forward_static",
    "hy3moe_route_planes", "router_split",
    "HY3MOE_ROUTE_SIGMOID_BIAS",
    "HY3MOE_ROUTE_SOFTMAX", "HY3MOE_ROUTER_FP32", "HY3MOE_ROUTER_SPLIT2_BF16",
    "Hy3MoEError", "alloc_workspace", "forward", "hy3moe_config", "hy3moe_forward",
    "hy3moe_quantize_e4m3", "hy3moe_route", "hy3moe_weights", "hy3moe_workspace_bytes", "hy3moe_workspace_layout",
    "hy3moe_ws_layout", "load", "make_config", "route", "strerror",
    "ATTN_EXPORTED_SYMBOLS", "ATTN_TILE", "AttnPlan", "attn_decode", "attn_plan",
]
