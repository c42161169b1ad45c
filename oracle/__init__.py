"""CPU oracle of the MoE FFN layer (float64).  TEST INFRASTRUCTURE ONLY:
imported by tests, the smoke check and the benchmark's CPU-baseline leg,
never by the product path."""
from .moe import (AS_ROUTED, E4M3_MAX, ROUTE_SIGMOID_BIAS, ROUTE_SOFTMAX, Route, combine_weights,
                  dense_masked, expert_h, forward_by_expert,
                  dequant_fp8, dequant_mxfp4, e8m0_value, forward, forward_given_route,
                  fp4_e2m1_value, fp8_e4m3_value,
                  dequant_mxfp8, layer_flops, quant_dequant_e4m3, quant_dequant_mxfp8,
                  quant_e4m3, quant_mxfp8, round_bf16, route,
                  route_from_logits, router_logits, sigmoid, silu,
                  softmax_rows, swiglu_expert, topk_desc)

__all__ = [
    "AS_ROUTED", "E4M3_MAX", "ROUTE_SIGMOID_BIAS", "ROUTE_SOFTMAX", "Route", "combine_weights",
    "dense_masked", "dequant_fp8", "expert_h", "forward_by_expert",
    "dequant_mxfp4", "e8m0_value", "fp4_e2m1_value",
    "forward", "forward_given_route", "fp8_e4m3_value", "layer_flops", "quant_dequant_e4m3",
    "quant_e4m3", "route", "route_from_logits", "dequant_mxfp8", "quant_dequant_mxfp8",
    "quant_mxfp8", "round_bf16",
    "router_logits", "sigmoid", "silu", "softmax_rows", "swiglu_expert", "topk_desc",
]
