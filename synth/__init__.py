"""Seeded synthetic inputs (shapes and distributions only; no MoE arithmetic)."""
from .inputs import (CONFIGS, HY3_SCALE, ROUTE_SIGMOID_BIAS, ROUTE_SOFTMAX,
                     ROUTER_SWEEP_M, MoEConfig, MoEInputs, bf16_bits_to_f32,
                     bf16_bits_to_f64, f32_to_bf16_bits, make_inputs,
                     random_small, to_f64)

__all__ = [
    "CONFIGS", "HY3_SCALE", "ROUTE_SIGMOID_BIAS", "ROUTE_SOFTMAX", "ROUTER_SWEEP_M",
    "MoEConfig", "MoEInputs", "bf16_bits_to_f32", "bf16_bits_to_f64",
    "f32_to_bf16_bits", "make_inputs", "random_small", "to_f64",
]
