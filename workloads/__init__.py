"""Seeded synthetic workloads for the sparse MoE layer forward pass.

This package only produces inputs (shapes, distributions, stored dtypes).  It
is shared by the oracle tests and the GPU path and contains none of the
layer's arithmetic.
"""
from .configs import (CANONICAL, CONFIGS, DEEPSEEK, MIXTRAL, P1_GELU, STRESS,
                      SWITCH, SWITCH_DROP, SWITCH_GELU, TINY, MoEConfig,
                      get_config, shrink)
from .encode import (bf16_bits_to_f32, e4m3_scales, f32_to_bf16_bits,
                     f32_to_e4m3, quantize_rows_e4m3)
from .gen import (gen_expert, gen_experts, gen_noisy_gate, gen_router, gen_x,
                  generate)

__all__ = [
    "CANONICAL", "CONFIGS", "DEEPSEEK", "MIXTRAL", "P1_GELU", "STRESS", "SWITCH",
    "SWITCH_DROP", "SWITCH_GELU", "TINY", "MoEConfig", "get_config", "shrink",
    "bf16_bits_to_f32", "e4m3_scales", "f32_to_bf16_bits", "f32_to_e4m3",
    "quantize_rows_e4m3", "gen_expert", "gen_experts", "gen_noisy_gate",
    "gen_router", "gen_x",
    "generate",
]
