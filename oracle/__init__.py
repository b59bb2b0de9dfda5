"""CPU oracle (float64) for the sparse MoE layer forward pass.

TEST INFRASTRUCTURE ONLY: imported by tests, by the smoke check and by the
CPU-baseline leg of the benchmark, never by the product library.
"""
from .moe_oracle import (E4M3_TABLE, aux_loss, bf16_to_f64, capacity, combine,
                         decode_weights, dense_moe, dispatch, e4m3_to_f64,
                         expert_ffn, experts_packed, forward, gates, gelu,
                         near_tie_mask, noisy_router, noisy_router_logits,
                         permute, router_logits, shared_experts, silu,
                         softmax, softplus, to_f64, topk_select)

__all__ = [
    "E4M3_TABLE", "aux_loss", "bf16_to_f64", "capacity", "combine",
    "decode_weights", "dense_moe", "dispatch", "e4m3_to_f64", "expert_ffn",
    "experts_packed", "forward", "gates", "gelu", "near_tie_mask", "noisy_router",
    "noisy_router_logits", "permute", "router_logits", "shared_experts",
    "silu", "softmax", "softplus", "to_f64", "topk_select",
]
