"""fp64 CPU oracle of the MoE layer forward.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
bench's CPU-baseline leg, never by the product path.
"""
from .moe_oracle import (  # noqa: F401
    GATINGS, boundary_near_tie, combine, dense_bruteforce, dispatch, expert_capacity,
    expert_ffn, expert_ffn_block, forward, forward_tokens, gate_weights, gather_rows,
    gelu_tanh, route, router_logits, topk_ids,
)
