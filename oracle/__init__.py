"""fp64 CPU oracle of the MoE layer forward and backward.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
bench's CPU-baseline leg, never by the product path.
"""
from .moe_oracle import (  # noqa: F401
    GATINGS, backward, boundary_near_tie, combine, dense_bruteforce, dispatch,
    expert_block_backward, expert_capacity, expert_ffn, expert_ffn_backward, expert_ffn_block,
    forward, forward_tokens, gate_weights, gate_weights_grad, gather_rows, gelu_tanh,
    gelu_tanh_grad, route, router_logits, topk_ids,
)
