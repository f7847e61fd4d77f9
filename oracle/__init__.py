"""CPU oracle of the DiT-MoE sparse MoE layer -- test infrastructure only.

Imported by the tests, the smoke check and the benchmark's CPU-baseline leg;
never by the product path.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (balance_stats, balance_grad, decision_scores,
                         expert_mlp, expert_mlp_backward, forward,
                         gelu_tanh_grad, layer_backward, softmax_backward,
                         gate_logits, gelu_tanh, layer_output, permute,
                         race_select, route, routed_output, selection_indicator,
                         shared_output, slot_weights, softmax, topk_select,
                         NEAR_TIE, GELU_A, GELU_C)
