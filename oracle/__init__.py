"""fp64 CPU oracle of the sparse MoE FFN layer forward.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.
"""
from .moe_ref import (  # noqa: F401
    aux_statistic, bias_update, bias_update_seq, capacity, dispatch,
    expert_choice_dispatch, expert_choice_select, gate_weights, moe_layer_ec,
    group_candidates, moe_layer, router_logits, scores_from_logits,
    router_stats, selection_keys, silu, swiglu_ffn, topk_select,
    MX_BLOCK, E4M3_MAX, e4m3_decode, e4m3_encode, mx_quantize, mx_dequantize,
    mx_round, swiglu_ffn_mx, moe_layer_latent,
)
