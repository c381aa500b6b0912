"""CPU oracle of the fine-grained MoE layer (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package; the product path never does.
"""
from .moe_oracle import (LayerSpec, SOFTMAX, SIGMOID, LOWRANK_GRADS, round_bf16, silu,  # noqa: F401
                         sigmoid,
                         router_logits, router_scores, select_topk, token_gates,
                         dispatch, swiglu, lowrank_apply, lowrank_swiglu, Experts,
                         aux_statistic, bias_update, route, layer_forward, layer_forward_batched,
                         dsilu,
                         layer_backward, layer_backward_batched, E4M3_MAX, e4m3_round,
                         fp8_scale_exp, fp8_quantize, swiglu_fp8)
