"""fp64 CPU oracle of the sparse MoE layer -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the HIP library and is never a fallback
for it.
"""
from .moe_oracle import (to_f64, router_logits, softmax_rows, top_k_desc, route, selection_gap,
                         dispatch, Dispatch, silu, gelu, ffn_swiglu, ffn_gelu, expert_apply,
                         aux_loss, bias_step, oracle_route, oracle_layer, RouteResult,
                         GATE_TOPK_SOFTMAX, GATE_SOFTMAX_RENORM, GATE_SWITCH_TOP1,
                         E4M3_MAX, e4m3_value, e4m3_round, quantize_fp8_rows, dequantize_fp8_rows,
                         fp8_expert_weights, silu_grad, gelu_grad, softmax_backward, gate_backward,
                         aux_loss_backward, expert_backward, oracle_layer_backward, oracle_backward_rows,
                         oracle_expert_grad_columns, oracle_shared_grad_columns)
