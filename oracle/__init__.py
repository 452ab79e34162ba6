"""CPU oracle of the MoE layer hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product (the HIP library and its
Python binding in ``mixture_experts_layer_amd``) never does, and the two share
no code. Everything here is float64 NumPy with explicit float32/bfloat16/e4m3
rounding at the points where the GPU path stores narrower types.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (SOFTMAX_PRE_RENORM, SOFTMAX_POST, SIGMOID, SQRTSOFTPLUS,  # noqa: F401
                         SOFTMAX_PRE, SOFTMAX_KINDS, aux_scores, aux_loss, aux_loss_backward,
                         E4M3_MAX,
                         bf16_bits_to_f64, f32_to_bf16_bits, as_values, to_f32, to_bf16,
                         e4m3_decode, e4m3_encode, topk_select, topk_probs, router_topk,
                         dispatch_meta, permute, quantize_rows_e4m3, quantize_cols_e4m3,
                         silu, grouped_gemm, swiglu_from_gu, expert_mlp, dense_mlp, combine,
                         moe_forward, swiglu_backward, grouped_gemm_dw, moe_backward,
                         gate_logits, router_backward, prob_grad, softplus, score_values,
                         selection_keys, topk_select_ext, pack_routing_map, expert_bias_update,
                         PLACE_COMBINE, PLACE_INPUT, PLACE_ACTIVATION, row_weights, dispatch_meta_padded,
                         MX_BLOCK, quantize_mx_e4m3, mx_decode, grouped_gemm_mx, expert_mlp_mx,
                         MX_COL_ALIGN, mx_col_offsets, quantize_mx_cols,
                         grouped_gemm_mx_wgrad, expert_mlp_mx_backward)
