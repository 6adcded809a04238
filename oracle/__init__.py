"""CPU float64 oracle for the GQE prefill layer -- test infrastructure only.

Importable by the tests, the smoke check and the benchmark's CPU-baseline leg;
never by the product path.
"""
from .gqe_oracle import (OUTPUT_MODES, ablation_slots, attention_backward,  # noqa: F401
                         attention_flops, causal_attention, dispatch, expert_head, gqa_backward, gqa_decode_step,
                         gqa_forward, gqe_backward, gqe_decode_step, gqe_forward,
                         gqe_backward_group_k, gqe_decode_step_group_k, gqe_forward_group_k,
                         group_offsets, load_balance_loss_group_k,
                         route_group_k, dispatch_group_k,
                         group_softmax, kv_project, load_balance_loss, output_projection, renormalize, route,
                         router_logits, slot_vector, slot_width, softmax_backward, topk_in_group,
                         weighted_slot)
