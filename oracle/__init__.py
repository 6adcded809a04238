"""CPU float64 oracle for the GQE prefill layer -- test infrastructure only.

Importable by the tests, the smoke check and the benchmark's CPU-baseline leg;
never by the product path.
"""
from .gqe_oracle import (OUTPUT_MODES, ablation_slots, attention_flops,  # noqa: F401
                         causal_attention, dispatch, expert_head, gqa_decode_step,
                         gqa_forward, gqe_decode_step, gqe_forward,
                         group_softmax, kv_project, output_projection, renormalize, route,
                         router_logits, slot_vector, slot_width, topk_in_group, weighted_slot)
