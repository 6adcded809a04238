"""CPU float64 oracle for the GQE prefill layer -- test infrastructure only.

Importable by the tests, the smoke check and the benchmark's CPU-baseline leg;
never by the product path.
"""
from .gqe_oracle import (attention_flops, causal_attention, dispatch, expert_head,  # noqa: F401
                         gqa_forward, gqe_forward, group_softmax, kv_project,
                         output_projection, renormalize, route, router_logits, slot_vector,
                         topk_in_group, weighted_slot)
