"""CPU oracle for the MoE layer forward -- test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  It shares no code with the GPU library.
"""
from .moe_oracle import (aux_loss, capacity_from_factor, dispatch, expert_ffn, gelu,  # noqa: F401
                         moe_forward, router_logits, router_z_loss, selection_scores,
                         topk_select, topk_softmax)
