"""fp64 CPU oracle of the sparse MoE layer: test infrastructure only (see
moe_oracle's header for who may use it)."""
from .moe_oracle import (balance_stats, expert_param_count, moe_forward,  # noqa: F401
                         router_logits, routing_gaps, select_topk, silu,
                         swiglu_expert, to_f64, topk_gates)
