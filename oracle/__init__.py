"""fp64 CPU oracle of the sparse MoE layer: test infrastructure only (see
moe_oracle's header for who may use it)."""
from .moe_oracle import (balance_stats, expert_hidden, expert_param_count,  # noqa: F401
                         moe_forward,
                         router_logits, routing_gaps, select_topk, silu,
                         swiglu_expert, to_f64, topk_gates)
