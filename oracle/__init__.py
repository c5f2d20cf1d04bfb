"""fp64 CPU oracle of the sparse MoE layer: test infrastructure only (see
moe_oracle's header for who may use it)."""
from .moe_oracle import (balance_stats, block_forward, dequantize_int4,  # noqa: F401
                         expert_hidden, expert_param_count, moe_forward,
                         moe_backward, moe_backward_entries, moe_forward_int4, quantize_int4, rms_norm,
                         silu_grad,
                         router_logits, routing_gaps, select_topk, silu,
                         swiglu_expert, to_f64, topk_gates)
