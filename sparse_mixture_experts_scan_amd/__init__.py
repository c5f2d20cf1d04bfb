"""MI355X-native sparse Mixture-of-Experts feed-forward layer (forward pass).

The layer runs in hand-written HIP kernels for gfx950 behind a C ABI
(include/moe_ffn.h, built into libmoe_ffn.so); this package holds the
kernels' sources, the build step, the ctypes binding and the seeded workload
generator."""
from .binding import (EXPORTED, MOE_BF16, MOE_F32, MOE_W4A16, MoeError,  # noqa: F401
                      MoeOpts, MoeWsLayout, backward, forward, forward_int4, lib,
                      moe_block_forward, moe_block_workspace_layout, moe_block_workspace_size,
                      moe_ffn_backward, moe_ffn_backward_workspace_size, moe_ffn_forward,
                      moe_ffn_forward_noalloc, moe_ffn_forward_int4, moe_ffn_workspace_layout,
                      moe_ffn_workspace_size, moe_last_error, moe_opts_init,
                      moe_quantize_int4, moe_release, moe_status_string, moe_version,
                      quantize_int4)
