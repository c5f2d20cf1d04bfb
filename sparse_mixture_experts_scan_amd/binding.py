"""ctypes binding of libmoe_ffn.so: the C ABI's entry points under the same
names, plus `forward`, which marshals torch device tensors into one
`moe_ffn_forward` call.  Argument marshalling only: every step of the layer
runs in the library's HIP kernels.  There is no fallback: if the library is
not built, every call raises."""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_ffn.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_BF16, MOE_F32, MOE_W4A16 = 0, 1, 2

EXPORTED = ("moe_opts_init", "moe_ffn_forward", "moe_ffn_forward_noalloc", "moe_block_forward", "moe_quantize_int4",
            "moe_ffn_forward_int4", "moe_ffn_backward", "moe_ffn_backward_workspace_size",
            "moe_ffn_workspace_size", "moe_block_workspace_size",
            "moe_ffn_workspace_layout", "moe_block_workspace_layout", "moe_status_string", "moe_last_error",
            "moe_release", "moe_version")


class MoeOpts(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32),
                ("stream", ctypes.c_void_p),
                ("router_bias", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t),
                ("topk_idx_out", ctypes.c_void_p),
                ("topk_w_out", ctypes.c_void_p),
                ("expert_counts_out", ctypes.c_void_p),
                ("router_prob_out", ctypes.c_void_p),
                ("balance_loss_out", ctypes.c_void_p),
                ("stage_events", ctypes.c_void_p)]

MOE_NUM_STAGES = 6
STAGE_NAMES = ("router", "scan", "scatter", "gateup", "down", "combine")
MOE_BWD_NUM_STAGES = 8
BWD_STAGE_NAMES = ("routing", "recompute", "z", "rows_router", "dxs", "dx", "dw_down",
                   "dw_gate_up")


class MoeWsLayout(ctypes.Structure):
    _fields_ = [("block_rows", ctypes.c_int64),
                ("max_rows", ctypes.c_int64),
                ("router_blocks", ctypes.c_int64),
                ("y_part_rows", ctypes.c_int64),
                ("gemm_variant", ctypes.c_int32),
                ("down_splits", ctypes.c_int32),
                ("tokens_in_place", ctypes.c_int32),
                ("y_weighted", ctypes.c_int32)] + [
        (name, ctypes.c_size_t) for name in
        ("topk_idx", "topk_w", "block_counts", "counts", "offsets", "num_tiles",
         "tile_expert", "row_token", "tok_row", "row_w", "xs", "h", "y", "y_parts",
         "down_sched",
         "block_probs", "norm_rs", "xn",
         "router_partial", "wdeq", "total")]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {moe_status_string(status)} ({status}): {moe_last_error()}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run "
                               "`python -m sparse_mixture_experts_scan_amd.build` first")
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
        L.moe_opts_init.argtypes = [ctypes.POINTER(MoeOpts)]
        L.moe_opts_init.restype = None
        L.moe_ffn_forward.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32,
                                      ctypes.POINTER(MoeOpts)]
        L.moe_ffn_forward.restype = ctypes.c_int
        L.moe_ffn_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32,
                                              ctypes.POINTER(MoeOpts)]
        L.moe_ffn_forward_noalloc.restype = ctypes.c_int
        L.moe_block_forward.argtypes = [vp, vp, ctypes.c_float, vp, vp, vp, vp, vp, i64, i64,
                                        i64, i32, i32, ctypes.POINTER(MoeOpts)]
        L.moe_block_forward.restype = ctypes.c_int
        L.moe_quantize_int4.argtypes = [vp, i32, i64, i64, i64, i32, vp, vp, vp]
        L.moe_quantize_int4.restype = ctypes.c_int
        L.moe_ffn_forward_int4.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, i64, i64,
                                           i64, i32, i32, ctypes.POINTER(MoeOpts)]
        L.moe_ffn_forward_int4.restype = ctypes.c_int
        L.moe_ffn_backward.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, vp,
                                       vp, i64, i64, i64, i32, i32, ctypes.POINTER(MoeOpts)]
        L.moe_ffn_backward.restype = ctypes.c_int
        L.moe_ffn_backward_workspace_size.argtypes = [i64, i64, i64, i32, i32]
        L.moe_ffn_backward_workspace_size.restype = sz
        L.moe_ffn_workspace_size.argtypes = [i64, i64, i64, i32, i32, i32]
        L.moe_ffn_workspace_size.restype = sz
        L.moe_ffn_workspace_layout.argtypes = [i64, i64, i64, i32, i32, i32,
                                               ctypes.POINTER(MoeWsLayout)]
        L.moe_ffn_workspace_layout.restype = ctypes.c_int
        L.moe_block_workspace_size.argtypes = [i64, i64, i64, i32, i32, i32]
        L.moe_block_workspace_size.restype = sz
        L.moe_block_workspace_layout.argtypes = [i64, i64, i64, i32, i32, i32,
                                                 ctypes.POINTER(MoeWsLayout)]
        L.moe_block_workspace_layout.restype = ctypes.c_int
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_release.argtypes = []
        L.moe_release.restype = None
        L.moe_version.argtypes = []
        L.moe_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


# ---------------------------------------------------------------- raw C ABI
def moe_opts_init() -> MoeOpts:
    o = MoeOpts()
    lib().moe_opts_init(ctypes.byref(o))
    return o


def moe_ffn_forward(x, W_router, W_gate, W_up, W_down, out, T, d_model, d_ff, E, k,
                    opts: Optional[MoeOpts] = None) -> int:
    """Raw entry point: integer device addresses, returns the status code."""
    return lib().moe_ffn_forward(x, W_router, W_gate, W_up, W_down, out, T, d_model, d_ff, E,
                                 k, ctypes.byref(opts) if opts is not None else None)


def moe_ffn_forward_noalloc(x, W_router, W_gate, W_up, W_down, out, T, d_model, d_ff, E, k,
                            opts: Optional[MoeOpts] = None) -> int:
    """Raw entry point of the forward that allocates nothing (library scratch)."""
    return lib().moe_ffn_forward_noalloc(x, W_router, W_gate, W_up, W_down, out, T, d_model,
                                         d_ff, E, k,
                                         ctypes.byref(opts) if opts is not None else None)


def moe_block_forward(x, norm_weight, eps, W_router, W_gate, W_up, W_down, out, T, d_model,
                      d_ff, E, k, opts: Optional[MoeOpts] = None) -> int:
    """Raw entry point of the block wrapper out = x + layer(RMSNorm(x))."""
    return lib().moe_block_forward(x, norm_weight, eps, W_router, W_gate, W_up, W_down, out, T,
                                   d_model, d_ff, E, k,
                                   ctypes.byref(opts) if opts is not None else None)


def moe_quantize_int4(W, dtype, batch, N, K, group, packed, scales, stream=None) -> int:
    """Raw entry point of the INT4 quantizer."""
    return lib().moe_quantize_int4(W, dtype, batch, N, K, group, packed, scales, stream)


def moe_ffn_forward_int4(x, W_router, Wg_q, Wg_s, Wu_q, Wu_s, Wd_q, Wd_s, group, out, T,
                         d_model, d_ff, E, k, opts: Optional[MoeOpts] = None) -> int:
    """Raw entry point of the layer with INT4 expert weights."""
    return lib().moe_ffn_forward_int4(x, W_router, Wg_q, Wg_s, Wu_q, Wu_s, Wd_q, Wd_s, group,
                                      out, T, d_model, d_ff, E, k,
                                      ctypes.byref(opts) if opts is not None else None)


def moe_ffn_backward(x, W_router, W_gate, W_up, W_down, dout, alpha, dx, dW_router, dbias,
                     dW_gate, dW_up, dW_down, T, d_model, d_ff, E, k,
                     opts: Optional[MoeOpts] = None) -> int:
    """Raw entry point of the backward pass."""
    return lib().moe_ffn_backward(x, W_router, W_gate, W_up, W_down, dout, alpha, dx, dW_router,
                                  dbias, dW_gate, dW_up, dW_down, T, d_model, d_ff, E, k,
                                  ctypes.byref(opts) if opts is not None else None)


def moe_ffn_backward_workspace_size(T, d_model, d_ff, E, k) -> int:
    return lib().moe_ffn_backward_workspace_size(T, d_model, d_ff, E, k)


def moe_ffn_workspace_size(T, d_model, d_ff, E, k, dtype=MOE_BF16) -> int:
    return lib().moe_ffn_workspace_size(T, d_model, d_ff, E, k, dtype)


def moe_ffn_workspace_layout(T, d_model, d_ff, E, k, dtype=MOE_BF16) -> MoeWsLayout:
    lay = MoeWsLayout()
    st = lib().moe_ffn_workspace_layout(T, d_model, d_ff, E, k, dtype, ctypes.byref(lay))
    if st != MOE_OK:
        raise MoeError(st, "moe_ffn_workspace_layout")
    return lay


def moe_block_workspace_size(T, d_model, d_ff, E, k, dtype=MOE_BF16) -> int:
    return lib().moe_block_workspace_size(T, d_model, d_ff, E, k, dtype)


def moe_block_workspace_layout(T, d_model, d_ff, E, k, dtype=MOE_BF16) -> MoeWsLayout:
    lay = MoeWsLayout()
    st = lib().moe_block_workspace_layout(T, d_model, d_ff, E, k, dtype, ctypes.byref(lay))
    if st != MOE_OK:
        raise MoeError(st, "moe_block_workspace_layout")
    return lay


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def moe_last_error() -> str:
    return lib().moe_last_error().decode()


def moe_release() -> None:
    lib().moe_release()


def moe_version() -> str:
    return lib().moe_version().decode()


# ---------------------------------------------------------------- torch marshalling
def _check(t, shape, dtype, x):
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"tensor {tuple(t.shape)} {t.dtype}: expected {tuple(shape)} {dtype}")
    if not t.is_cuda or not t.is_contiguous() or t.device != x.device:
        raise ValueError("every tensor must be a contiguous device tensor on x's device")


def _opts(x, E, k, dtype, bias, out, workspace, topk_idx, topk_w, expert_counts, stream,
          stage_events, router_probs, balance_loss):
    """Checks the common tensors and fills a MoeOpts; returns (opts, out, keepalive)."""
    import torch

    T, d = x.shape
    if out is None:
        out = torch.empty_like(x)
    checks = [(out, (T, d), x.dtype)]
    if bias is not None:
        checks.append((bias, (E,), torch.float32))
    for t, shape in ((topk_idx, (T, k)), (expert_counts, (E,))):
        if t is not None:
            checks.append((t, shape, torch.int32))
    if topk_w is not None:
        checks.append((topk_w, (T, k), torch.float32))
    if router_probs is not None:
        checks.append((router_probs, (E,), torch.float32))
    if balance_loss is not None:
        checks.append((balance_loss, (1,), torch.float32))
    for t, shape, dt in checks:
        _check(t, shape, dt, x)
    o = moe_opts_init()
    o.dtype = dtype
    st = stream if stream is not None else torch.cuda.current_stream(x.device)
    o.stream = st.cuda_stream
    o.router_bias = bias.data_ptr() if bias is not None else None
    if workspace is not None:
        if workspace.device != x.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on x's device")
        o.workspace = workspace.data_ptr()
        o.workspace_bytes = workspace.numel() * workspace.element_size()
    o.topk_idx_out = topk_idx.data_ptr() if topk_idx is not None else None
    o.topk_w_out = topk_w.data_ptr() if topk_w is not None else None
    o.expert_counts_out = expert_counts.data_ptr() if expert_counts is not None else None
    o.router_prob_out = router_probs.data_ptr() if router_probs is not None else None
    o.balance_loss_out = balance_loss.data_ptr() if balance_loss is not None else None
    arr = None
    if stage_events is not None:
        # MOE_NUM_STAGES + 1 created torch.cuda.Event objects (record() once first)
        if len(stage_events) != MOE_NUM_STAGES + 1:
            raise ValueError("stage_events needs MOE_NUM_STAGES + 1 events")
        arr = (ctypes.c_void_p * len(stage_events))(*[ev.cuda_event for ev in stage_events])
        o.stage_events = ctypes.cast(arr, ctypes.c_void_p)
    return o, out, arr


def forward(x, W_router, W_gate, W_up, W_down, k: int, *, bias=None, out=None,
            workspace=None, topk_idx=None, topk_w=None, expert_counts=None, stream=None,
            stage_events=None, router_probs=None, balance_loss=None, norm_weight=None,
            eps=1e-5, noalloc=False):
    """One moe_ffn_forward call on torch device tensors.

    x [T][d] (bf16 or fp32), W_router [d][E] fp32, W_gate/W_up [E][d_ff][d],
    W_down [E][d][d_ff] (x's dtype), bias [E] fp32 or None.  Optional outputs
    topk_idx [T][k] int32, topk_w [T][k] fp32, expert_counts [E] int32,
    router_probs [E] fp32 (mean full-softmax probability p_i) and
    balance_loss [1] fp32 (N * sum_i f_i p_i) are filled when given.  With
    norm_weight [d] fp32 the call is the block wrapper
    out = x + layer(RMSNorm(x)) (moe_block_forward, with `eps`).  `workspace`
    is a uint8 device tensor (see moe_ffn_workspace_size) or None for the
    library's own.  noalloc: call moe_ffn_forward_noalloc (no workspace, the
    library's fixed scratch; the bare layer only).  Returns out."""
    import torch

    T, d = x.shape
    E = W_router.shape[1]
    d_ff = W_gate.shape[1]
    if x.dtype == torch.bfloat16:
        dtype = MOE_BF16
    elif x.dtype == torch.float32:
        dtype = MOE_F32
    else:
        raise TypeError("x must be bfloat16 or float32")
    _check(x, (T, d), x.dtype, x)
    for t, shape, dt in ((W_router, (d, E), torch.float32), (W_gate, (E, d_ff, d), x.dtype),
                         (W_up, (E, d_ff, d), x.dtype), (W_down, (E, d, d_ff), x.dtype)):
        _check(t, shape, dt, x)
    if norm_weight is not None:
        _check(norm_weight, (d,), torch.float32, x)
    if noalloc and (norm_weight is not None or workspace is not None):
        raise ValueError("noalloc is the bare layer with the library's scratch: "
                         "no norm_weight, no workspace")
    o, out, _keep = _opts(x, E, k, dtype, bias, out, workspace, topk_idx, topk_w,
                          expert_counts, stream, stage_events, router_probs, balance_loss)
    with torch.cuda.device(x.device):
        if norm_weight is not None:
            status = moe_block_forward(x.data_ptr(), norm_weight.data_ptr(), float(eps),
                                       W_router.data_ptr(), W_gate.data_ptr(), W_up.data_ptr(),
                                       W_down.data_ptr(), out.data_ptr(), T, d, d_ff, E, k, o)
        else:
            entry = moe_ffn_forward_noalloc if noalloc else moe_ffn_forward
            status = entry(x.data_ptr(), W_router.data_ptr(), W_gate.data_ptr(),
                           W_up.data_ptr(), W_down.data_ptr(), out.data_ptr(), T, d, d_ff, E, k,
                           o)
    if status != MOE_OK:
        raise MoeError(status, "moe_ffn_forward")
    return out


def quantize_int4(W, group: int = 128, stream=None):
    """INT4 codes and scales of a bf16 or fp32 device tensor [..., N, K]
    (matrices of N rows over K input features) through moe_quantize_int4.
    Returns (packed uint8 [..., N, K/2], scales float32 [..., K/group, N])."""
    import torch

    if W.dtype == torch.bfloat16:
        dtype = MOE_BF16
    elif W.dtype == torch.float32:
        dtype = MOE_F32
    else:
        raise TypeError("W must be bfloat16 or float32")
    if not W.is_cuda or not W.is_contiguous():
        raise ValueError("W must be a contiguous device tensor")
    if W.dim() < 2:
        raise ValueError("W must be [..., N, K]")
    N, K = W.shape[-2], W.shape[-1]
    batch = W.numel() // (N * K)
    packed = torch.empty(W.shape[:-1] + (K // 2,), dtype=torch.uint8, device=W.device)
    scales = torch.empty(W.shape[:-2] + (K // group, N), dtype=torch.float32, device=W.device)
    st = stream if stream is not None else torch.cuda.current_stream(W.device)
    with torch.cuda.device(W.device):
        status = moe_quantize_int4(W.data_ptr(), dtype, batch, N, K, group, packed.data_ptr(),
                                   scales.data_ptr(), st.cuda_stream)
    if status != MOE_OK:
        raise MoeError(status, "moe_quantize_int4")
    return packed, scales


def forward_int4(x, W_router, W_gate, W_up, W_down, group: int, k: int, *, bias=None, out=None,
                 workspace=None, topk_idx=None, topk_w=None, expert_counts=None, stream=None,
                 stage_events=None, router_probs=None, balance_loss=None):
    """One moe_ffn_forward_int4 call.  x [T][d] bf16; W_gate, W_up, W_down are
    (packed, scales) pairs as quantize_int4 returns them for the [E][d_ff][d],
    [E][d_ff][d] and [E][d][d_ff] stacks.  Other arguments as forward."""
    import torch

    T, d = x.shape
    E = W_router.shape[1]
    d_ff = W_gate[0].shape[1]
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    _check(x, (T, d), x.dtype, x)
    _check(W_router, (d, E), torch.float32, x)
    for (q, sc), N, K in ((W_gate, d_ff, d), (W_up, d_ff, d), (W_down, d, d_ff)):
        _check(q, (E, N, K // 2), torch.uint8, x)
        _check(sc, (E, K // group, N), torch.float32, x)
    o, out, _keep = _opts(x, E, k, MOE_W4A16, bias, out, workspace, topk_idx, topk_w,
                          expert_counts, stream, stage_events, router_probs, balance_loss)
    with torch.cuda.device(x.device):
        status = moe_ffn_forward_int4(x.data_ptr(), W_router.data_ptr(), W_gate[0].data_ptr(),
                                      W_gate[1].data_ptr(), W_up[0].data_ptr(),
                                      W_up[1].data_ptr(), W_down[0].data_ptr(),
                                      W_down[1].data_ptr(), group, out.data_ptr(), T, d, d_ff,
                                      E, k, o)
    if status != MOE_OK:
        raise MoeError(status, "moe_ffn_forward_int4")
    return out


def backward(x, W_router, W_gate, W_up, W_down, dout, k: int, *, alpha=0.0, bias=None,
             want_dbias=False, workspace=None, stream=None, stage_events=None):
    """One moe_ffn_backward call on bf16 device tensors.  Returns a dict of
    new tensors: dx [T][d] bf16, dW_router [d][E] fp32, dW_gate, dW_up,
    dW_down (bf16, the stacks' shapes) and, with want_dbias, dbias [E] fp32."""
    import torch

    T, d = x.shape
    E = W_router.shape[1]
    d_ff = W_gate.shape[1]
    if x.dtype != torch.bfloat16:
        raise TypeError("the backward takes bfloat16 tensors")
    for t, shape, dt in ((x, (T, d), torch.bfloat16), (dout, (T, d), torch.bfloat16),
                         (W_router, (d, E), torch.float32),
                         (W_gate, (E, d_ff, d), torch.bfloat16),
                         (W_up, (E, d_ff, d), torch.bfloat16),
                         (W_down, (E, d, d_ff), torch.bfloat16)):
        _check(t, shape, dt, x)
    g = dict(dx=torch.empty_like(x),
             dW_router=torch.empty((d, E), dtype=torch.float32, device=x.device),
             dW_gate=torch.empty_like(W_gate), dW_up=torch.empty_like(W_up),
             dW_down=torch.empty_like(W_down))
    if want_dbias:
        g["dbias"] = torch.empty((E,), dtype=torch.float32, device=x.device)
    o, _, _keep = _opts(x, E, k, MOE_BF16, bias, g["dx"], workspace, None, None, None, stream,
                        None, None, None)
    arr = None
    if stage_events is not None:
        if len(stage_events) != MOE_BWD_NUM_STAGES + 1:
            raise ValueError("stage_events needs MOE_BWD_NUM_STAGES + 1 events")
        arr = (ctypes.c_void_p * len(stage_events))(*[ev.cuda_event for ev in stage_events])
        o.stage_events = ctypes.cast(arr, ctypes.c_void_p)
    with torch.cuda.device(x.device):
        status = moe_ffn_backward(x.data_ptr(), W_router.data_ptr(), W_gate.data_ptr(),
                                  W_up.data_ptr(), W_down.data_ptr(), dout.data_ptr(),
                                  float(alpha), g["dx"].data_ptr(), g["dW_router"].data_ptr(),
                                  g["dbias"].data_ptr() if want_dbias else None,
                                  g["dW_gate"].data_ptr(), g["dW_up"].data_ptr(),
                                  g["dW_down"].data_ptr(), T, d, d_ff, E, k, o)
    if status != MOE_OK:
        raise MoeError(status, "moe_ffn_backward")
    return g
