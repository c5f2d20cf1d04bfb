"""moe_ffn_forward_noalloc (the forward that allocates nothing: its
intermediates live in the library's fixed device scratch array) through the
C ABI, against moe_ffn_forward with a caller workspace on the same inputs.
The two run the same kernels, so out, the routing and the expert counts must
agree bit for bit; the reference entry point's output is also held to the
layer's bf16 / fp32 tolerance against the fp64 oracle.  Several calls in a
row, each smaller than or shaped differently from the one before, so a call
that relied on scratch contents left by the previous one would fail."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import sparse_mixture_experts_scan_amd as moe  # noqa: E402
from sparse_mixture_experts_scan_amd.inputs import MoEConfig, make_inputs  # noqa: E402
from tests import gpu_harness as H  # noqa: E402

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[gpu-noalloc] {msg}", file=sys.stderr, flush=True)


def run_pair(cfg, seed):
    announce(f"case {cfg.name} T={cfg.T} d={cfg.d_model} f={cfg.d_ff} E={cfg.E} k={cfg.k} "
             f"{cfg.dtype}")
    inp = make_inputs(cfg, seed)
    d = H.upload(inp)
    T, E, k = cfg.T, cfg.E, cfg.k
    dt = moe.MOE_BF16 if cfg.dtype == "bf16" else moe.MOE_F32
    assert moe.moe_ffn_workspace_size(T, cfg.d_model, cfg.d_ff, E, k, dt) <= (64 << 20)
    res = {}
    for name, noalloc in (("ref", False), ("noalloc", True)):
        ws = (None if noalloc else
              torch.empty(moe.moe_ffn_workspace_size(T, cfg.d_model, cfg.d_ff, E, k, dt),
                          dtype=torch.uint8, device="cuda"))
        idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
        w = torch.full((T, k), -7.0, dtype=torch.float32, device="cuda")
        cnt = torch.full((E,), -7, dtype=torch.int32, device="cuda")
        out = torch.full_like(d["x"], float("nan"))
        moe.forward(d["x"], d["W_router"], d["W_gate"], d["W_up"], d["W_down"], k,
                    bias=d["bias"], out=out, workspace=ws, topk_idx=idx, topk_w=w,
                    expert_counts=cnt, noalloc=noalloc)
        torch.cuda.synchronize()
        res[name] = dict(out=H.to_host(out), idx=idx.cpu().numpy(), w=w.cpu().numpy(),
                         cnt=cnt.cpu().numpy())
    for key in ("out", "idx", "w", "cnt"):
        np.testing.assert_array_equal(res["noalloc"][key], res["ref"][key], err_msg=key)
    return inp, res["ref"]


def test_noalloc_matches_forward_on_calls_in_a_row():
    cases = [
        # LDS-tiled GEMMs (about 250 rows per expert), then weight-streaming
        # ones on a smaller batch, then a smaller one still
        MoEConfig("noalloc_tile", 1000, 256, 384, 8, 2, "bf16"),
        MoEConfig("noalloc_stream", 300, 256, 512, 8, 2, "bf16"),
        MoEConfig("noalloc_small", 40, 256, 512, 8, 2, "bf16"),
        MoEConfig("noalloc_f32", 64, 128, 512, 8, 2, "f32"),
    ]
    for i, cfg in enumerate(cases):
        inp, ref = run_pair(cfg, seed=40 + i)
        toks = np.arange(cfg.T) if cfg.T <= 300 else np.arange(0, cfg.T, 7)
        err = H.check_values(cfg, inp, dict(out=ref["out"], idx=ref["idx"]), toks)
        announce(f"  ok: bitwise equal to moe_ffn_forward; max|err|/max|ref| = {err:.2e}")


def test_noalloc_mixtral_decode_then_single_token():
    # the Mixtral 8x7B layer at decode size, then one token
    for T in (64, 1):
        cfg = MoEConfig("noalloc_mixtral", T, 4096, 14336, 8, 2, "bf16")
        run_pair(cfg, seed=0)
        announce("  ok: bitwise equal to moe_ffn_forward")
