"""HIP graph capture of the entry points with caller-owned workspaces: the
captured forward (bf16 and INT4) and backward replay to the eager results,
bit for bit, several times, with other eager work and synchronisations in
between (each replay starts from cleared outputs)."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import sparse_mixture_experts_scan_amd as moe  # noqa: E402
from sparse_mixture_experts_scan_amd.inputs import MoEConfig, make_dout, make_inputs  # noqa: E402
from tests import gpu_harness as H  # noqa: E402

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[gpu-graph] {msg}", file=sys.stderr, flush=True)


def capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("cfg", [MoEConfig("graph_stream", 48, 256, 512, 8, 2, "bf16"),
                                 # one router block: the select pass runs the scan
                                 MoEConfig("graph_decode", 16, 512, 1024, 8, 2, "bf16"),
                                 MoEConfig("graph_tile", 1000, 256, 384, 8, 2, "bf16"),
                                 # top-4: the tiled form reads the tokens in place
                                 MoEConfig("graph_tile_k4", 600, 256, 256, 8, 4, "bf16")],
                         ids=lambda c: c.name)
def test_forward_graph_replays(cfg):
    announce(f"case {cfg.name}")
    d = H.upload(make_inputs(cfg, seed=31))
    T, k, E = cfg.T, cfg.k, cfg.E
    ws = torch.empty(moe.moe_ffn_workspace_size(T, cfg.d_model, cfg.d_ff, E, k),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(d["x"])
    cnt = torch.empty((E,), dtype=torch.int32, device="cuda")

    def fwd():
        moe.forward(d["x"], d["W_router"], d["W_gate"], d["W_up"], d["W_down"], k,
                    bias=d["bias"], out=out, workspace=ws, expert_counts=cnt)

    fwd()
    torch.cuda.synchronize()
    ref, ref_cnt = out.clone(), cnt.clone()
    g = capture(fwd)
    for rep in range(3):
        out.zero_()
        cnt.zero_()
        junk = torch.randn(256, 256, device="cuda") @ torch.randn(256, 256, device="cuda")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), rep
        assert torch.equal(cnt, ref_cnt), rep
        del junk


def test_int4_forward_graph_replays():
    cfg = MoEConfig("graph_int4", 16, 256, 512, 8, 2, "bf16")
    d = H.upload(make_inputs(cfg, seed=32))
    q = {n: moe.quantize_int4(d[n], 128) for n in ("W_gate", "W_up", "W_down")}
    ws = torch.empty(moe.moe_ffn_workspace_size(cfg.T, cfg.d_model, cfg.d_ff, cfg.E, cfg.k,
                                                moe.MOE_W4A16), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(d["x"])

    def fwd():
        moe.forward_int4(d["x"], d["W_router"], q["W_gate"], q["W_up"], q["W_down"], 128, cfg.k,
                         out=out, workspace=ws)

    fwd()
    torch.cuda.synchronize()
    ref = out.clone()
    g = capture(fwd)
    for rep in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), rep


def test_backward_graph_replays():
    cfg = MoEConfig("graph_bwd", 96, 256, 256, 8, 2, "bf16")
    inp = make_inputs(cfg, seed=33)
    d = H.upload(inp)
    dout = H.dev_tensor(make_dout(cfg, seed=33))
    ws = torch.empty(moe.moe_ffn_backward_workspace_size(cfg.T, cfg.d_model, cfg.d_ff, cfg.E,
                                                         cfg.k), dtype=torch.uint8, device="cuda")
    res = {}

    def bwd():
        res["g"] = moe.backward(d["x"], d["W_router"], d["W_gate"], d["W_up"], d["W_down"], dout,
                                cfg.k, alpha=0.02, workspace=ws)

    bwd()
    torch.cuda.synchronize()
    ref = {n: t.clone() for n, t in res["g"].items()}
    g = capture(bwd)
    outs = res["g"]                       # tensors owned by the graph's pool
    for rep in range(3):
        for t in outs.values():
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, t in outs.items():
            assert torch.equal(t, ref[n]), (rep, n)
