"""The normalised MoE sub-block out = x + layer(RMSNorm(x)) through the C ABI
(moe_block_forward) against the fp64 oracle's block_forward, and the empty
batch (T = 0).

"Mistral/Mixtralのアーキテクチャ", section "Mixtralのアーキテクチャ": each
block's second half is RMSNorm, the MoE layer, then a residual connection.
Bars: 1/rms per token within 1e-5 relative; the normalised tokens the
experts read within one rounding of the element type (bf16: 2^-8 relative,
fp32: 1e-5); routing exact away from near ties (scores of the normalised
tokens); out within the layer's value tolerance; W_down = 0 gives out == x
bit for bit (the layer adds an exact zero)."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import sparse_mixture_experts_scan_amd as moe  # noqa: E402
from sparse_mixture_experts_scan_amd.inputs import MoEConfig, make_block_inputs  # noqa: E402
from tests import gpu_harness as H  # noqa: E402

pytestmark = pytest.mark.gpu

EPS = 1e-5
CASES = [
    MoEConfig("block_stream_bf16", 300, 256, 512, 8, 2, "bf16"),
    MoEConfig("block_f32", 100, 256, 256, 8, 2, "f32"),
    MoEConfig("block_tile_bf16", 1000, 512, 384, 8, 2, "bf16"),      # LDS-tiled GEMMs
    MoEConfig("block_tile_k4", 800, 256, 256, 8, 4, "bf16"),         # tiled, tokens read in place
    MoEConfig("block_split_router", 40, 2048, 256, 16, 4, "bf16"),   # router split over d
    MoEConfig("block_single", 1, 128, 128, 4, 2, "bf16"),
]


def announce(msg):
    print(f"[gpu-block] {msg}", file=sys.stderr, flush=True)


def run_block(cfg, inp, eps=EPS):
    announce(f"case {cfg.name} T={cfg.T} d={cfg.d_model} f={cfg.d_ff} E={cfg.E} k={cfg.k} "
             f"{cfg.dtype}")
    return H.run_gpu(cfg, H.upload(inp), block_eps=eps)


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_block_parity(cfg):
    inp = make_block_inputs(cfg, seed=3)
    res = run_block(cfg, inp)
    # RMSNorm: per-token 1/rms and the normalised tokens handed to the experts
    xf = H.as_f32(inp["x"]).astype(np.float64)
    rs_ref = 1.0 / np.sqrt((xf * xf).mean(axis=1) + EPS)
    np.testing.assert_allclose(res["norm_rs"], rs_ref, rtol=1e-5)
    xn_ref = oracle.rms_norm(inp["x"], inp["norm_weight"], EPS)
    xn_gpu = H.as_f32(res["xn"]).astype(np.float64)
    tol = 2.0 ** -8 * 1.001 if cfg.dtype == "bf16" else 1e-5
    assert (np.abs(xn_gpu - xn_ref) <= tol * np.abs(xn_ref) + 1e-30).all()
    # routing on the normalised tokens
    s = oracle.router_logits(xn_ref, inp["W_router"], inp["bias"])
    idx = oracle.select_topk(s, cfg.k)
    gap, order_gap = oracle.routing_gaps(s, cfg.k)
    rinfo = H.check_routing(cfg, dict(idx=idx, gates=oracle.topk_gates(s, idx), gap=gap,
                                      order_gap=order_gap), res)
    H.check_permutation(cfg, inp, res)
    # values, routed as the GPU routed them
    r = oracle.block_forward(inp["x"], inp["norm_weight"], EPS, inp["W_router"], inp["W_gate"],
                             inp["W_up"], inp["W_down"], cfg.k, bias=inp["bias"],
                             forced_idx=res["idx"].astype(np.int64))
    got = H.as_f32(res["out"]).astype(np.float64)
    err = np.abs(got - r["out"]).max() / np.abs(r["out"]).max()
    assert err <= H.TOL[cfg.dtype], err
    part = check_moe_part(cfg, got, xf, r["moe_out"])
    announce(f"  ok: out err {err:.2e}, moe part {part:.2e}, "
             f"near_ties={rinfo['near_ties']}")


def test_block_zero_down_is_identity():
    cfg = MoEConfig("block_identity", 257, 256, 256, 8, 2, "bf16")
    inp = make_block_inputs(cfg, seed=4)
    inp["W_down"] = np.zeros_like(inp["W_down"])
    res = run_block(cfg, inp)
    np.testing.assert_array_equal(res["out"], inp["x"])


def test_block_eps_dominates_tiny_tokens():
    # a zero token normalises to zero (eps keeps it finite) and its output is
    # the layer applied to zeros: SiLU(0) * 0 = 0, so out == x == 0
    cfg = MoEConfig("block_zero_rows", 64, 128, 256, 8, 2, "f32")
    inp = make_block_inputs(cfg, seed=5)
    inp["x"][::7] = 0.0
    res = run_block(cfg, inp, eps=1e-3)
    assert np.isfinite(res["out"]).all()
    assert (res["out"][::7] == 0).all()
    np.testing.assert_allclose(res["norm_rs"][::7], 1.0 / np.sqrt(1e-3), rtol=1e-6)


@pytest.mark.parametrize("block", [False, True], ids=["layer", "block"])
def test_empty_batch_clears_statistics(block):
    E, k, d, f = 8, 2, 256, 256
    x = torch.empty((0, d), dtype=torch.bfloat16, device="cuda")
    Wr = torch.zeros((d, E), dtype=torch.float32, device="cuda")
    Wg = torch.zeros((E, f, d), dtype=torch.bfloat16, device="cuda")
    Wd = torch.zeros((E, d, f), dtype=torch.bfloat16, device="cuda")
    cnt = torch.full((E,), -3, dtype=torch.int32, device="cuda")
    probs = torch.full((E,), -3.0, dtype=torch.float32, device="cuda")
    loss = torch.full((1,), -3.0, dtype=torch.float32, device="cuda")
    nw = torch.ones(d, dtype=torch.float32, device="cuda") if block else None
    out = moe.forward(x, Wr, Wg, Wg, Wd, k, expert_counts=cnt, router_probs=probs,
                      balance_loss=loss, norm_weight=nw)
    torch.cuda.synchronize()
    assert out.shape == (0, d)
    assert (cnt.cpu() == 0).all() and (probs.cpu() == 0).all() and float(loss.cpu()[0]) == 0.0


def check_moe_part(cfg, got, x_rows, moe_ref):
    """The MoE part alone, per token: (out - x) against the oracle's
    moe_out, allowing the one rounding of out.  Relative to each token's own
    max|moe_out| (out itself is dominated by the residual x, whose rows are
    scaled up to 2^3 by the block input recipe)."""
    ulp = 2.0 ** -8 if cfg.dtype == "bf16" else 2.0 ** -23
    moe_err = np.abs((got - x_rows) - moe_ref) - ulp * np.abs(got)
    rel = moe_err.max(axis=1) / np.abs(moe_ref).max(axis=1)
    assert rel.max() <= H.TOL[cfg.dtype], rel.max()
    return float(rel.max())


def test_block_prefill_sampled():
    # the normalised block at the full prefill shape: every token's routing,
    # and the output of a tile-stratified token sample (a row of every
    # (expert, token tile) pair of the grouped GEMMs)
    from sparse_mixture_experts_scan_amd.inputs import CONFIGS
    cfg = CONFIGS["prefill"]
    inp = make_block_inputs(cfg, seed=0)
    res = run_block(cfg, inp)
    xn_ref = oracle.rms_norm(inp["x"], inp["norm_weight"], EPS)
    s = oracle.router_logits(xn_ref, inp["W_router"], inp["bias"])
    gap, order_gap = oracle.routing_gaps(s, cfg.k)
    idx = oracle.select_topk(s, cfg.k)
    H.check_routing(cfg, dict(idx=idx, gates=oracle.topk_gates(s, idx), gap=gap,
                              order_gap=order_gap), res)
    H.check_permutation(cfg, inp, res)
    toks = H.tile_tokens(res, per_tile=1, seed=0)
    r = oracle.block_forward(inp["x"], inp["norm_weight"], EPS, inp["W_router"], inp["W_gate"],
                             inp["W_up"], inp["W_down"], cfg.k, bias=inp["bias"], tokens=toks,
                             forced_idx=res["idx"].astype(np.int64))
    got = H.as_f32(res["out"][toks]).astype(np.float64)
    err = np.abs(got - r["out"]).max() / np.abs(r["out"]).max()
    assert err <= H.TOL["bf16"], err
    xf = H.as_f32(inp["x"][toks]).astype(np.float64)
    part = check_moe_part(cfg, got, xf, r["moe_out"])
    announce(f"  prefill block ok: out err {err:.2e}, moe part {part:.2e} over {toks.size} tokens")
