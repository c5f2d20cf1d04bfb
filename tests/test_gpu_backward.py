"""Backward pass of the layer on the GPU (moe_ffn_backward through the C ABI)
against the fp64 oracle's moe_backward.

"Mistral/Mixtralのアーキテクチャ", section "ロードバランス損失": the gradients
of <dOut, MoE(x)> + alpha * N * sum f_i p_i.  Routing: the GPU forward's
indices (the backward recomputes the same routing with the same kernels),
exact away from near ties, handed to the oracle.  Values: every gradient
within max|err| / max|ref| <= 2e-2 (bf16 tensors, fp32 accumulation).
Also: an empty batch gives zero weight gradients, a zero W_down gives exactly
zero gradients below it, and two runs are bitwise equal."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import sparse_mixture_experts_scan_amd as moe  # noqa: E402
from sparse_mixture_experts_scan_amd.inputs import MoEConfig, make_dout, make_inputs  # noqa: E402
from tests import gpu_harness as H  # noqa: E402

pytestmark = pytest.mark.gpu
TOL = 2e-2
GRADS = ("dx", "dW_router", "dW_gate", "dW_up", "dW_down")


def announce(msg):
    print(f"[gpu-bwd] {msg}", file=sys.stderr, flush=True)


def run_bwd(cfg, inp, dout, alpha, want_dbias=False):
    d = H.upload(inp)
    ddo = H.dev_tensor(dout)
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    moe.forward(d["x"], d["W_router"], d["W_gate"], d["W_up"], d["W_down"], cfg.k,
                bias=d["bias"], topk_idx=idx)
    g = moe.backward(d["x"], d["W_router"], d["W_gate"], d["W_up"], d["W_down"], ddo, cfg.k,
                     alpha=alpha, bias=d["bias"], want_dbias=want_dbias)
    torch.cuda.synchronize()
    out = {n: H.as_f32(H.to_host(t)).astype(np.float64) for n, t in g.items()}
    out["idx"] = idx.cpu().numpy()
    return out


def compare(cfg, inp, dout, alpha, res, names=GRADS):
    s = oracle.router_logits(inp["x"], inp["W_router"], inp["bias"])
    ref_idx = oracle.select_topk(s, cfg.k)
    gap, _ = oracle.routing_gaps(s, cfg.k)
    ok = gap >= H.NEAR_TIE
    np.testing.assert_array_equal(np.sort(res["idx"][ok], axis=1), np.sort(ref_idx[ok], axis=1))
    ref = oracle.moe_backward(inp["x"], inp["W_router"], inp["W_gate"], inp["W_up"],
                              inp["W_down"], dout, cfg.k, bias=inp["bias"], alpha=alpha,
                              forced_idx=res["idx"].astype(np.int64))
    errs = {}
    for n in names:
        got, want = res[n], ref[n]
        assert got.shape == want.shape, n
        assert np.isfinite(got).all(), n
        errs[n] = float(np.abs(got - want).max() / max(np.abs(want).max(), 1e-30))
        assert errs[n] <= TOL, (n, errs[n])
    return errs


CASES = [
    (MoEConfig("bwd_small", 64, 128, 256, 8, 2, "bf16"), 0.0),
    (MoEConfig("bwd_alpha", 96, 256, 128, 8, 2, "bf16"), 0.05),
    (MoEConfig("bwd_ragged", 77, 256, 384, 6, 3, "bf16"), 0.01),
    (MoEConfig("bwd_fine", 130, 128, 128, 16, 4, "bf16"), 0.02),
    (MoEConfig("bwd_single", 1, 128, 128, 4, 2, "bf16"), 0.1),
    (MoEConfig("bwd_top1", 50, 128, 256, 4, 1, "bf16"), 0.0),
    (MoEConfig("bwd_tiles", 700, 512, 640, 8, 2, "bf16"), 0.01),   # several 128-row tiles
    # one router block (decode-sized): routing, scan and scores from one select pass
    (MoEConfig("bwd_decode", 16, 256, 384, 8, 2, "bf16"), 0.02),
    # widths that are multiples of 256: the 256 x 256 ping-pong GEMMs (k-strided operands
    # read through transposing LDS loads), one launch per contraction
    (MoEConfig("bwd256_small", 64, 256, 256, 8, 2, "bf16"), 0.0),
    (MoEConfig("bwd256_ragged", 77, 256, 512, 6, 3, "bf16"), 0.01),
    (MoEConfig("bwd256_fine", 130, 256, 256, 16, 4, "bf16"), 0.02),
    (MoEConfig("bwd256_single", 1, 256, 256, 4, 2, "bf16"), 0.1),
    (MoEConfig("bwd256_tiles", 900, 512, 768, 8, 2, "bf16"), 0.01),  # several 256-row tiles
    (MoEConfig("bwd256_many_e", 40, 256, 256, 64, 2, "bf16"), 0.0),  # experts left empty
    (MoEConfig("bwd256_e32", 96, 256, 256, 32, 4, "bf16"), 0.02),   # 17-32 experts
    (MoEConfig("bwd256_multi", 700, 256, 256, 4, 2, "bf16"), 0.01),  # two row tiles per expert
    (MoEConfig("bwd256_decode", 24, 256, 256, 8, 2, "bf16"), 0.01),  # one router block
]


@pytest.mark.parametrize("cfg,alpha", CASES, ids=lambda c: getattr(c, "name", str(c)))
def test_backward_parity(cfg, alpha):
    announce(f"case {cfg.name} T={cfg.T} d={cfg.d_model} f={cfg.d_ff} E={cfg.E} k={cfg.k} "
             f"alpha={alpha}")
    inp = make_inputs(cfg, seed=21)
    dout = make_dout(cfg, seed=21)
    res = run_bwd(cfg, inp, dout, alpha)
    errs = compare(cfg, inp, dout, alpha, res)
    announce("  ok: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))


def test_backward_router_bias_gradient():
    cfg = MoEConfig("bwd_bias", 128, 128, 256, 8, 2, "bf16", router_bias=(0.5, -0.2, 0, 0, 0.3, 0,
                                                                          0, -0.4))
    inp = make_inputs(cfg, seed=22)
    dout = make_dout(cfg, seed=22)
    res = run_bwd(cfg, inp, dout, 0.03, want_dbias=True)
    errs = compare(cfg, inp, dout, 0.03, res, names=GRADS + ("dbias",))
    announce("  bias ok: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))


def test_backward_zero_down_and_determinism():
    cfg = MoEConfig("bwd_zero", 80, 128, 128, 8, 2, "bf16")
    inp = make_inputs(cfg, seed=23)
    inp["W_down"] = np.zeros_like(inp["W_down"])
    dout = make_dout(cfg, seed=23)
    res = run_bwd(cfg, inp, dout, 0.0)
    for n in ("dx", "dW_router", "dW_gate", "dW_up"):
        assert (res[n] == 0).all(), n
    assert np.abs(res["dW_down"]).max() > 0
    cfg2 = MoEConfig("bwd_det", 200, 256, 256, 8, 2, "bf16")
    inp2 = make_inputs(cfg2, seed=24)
    dout2 = make_dout(cfg2, seed=24)
    a = run_bwd(cfg2, inp2, dout2, 0.01)
    b = run_bwd(cfg2, inp2, dout2, 0.01)
    for n in GRADS:
        np.testing.assert_array_equal(a[n], b[n])


def test_backward_empty_batch():
    E, k, d, f = 8, 2, 128, 256
    x = torch.empty((0, d), dtype=torch.bfloat16, device="cuda")
    Wr = torch.ones((d, E), dtype=torch.float32, device="cuda")
    Wg = torch.ones((E, f, d), dtype=torch.bfloat16, device="cuda")
    Wd = torch.ones((E, d, f), dtype=torch.bfloat16, device="cuda")
    g = moe.backward(x, Wr, Wg, Wg, Wd, x, k, want_dbias=True)
    torch.cuda.synchronize()
    for n in ("dW_router", "dW_gate", "dW_up", "dW_down", "dbias"):
        assert (g[n].float().cpu() == 0).all(), n
    assert g["dx"].shape == (0, d)


def row_chunk_tokens(idx, E, chunk, seed=0):
    """Tokens covering every `chunk`-row piece of every expert's rows in the
    permuted (token, slot) order the grouped GEMMs tile (one random pair of
    each piece, and every expert's last pair)."""
    k = idx.shape[1]
    rng = np.random.default_rng(seed)
    flat = idx.ravel()
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E)
    toks, pos = set(), 0
    for e in range(E):
        pairs = order[pos:pos + counts[e]]
        pos += counts[e]
        for c0 in range(0, pairs.size, chunk):
            piece = pairs[c0:c0 + chunk]
            toks.add(int(piece[rng.integers(piece.size)] // k))
        if pairs.size:
            toks.add(int(pairs[-1] // k))
    return np.array(sorted(toks), dtype=np.int64)


# smaller shapes whose token tiles fill four rounds of the CUs, so that dX
# runs as one K = 2 d_ff pass: at seed 0 the schedule splits the last 8 token
# tiles into K halves (the second in W3 alone), at seed 1 nothing is split
ONE_PART = {"onepart_split": (MoEConfig("bwd_onepart", 2048, 4096, 256, 16, 8, "bf16"), 0),
            "onepart": (MoEConfig("bwd_onepart", 2048, 4096, 256, 16, 8, "bf16"), 1)}


@pytest.mark.parametrize("workload", ["prefill", "fine", "skewed", "onepart_split", "onepart"])
def test_backward_prefill_sampled(workload):
    # the full shapes of the benchmark (T = 4096: the Mixtral layer, and 64
    # experts of d_ff 3584 with top-8; T = 8192 with skewed routing), checked
    # on stratified outputs.  The dX GEMM runs in two K parts on prefill and
    # in one K = 2 d_ff pass on the other two, and at seed 0 the skewed
    # routing leaves a partial last round that the schedule splits into K
    # halves.  The outputs: dx of
    # a token from every 128-row piece of every expert's rows (each row tile
    # of the recompute, Z and dX GEMMs, including the dX schedule's split
    # tiles), and of every expert, one feature from every 256-feature tile of
    # d_ff: its rows of dW_gate and dW_up and its column of dW_down (each tile
    # of the weight-gradient GEMMs along d_ff, all of their tiles along
    # d_model)
    from sparse_mixture_experts_scan_amd.inputs import CONFIGS
    cfg, seed = ONE_PART[workload] if workload in ONE_PART else (CONFIGS[workload], 0)
    announce(f"case {workload} T={cfg.T} d={cfg.d_model} f={cfg.d_ff} E={cfg.E} k={cfg.k} "
             f"seed={seed} stratified")
    inp = make_inputs(cfg, seed=seed)
    dout = make_dout(cfg, seed=seed)
    d = H.upload(inp)
    idx_t = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    moe.forward(d["x"], d["W_router"], d["W_gate"], d["W_up"], d["W_down"], cfg.k,
                bias=d["bias"], topk_idx=idx_t)
    g = moe.backward(d["x"], d["W_router"], d["W_gate"], d["W_up"], d["W_down"],
                     H.dev_tensor(dout), cfg.k, alpha=0.01, bias=d["bias"])
    torch.cuda.synchronize()
    res = {"idx": idx_t.cpu().numpy()}
    s = oracle.router_logits(inp["x"], inp["W_router"], inp["bias"])
    ref_idx = oracle.select_topk(s, cfg.k)
    gap, _ = oracle.routing_gaps(s, cfg.k)
    ok = gap >= H.NEAR_TIE
    np.testing.assert_array_equal(np.sort(res["idx"][ok], axis=1), np.sort(ref_idx[ok], axis=1))
    toks = row_chunk_tokens(res["idx"], cfg.E, 128)
    rng = np.random.default_rng(1)
    feats = [(e, int(f0 + rng.integers(256))) for e in range(cfg.E)
             for f0 in range(0, cfg.d_ff, 256)]
    ref = oracle.moe_backward_entries(inp["x"], inp["W_router"], inp["W_gate"], inp["W_up"],
                                      inp["W_down"], dout, cfg.k, toks, feats,
                                      bias=inp["bias"], alpha=0.01,
                                      forced_idx=res["idx"].astype(np.int64))

    def host(t):
        return H.as_f32(H.to_host(t.contiguous())).astype(np.float64)
    fe = torch.as_tensor([e for e, _ in feats], device="cuda")
    fi = torch.as_tensor([i for _, i in feats], device="cuda")
    got = {"dx": host(g["dx"][torch.as_tensor(toks, device="cuda")]),
           "dW_gate_rows": host(g["dW_gate"][fe, fi]),
           "dW_up_rows": host(g["dW_up"][fe, fi]),
           "dW_down_cols": host(g["dW_down"][fe, :, fi])}
    errs = {}
    for n, v in got.items():
        assert v.shape == ref[n].shape, n
        errs[n] = float(np.abs(v - ref[n]).max() / np.abs(ref[n]).max())
        assert errs[n] <= TOL, (n, errs[n])
    announce(f"  ok over {toks.size} tokens and {len(feats)} features: "
             + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
