"""INT4 expert weights on the GPU through the C ABI, against the oracle.

"Mixtral of Experts" (limitations, memory item) names INT4 weights; the
library's scheme is symmetric per-group absmax with float32 decisions.
Quantizer: codes and scales bit-exact against oracle.quantize_int4 (both
divide in IEEE float32 and round ties to even), including exact ties, zero
groups and float32 input.  Layer: routing exact away from near ties; values
within the layer's bf16 tolerance (max|err| / max|ref| <= 2e-2) of the oracle
layer on the oracle's own dequantized weights, routed as the GPU routed; both
GEMM forms (INT4 weight streaming, and dequantize-then-tile)."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import sparse_mixture_experts_scan_amd as moe  # noqa: E402
from sparse_mixture_experts_scan_amd.inputs import (CONFIGS, MoEConfig, f32_to_bf16_bits,  # noqa: E402
                                                    make_inputs)
from tests import gpu_harness as H  # noqa: E402

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[gpu-int4] {msg}", file=sys.stderr, flush=True)


def gpu_quantize(W_dev, group):
    p, s = moe.quantize_int4(W_dev, group)
    torch.cuda.synchronize()
    return p, s


# ---------------------------------------------------------------- quantizer
@pytest.mark.parametrize("rows,K,group,dtype", [
    (40, 256, 128, "bf16"), (33, 384, 32, "bf16"), (17, 512, 64, "f32"),
    (8, 1024, 256, "bf16"), (5, 640, 640, "f32"), (3, 65536, 128, "bf16"),
])
def test_quantizer_bit_exact(rows, K, group, dtype):
    announce(f"quantize rows={rows} K={K} group={group} {dtype}")
    rng = np.random.default_rng(rows * 7 + K)
    W = (rng.standard_normal((rows, K)) * np.exp(rng.uniform(-6, 2, (rows, 1)))).astype(np.float32)
    W[0, :group] = 0.0                                      # a zero group
    if K >= 2 * group:
        # exact ties: absmax 7s makes s exact and w / s = q + 1/2
        s = np.float32(0.375)
        W[1, group:2 * group] = s * (rng.integers(-7, 7, group) + 0.5)
        W[1, group] = 7 * s
    host = f32_to_bf16_bits(W) if dtype == "bf16" else W
    p_ref, s_ref = oracle.quantize_int4(host, group)
    p, s = gpu_quantize(H.dev_tensor(host), group)
    np.testing.assert_array_equal(s.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(p.cpu().numpy(), p_ref)


# ---------------------------------------------------------------- layer
def run_int4(cfg, inp, group):
    d = H.upload(inp)
    T, k, E = cfg.T, cfg.k, cfg.E
    q = {n: gpu_quantize(d[n], group) for n in ("W_gate", "W_up", "W_down")}
    idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, k), -7.0, dtype=torch.float32, device="cuda")
    cnt = torch.full((E,), -7, dtype=torch.int32, device="cuda")
    lay = moe.moe_ffn_workspace_layout(T, cfg.d_model, cfg.d_ff, E, k, moe.MOE_W4A16)
    ws = torch.empty(lay.total, dtype=torch.uint8, device="cuda")
    out = moe.forward_int4(d["x"], d["W_router"], q["W_gate"], q["W_up"], q["W_down"], group, k,
                           bias=d.get("bias"), workspace=ws, topk_idx=idx, topk_w=w,
                           expert_counts=cnt)
    torch.cuda.synchronize()
    return dict(out=H.to_host(out), idx=idx.cpu().numpy(), w=w.cpu().numpy(),
                counts=cnt.cpu().numpy(), layout=lay, q=q)


class _LazyQuant:
    """Oracle INT4 codes or scales of one stack, quantized one expert at a
    time on first use (full-size stacks)."""

    def __init__(self, W, group, cache, which):
        self.W, self.group, self.cache, self.which = W, group, cache, which

    def __getitem__(self, e):
        if e not in self.cache:
            self.cache[e] = oracle.quantize_int4(self.W[e], self.group)
        return self.cache[e][self.which]


def oracle_qweights(inp, group, lazy=False):
    if not lazy:
        return {n: oracle.quantize_int4(inp[n], group) for n in ("W_gate", "W_up", "W_down")}
    out = {}
    for n in ("W_gate", "W_up", "W_down"):
        cache = {}
        out[n] = (_LazyQuant(inp[n], group, cache, 0), _LazyQuant(inp[n], group, cache, 1))
    return out


def check_layer(cfg, inp, group, res, tokens=None, lazy=False):
    s = oracle.router_logits(inp["x"], inp["W_router"], inp["bias"])
    idx = oracle.select_topk(s, cfg.k)
    gap, order_gap = oracle.routing_gaps(s, cfg.k)
    rinfo = H.check_routing(cfg, dict(idx=idx, gates=oracle.topk_gates(s, idx), gap=gap,
                                      order_gap=order_gap), res)
    np.testing.assert_array_equal(res["counts"], np.bincount(res["idx"].ravel(),
                                                             minlength=cfg.E))
    toks = np.arange(cfg.T) if tokens is None else np.asarray(tokens)
    r = oracle.moe_forward_int4(inp["x"], inp["W_router"], oracle_qweights(inp, group, lazy),
                                group, cfg.k, bias=inp["bias"], tokens=toks,
                                forced_idx=res["idx"].astype(np.int64))
    got = H.as_f32(res["out"][toks]).astype(np.float64)
    assert np.isfinite(got).all()
    err = np.abs(got - r["out"]).max() / np.abs(r["out"]).max()
    assert err <= H.TOL["bf16"], err
    return err, rinfo


CASES = [
    (MoEConfig("q4_decode_small", 16, 256, 512, 8, 2, "bf16"), 128, 0),
    (MoEConfig("q4_ragged", 33, 384, 256, 6, 3, "bf16"), 64, 0),
    (MoEConfig("q4_group32", 20, 256, 384, 4, 2, "bf16"), 32, 0),
    (MoEConfig("q4_group256", 24, 512, 256, 8, 2, "bf16"), 256, 0),  # two chunks per group
    # three chunks per group: a 256-K run of the LDS-staged form straddles two groups
    (MoEConfig("q4_group384", 24, 768, 768, 8, 2, "bf16"), 384, 0),
    (MoEConfig("q4_bt32", 300, 256, 256, 8, 2, "bf16"), 128, 0),     # 32-row token tiles
    (MoEConfig("q4_single", 1, 128, 128, 4, 1, "bf16"), 128, 0),
    (MoEConfig("q4_tiled", 1000, 256, 384, 8, 2, "bf16"), 128, 1),   # dequantize + tile
    (MoEConfig("q4_tiled_k4", 600, 256, 256, 8, 4, "bf16"), 128, 1),  # tiled, tokens in place
    (MoEConfig("q4_fine", 200, 128, 256, 64, 8, "bf16"), 128, 0),
]


@pytest.mark.parametrize("cfg,group,variant", CASES, ids=lambda c: getattr(c, "name", str(c)))
def test_int4_layer(cfg, group, variant):
    announce(f"case {cfg.name} T={cfg.T} d={cfg.d_model} f={cfg.d_ff} E={cfg.E} k={cfg.k} "
             f"group={group}")
    inp = make_inputs(cfg, seed=11)
    res = run_int4(cfg, inp, group)
    assert res["layout"].gemm_variant == variant
    # the GPU's codes are the oracle's
    for n in ("W_gate", "W_down"):
        p_ref, s_ref = oracle.quantize_int4(inp[n], group)
        np.testing.assert_array_equal(res["q"][n][0].cpu().numpy(), p_ref)
        np.testing.assert_array_equal(res["q"][n][1].cpu().numpy(), s_ref)
    err, rinfo = check_layer(cfg, inp, group, res)
    announce(f"  ok: max|err|/max|ref| {err:.2e}, near_ties={rinfo['near_ties']}")


def test_int4_zero_down_gives_zero():
    cfg = MoEConfig("q4_zero", 40, 256, 256, 8, 2, "bf16")
    inp = make_inputs(cfg, seed=12)
    inp["W_down"] = np.zeros_like(inp["W_down"])
    res = run_int4(cfg, inp, 128)
    assert (res["out"] == 0).all()


def test_int4_decode_workload():
    cfg = CONFIGS["decode"]
    announce(f"case decode T={cfg.T} d={cfg.d_model} f={cfg.d_ff} E={cfg.E} k={cfg.k} group=128")
    inp = make_inputs(cfg, seed=0)
    res = run_int4(cfg, inp, 128)
    assert res["layout"].gemm_variant == 0
    # sampled rows of the GPU's codes against the oracle's
    rng = np.random.default_rng(0)
    for n in ("W_gate", "W_up", "W_down"):
        e = int(rng.integers(cfg.E))
        rows = np.sort(rng.choice(inp[n].shape[1], 64, replace=False))
        p_ref, s_ref = oracle.quantize_int4(inp[n][e][rows], 128)
        trows = torch.as_tensor(rows, device="cuda")
        np.testing.assert_array_equal(res["q"][n][0][e][trows].cpu().numpy(), p_ref)
        np.testing.assert_array_equal(res["q"][n][1][e][:, trows].cpu().numpy(), s_ref)
    err, _ = check_layer(cfg, inp, 128, res, lazy=True)
    announce(f"  ok: max|err|/max|ref| {err:.2e}")


def test_int4_prefill_sampled():
    # the dequantize-then-tile path at the full prefill shape, sampled tokens
    cfg = CONFIGS["prefill"]
    announce(f"case prefill T={cfg.T} d={cfg.d_model} f={cfg.d_ff} E={cfg.E} k={cfg.k} group=128")
    inp = make_inputs(cfg, seed=0)
    res = run_int4(cfg, inp, 128)
    assert res["layout"].gemm_variant == 1
    s = oracle.router_logits(inp["x"], inp["W_router"], inp["bias"])
    toks = H.sample_tokens(cfg, oracle.select_topk(s, cfg.k), 24)
    err, _ = check_layer(cfg, inp, 128, res, tokens=toks, lazy=True)
    announce(f"  ok: max|err|/max|ref| {err:.2e}")
