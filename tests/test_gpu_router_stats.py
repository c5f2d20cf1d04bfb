"""Router statistics and load-balancing loss forward ("ロードバランス損失" on
the architecture page): f_i = fraction of tokens routed to i, p_i = mean over
tokens of the full softmax over all N experts, N * sum_i f_i p_i; GPU values
through the C ABI against the fp64 oracle's balance_stats."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import sparse_mixture_experts_scan_amd as moe  # noqa: E402
from sparse_mixture_experts_scan_amd.inputs import CONFIGS, MoEConfig, make_inputs  # noqa: E402
from tests import gpu_harness as H  # noqa: E402

pytestmark = pytest.mark.gpu

CASES = [
    MoEConfig("stats_fused", 5000, 256, 256, 16, 2, "bf16"),        # many token blocks
    MoEConfig("stats_split", 100, 512, 128, 64, 8, "bf16"),         # router split over d_model
    MoEConfig("stats_f32", 64, 128, 512, 8, 2, "f32"),
    # one router block: the select pass also runs the statistics and the scan
    MoEConfig("stats_single_block", 16, 512, 256, 8, 2, "bf16"),
    MoEConfig("stats_single_e64", 27, 256, 256, 64, 8, "bf16"),
]


def run_stats(cfg, inp):
    d = H.upload(inp)
    probs = torch.full((cfg.E,), -1.0, dtype=torch.float32, device="cuda")
    loss = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((cfg.E,), dtype=torch.int32, device="cuda")
    moe.forward(d["x"], d["W_router"], d["W_gate"], d["W_up"], d["W_down"], cfg.k,
                bias=d["bias"], topk_idx=idx, expert_counts=cnt, router_probs=probs,
                balance_loss=loss)
    torch.cuda.synchronize()
    return probs.cpu().numpy(), float(loss.cpu()[0]), idx.cpu().numpy(), cnt.cpu().numpy()


def check(cfg, inp):
    print(f"[router-stats] case {cfg.name} T={cfg.T} E={cfg.E} k={cfg.k}", file=sys.stderr,
          flush=True)
    p_gpu, l_gpu, idx, cnt = run_stats(cfg, inp)
    s = oracle.router_logits(inp["x"], inp["W_router"], inp["bias"])
    ref = oracle.balance_stats(s, idx, alpha=1.0)      # f from the GPU's routing
    np.testing.assert_array_equal(cnt, np.round(ref["f"] * cfg.T).astype(np.int64))
    np.testing.assert_allclose(p_gpu, ref["p"], rtol=1e-5, atol=1e-7)
    assert abs(p_gpu.sum() - 1.0) < 1e-5
    assert l_gpu == pytest.approx(ref["loss"], rel=1e-5)
    return p_gpu, l_gpu


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_router_statistics(cfg):
    lay = moe.moe_ffn_workspace_layout(cfg.T, cfg.d_model, cfg.d_ff, cfg.E, cfg.k,
                                       moe.MOE_BF16 if cfg.dtype == "bf16" else moe.MOE_F32)
    check(cfg, make_inputs(cfg, seed=5))


def test_zero_router_closed_form():
    # all scores equal: p_i = 1/N and the first k experts take every token,
    # so N * sum_i f_i p_i = k
    cfg = MoEConfig("stats_zero", 300, 128, 128, 8, 2, "bf16")
    inp = make_inputs(cfg, seed=6)
    inp["W_router"] = np.zeros_like(inp["W_router"])
    p, l, _, _ = run_stats(cfg, inp)
    np.testing.assert_allclose(p, 1.0 / 8, rtol=1e-6)
    assert l == pytest.approx(2.0, rel=1e-6)


def test_skewed_workload_loss_exceeds_uniform():
    cfg = CONFIGS["skewed"]
    p, l = check(cfg, make_inputs(cfg, seed=0))
    # skewed routing: the loss is well above its uniform value k
    assert l > 1.2 * cfg.k
