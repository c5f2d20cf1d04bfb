"""The seeded input generator: reproducible, thread-count independent, and
its bfloat16 rounding agrees with torch's (round to nearest, ties to even)."""
import numpy as np
import torch

from sparse_mixture_experts_scan_amd.inputs import (CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits,
                                                    make_inputs)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    v = rng.standard_normal(100000).astype(np.float32) * 10
    # exact ties between two bf16 values, both parities, and signed zeros
    ties = (np.arange(1, 2000, dtype=np.uint32) << np.uint32(16)) | np.uint32(0x8000)
    v = np.concatenate([v, ties.view(np.float32), -ties.view(np.float32),
                        np.array([0.0, -0.0, 1e-40, 3.3e38], dtype=np.float32)])
    ours = f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(bf16_bits_to_f32(ours),
                                  torch.from_numpy(v).to(torch.bfloat16).float().numpy())


def test_reproducible_and_thread_independent():
    cfg = CONFIGS["tiny"]
    a = make_inputs(cfg, seed=3, threads=1)
    b = make_inputs(cfg, seed=3, threads=5)
    c = make_inputs(cfg, seed=4, threads=2)
    for key in ("x", "W_router", "W_gate", "W_up", "W_down"):
        np.testing.assert_array_equal(a[key], b[key])
        assert not np.array_equal(a[key], c[key])


def test_shapes_dtypes_and_scales():
    cfg = CONFIGS["fine"].with_T(256)
    inp = make_inputs(cfg.__class__(**{**cfg.__dict__, "d_model": 256, "d_ff": 512}), seed=0)
    assert inp["x"].dtype == np.uint16 and inp["x"].shape == (256, 256)
    assert inp["W_router"].dtype == np.float32 and inp["W_router"].shape == (256, 64)
    assert inp["W_gate"].shape == (64, 512, 256) and inp["W_down"].shape == (64, 256, 512)
    g = bf16_bits_to_f32(inp["W_gate"])
    dn = bf16_bits_to_f32(inp["W_down"])
    assert abs(g.std() * np.sqrt(256) - 1) < 0.01
    assert abs(dn.std() * np.sqrt(512) - 1) < 0.01
    assert inp["bias"] is None
    sk = make_inputs(CONFIGS["skewed"].with_T(8), weights=False)
    assert sk["bias"].tolist()[:2] == [np.float32(1.2), np.float32(1.2)]
