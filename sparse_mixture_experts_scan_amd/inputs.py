"""Seeded synthetic inputs for the sparse MoE feed-forward layer.

This module only draws and encodes numbers; it holds none of the layer's
arithmetic, so both the HIP path and the fp64 oracle can take their inputs
from it without sharing any of the method's code.

Workloads follow the shapes of Mixtral 8x7B's MoE layer as described on
"Mistral/Mixtralのアーキテクチャ" (disassemble-channel.com), section
"各エキスパートの構造": d_model = 4096, d_ff = 14336, N = 8 experts, top-2.
Distributions: x ~ N(0, 1); every weight ~ N(0, 1/fan_in), fan_in being the
input width of that matrix (d_model for the router, gate and up projections,
d_ff for the down projection).  Random-init weights stand in for trained
Mixtral weights, which are not available.

Random streams: each tensor (and each expert's slice of a weight stack) has
its own ``numpy.random.PCG64`` stream, seeded by
``SeedSequence([seed, tensor_id, expert])``, so the draw is identical whatever
the number of worker threads.  Values are drawn as float32 standard normals,
scaled in float32 by 1/sqrt(fan_in) and, for bf16 workloads, rounded to
bfloat16 with round-to-nearest-even.  bfloat16 arrays are carried as their
16-bit patterns in ``numpy.uint16`` arrays (numpy has no bfloat16 type).
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

X_ID, ROUTER_ID, GATE_ID, UP_ID, DOWN_ID, NORM_ID, DOUT_ID = 0, 1, 2, 3, 4, 5, 6


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    """One workload: T tokens through one MoE layer of E SwiGLU experts, top-k."""

    name: str
    T: int
    d_model: int
    d_ff: int
    E: int
    k: int
    dtype: str  # "bf16": x, expert weights and out in bfloat16; "f32": all float32
    router_bias: Optional[tuple] = None  # per-expert fp32 bias added to the logits
    note: str = ""

    def with_T(self, T: int) -> "MoEConfig":
        return dataclasses.replace(self, T=T)

    @property
    def expert_bytes(self) -> int:
        """Bytes of one expert's three matrices (gate, up, down)."""
        return 3 * self.d_model * self.d_ff * (2 if self.dtype == "bf16" else 4)


# Skewed workload: a positive bias on experts 0 and 1 and a negative one on the
# last expert; with logits of unit spread this sends about 60% of all
# assignments to experts 0 and 1 and under 2% to expert 7.
SKEW_BIAS = (1.2, 1.2, 0.0, 0.0, 0.0, 0.0, 0.0, -1.0)

CONFIGS = {
    "tiny": MoEConfig("tiny", 64, 128, 512, 8, 2, "f32",
                      note="tiny fp32 case, oracle-sized"),
    "decode": MoEConfig("decode", 16, 4096, 14336, 8, 2, "bf16",
                        note="Mixtral-shaped decode step, weight-streaming"),
    "prefill": MoEConfig("prefill", 4096, 4096, 14336, 8, 2, "bf16",
                         note="Mixtral-shaped prefill, near-uniform routing"),
    "skewed": MoEConfig("skewed", 8192, 4096, 14336, 8, 2, "bf16", SKEW_BIAS,
                        note="router bias sends ~60% of assignments to experts 0,1"),
    "fine": MoEConfig("fine", 4096, 4096, 3584, 64, 8, "bf16",
                      note="fine-grained: 64 experts of d_ff 3584, top-8"),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return the
    16-bit patterns.  Inputs are finite (normal draws), so no NaN handling."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 patterns to float32 (for host-side checks)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def _stream(seed: int, tensor_id: int, expert: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([seed, tensor_id, expert])))


def _draw(seed, tensor_id, expert, shape, std, bf16):
    g = _stream(seed, tensor_id, expert)
    v = g.standard_normal(int(np.prod(shape)), dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    v = v.reshape(shape)
    return f32_to_bf16_bits(v) if bf16 else v


def _draw_stack(seed, tensor_id, E, shape, std, bf16, pool):
    out = np.empty((E,) + tuple(shape), dtype=np.uint16 if bf16 else np.float32)

    def one(e):
        out[e] = _draw(seed, tensor_id, e, shape, std, bf16)

    list(pool.map(one, range(E)))
    return out


def make_inputs(cfg: MoEConfig, seed: int = 0, threads: Optional[int] = None,
                weights: bool = True) -> dict:
    """Draw one workload.

    Returns a dict of host arrays, all C-contiguous:
      x         [T][d_model]        bf16 bits (uint16) or float32
      W_router  [d_model][E]        float32 (always)
      W_gate    [E][d_ff][d_model]  bf16 bits or float32  (nn.Linear [out][in])
      W_up      [E][d_ff][d_model]
      W_down    [E][d_model][d_ff]
      bias      [E] float32 or None
    ``weights=False`` skips the expert stacks (router-only checks).
    """
    bf16 = cfg.dtype == "bf16"
    d, f, E = cfg.d_model, cfg.d_ff, cfg.E
    threads = threads or min(16, os.cpu_count() or 1)
    res = {
        "x": _draw(seed, X_ID, 0, (cfg.T, d), 1.0, bf16),
        "W_router": _draw(seed, ROUTER_ID, 0, (d, E), 1.0 / np.sqrt(d), False),
        "bias": (np.asarray(cfg.router_bias, dtype=np.float32)
                 if cfg.router_bias is not None else None),
    }
    if res["bias"] is not None and res["bias"].shape != (E,):
        raise ValueError("router bias must have E entries")
    if weights:
        with ThreadPoolExecutor(threads) as pool:
            res["W_gate"] = _draw_stack(seed, GATE_ID, E, (f, d), 1.0 / np.sqrt(d), bf16, pool)
            res["W_up"] = _draw_stack(seed, UP_ID, E, (f, d), 1.0 / np.sqrt(d), bf16, pool)
            res["W_down"] = _draw_stack(seed, DOWN_ID, E, (d, f), 1.0 / np.sqrt(f), bf16, pool)
    return res


def make_block_inputs(cfg: MoEConfig, seed: int = 0, threads: Optional[int] = None) -> dict:
    """make_inputs plus what the normalised block needs, with x given the
    spread of scales a residual stream has:
      x            rows of N(0, 1) scaled by 2**u, u ~ U(-4, 4) per token (the
                   scale is a power of two, so bf16 rows stay exact)
      norm_weight  [d_model] float32, 1 + 0.25 * N(0, 1)
    """
    res = make_inputs(cfg, seed, threads)
    g = _stream(seed, NORM_ID, 0)
    u = np.floor(g.uniform(-4.0, 4.0, size=cfg.T)).astype(np.int32)
    scale = np.ldexp(np.float32(1.0), u).astype(np.float32)[:, None]
    if res["x"].dtype == np.uint16:
        res["x"] = f32_to_bf16_bits(bf16_bits_to_f32(res["x"]) * scale)
    else:
        res["x"] = (res["x"] * scale).astype(np.float32)
    res["norm_weight"] = (1.0 + 0.25 * g.standard_normal(cfg.d_model, dtype=np.float32)
                          ).astype(np.float32)
    return res


def make_dout(cfg: MoEConfig, seed: int = 0) -> np.ndarray:
    """Upstream gradient of the layer's output for the backward pass:
    [T][d_model] N(0, 1), in the workload's element type."""
    return _draw(seed, DOUT_ID, 0, (cfg.T, cfg.d_model), 1.0, cfg.dtype == "bf16")
