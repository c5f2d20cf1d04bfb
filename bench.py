"""Benchmark of the sparse MoE feed-forward layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode]

A step is one full forward of the layer (router, permutation, gate/up GEMM,
down GEMM, combine) over one batch of seeded synthetic tokens, with inputs and
weights already resident in HBM.  The default workload is the Mixtral-shaped
decode layer (T = 16, d_model 4096, d_ff 14336, 8 experts, top-2, bf16), the
HBM-bound half of the metric; the same run then times the MFMA-bound half,
the prefill layer (T = 4096, same weights), in the same process and reports
it as a nested "prefill" object.  Prints one JSON line: tokens/s, the
roofline of the dominant kernel (timed live with HIP events recorded on the
launch stream), measured HBM and MFMA ceilings beside the datasheet peaks, a
check of each leg's timed output against the fp64 oracle (routing on every
token, values on a tile-stratified token sample) and the oracle itself timed
on a bounded sample of the same workload."""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

from sparse_mixture_experts_scan_amd.inputs import (CONFIGS, make_block_inputs, make_dout,
                                                    make_inputs)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6        # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3         # MI355X dense fp32 MFMA / vector


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="decode", choices=sorted(CONFIGS))
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-tokens", type=int, default=0,
                   help="tokens of the oracle sample (0 = per-workload default)")
    p.add_argument("--router-stats", action="store_true",
                   help="also produce the router statistics p_i and the load-balancing loss "
                        "in every step")
    p.add_argument("--weights", default="bf16", choices=("bf16", "int4"),
                   help="expert weights as given (bf16) or INT4 with per-group float32 "
                        "scales (quantized on the GPU before warmup)")
    p.add_argument("--group", type=int, default=128, help="INT4 scale group size")
    p.add_argument("--backward", action="store_true",
                   help="time the backward pass (gradients of <dOut, out> + alpha * balance "
                        "loss, routing and pre-activations recomputed) instead of the forward")
    p.add_argument("--alpha", type=float, default=0.01, help="balance-loss weight (--backward)")
    p.add_argument("--block", action="store_true",
                   help="time the normalised block out = x + layer(RMSNorm(x)) instead of "
                        "the bare layer")
    p.add_argument("--no-prefill-leg", action="store_true",
                   help="with the default decode workload, do not also time the prefill layer")
    p.add_argument("--no-measured-peaks", action="store_true",
                   help="skip the HBM / MFMA microbenchmarks")
    p.add_argument("--no-output-check", action="store_true",
                   help="skip the oracle check of the timed output")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="before warmup, run one device-to-device copy of this many MiB "
                        "(a known-size reference for HBM byte counters)")
    return p.parse_args()


def algorithmic_work(cfg, counts, group=0):
    """Per-step bytes the method must move and flops it must do (no padding,
    no intermediates, only the experts that received tokens), and the same
    per kernel for the two GEMMs.  group > 0: INT4 expert weights (half a
    byte per weight plus one float32 scale per group)."""
    w = 2 if cfg.dtype == "bf16" else 4
    T, d, f, E, k = cfg.T, cfg.d_model, cfg.d_ff, cfg.E, cfg.k
    A = T * k
    touched = int((counts > 0).sum())
    ww = (0.5 + 4.0 / group) if group else w        # bytes per expert weight
    layer_bytes = touched * 3 * d * f * ww + 2 * T * d * w + d * E * 4
    layer_flops = 2 * A * 3 * d * f + 2 * T * d * E
    gateup_bytes = touched * 2 * d * f * ww + A * d * w + A * f * w
    gateup_flops = 2 * A * 2 * d * f
    down_bytes = touched * d * f * ww + A * f * w + A * d * 4
    down_flops = 2 * A * d * f
    return dict(touched=touched, layer_bytes=layer_bytes, layer_flops=layer_flops,
                gateup=(gateup_bytes, gateup_flops), down=(down_bytes, down_flops))


def measured_traffic(workload, kernel, variant):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 counter summary (profiles/traffic.json), or None when there is
    none or the kernel's source has changed since the counters were taken."""
    from sparse_mixture_experts_scan_amd import prof_summary
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "traffic.json")
    try:
        with open(path) as fh:
            rec = json.load(fh)[workload][kernel]
    except (OSError, KeyError, ValueError):
        return None
    files = prof_summary.KERNEL_SOURCES.get(kernel, {}).get(variant)
    if files is None:
        return None
    if rec.get("source_files") != files or rec.get("source_sha256") != prof_summary.source_hash(files):
        return None
    return rec["bytes"]


def host_cpu():
    """(logical CPUs, model name) of this host."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return os.cpu_count() or 1, model


def cpu_baseline(cfg, inp, n_tokens, block=False):
    """The fp64 oracle as it stands, timed on a bounded token sample."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        blas = ",".join(sorted({i.get("internal_api", "?") for i in threadpool_info()
                                if i.get("user_api") == "blas"})) or "?"
    except Exception:  # pragma: no cover
        threads, blas = 1, "?"
    ncpu, model = host_cpu()
    rng = np.random.default_rng(123)
    toks = np.sort(rng.choice(cfg.T, size=min(n_tokens, cfg.T), replace=False))
    t0 = time.perf_counter()
    if block:
        oracle.block_forward(inp["x"], inp["norm_weight"], 1e-5, inp["W_router"], inp["W_gate"],
                             inp["W_up"], inp["W_down"], cfg.k, bias=inp["bias"], tokens=toks)
    else:
        oracle.moe_forward(inp["x"], inp["W_router"], inp["W_gate"], inp["W_up"],
                           inp["W_down"], cfg.k, bias=inp["bias"], tokens=toks)
    dt = time.perf_counter() - t0
    return {"value": len(toks) / dt, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "host_cpus": ncpu, "cpu_model": model,
            "sample": f"{len(toks)} of {cfg.T} tokens of the {cfg.name} workload "
                      f"(routing for all {cfg.T}), fp64 numpy oracle with {threads} "
                      f"{blas} BLAS threads, {dt:.2f} s"}


def tile_tokens(idx, E, tile=256, per_tile=1, seed=0):
    """Tokens that reach every (expert, token tile) unit of the grouped GEMMs:
    in each expert's rows, ordered by (token, slot) as the permutation lays
    them out, one random row of every `tile`-row piece and the last row."""
    k = idx.shape[1]
    rng = np.random.default_rng(seed)
    flat = idx.ravel()
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E)
    toks, pos = {0, idx.shape[0] - 1}, 0
    for e in range(E):
        pairs = order[pos:pos + counts[e]]
        pos += counts[e]
        for c0 in range(0, pairs.size, tile):
            piece = pairs[c0:c0 + tile]
            toks.update((rng.choice(piece, size=min(per_tile, piece.size), replace=False)
                         // k).tolist())
        if pairs.size:
            toks.add(int(pairs[-1] // k))
    return np.array(sorted(toks), dtype=np.int64)


def output_check(cfg, inp, out, idx, tile_rows):
    """The timed step's output against the fp64 oracle: routing on every
    token (indices exact except where the k-th/(k+1)-th score gap, or a gap
    inside the selected set, is below 1e-4), values on every token when T is
    small, else on a tile-stratified sample, routed as the GPU routed them."""
    import oracle
    near = 1e-4
    s = oracle.router_logits(inp["x"], inp["W_router"], inp["bias"])
    oidx = oracle.select_topk(s, cfg.k)
    gap, order_gap = oracle.routing_gaps(s, cfg.k)
    robust = (gap >= near) & (order_gap >= near)
    mism = int((idx[robust] != oidx[robust]).any(axis=1).sum())
    set_robust = (gap >= near) & (order_gap < near)
    mism += int(sum(set(idx[t]) != set(oidx[t]) for t in np.nonzero(set_robust)[0]))
    tie_mism = int(sum(set(idx[t]) != set(oidx[t]) for t in np.nonzero(gap < near)[0]))
    toks = (np.arange(cfg.T) if cfg.T <= 256 else tile_tokens(idx, cfg.E, tile_rows))
    r = oracle.moe_forward(inp["x"], inp["W_router"], inp["W_gate"], inp["W_up"], inp["W_down"],
                           cfg.k, bias=inp["bias"], tokens=toks, forced_idx=idx.astype(np.int64))
    got = out[toks].astype(np.float64)
    err = float(np.abs(got - r["out"]).max() / max(np.abs(r["out"]).max(), 1e-30))
    tol = 2e-2 if cfg.dtype == "bf16" else 1e-4
    counts = np.bincount(idx.ravel(), minlength=cfg.E)
    return {"max_err_rel": err, "tol": tol, "pass": bool(err <= tol and mism == 0),
            "tokens_checked": int(toks.size),
            "sample": "all tokens" if toks.size == cfg.T else
                      f"tile-stratified: a row of every ({tile_rows}-row token tile, expert) "
                      "pair, each expert's last row, first and last token",
            "index_mismatches": mism, "near_ties": int((gap < near).sum()),
            "near_tie_mismatches": tie_mism, "order_ties": int((set_robust).sum()),
            "histogram": counts.tolist(), "experts_touched": int((counts > 0).sum())}


def bench_backward(args, cfg, d, dev, stream):
    """--backward: one step is one moe_ffn_backward call."""
    import torch
    import sparse_mixture_experts_scan_amd as moe
    from sparse_mixture_experts_scan_amd.binding import BWD_STAGE_NAMES, MOE_BWD_NUM_STAGES

    if cfg.dtype != "bf16" or args.block or args.weights != "bf16":
        print("the backward takes bf16 tensors and the bare layer", file=sys.stderr)
        sys.exit(2)
    T, E, k = cfg.T, cfg.E, cfg.k
    dout = torch.from_numpy(make_dout(cfg, args.seed).view(np.int16)).view(torch.bfloat16).to(dev)
    ws = torch.empty(moe.moe_ffn_backward_workspace_size(T, cfg.d_model, cfg.d_ff, E, k),
                     dtype=torch.uint8, device=dev)

    def step(events=None):
        return moe.backward(d["x"], d["W_router"], d["W_gate"], d["W_up"], d["W_down"], dout, k,
                            alpha=args.alpha, bias=d["bias"], workspace=ws, stream=stream,
                            stage_events=events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    evs = []
    for _ in range(args.steps):
        row = [torch.cuda.Event(enable_timing=True) for _ in range(MOE_BWD_NUM_STAGES + 1)]
        for ev in row:
            ev.record(stream)
        evs.append(row)
    torch.cuda.synchronize()
    for row in evs:
        step(row)
    torch.cuda.synchronize()
    split = {name: float(np.mean([row[i].elapsed_time(row[i + 1]) for row in evs]))
             for i, name in enumerate(BWD_STAGE_NAMES)}
    A, dm, f = T * k, cfg.d_model, cfg.d_ff
    flops = {"recompute": 4 * A * dm * f, "z": 2 * A * dm * f, "dxs": 4 * A * dm * f,
             "dw_down": 2 * A * dm * f, "dw_gate_up": 4 * A * dm * f}
    dom = max(flops, key=lambda n: split[n])
    achieved = flops[dom] / (split[dom] * 1e-3) / 1e12
    total = sum(flops.values()) + 4 * T * dm * E
    secs = ms_step * 1e-3
    record = {
        "metric": "MoE-layer backward tokens/s (routing and pre-activations recomputed)",
        "value": T / secs, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) tokens and upstream gradient, N(0,1/fan_in) weights)",
        "config": {"workload": cfg.name, "T": T, "d_model": dm, "d_ff": f, "E": E, "k": k,
                   "alpha": args.alpha, "parallelism": "single GPU"},
        "layer": {"TFLOP/s": total / secs / 1e12,
                  "mfma_frac": total / secs / 1e12 / BF16_PEAK_TFLOPS, "kernel_ms": split},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / BF16_PEAK_TFLOPS, "traffic": None,
                     "kernel": dom, "kernel_ms": split[dom]},
    }
    print(json.dumps(record), flush=True)


def upload(a, dev):
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(a).to(dev)


def roofline(cfg, work, split, form, workload_key):
    """The dominant kernel's (gate/up's) roofline: HBM for few rows per
    expert, MFMA (in the element type's peak) for many."""
    gateup_bytes, gateup_flops = work["gateup"]
    gu_s = split["gateup"] * 1e-3
    if cfg.dtype == "f32":
        roof = {"bound": "mfma", "achieved": gateup_flops / gu_s / 1e12, "peak": FP32_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    elif cfg.T * cfg.k / cfg.E <= 64:
        roof = {"bound": "hbm", "achieved": gateup_bytes / gu_s / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": gateup_flops / gu_s / 1e12,
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(workload_key, "gateup", form)
    roof["kernel"] = "gateup"
    roof["kernel_ms"] = split["gateup"]
    return roof


def run_leg(args, cfg, d, x, step_fn, stream, group=0):
    """Warm up, time exactly args.steps steps between two synchronisations,
    then time the per-kernel split with the library's stage events (one row
    of events per step, a second pass over args.steps steps).  Returns the
    timings, the counts and routing of the last step, and its output."""
    import torch
    from sparse_mixture_experts_scan_amd.binding import MOE_NUM_STAGES, STAGE_NAMES
    T, E, k = cfg.T, cfg.E, cfg.k
    dev = x.device
    out = torch.empty_like(x)
    counts = torch.zeros(E, dtype=torch.int32, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)

    def step(events=None):
        step_fn(x, out, counts, idx, events)

    print(f"[bench] {cfg.name}: warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for _ in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    print(f"[bench] {cfg.name}: timed {args.steps} steps: {ms_step:.4f} ms/step",
          file=sys.stderr, flush=True)
    evs = []
    for _ in range(args.steps):
        row = [torch.cuda.Event(enable_timing=True) for _ in range(MOE_NUM_STAGES + 1)]
        for ev in row:
            ev.record(stream)          # creates the underlying event
        evs.append(row)
    torch.cuda.synchronize()
    for row in evs:
        step(row)
    torch.cuda.synchronize()
    split = {name: float(np.mean([row[i].elapsed_time(row[i + 1]) for row in evs]))
             for i, name in enumerate(STAGE_NAMES)}
    cnt = counts.cpu().numpy()
    work = algorithmic_work(cfg, cnt, group)
    secs = ms_step * 1e-3
    layer = {"GB/s": work["layer_bytes"] / secs / 1e9,
             "hbm_frac": work["layer_bytes"] / secs / 1e9 / HBM_PEAK_GBS,
             "TFLOP/s": work["layer_flops"] / secs / 1e12,
             "mfma_frac": work["layer_flops"] / secs / 1e12 / (
                 BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else FP32_PEAK_TFLOPS),
             "experts_touched": work["touched"], "kernel_ms": split}
    host_out = out.float().cpu().numpy() if cfg.dtype == "bf16" else out.cpu().numpy()
    return dict(ms_step=ms_step, split=split, work=work, layer=layer, counts=cnt,
                idx=idx.cpu().numpy(), out=host_out)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer's multi-GPU sharding is a design note, not built)", file=sys.stderr)
        sys.exit(2)
    import torch
    import sparse_mixture_experts_scan_amd as moe

    cfg = CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] workload {cfg.name}: generating inputs", file=sys.stderr, flush=True)
    inp = (make_block_inputs if args.block else make_inputs)(cfg, seed=args.seed)
    d = {k: upload(v, dev) for k, v in inp.items()}
    E, k = cfg.E, cfg.k
    dt = moe.MOE_BF16 if cfg.dtype == "bf16" else moe.MOE_F32
    int4 = args.weights == "int4"
    if int4:
        if cfg.dtype != "bf16" or args.block:
            print("INT4 weights take bf16 activations and the bare layer", file=sys.stderr)
            sys.exit(2)
        dt = moe.MOE_W4A16
        q = {n: moe.quantize_int4(d[n], args.group) for n in ("W_gate", "W_up", "W_down")}
        for n in ("W_gate", "W_up", "W_down"):
            del d[n]                   # only the INT4 copies stay resident
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    if args.backward:
        bench_backward(args, cfg, d, dev, stream)
        return
    probs = torch.zeros(E, dtype=torch.float32, device=dev) if args.router_stats else None
    bloss = torch.zeros(1, dtype=torch.float32, device=dev) if args.router_stats else None

    def make_step(leg_cfg):
        size = moe.moe_block_workspace_size if args.block else moe.moe_ffn_workspace_size
        ws = torch.empty(size(leg_cfg.T, cfg.d_model, cfg.d_ff, E, k, dt), dtype=torch.uint8,
                         device=dev)

        def step(x, out, counts, idx, events):
            if int4:
                moe.forward_int4(x, d["W_router"], q["W_gate"], q["W_up"], q["W_down"],
                                 args.group, k, bias=d["bias"], out=out, workspace=ws,
                                 expert_counts=counts, topk_idx=idx, stream=stream,
                                 stage_events=events, router_probs=probs, balance_loss=bloss)
                return
            moe.forward(x, d["W_router"], d["W_gate"], d["W_up"], d["W_down"], k,
                        bias=d["bias"], out=out, workspace=ws, expert_counts=counts,
                        topk_idx=idx, stream=stream, stage_events=events, router_probs=probs,
                        balance_loss=bloss, norm_weight=d.get("norm_weight"), eps=1e-5)
        return step

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)                 # runtime blit kernel
        torch.add(src, 1, out=dst)     # plain elementwise kernel: reads n, writes n bytes
        torch.cuda.synchronize()
        del src, dst

    def form_of(leg_cfg):
        variant = moe.moe_ffn_workspace_layout(leg_cfg.T, cfg.d_model, cfg.d_ff, E, k,
                                               dt).gemm_variant
        tile = 256 if variant == 1 else moe.moe_ffn_workspace_layout(
            leg_cfg.T, cfg.d_model, cfg.d_ff, E, k, dt).block_rows
        return (("q4" if variant == 0 else "q4tile") if int4 else
                ("tile" if variant == 1 else "stream")), int(tile)

    def check(leg_cfg, leg_inp, leg, tile):
        if args.no_output_check or int4 or args.block:
            return None
        print(f"[bench] {leg_cfg.name}: checking the timed output against the oracle",
              file=sys.stderr, flush=True)
        return output_check(leg_cfg, leg_inp, leg["out"], leg["idx"], tile)

    group = args.group if int4 else 0
    leg = run_leg(args, cfg, d, d["x"], make_step(cfg), stream, group)
    form, tile = form_of(cfg)
    ms_step = leg["ms_step"]
    secs = ms_step * 1e-3
    record = {
        "metric": "MoE-layer tokens/s + % of HBM BW (T=16) / % bf16 MFMA peak (T=4096)",
        "value": cfg.T / secs,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) tokens, N(0,1/fan_in) random-init weights)",
        "config": {"workload": cfg.name, "T": cfg.T, "d_model": cfg.d_model, "d_ff": cfg.d_ff,
                   "E": E, "k": k, "router_bias": cfg.router_bias, "seed": args.seed,
                   "block": bool(args.block),
                   "weights": f"int4 (group {args.group}, fp32 scales)" if int4 else cfg.dtype,
                   "parallelism": "single GPU"},
        "layer": leg["layer"],
        "router_stats": ({"balance_loss_unscaled": float(bloss.cpu()[0]),
                          "p": [round(float(v), 6) for v in probs.cpu()]}
                         if args.router_stats else None),
        "roofline": roofline(cfg, leg["work"], leg["split"], form,
                             cfg.name + ("_int4" if int4 else "")),
        "check": check(cfg, inp, leg, tile),
    }
    del leg

    if cfg.name == "decode" and not args.no_prefill_leg and not args.block:
        # the MFMA-bound half of the metric, on the same resident weights
        # (drawn from the same seeded streams, so only x is new)
        pcfg = CONFIGS["prefill"]
        print(f"[bench] prefill leg: generating tokens", file=sys.stderr, flush=True)
        pinp = make_inputs(pcfg, seed=args.seed, weights=False)
        pinp.update({n: inp[n] for n in ("W_gate", "W_up", "W_down") if n in inp})
        px = upload(pinp["x"], dev)
        pleg = run_leg(args, pcfg, d, px, make_step(pcfg), stream, group)
        pform, ptile = form_of(pcfg)
        psecs = pleg["ms_step"] * 1e-3
        record["prefill"] = {
            "workload": "prefill", "T": pcfg.T, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": pleg["ms_step"], "tokens/s": pcfg.T / psecs,
            "TFLOP/s": pleg["work"]["layer_flops"] / psecs / 1e12,
            "layer": pleg["layer"],
            "roofline": roofline(pcfg, pleg["work"], pleg["split"], pform,
                                 pcfg.name + ("_int4" if int4 else "")),
            "check": check(pcfg, pinp, pleg, ptile),
        }
        del pleg, px

    if not args.no_measured_peaks:
        from sparse_mixture_experts_scan_amd import probe
        print("[bench] measured peaks", file=sys.stderr, flush=True)
        peaks = probe.measured_peaks(dev)
        for roof in [record["roofline"]] + ([record["prefill"]["roofline"]]
                                            if "prefill" in record else []):
            if roof["unit"] == "GB/s":
                mp = peaks["hbm_read_GBs"]
                what = "16-byte streaming read of 4 GiB"
            elif roof["peak"] == BF16_PEAK_TFLOPS:
                mp = peaks["mfma_bf16_TFLOPs"]
                what = "register-operand v_mfma_f32_32x32x16_bf16 loop, 2 waves per SIMD"
            else:
                continue
            roof["measured_peak"] = {"value": mp, "unit": roof["unit"], "what": what,
                                     "frac": roof["achieved"] / mp}
        record["measured_peaks"] = peaks
    if not args.no_cpu_baseline and not int4:
        n = args.cpu_sample_tokens or {"tiny": 64, "decode": 16}.get(cfg.name, 64)
        print(f"[bench] cpu baseline on {n} tokens", file=sys.stderr, flush=True)
        record["cpu_baseline"] = cpu_baseline(cfg, inp, n, block=args.block)
    print(json.dumps(record), flush=True)


if __name__ == "__main__":
    main()
