"""Shared helpers of the GPU parity tests: move seeded inputs to the device,
run the HIP layer through the C ABI with a caller workspace, read back the
intermediates, and compare against the fp64 oracle.

Bars (the layer's stated tolerances): routing indices equal the oracle's on
every token whose k-th/(k+1)-th score gap is >= 1e-4 (tokens below are
counted; on them the GPU's own choice is value-checked through the oracle's
forced routing); outputs within max|err| / max|ref| <= 2e-2 for bf16 and
<= 1e-4 for fp32.  Integer work (counts, offsets, row maps, gathered rows) is
checked bit-exactly against a host recomputation from the GPU's indices."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import sparse_mixture_experts_scan_amd as moe
from sparse_mixture_experts_scan_amd.inputs import MoEConfig

NEAR_TIE = 1e-4
TOL = {"bf16": 2e-2, "f32": 1e-4}


def dev_tensor(a: np.ndarray, device="cuda"):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def as_f32(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return a.astype(np.float32)


def upload(inp: dict, device="cuda") -> dict:
    return {k: (dev_tensor(v, device) if v is not None else None) for k, v in inp.items()}


def run_gpu(cfg: MoEConfig, dinp: dict, *, device="cuda", keep_ws=True, block_eps=None) -> dict:
    """One forward through the C ABI with a caller workspace; returns host
    copies of out, routing outputs and (keep_ws) the workspace intermediates.
    block_eps given: the normalised block (dinp["norm_weight"], that eps)."""
    T, d, f, E, k = cfg.T, cfg.d_model, cfg.d_ff, cfg.E, cfg.k
    dt = moe.MOE_BF16 if cfg.dtype == "bf16" else moe.MOE_F32
    lay = (moe.moe_block_workspace_layout(T, d, f, E, k, dt) if block_eps is not None
           else moe.moe_ffn_workspace_layout(T, d, f, E, k, dt))
    ws = torch.empty(lay.total, dtype=torch.uint8, device=device)
    idx = torch.full((T, k), -7, dtype=torch.int32, device=device)
    w = torch.full((T, k), -7.0, dtype=torch.float32, device=device)
    cnt = torch.full((E,), -7, dtype=torch.int32, device=device)
    out = moe.forward(dinp["x"], dinp["W_router"], dinp["W_gate"], dinp["W_up"], dinp["W_down"],
                      k, bias=dinp.get("bias"), workspace=ws, topk_idx=idx, topk_w=w,
                      expert_counts=cnt,
                      norm_weight=dinp["norm_weight"] if block_eps is not None else None,
                      eps=block_eps if block_eps is not None else 0.0)
    torch.cuda.synchronize()
    res = dict(out=to_host(out), idx=idx.cpu().numpy(), w=w.cpu().numpy(),
               counts=cnt.cpu().numpy(), layout=lay)
    if keep_ws:
        def i32(off, n):
            return ws[off:off + 4 * n].view(torch.int32).cpu().numpy()
        R = lay.max_rows
        res.update(
            ws_counts=i32(lay.counts, E), offsets=i32(lay.offsets, E + 1),
            num_tiles=int(i32(lay.num_tiles, 1)[0]),
            tile_expert=i32(lay.tile_expert, R // lay.block_rows),
            row_token=i32(lay.row_token, R), tok_row=i32(lay.tok_row, T * k).reshape(T, k))
        # the down GEMM's schedule: K parts of the split token tiles, first split row
        res["down_sched"] = (tuple(int(v) for v in i32(lay.down_sched, 2))
                             if lay.gemm_variant == 1 else (1, R))
        if lay.y_weighted:   # gate weight of each permuted row (tiled form)
            res["row_w"] = ws[lay.row_w:lay.row_w + 4 * R].view(torch.float32).cpu().numpy()
        if block_eps is not None:
            res["norm_rs"] = ws[lay.norm_rs:lay.norm_rs + 4 * T].view(torch.float32).cpu().numpy()
            es = 2 if cfg.dtype == "bf16" else 4
            b = ws[lay.xn:lay.xn + es * T * d]
            res["xn"] = (b.view(torch.int16).cpu().numpy().view(np.uint16) if es == 2
                         else b.view(torch.float32).cpu().numpy()).reshape(T, d)
        res["_ws"] = ws
    return res


def ws_rows(res, cfg: MoEConfig, which: str, rows) -> np.ndarray:
    """Rows of a workspace matrix (xs, h: element type; y: fp32, or bf16 when
    the layout's y_weighted is set; for rows of the token tiles the down GEMM
    split along K the sum of their parts in y and y_parts (fp32), in part
    order) as float32 (float64 for y)."""
    lay = res["layout"]
    ws = res["_ws"]
    width = cfg.d_ff if which == "h" else cfg.d_model
    if which == "y":
        es = 2 if lay.y_weighted else 4
    else:
        es = 4 if cfg.dtype == "f32" else 2
    off = getattr(lay, which)
    sparts, split_row0 = res.get("down_sched", (1, lay.max_rows))
    out = []
    for r in rows:
        acc = None
        parts = sparts if (which == "y" and r >= split_row0) else 1
        for p in range(parts):
            if p == 0:
                base, rr, pes = off, r, es
            else:
                pes = 4
                base = lay.y_parts + (p - 1) * lay.y_part_rows * width * pes
                rr = r - split_row0
            b = ws[base + rr * width * pes: base + (rr + 1) * width * pes]
            if pes == 2:
                v = as_f32(b.view(torch.int16).cpu().numpy().view(np.uint16))
            else:
                v = b.view(torch.float32).cpu().numpy()
            acc = v.astype(np.float64) if acc is None else acc + v
        out.append(acc if which == "y" else acc.astype(np.float32))
    return np.array(out)


# ---------------------------------------------------------------- checks
def check_permutation(cfg: MoEConfig, inp: dict, res: dict):
    """Integer work, bit-exact, recomputed on the host from the GPU's own
    indices: counts, padded offsets, tile table, stable row maps."""
    T, E, k = cfg.T, cfg.E, cfg.k
    idx = res["idx"]
    assert idx.min() >= 0 and idx.max() < E
    for t in range(0, T, max(1, T // 512)):           # distinct experts per token
        assert len(set(idx[t].tolist())) == k
    counts = np.bincount(idx.ravel(), minlength=E)
    np.testing.assert_array_equal(res["counts"], counts)
    np.testing.assert_array_equal(res["ws_counts"], counts)
    BT = res["layout"].block_rows
    padded = (counts + BT - 1) // BT * BT
    offs = np.concatenate([[0], np.cumsum(padded)])
    np.testing.assert_array_equal(res["offsets"], offs)
    assert res["num_tiles"] == offs[-1] // BT
    te = np.full(res["tile_expert"].shape, -1)
    for e in range(E):
        te[offs[e] // BT: offs[e + 1] // BT] = e
    np.testing.assert_array_equal(res["tile_expert"], te)
    # stable order: (token, slot) ascending inside each expert segment
    want_rt = np.full(res["row_token"].shape, -1)
    want_tr = np.empty((T, k), dtype=np.int64)
    flat_e = idx.ravel()
    order = np.argsort(flat_e, kind="stable")          # pairs grouped by expert, (t,j) order kept
    pos = 0
    for e in range(E):
        pairs = order[pos:pos + counts[e]]
        pos += counts[e]
        rows = offs[e] + np.arange(counts[e])
        want_rt[rows] = pairs // k
        want_tr.reshape(-1)[pairs] = rows
    np.testing.assert_array_equal(res["row_token"], want_rt)
    np.testing.assert_array_equal(res["tok_row"], want_tr)
    if "row_w" in res:   # each row carries its (token, slot)'s gate (padding: unwritten)
        np.testing.assert_array_equal(res["row_w"][want_tr.ravel()], res["w"].ravel())


def check_gather(cfg: MoEConfig, inp: dict, res: dict, rows):
    """Xs rows are bit copies of their tokens' x rows."""
    xs = ws_rows(res, cfg, "xs", rows)
    x = as_f32(inp["x"])
    for i, r in enumerate(rows):
        t = res["row_token"][r]
        assert t >= 0
        np.testing.assert_array_equal(xs[i], x[t])


def check_routing(cfg: MoEConfig, orc: dict, res: dict) -> dict:
    """Indices bit-exact except near ties; gate weights to 1e-5."""
    idx, w = res["idx"], res["w"]
    oidx, og = orc["idx"], orc["gates"]
    near = orc["gap"] < NEAR_TIE
    order_near = orc["order_gap"] < NEAR_TIE
    ok = ~near
    same_order = ok & ~order_near
    np.testing.assert_array_equal(idx[same_order], oidx[same_order])
    np.testing.assert_allclose(w[same_order], og[same_order], rtol=0, atol=1e-5)
    for t in np.nonzero(ok & order_near)[0]:           # robust set, tie inside: compare as sets
        assert set(idx[t].tolist()) == set(oidx[t].tolist())
        gmap = dict(zip(oidx[t].tolist(), og[t].tolist()))
        for e, v in zip(idx[t].tolist(), w[t].tolist()):
            assert abs(gmap[e] - v) <= 1e-5
    mismatched = [int(t) for t in np.nonzero(near)[0]
                  if set(idx[t].tolist()) != set(oidx[t].tolist())]
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-5)
    return dict(near_ties=int(near.sum()), near_tie_mismatches=mismatched,
                order_ties=int((ok & order_near).sum()))


def check_values(cfg: MoEConfig, inp: dict, res: dict, tokens, orc_full=None) -> float:
    """out rows of `tokens` vs the oracle's, routed as the GPU routed them
    (identical to the oracle's own routing except on near ties)."""
    tokens = np.asarray(tokens)
    r = oracle.moe_forward(inp["x"], inp["W_router"], inp["W_gate"], inp["W_up"], inp["W_down"],
                           cfg.k, bias=inp.get("bias"), tokens=tokens,
                           forced_idx=res["idx"].astype(np.int64))
    ref = r["out"]
    got = as_f32(res["out"][tokens]).astype(np.float64)
    assert np.isfinite(got).all()
    err = np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30)
    assert err <= TOL[cfg.dtype], f"max|err|/max|ref| = {err:.3e} > {TOL[cfg.dtype]}"
    return float(err)


def check_hidden_and_expert_outputs(cfg: MoEConfig, inp: dict, res: dict, rows) -> tuple:
    """H = SiLU(W1 x) * W3 x and Y = W2 H of the given permuted rows vs the
    oracle's expert_hidden / swiglu_expert, one oracle call per expert on
    all of that expert's sampled rows.  When the layout stores gate-weighted
    rows (y_weighted), Y is compared with the row's gate times the oracle's
    (the gates themselves are checked by check_routing and check_permutation)."""
    rows = np.asarray(rows, dtype=np.int64)
    rt = res["row_token"]
    offs = res["offsets"]
    expert_of = np.searchsorted(offs, rows, side="right") - 1
    h = ws_rows(res, cfg, "h", rows).astype(np.float64)
    y = ws_rows(res, cfg, "y", rows)
    errs_h, errs_y = [], []
    for e in np.unique(expert_of):
        sel = np.nonzero(expert_of == e)[0]
        toks = rt[rows[sel]]
        assert (toks >= 0).all(), "sampled a padding row"
        xr = inp["x"][toks]
        href = oracle.expert_hidden(xr, inp["W_gate"][e], inp["W_up"][e])
        yref = oracle.swiglu_expert(xr, inp["W_gate"][e], inp["W_up"][e], inp["W_down"][e])
        if res["layout"].y_weighted:
            yref = yref * res["row_w"][rows[sel]].astype(np.float64)[:, None]
        for i, n in enumerate(sel):
            errs_h.append(np.abs(h[n] - href[i]).max() / max(np.abs(href[i]).max(), 1e-30))
            errs_y.append(np.abs(y[n] - yref[i]).max() / max(np.abs(yref[i]).max(), 1e-30))
    eh, ey = max(errs_h), max(errs_y)
    assert eh <= TOL[cfg.dtype] and ey <= TOL[cfg.dtype], (eh, ey)
    return eh, ey


def tile_rows(res: dict, per_tile: int = 1, seed: int = 0) -> np.ndarray:
    """Permuted rows that reach every unit of the grouped GEMMs' work:
    `per_tile` random valid rows of every token tile in use (so every
    (expert, token tile) pair, and with it every XCD share of the tile
    order, is value-checked) plus the first and last valid row of every
    expert segment (the ragged end of its last tile)."""
    lay = res["layout"]
    BT = int(lay.block_rows)
    rt = res["row_token"]
    rng = np.random.default_rng(seed)
    rows = set()
    for t in range(int(res["num_tiles"])):
        valid = np.nonzero(rt[t * BT:(t + 1) * BT] >= 0)[0]
        if valid.size:
            pick = rng.choice(valid, size=min(per_tile, valid.size), replace=False)
            rows.update((t * BT + pick).tolist())
    offs, cnt = res["offsets"], res["ws_counts"]
    for e in range(cnt.size):
        if cnt[e]:
            rows.update([int(offs[e]), int(offs[e] + cnt[e] - 1)])
    return np.array(sorted(rows), dtype=np.int64)


def tile_tokens(res: dict, per_tile: int = 1, seed: int = 0) -> np.ndarray:
    """Tokens whose (token, slot) rows include tile_rows(res, per_tile), plus
    the first, the last and a ragged-tail token."""
    T = res["idx"].shape[0]
    toks = set(res["row_token"][tile_rows(res, per_tile, seed)].tolist())
    toks.update({0, T - 1, max(0, T - 1 - (T % 32))})
    return np.array(sorted(toks), dtype=np.int64)


def sample_tokens(cfg: MoEConfig, orc_idx: np.ndarray, n: int, seed: int = 0) -> np.ndarray:
    """First, last, a ragged-tail token, a random spread, and at least one
    token of every expert that received any."""
    T = cfg.T
    rng = np.random.default_rng(seed)
    picks = {0, T - 1, max(0, T - 1 - (T % 32))}
    picks.update(rng.choice(T, size=min(n, T), replace=False).tolist())
    for e in range(cfg.E):
        hit = np.nonzero((orc_idx == e).any(axis=1))[0]
        if hit.size:
            picks.add(int(hit[rng.integers(hit.size)]))
    return np.array(sorted(picks))
