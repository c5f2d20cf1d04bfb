"""Plain CPU fp64 oracle of the Mixtral-style sparse MoE feed-forward layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the package entry's smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP path; the
two meet only in the seeded inputs they are both handed.

Every step follows the definitions on the pages, in fp64, with numpy's matmul
and sort as library primitives and no blocking, fusion or reordering beyond
what the definitions state:

* "Mistral/Mixtralのアーキテクチャ" (disassemble-channel.com), section
  "Top-2ゲーティングの定式化": router scores s = W_g x with no bias term;
  the top-2 indices i1, i2 with s_i1 >= s_i2; gates g_ik = exp(s_ik) /
  (exp(s_i1) + exp(s_i2)), a softmax over the selected scores only; and
  MoE(x) = g_i1 E_i1(x) + g_i2 E_i2(x).
* same page, section "各エキスパートの構造": E_i(x) applies SiLU to W1 x,
  multiplies elementwise by W3 x and projects with W2, where W1, W3 are
  d_ff x d_model, W2 is d_model x d_ff and SiLU(z) = z * sigma(z).  The
  equation as printed right-multiplies by W2, which does not type-check with
  those shapes; the page's SwiGLUExpert code (section "MoEレイヤー全体の実装")
  applies w2 to silu(w1 x) * w3 x, and that reading is taken here.
* same page, section "ロードバランス損失": f_i, p_i and L_balance.
* "Mixtral of Experts" (singularity-lens.com), the layer-output formula
  y = sum_i g_i(x) E_i(x) with g(x) = Softmax(KeepTopK(H(x), 2)) and
  H(x)_i = (x . W_g)_i: the router matrix is stored here as W_router[d][E],
  the orientation of that formula.

Readings where the pages are silent (each also listed in the design notes):
top-k is generalised from top-2 to any 1 <= k <= E; equal scores are broken
in favour of the lower expert index, both for membership and for order; an
optional per-expert router bias (an extension the pages do not have) is added
to the scores before both the selection and the softmax; every token is
routed to exactly k experts (no capacity limit or token dropping).

* "Mistral/Mixtralのアーキテクチャ", section "ロードバランス損失": the
  training loss is the language-model loss plus L_balance; moe_backward
  gives the layer's part of its gradient, that of
  <dOut, MoE(x)> + alpha * N * sum_i f_i p_i for an upstream gradient dOut.
* "Mixtral of Experts" (singularity-lens.com), its list of limitations, the
  item on memory requirements and offloading: the model needs INT4
  quantisation to fit in about 25-30 GB.  The pages give no scheme; the plain
  weight-only symmetric per-group reading is taken (quantize_int4 below).

Parity pins: every function here is pinned by tests/test_oracle_pins.py
against closed forms, brute force and special cases fixed by the pages.
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------
# input decoding (exact): bf16 patterns -> float64, float32 -> float64
# ----------------------------------------------------------------------------

def to_f64(a: np.ndarray) -> np.ndarray:
    """Exact conversion of a host array to float64.  uint16 arrays hold
    bfloat16 bit patterns (the top half of a float32)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if a.dtype in (np.float32, np.float64):
        return a.astype(np.float64)
    raise TypeError(f"unsupported dtype {a.dtype}")


# ----------------------------------------------------------------------------
# router
# ----------------------------------------------------------------------------

def router_logits(x, W_router, bias=None) -> np.ndarray:
    """Scores s[t][e] = sum_j x[t][j] * W_router[j][e]  (+ bias[e]).

    "Top-2ゲーティングの定式化" eq. s = W_g x (W_g in R^{N x d}); stored
    transposed as W_router[d][E], i.e. H(x)_i = (x . W_g)_i of the
    "Mixtral of Experts" layer formula.  The pages' router has no bias; the
    optional bias is an extension used only by the skewed workload."""
    s = to_f64(x) @ to_f64(W_router)
    if bias is not None:
        s = s + to_f64(bias)[None, :]
    return s


def select_topk(s: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores per token, in descending score order;
    equal scores go to the lower expert index first.

    "Top-2ゲーティングの定式化": {i1, i2} = Top-2(s) with s_i1 >= s_i2,
    generalised to k."""
    T, E = s.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    order = np.argsort(-s, axis=1, kind="stable")
    return np.ascontiguousarray(order[:, :k])


def topk_gates(s: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Gate weights: softmax over the selected scores only.

    "Top-2ゲーティングの定式化" eq. g_ik = exp(s_ik) / sum_l exp(s_il).
    Subtracting the largest selected score first leaves the ratio unchanged
    and keeps exp finite."""
    sel = np.take_along_axis(s, idx, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def routing_gaps(s: np.ndarray, k: int):
    """(gap, order_gap) per token.  gap = k-th largest score minus the
    (k+1)-th (+inf when k = E): below a small threshold the selected set is
    not robustly defined.  order_gap = the smallest difference between
    adjacent selected scores (+inf when k = 1): below a threshold the order
    inside the set is not robust."""
    T, E = s.shape
    srt = -np.sort(-s, axis=1)
    gap = srt[:, k - 1] - srt[:, k] if k < E else np.full(T, np.inf)
    if k > 1:
        order_gap = (srt[:, :k - 1] - srt[:, 1:k]).min(axis=1)
    else:
        order_gap = np.full(T, np.inf)
    return gap, order_gap


# ----------------------------------------------------------------------------
# expert
# ----------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigma(z), sigma the logistic function
    ("各エキスパートの構造")."""
    return z / (1.0 + np.exp(-z))


def expert_hidden(xrows, W_gate_e, W_up_e) -> np.ndarray:
    """The expert's hidden activation SiLU(W1 x) * W3 x, [n][d_ff], with
    W_gate = W1 [d_ff][d] and W_up = W3 [d_ff][d] ("各エキスパートの構造")."""
    xr = to_f64(xrows)
    u = xr @ to_f64(W_gate_e).T        # W1 x       [n][d_ff]
    v = xr @ to_f64(W_up_e).T          # W3 x       [n][d_ff]
    return silu(u) * v


def swiglu_expert(xrows, W_gate_e, W_up_e, W_down_e) -> np.ndarray:
    """One expert on a block of rows: W2 (SiLU(W1 x) * W3 x), W_down = W2
    [d][d_ff] ("各エキスパートの構造"; the page's SwiGLUExpert code fixes the
    order: w2 is applied to the product)."""
    return expert_hidden(xrows, W_gate_e, W_up_e) @ to_f64(W_down_e).T   # [n][d]


# ----------------------------------------------------------------------------
# layer
# ----------------------------------------------------------------------------

def moe_forward(x, W_router, W_gate, W_up, W_down, k, bias=None, tokens=None,
                forced_idx=None, keep_expert_outputs=False) -> dict:
    """The MoE layer, MoE(x) = sum_j g_ij E_ij(x) over the k selected experts
    ("Top-2ゲーティングの定式化", last equation; "Mixtral of Experts" layer
    formula), token by token.

    tokens:      optional 1-D array of token ids: the routing is computed for
                 every token, the expert outputs only for these (rows of
                 ``out`` follow this order).
    forced_idx:  optional [T][k] expert ids to use instead of the router's
                 choice (gates are then the softmax over those scores); used
                 to value-check tokens whose selection is a near tie.
    Returns a dict: out [n][d] fp64, idx [T][k], gates [T][k], logits [T][E],
    counts [E], gap [T], order_gap [T], tokens [n], and with
    keep_expert_outputs the per-(token, slot) expert outputs y [n][k][d]."""
    xf = to_f64(x)
    T = xf.shape[0]
    E = np.asarray(W_router).shape[1]
    s = router_logits(xf, W_router, bias)
    idx = select_topk(s, k) if forced_idx is None else np.asarray(forced_idx, dtype=np.int64)
    if idx.shape != (T, k):
        raise ValueError("forced_idx must be [T][k]")
    g = topk_gates(s, idx)
    gap, order_gap = routing_gaps(s, k)
    counts = np.bincount(idx.reshape(-1), minlength=E)

    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    n = tok.shape[0]
    d = xf.shape[1]
    y = np.zeros((n, k, d))
    sub_idx = idx[tok]                                  # [n][k]
    for e in range(E):
        rows, slots = np.nonzero(sub_idx == e)
        if rows.size == 0:
            continue
        y[rows, slots] = swiglu_expert(xf[tok[rows]], W_gate[e], W_up[e], W_down[e])
    out = np.zeros((n, d))
    for j in range(k):                                  # sum in slot order
        out += g[tok, j][:, None] * y[:, j]
    res = dict(out=out, idx=idx, gates=g, logits=s, counts=counts, gap=gap,
               order_gap=order_gap, tokens=tok)
    if keep_expert_outputs:
        res["y"] = y
    return res


# ----------------------------------------------------------------------------
# transformer-block wrapper: RMSNorm before, residual after
# ----------------------------------------------------------------------------

def rms_norm(x, weight, eps) -> np.ndarray:
    """RMSNorm(x) = x / sqrt(mean_j x_j^2 + eps) * weight, per token.

    The architecture page (section on Mixtral's block structure) places an
    RMSNorm before the MoE layer and a residual connection after it, without
    defining RMSNorm; this is its plain definition, with a per-feature weight
    and eps as parameters."""
    xf = to_f64(x)
    ms = (xf * xf).mean(axis=1, keepdims=True)
    return xf / np.sqrt(ms + float(eps)) * to_f64(weight)[None, :]


def block_forward(x, norm_weight, eps, W_router, W_gate, W_up, W_down, k, bias=None,
                  tokens=None, forced_idx=None) -> dict:
    """One MoE sub-block: out = x + MoE(RMSNorm(x)) ("Mistral/Mixtralの
    アーキテクチャ", section "Mixtralのアーキテクチャ": normalisation, the MoE
    layer, then a residual connection).  Returns moe_forward's dict with
    `out` replaced by the block output and `moe_out` the MoE part."""
    xn = rms_norm(x, norm_weight, eps)
    r = moe_forward(xn, W_router, W_gate, W_up, W_down, k, bias=bias, tokens=tokens,
                    forced_idx=forced_idx)
    r["moe_out"] = r["out"]
    r["out"] = to_f64(x)[r["tokens"]] + r["moe_out"]
    r["x_norm"] = xn
    return r


# ----------------------------------------------------------------------------
# router statistics and load-balancing loss (forward value only)
# ----------------------------------------------------------------------------

def balance_stats(logits: np.ndarray, idx: np.ndarray, alpha: float = 0.01) -> dict:
    """Router statistics of "ロードバランス損失":
      f_i = (1/T) sum_t 1[i in TopK(s_t)]   (fraction of tokens routed to i)
      p_i = (1/T) sum_t softmax(s_t)_i      (full softmax over all N experts)
      L   = alpha * N * sum_i f_i p_i
    f sums to k (the page's own uniform example has f_i = 2/N for top-2), so
    under uniform routing L = k * alpha.  The page's remark that uniform use
    gives L = alpha conflicts with that example; the definitions are taken
    as written."""
    s = np.asarray(logits, dtype=np.float64)
    T, E = s.shape
    f = np.bincount(np.asarray(idx).reshape(-1), minlength=E) / T
    z = np.exp(s - s.max(axis=1, keepdims=True))
    p = (z / z.sum(axis=1, keepdims=True)).mean(axis=0)
    return dict(f=f, p=p, loss=alpha * E * float((f * p).sum()))


def expert_param_count(d_model: int, d_ff: int) -> int:
    """Parameters of one SwiGLU expert: W1, W3 (d_ff x d_model) and W2
    (d_model x d_ff), "各エキスパートの構造"."""
    return 3 * d_model * d_ff


# ----------------------------------------------------------------------------
# weight-only INT4 expert weights
# ----------------------------------------------------------------------------

INT4_QMAX = 7          # largest code magnitude used by the scale
INT4_OFFSET = 8        # stored nibble = code + 8, codes in [-8, 7]


def _as_f32(W) -> np.ndarray:
    """bf16 bit patterns (uint16) or float arrays -> float32, exactly."""
    W = np.asarray(W)
    if W.dtype == np.uint16:
        return (W.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return W.astype(np.float32)


def quantize_int4(W, group: int):
    """Weight-only INT4 quantisation of weight matrices W [..., N, K] (N
    output rows, K input features) in groups of `group` consecutive input
    features of one row.

    "Mixtral of Experts" (limitations, memory item) names INT4 quantisation
    without a scheme; the reading taken is symmetric per group:
        s   = max_{k in group} |w_k| / 7                  (float32)
        q_k = clamp(rint(w_k / s), -8, 7), q_k = 0 if s = 0 (float32 division,
                                                           ties to even)
    The scale and every code are decided in float32 (the precision of the
    stored scale), so any implementation that divides with IEEE rounding
    reaches the same codes.  Storage: nibble u = q + 8; element 2b of a row in
    the low nibble of byte b and element 2b + 1 in the high nibble; scales
    group-major, [..., K/group, N] (the scales of one group of all rows are
    adjacent).

    Returns (packed uint8 [..., N, K/2], scales float32 [..., K/group, N])."""
    Wf = _as_f32(W)
    if Wf.ndim < 2:
        raise ValueError("W must be [..., N, K]")
    K = Wf.shape[-1]
    if K % group or K % 2:
        raise ValueError("K must be a multiple of the group size and even")
    G = Wf.reshape(Wf.shape[:-1] + (K // group, group))
    absmax = np.abs(G).max(axis=-1)                                 # exact in f32
    scale = (absmax / np.float32(INT4_QMAX)).astype(np.float32)    # one f32 rounding
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    ratio = (G / safe[..., None]).astype(np.float32)                 # one f32 rounding
    q = np.clip(np.rint(ratio), -INT4_OFFSET, INT4_QMAX)
    q = np.where(scale[..., None] > 0, q, 0).astype(np.int64)
    u = (q + INT4_OFFSET).reshape(Wf.shape).astype(np.uint8)
    packed = (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)
    return packed, np.ascontiguousarray(np.swapaxes(scale, -1, -2))


def dequantize_int4(packed, scales, group: int) -> np.ndarray:
    """fp64 weights s * q [..., N, K] from quantize_int4's storage (exact: s
    is float32 and q a small integer)."""
    packed = np.asarray(packed, dtype=np.uint8)
    lo = (packed & 0x0F).astype(np.int64) - INT4_OFFSET
    hi = (packed >> 4).astype(np.int64) - INT4_OFFSET
    q = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.int64)
    q[..., 0::2] = lo
    q[..., 1::2] = hi
    s = np.repeat(np.swapaxes(np.asarray(scales, dtype=np.float64), -1, -2), group, axis=-1)
    return q.astype(np.float64) * s


class _Int4Stack:
    """An expert stack of INT4 weights; indexing expert e gives its
    dequantized fp64 matrix (one expert at a time, so full-size stacks need
    no fp64 copy of every expert)."""

    def __init__(self, packed, scales, group):
        self.packed, self.scales, self.group = packed, scales, group

    def __getitem__(self, e):
        return dequantize_int4(self.packed[e], self.scales[e], self.group)


def moe_forward_int4(x, W_router, qweights: dict, group: int, k, bias=None, tokens=None,
                     forced_idx=None) -> dict:
    """The layer with INT4 expert weights: moe_forward on the dequantized
    weights s * q.  qweights holds (packed, scales) for "W_gate", "W_up" and
    "W_down" as quantize_int4 returns them."""
    W = {n: _Int4Stack(*qweights[n], group) for n in ("W_gate", "W_up", "W_down")}
    return moe_forward(x, W_router, W["W_gate"], W["W_up"], W["W_down"], k, bias=bias,
                       tokens=tokens, forced_idx=forced_idx)


# ----------------------------------------------------------------------------
# backward pass
# ----------------------------------------------------------------------------

def silu_grad(z: np.ndarray) -> np.ndarray:
    """d/dz SiLU(z) = sigma(z) * (1 + z * (1 - sigma(z)))."""
    sig = 1.0 / (1.0 + np.exp(-z))
    return sig * (1.0 + z * (1.0 - sig))


def moe_backward(x, W_router, W_gate, W_up, W_down, dout, k, bias=None, alpha=0.0,
                 forced_idx=None) -> dict:
    """Gradients of  L = <dOut, MoE(x)> + alpha * N * sum_i f_i p_i  with
    respect to x, W_router, the bias and the three expert stacks.

    "ロードバランス損失" adds the balance loss to the language-model loss; the
    layer's part of the total gradient is the chain rule through
    MoE(x) = sum_j g_j E_ij(x) (the upstream gradient dOut stands for the
    language-model loss above the layer) plus the balance loss's own term.
    f_i counts top-k selections, which are piecewise constant, so only p_i
    (the mean full softmax) carries gradient.  Steps, per routed (t, j) with
    expert e, a = W1 x_t, b = W3 x_t, h = SiLU(a) * b, y = W2 h:
        dg_tj = <dOut_t, y>,  dy = g_tj dOut_t,  dh = W2^T dy,
        da = dh * b * SiLU'(a),  db = dh * SiLU(a),
        dx_t += W1^T da + W3^T db,  dW2 += dy h^T,  dW1 += da x^T,  dW3 += db x^T;
    the softmax over the selected scores: ds_tij = g_tj (dg_tj - sum_l g_tl dg_tl);
    the balance term: ds_tm += (alpha N / T) P_tm (f_m - sum_i f_i P_ti);
    then dW_router = x^T ds, dbias = sum_t ds_t, dx += ds W_router^T.
    Returns fp64 arrays dx [T][d], dW_router [d][E], dbias [E], dW_gate,
    dW_up [E][d_ff][d], dW_down [E][d][d_ff], and the routing (idx, gates)."""
    xf = to_f64(x)
    T, d = xf.shape
    Wr = to_f64(W_router)
    E = Wr.shape[1]
    go = to_f64(dout)
    s = router_logits(xf, Wr, bias)
    idx = select_topk(s, k) if forced_idx is None else np.asarray(forced_idx, dtype=np.int64)
    g = topk_gates(s, idx)
    f_dim = np.asarray(W_gate[0]).shape[0]
    dx = np.zeros((T, d))
    dg = np.zeros((T, k))
    dW1 = np.zeros((E, f_dim, d))
    dW3 = np.zeros((E, f_dim, d))
    dW2 = np.zeros((E, d, f_dim))
    for e in range(E):
        rows, slots = np.nonzero(idx == e)          # a token picks an expert at most once
        if rows.size == 0:
            continue
        W1, W3, W2 = to_f64(W_gate[e]), to_f64(W_up[e]), to_f64(W_down[e])
        X = xf[rows]
        a = X @ W1.T
        b = X @ W3.T
        h = silu(a) * b
        y = h @ W2.T
        dg[rows, slots] = (go[rows] * y).sum(axis=1)
        dy = g[rows, slots][:, None] * go[rows]
        dh = dy @ W2
        da = dh * b * silu_grad(a)
        db = dh * silu(a)
        dx[rows] += da @ W1 + db @ W3
        dW2[e] = dy.T @ h
        dW1[e] = da.T @ X
        dW3[e] = db.T @ X
    ds = np.zeros((T, E))
    ds_sel = g * (dg - (g * dg).sum(axis=1, keepdims=True))
    np.put_along_axis(ds, idx, ds_sel, axis=1)
    if alpha:
        f = np.bincount(idx.reshape(-1), minlength=E) / T
        z = np.exp(s - s.max(axis=1, keepdims=True))
        P = z / z.sum(axis=1, keepdims=True)
        c = alpha * E * f / T
        ds += P * (c[None, :] - (P * c[None, :]).sum(axis=1, keepdims=True))
    dx += ds @ Wr.T
    return dict(dx=dx, dW_router=xf.T @ ds, dbias=ds.sum(axis=0), dW_gate=dW1, dW_up=dW3,
                dW_down=dW2, idx=idx, gates=g, ds=ds, dg=dg)


def moe_backward_entries(x, W_router, W_gate, W_up, W_down, dout, k, tokens, feats,
                         bias=None, alpha=0.0, forced_idx=None) -> dict:
    """Parts of moe_backward's result at sizes where the whole is too costly,
    each from the same definitions, expert by expert:
      dx[t] for t in `tokens`;
      dW_gate[e][i][:], dW_up[e][i][:] (rows) and dW_down[e][:][i] (columns)
      for (e, i) in `feats`, i a d_ff index.
    dx needs the gate gradients of only its own token; the weight gradients
    need, per routed row of e, only feature i of a, b, W2^T dOut and h.
    Returns dx [len(tokens)][d] and gate/up/down [len(feats)][d] (fp64)."""
    xf = to_f64(x)
    T, d = xf.shape
    Wr = to_f64(W_router)
    E = Wr.shape[1]
    s = router_logits(xf, Wr, bias)
    idx = select_topk(s, k) if forced_idx is None else np.asarray(forced_idx, dtype=np.int64)
    g = topk_gates(s, idx)
    counts = np.bincount(idx.reshape(-1), minlength=E)
    tokens = np.asarray(tokens, dtype=np.int64)
    go_tok = to_f64(dout[tokens])
    dx = np.zeros((tokens.size, d))
    dg = np.zeros((tokens.size, k))
    gate = np.zeros((len(feats), d))
    up = np.zeros((len(feats), d))
    down = np.zeros((len(feats), d))
    for e in range(E):
        mine = [n for n, (fe, _) in enumerate(feats) if fe == e]
        sel = [(n, j) for n, t in enumerate(tokens) for j in range(k) if idx[t, j] == e]
        if not mine and not sel:
            continue
        W1, W3, W2 = to_f64(W_gate[e]), to_f64(W_up[e]), to_f64(W_down[e])
        if sel:                                            # dx of sampled tokens
            ns = np.array([n for n, _ in sel])
            js = np.array([j for _, j in sel])
            ts = tokens[ns]
            Xt = xf[ts]                                    # one row per (token, slot)
            a, b = Xt @ W1.T, Xt @ W3.T
            h = silu(a) * b
            dg[ns, js] = (go_tok[ns] * (h @ W2.T)).sum(axis=1)
            dh = (g[ts, js][:, None] * go_tok[ns]) @ W2
            # a token routes to e in at most one slot, so the rows of ns differ
            dx[ns] += (dh * b * silu_grad(a)) @ W1 + (dh * silu(a)) @ W3
        if mine:
            rows = np.nonzero((idx == e).any(axis=1))[0]   # tokens routed to e
            slot = np.argmax(idx[rows] == e, axis=1)
            gr = g[rows, slot]
            X = xf[rows]
            Go = to_f64(dout[rows])
            for n in mine:
                i = feats[n][1]
                a, b = X @ W1[i], X @ W3[i]
                dh = gr * (Go @ W2[:, i])
                gate[n] = (dh * b * silu_grad(a)) @ X
                up[n] = (dh * silu(a)) @ X
                down[n] = (gr * silu(a) * b) @ Go
    ds = np.zeros((tokens.size, E))
    gt = g[tokens]
    np.put_along_axis(ds, idx[tokens], gt * (dg - (gt * dg).sum(axis=1, keepdims=True)), axis=1)
    if alpha:
        z = np.exp(s[tokens] - s[tokens].max(axis=1, keepdims=True))
        P = z / z.sum(axis=1, keepdims=True)
        c = alpha * E * (counts / T) / T
        ds += P * (c[None, :] - (P * c[None, :]).sum(axis=1, keepdims=True))
    dx += ds @ Wr.T
    return dict(dx=dx, dW_gate_rows=gate, dW_up_rows=up, dW_down_cols=down, idx=idx)
