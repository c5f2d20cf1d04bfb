"""The oracle's pins are sensitive: each plausible mistake planted in the
oracle (on the CPU, by monkeypatching) makes at least one pin fail."""
import numpy as np
import pytest

import oracle
from oracle import moe_oracle as om
from tests import test_oracle_pins as pins


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(om, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def swapped_gate_up(xrows, Wg, Wu, Wd):
    xr = om.to_f64(xrows)
    return (om.silu(xr @ om.to_f64(Wu).T) * (xr @ om.to_f64(Wg).T)) @ om.to_f64(Wd).T


def down_not_transposed(xrows, Wg, Wu, Wd):
    xr = om.to_f64(xrows)
    return (om.silu(xr @ om.to_f64(Wg).T) * (xr @ om.to_f64(Wu).T)) @ om.to_f64(Wd)


def silu_wrong_sign(z):
    return z / (1.0 + np.exp(z))


def topk_ties_high(s, k):
    order = np.argsort(-s[:, ::-1], axis=1, kind="stable")
    return np.ascontiguousarray((s.shape[1] - 1 - order)[:, :k])


def topk_smallest(s, k):
    return np.ascontiguousarray(np.argsort(s, axis=1, kind="stable")[:, :k])


def gates_full_softmax(s, idx):
    z = np.exp(s - s.max(axis=1, keepdims=True))
    return np.take_along_axis(z / z.sum(axis=1, keepdims=True), idx, axis=1)


def router_transposed(x, W_router, bias=None):
    # reads a [d][E] matrix as if it were stored [E][d]
    W = om.to_f64(W_router)
    return om.to_f64(x) @ W.reshape(W.shape[1], W.shape[0]).T


def rms_mean_abs(x, weight, eps):
    xf = om.to_f64(x)
    return xf / (np.abs(xf).mean(axis=1, keepdims=True) + eps) * om.to_f64(weight)[None, :]


def rms_centred(x, weight, eps):
    xf = om.to_f64(x)
    return (xf - xf.mean(axis=1, keepdims=True)) / np.sqrt(xf.var(axis=1, keepdims=True) + eps) \
        * om.to_f64(weight)[None, :]


def _q4_variant(nibble_swap=False, scale_div=7.0, half_away=False):
    def q4(W, group):
        Wf = om._as_f32(W)
        K = Wf.shape[-1]
        G = Wf.reshape(Wf.shape[:-1] + (K // group, group))
        scale = (np.abs(G).max(axis=-1) / np.float32(scale_div)).astype(np.float32)
        safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
        r = (G / safe[..., None]).astype(np.float32)
        q = np.sign(r) * np.floor(np.abs(r) + 0.5) if half_away else np.rint(r)
        q = np.where(scale[..., None] > 0, np.clip(q, -8, 7), 0).astype(np.int64)
        u = (q + 8).reshape(Wf.shape).astype(np.uint8)
        a, b = (u[..., 1::2], u[..., 0::2]) if nibble_swap else (u[..., 0::2], u[..., 1::2])
        return (a | (b << 4)).astype(np.uint8), np.ascontiguousarray(np.swapaxes(scale, -1, -2))
    return q4


def deq4_no_offset(packed, scales, group):
    packed = np.asarray(packed, dtype=np.uint8)
    q = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.int64)
    q[..., 0::2] = packed & 15
    q[..., 1::2] = packed >> 4
    return q * np.repeat(np.swapaxes(np.asarray(scales, dtype=np.float64), -1, -2), group,
                         axis=-1)


def silu_grad_sigma_only(z):
    return 1.0 / (1.0 + np.exp(-z))


MUTANTS = {
    "silu_grad:sigma_only": ("silu_grad", silu_grad_sigma_only,
                             [lambda: pins.test_backward_matches_central_differences(0.0, False, 2)]),
    "quantize_int4:nibbles_swapped": ("quantize_int4", _q4_variant(nibble_swap=True),
                                      [pins.test_int4_worked_example]),
    "quantize_int4:scale_over_8": ("quantize_int4", _q4_variant(scale_div=8.0),
                                   [pins.test_int4_exact_recovery,
                                    pins.test_int4_error_bound_and_range]),
    "quantize_int4:round_half_away": ("quantize_int4", _q4_variant(half_away=True),
                                      [pins.test_int4_worked_example]),
    "dequantize_int4:no_offset": ("dequantize_int4", deq4_no_offset,
                                  [pins.test_int4_exact_recovery,
                                   pins.test_int4_error_bound_and_range]),
    "rms_norm:mean_abs": ("rms_norm", rms_mean_abs, [pins.test_rms_norm_closed_forms]),
    "rms_norm:centred": ("rms_norm", rms_centred, [pins.test_rms_norm_closed_forms]),
    "swiglu_expert:swapped_gate_up": ("swiglu_expert", swapped_gate_up,
                                      [pins.test_expert_scalar_worked_example]),
    "swiglu_expert:down_not_transposed": ("swiglu_expert", down_not_transposed,
                                          [pins.test_expert_brute_force]),
    "silu:wrong_sign": ("silu", silu_wrong_sign, [pins.test_silu_closed_forms]),
    "select_topk:ties_high": ("select_topk", topk_ties_high, [pins.test_topk_ties_go_to_lower_index]),
    "select_topk:smallest": ("select_topk", topk_smallest,
                             [lambda: pins.test_topk_matches_brute_force_enumeration(5)]),
    "topk_gates:full_softmax": ("topk_gates", gates_full_softmax, [pins.test_gates_closed_forms]),
    "router_logits:transposed": ("router_logits", router_transposed,
                                 [pins.test_logits_orientation_one_hot_rows]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn, checks = MUTANTS[name]
    _patch(monkeypatch, attr, fn)
    for check in checks:
        with pytest.raises(Exception):
            check()
    # the whole-layer pin catches every mistake in the layer's arithmetic too
    if attr in ("swiglu_expert", "silu", "topk_gates"):
        with pytest.raises(Exception):
            pins.test_layer_equals_dense_keep_topk_formulation(4, 2)


def test_int4_mutant_base_is_the_oracle():
    # the INT4 mutants differ from the oracle only by the planted mistake
    rng = np.random.default_rng(3)
    W = rng.standard_normal((5, 64)).astype(np.float32)
    for g in (32, 64):
        p0, s0 = oracle.quantize_int4(W, g)
        p1, s1 = _q4_variant()(W, g)
        np.testing.assert_array_equal(p0, p1)
        np.testing.assert_array_equal(s0, s1)


# mistakes planted inside moe_backward by editing one line of its source
BACKWARD_EDITS = {
    "k_softmax_without_subtraction": ("ds_sel = g * (dg - (g * dg).sum(axis=1, keepdims=True))",
                                      "ds_sel = g * dg"),
    "gate_up_swapped_in_dx": ("dx[rows] += da @ W1 + db @ W3", "dx[rows] += da @ W3 + db @ W1"),
    "up_grad_without_silu": ("db = dh * silu(a)", "db = dh * a"),
    "balance_sign": ("ds += P * (c[None, :] - (P * c[None, :]).sum(axis=1, keepdims=True))",
                     "ds -= P * (c[None, :] - (P * c[None, :]).sum(axis=1, keepdims=True))"),
    "gate_scale_missing": ("dy = g[rows, slots][:, None] * go[rows]", "dy = go[rows]"),
    "router_path_dropped": ("dx += ds @ Wr.T", "dx += (ds @ Wr.T) * 0"),
}


def _edited_backward(old, new):
    import inspect
    import textwrap
    src = textwrap.dedent(inspect.getsource(om.moe_backward))
    assert src.count(old) == 1, old
    ns = dict(vars(om))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    return ns["moe_backward"]


@pytest.mark.parametrize("edit", sorted(BACKWARD_EDITS))
def test_backward_pins_catch_planted_mistake(edit, monkeypatch):
    _patch(monkeypatch, "moe_backward", _edited_backward(*BACKWARD_EDITS[edit]))
    failed = 0
    for args in ((0.0, False, 2), (0.05, True, 2)):
        try:
            pins.test_backward_matches_central_differences(*args)
        except AssertionError:
            failed += 1
    assert failed > 0


def test_backward_edit_base_is_the_oracle():
    fn = _edited_backward("dx += ds @ Wr.T", "dx += ds @ Wr.T")
    args = pins._bwd_case(5)
    a = fn(*args[:5], args[6], 2, bias=args[5], alpha=0.1)
    b = om.moe_backward(*args[:5], args[6], 2, bias=args[5], alpha=0.1)
    for n in ("dx", "dW_router", "dW_gate", "dW_up", "dW_down", "dbias"):
        np.testing.assert_array_equal(a[n], b[n])
