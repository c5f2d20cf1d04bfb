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


MUTANTS = {
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
