"""Plant plausible mistakes in the oracle (on the CPU) and check that its pins catch them.

A pin is only worth something if a wrong oracle fails it.  Each case below
replaces one oracle function with a subtly wrong variant and runs the pin
tests that should notice; the test passes when at least one of them fails.
"""
import math

import numpy as np
import pytest

import oracle as o
import oracle.moe_oracle as om
from tests import test_oracle_backward as bpins
from tests import test_oracle_pins as pins


def _topk_ties_high(logits, k):
    l = np.asarray(logits, dtype=np.float32)
    T, E = l.shape
    order = np.lexsort((-np.broadcast_to(np.arange(E), (T, E)), -l), axis=1)
    return order[:, :k].astype(np.int32)


def _weights_no_renorm(logits, idx):
    p = om.softmax(logits)
    return np.take_along_axis(p, np.asarray(idx, dtype=np.int64), 1).astype(np.float32)


def _capacity_without_k(T, E, k, cf):
    cf = float(np.float32(cf))
    if cf <= 0:
        return None
    C = int(math.floor(cf * T / E))
    return None if C == 0 else C


def _gelu_tanh(z):
    return 0.5 * z * (1 + np.tanh(math.sqrt(2 / math.pi) * (z + 0.044715 * z ** 3)))


def _aux_counts_over_T(counts, probs, T, k, E):
    return float(E * np.sum(np.asarray(counts, float) / T * np.asarray(probs).sum(0) / T))


def _logits_no_bias(x, W_gate, logit_bias, dtype):
    return _orig["router_logits"](x, W_gate, None, dtype)


def _permute_unstable(topk_idx, E, C):
    counts, offsets, sorted_slot, slot_pos = _orig["permute"](topk_idx, E, C)
    # reverse the order inside each segment (a sort that is not stable)
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        seg = sorted_slot[a:b][::-1].copy()
        sorted_slot[a:b] = seg
        slot_pos[seg] = np.arange(a, b)
    return counts, offsets, sorted_slot, slot_pos


def _silu_sign(z):
    return z / (1.0 + np.exp(z))


def _binned_keep_last(topk_idx, E, C):
    # fills the buckets with the last C assignments of each expert instead of the first C
    flat = np.asarray(topk_idx).reshape(-1)
    rev = flat[::-1].reshape(-1, 1)
    bins, sp = _orig["binned_layout"](rev, E, C)
    n = flat.size
    bins = np.where(bins >= 0, n - 1 - bins, -1).astype(np.int32)
    return bins, sp[::-1].copy()


def _binned_capacity_no_minimum(T, E, k, cf, min_capacity, counts):
    return _orig["binned_capacity"](T, E, k, cf, 0, counts)


def _softmax_t_times(logits, temperature):
    # multiplies by the temperature instead of dividing
    return _orig["softmax_t"](logits, 1.0 / float(temperature))


def _uniform_transposed(T, k, E):
    return ((np.arange(k)[None, :] * T + np.arange(T)[:, None]) % E).astype(np.int32)


def _noise_ignored(logits, noise):
    return np.asarray(logits, dtype=np.float32)


def _silu_grad_first_term(z):
    return 1.0 / (1.0 + np.exp(-z))


def _gelu_grad_cdf_only(z):
    return 0.5 * (1.0 + om._erf(z / math.sqrt(2.0)))


def _scale_no_abs_on_W2(X, dy_rows, w_rows, a, g, hm_r, W1e, W3e, W2e, act):
    # the magnitude chain with |W2| replaced by W2 (a dropped abs)
    return _orig["expert_grad_scale"](X, dy_rows, w_rows, a, g, hm_r, W1e, W3e, W2e, act) | dict(
        dX=_scale_chain_dx(X, dy_rows, w_rows, a, g, W1e, W3e, W2e, act, abs_w2=False))


def _scale_chain_dx(X, dy_rows, w_rows, a, g, W1e, W3e, W2e, act, abs_w2):
    dO_m = np.abs(w_rows)[:, None] * np.abs(dy_rows)
    dHm_m = dO_m @ (np.abs(W2e) if abs_w2 else W2e).T
    if act == "swiglu":
        return (dHm_m * np.abs(g * om.silu_grad(a))) @ np.abs(W1e).T + (dHm_m * np.abs(om.silu(a))) @ np.abs(W3e).T
    return (dHm_m * np.abs(om.gelu_grad(a))) @ np.abs(W1e).T


def _scale_dg_term_doubled(X, dy_rows, w_rows, a, g, hm_r, W1e, W3e, W2e, act):
    # |W3| enters only the dX chain's dg term: doubling it doubles that term
    return _orig["expert_grad_scale"](X, dy_rows, w_rows, a, g, hm_r, W1e, None if W3e is None else 2 * W3e,
                                      W2e, act)


def _router_scale_difference(l, idx, w, dw_m, counts, d_aux, k, temperature=1.0, soft=False):
    # the renormalisation's two terms subtracted instead of added in the magnitude
    T, E = l.shape
    p = om.softmax_t(l, temperature)
    wk = np.abs(np.asarray(w, np.float64))
    s_m = np.sum(wk * dw_m, axis=1, keepdims=True)
    rows = np.repeat(np.arange(T), k)
    out = np.zeros((T, E))
    if soft:
        gm = np.zeros((T, E))
        np.add.at(gm, (rows, np.asarray(idx).reshape(-1)), dw_m.reshape(-1))
        out += p * np.abs(gm - s_m) / temperature
    else:
        np.add.at(out, (rows, np.asarray(idx).reshape(-1)), (wk * np.abs(dw_m - s_m) / temperature).reshape(-1))
    fe = np.asarray(counts, np.float64) / (T * k)
    out += abs(d_aux) * (E / T) * p * (fe[None, :] + np.sum(p * fe[None, :], 1, keepdims=True)) / temperature
    return out


def _soft_renormalised(logits, topk_idx, temperature, soft=False):
    # the earlier reading: a temperature on the hard top-k, renormalised over the k
    return _orig["topk_weights_t"](logits, topk_idx, temperature, False)


def _soft_grad_selected_only(l, idx, w, dw, counts, d_aux, k, temperature=1.0, soft=False):
    # the soft router's gradient kept only at the selected experts
    dl = _orig["router_logit_grad"](l, idx, w, dw, counts, d_aux, k, temperature, soft)
    if soft:
        aux_only = _orig["router_logit_grad"](l, idx, w, np.zeros_like(dw), counts, d_aux, k, temperature, soft)
        sel = np.zeros(dl.shape, bool)
        np.put_along_axis(sel, np.asarray(idx, np.int64), True, axis=1)
        dl = np.where(sel, dl, aux_only)
    return dl


_orig = {n: getattr(om, n) for n in ("router_logits", "permute", "binned_layout", "binned_capacity", "softmax_t",
                                     "expert_grad_scale", "topk_weights_t", "router_logit_grad")}

MUTANTS = [
    ("select_topk", _topk_ties_high, ["test_topk_ties_and_signed_zero"]),
    ("topk_weights", _weights_no_renorm, ["test_top2_worked_example", "test_topk_weights_invariants"]),
    ("expert_capacity", _capacity_without_k, ["test_capacity_closed_forms"]),
    ("gelu", _gelu_tanh, ["test_gelu_silu_vs_math"]),
    ("aux_loss", _aux_counts_over_T, ["test_aux_uniform_counts_is_one_and_collapse_is_E"]),
    ("router_logits", _logits_no_bias, ["test_k_equals_E_is_dense_softmax_mixture"]),
    ("permute", _permute_unstable, ["test_histogram_worked_example_dropless"]),
    ("silu", _silu_sign, ["test_gelu_silu_vs_math", "test_single_expert_is_plain_ffn"]),
    ("binned_layout", _binned_keep_last, ["test_binned_worked_example"]),
    ("binned_capacity", _binned_capacity_no_minimum, ["test_binned_capacity_rules", "test_binned_worked_example"]),
    ("softmax_t", _softmax_t_times, ["test_temperature_closed_form_on_the_worked_example"]),
    ("uniform_assignment", _uniform_transposed, ["test_uniform_assignment_ids_counts_and_aux"]),
    ("noisy_logits", _noise_ignored, ["test_noise_decides_the_selection"]),
    ("silu_grad", _silu_grad_first_term, ["backward:swiglu"]),
    ("gelu_grad", _gelu_grad_cdf_only, ["backward:gelu"]),
    ("expert_grad_scale", _scale_no_abs_on_W2, ["scale:bounds", "scale:brute"]),
    ("expert_grad_scale", _scale_dg_term_doubled, ["scale:equal", "scale:brute"]),
    ("router_logit_grad_scale", _router_scale_difference, ["scale:bounds", "scale:brute"]),
    ("topk_weights_t", _soft_renormalised, ["test_soft_topk_closed_form_on_the_worked_example"]),
    ("router_logit_grad", _soft_grad_selected_only, ["backward:soft", "backward:soft-unselected"]),
]


def _run(test_name):
    if test_name == "backward:soft":
        return bpins.test_backward_router_variants_vs_torch_autograd("soft-temperature-noise", "swiglu", 0.6, 0.8)
    if test_name == "backward:soft-unselected":
        return bpins.test_soft_topk_reaches_unselected_experts()
    if test_name.startswith("backward:"):
        act = test_name.split(":")[1]
        return bpins.test_backward_vs_torch_autograd(act, 0.0, 0.5, 2, 5)
    if test_name == "scale:bounds":
        for args in (("swiglu", 0.0, 0.0, 2, None), ("swiglu", 0.6, 0.7, 3, "soft"), ("gelu", 0.5, 1.1, 2, None)):
            bpins.test_grad_scale_bounds_every_gradient(*args)
        return None
    if test_name == "scale:equal":
        return bpins.test_grad_scale_equals_gradient_without_cancellation("swiglu")
    if test_name == "scale:brute":
        return bpins.test_grad_scale_vs_brute_force_chain()
    fn = getattr(pins, test_name)
    if test_name == "test_k_equals_E_is_dense_softmax_mixture":
        return fn("swiglu")
    return fn()


@pytest.mark.parametrize("target,mutant,catchers", MUTANTS, ids=[m[1].__name__.lstrip("_") for m in MUTANTS])
def test_pins_catch_planted_mistake(monkeypatch, target, mutant, catchers):
    monkeypatch.setattr(om, target, mutant)
    monkeypatch.setattr(o, target, mutant, raising=False)
    caught = False
    for name in catchers:
        try:
            _run(name)
        except AssertionError:
            caught = True
    assert caught, f"no pin caught the planted mistake in {target}"
