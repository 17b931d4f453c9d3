"""GPU parity of the router variants (moe_route_ex, moe_layer_forward_ex) against the
oracle's route / layer_forward with the same variant inputs.

Mode A as elsewhere: the oracle selects on the GPU router's fp32 logits (with jitter,
the logits of the jittered input, which are themselves compared with the oracle's),
so every integer decision is shared and compared bit for bit.
"""
import numpy as np
import pytest

import moe_workloads as mw
import oracle as o
import top_routing_expert_moe_amd as moe
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

VARIANTS = {
    "noise": dict(noise=True),
    "temperature-0.5": dict(temperature=0.5),
    "noise-temperature-2": dict(noise=True, temperature=2.0),
    "uniform": dict(uniform=True),
    "jitter": dict(jitter=True),
    "all": dict(jitter=True, noise=True, temperature=0.7, uniform=True),
    "soft": dict(soft=True),
    "soft-temperature-0.5": dict(soft=True, temperature=0.5),
    "soft-noise-jitter-1.5": dict(soft=True, noise=True, jitter=True, temperature=1.5),
}


def _say(*a):
    print(*a, flush=True)


def _variant_args(w, spec, dev_dtype):
    vi = mw.router_variant_inputs(w)
    host = dict(jitter=vi["jitter"] if spec.get("jitter") else None,
                noise=vi["noise"] if spec.get("noise") else None,
                temperature=spec.get("temperature", 1.0), uniform=spec.get("uniform", False),
                soft=spec.get("soft", False))
    dev = dict(jitter=gu.to_dev(host["jitter"], dev_dtype) if host["jitter"] is not None else None,
               noise=gu.to_dev(host["noise"], "f32") if host["noise"] is not None else None,
               temperature=host["temperature"], uniform=host["uniform"], soft=host["soft"])
    return host, dev


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("name", ["tiny-fp32", "decode-mixtral", "prefill-mixtral", "capacity-e64",
                                  "finegrained-e256"])
def test_route_variant_parity(name, variant):
    torch = gu.torch()
    w = mw.by_name(name)
    _say(f"route {name} {variant}")
    d = mw.make_inputs(w, with_weights=False)
    x = gu.to_dev(d["x"], w.dtype)
    Wg = gu.to_dev(d["W_gate"], "f32")
    b = gu.to_dev(d["logit_bias"], "f32")
    host, dev = _variant_args(w, VARIANTS[variant], w.dtype)
    logits, idx, wt, ps = moe.route(x, Wg, b, w.k, with_prob_sum=True, **dev)
    torch.cuda.synchronize()
    gl = gu.from_dev(logits)
    xr = d["x"] if host["jitter"] is None else o.jitter_input(d["x"], host["jitter"], w.dtype)
    gu.check_rel_rms(gl, o.router_logits(xr, d["W_gate"], d["logit_bias"], w.dtype), 1e-5, "logits")
    ref = o.route(gl, w.k, noise=host["noise"], temperature=host["temperature"], uniform=host["uniform"],
                  soft=host["soft"])
    assert np.array_equal(gu.from_dev(idx), ref["topk_idx"])
    gu.check_rel_rms(gu.from_dev(wt), ref["topk_w"], 1e-5, "topk_w")
    if host["soft"] and w.k < w.E:
        assert (gu.from_dev(wt).astype(np.float64).sum(1) < 1.0).all()   # mass left to unselected experts
    gu.check_rel_rms(gu.from_dev(ps), ref["probs"].sum(0), 1e-5, "prob_sum")


@pytest.mark.parametrize("name,variant", [("tiny-fp32", "all"), ("capacity-e64", "noise-temperature-2"),
                                          ("capacity-e64", "jitter"), ("prefill-mixtral", "uniform"),
                                          ("decode-mixtral", "all"), ("decode-mixtral", "soft"),
                                          ("prefill-mixtral", "soft-temperature-0.5"),
                                          ("capacity-e64", "soft-noise-jitter-1.5"), ("tiny-fp32", "soft"),
                                          ("prefill-mixtral", "all"), ("prefill-mixtral", "noise-temperature-2")])
def test_layer_forward_variant_parity(name, variant):
    torch = gu.torch()
    _say(f"layer {name} {variant}")
    w, host_in, dd = gu.workload(name)
    host, dev = _variant_args(w, VARIANTS[variant], w.dtype)
    args = (dd["x"], dd["W_gate"], dd["logit_bias"], dd["W1"], dd["W3"], dd["W2"])
    y, aux, counts = moe.layer_forward(*args, k=w.k, capacity_factor=w.cf, act=w.act, **dev)
    logits, _, _, _ = moe.route(dd["x"], dd["W_gate"], dd["logit_bias"], w.k, jitter=dev["jitter"])
    torch.cuda.synchronize()
    if w.T <= 64:
        tokens = np.arange(w.T)
    else:
        tokens = np.sort(np.random.default_rng(77).choice(w.T, 256, replace=False))
    ref = o.layer_forward(host_in["x"], host_in["W_gate"], host_in["logit_bias"], host_in["W1"], host_in["W3"],
                          host_in["W2"], k=w.k, capacity_factor=w.cf, act=w.act, dtype=w.dtype,
                          logits=gu.from_dev(logits), tokens=tokens, noise=host["noise"],
                          temperature=host["temperature"], uniform=host["uniform"], soft=host["soft"])
    assert np.array_equal(gu.from_dev(counts), ref["counts"])
    if host["uniform"]:
        assert len(set(ref["counts"].tolist())) <= 2   # balanced up to one when E does not divide T*k
    a = float(gu.from_dev(aux))
    assert abs(a - ref["aux"]) <= 1e-5 * abs(ref["aux"]), (a, ref["aux"])
    got = gu.as_f64(gu.from_dev(y)[tokens], w.dtype)
    if w.dtype == "bf16":
        raw, beyond = gu.check_bf16_out(got, ref["y64"], "y")
        _say(f"  y max|d|/RMS = {raw:.4f} (beyond the output's own bf16 rounding: {beyond:.4f})")
    else:
        gu.check_rel_rms(got, ref["y64"], 1e-5, "y")


def test_zero_noise_through_the_variant_entry_point_is_the_plain_layer():
    torch = gu.torch()
    w, _, dd = gu.workload("capacity-e64")
    args = (dd["x"], dd["W_gate"], dd["logit_bias"], dd["W1"], dd["W3"], dd["W2"])
    kw = dict(k=w.k, capacity_factor=w.cf, act=w.act)
    y0, aux0, c0 = moe.layer_forward(*args, **kw)
    zero = torch.zeros((w.T, w.E), dtype=torch.float32, device=dd["x"].device)
    y1, aux1, c1 = moe.layer_forward(*args, **kw, noise=zero)
    torch.cuda.synchronize()
    assert np.array_equal(gu.from_dev(y0), gu.from_dev(y1))
    assert np.array_equal(gu.from_dev(c0), gu.from_dev(c1))
    assert float(gu.from_dev(aux0)) == float(gu.from_dev(aux1))
