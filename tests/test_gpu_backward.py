"""GPU parity of the layer's backward pass (moe_layer_backward) against the oracle's
layer_backward.

The oracle routes on the GPU router's fp32 logits (Mode A), so the selection, the
capacity drops and the counts that enter the aux gradient are shared.  Gradients are
compared elementwise: fp32 workloads within 1e-4 (|ref| + RMS) -- the GPU chains five
fp32-accumulated products; bf16 workloads within 2^-5 of the oracle's magnitude scale
(the gradient's chain of products over absolute values, see layer_backward), plus half
a bf16 ulp for the bf16 dx.  The GPU rounds dO and da | dg to bf16 (2^-9 each, relative
to the scale), its forward's bf16 Hm may round one ulp away from the oracle's where the
fp32 pre-activation sits on a rounding boundary (up to 2^-7), and it accumulates
K <= 2f terms in fp32: at most about 2^-6.5 together, so 2^-5 leaves twice that.
Full-size prefill and fine-grained layers compare dx on sampled tokens and the weight
gradients of the expert with the fewest rows (the oracle's fp64 work is bounded to
those).
"""
import math

import numpy as np
import pytest

import moe_workloads as mw
import oracle as o
import top_routing_expert_moe_amd as moe
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

D_AUX = 0.5


def _say(*a):
    print(*a, flush=True)


def _dy(T, h, dtype, seed=17):
    a = np.random.default_rng(seed).standard_normal((T, h)).astype(np.float32)
    return mw.f32_to_bf16_bits(a) if dtype == "bf16" else a


def _run(w, dd, dy_host):
    torch = gu.torch()
    dt = moe.BF16 if w.dtype == "bf16" else moe.F32
    a = moe.SWIGLU if w.act == "swiglu" else moe.GELU
    fws = moe._ws(moe.workspace_bytes(w.T, w.h, w.f, w.E, w.k, w.cf, dt, a), dd["x"].device)
    args = (dd["x"], dd["W_gate"], dd["logit_bias"], dd["W1"], dd["W3"], dd["W2"])
    moe.layer_forward(*args, k=w.k, capacity_factor=w.cf, act=w.act, ws=fws)
    logits, _, _, _ = moe.route(dd["x"], dd["W_gate"], dd["logit_bias"], w.k)
    dy = gu.to_dev(dy_host, w.dtype)
    g = moe.layer_backward(dd["x"], dd["W_gate"], dd["W1"], dd["W3"], dd["W2"], dy, k=w.k, capacity_factor=w.cf,
                           act=w.act, fwd_ws=fws, d_aux=D_AUX)
    torch.cuda.synchronize()
    return g, gu.from_dev(logits)


def _cmp(got, ref, dtype, what, scale=None, bf16_out=False):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if dtype == "bf16":
        d = np.abs(got - ref)
        bound = 2.0 ** -5 * np.asarray(scale, np.float64)
        if bf16_out:
            bound = bound + gu.half_ulp_bf16(ref)
        bound = bound + 1e-30
        bad = d > bound
        rms = float(np.sqrt(np.mean(ref ** 2))) or 1.0
        assert not bad.any(), (f"{what}: {int(bad.sum())} of {d.size} beyond 2^-5 scale; worst ratio "
                               f"{float((d / bound).max()):.2f}")
        _say(f"  {what}: max|d|/RMS {d.max() / rms:.4f}, max |d| / bound {float((d / bound).max()):.3f}")
    else:
        gu.check_rel_rms(got, ref, 1e-4, what)


def _check_all(w, host, g, gl, dy_host, tokens=None, experts=None, with_w_gate=True, variants=None):
    ref = o.layer_backward(host["x"], host["W_gate"], host["logit_bias"], host["W1"], host["W3"], host["W2"],
                           dy_host, D_AUX, k=w.k, capacity_factor=w.cf, act=w.act, dtype=w.dtype, logits=gl,
                           tokens=tokens, experts=experts, with_w_gate=with_w_gate, with_scale=True,
                           **(variants or {}))
    sc = ref["scale"]
    tok = np.arange(w.T) if tokens is None else np.asarray(tokens)
    dx = gu.as_f64(gu.from_dev(g["dx"])[tok], w.dtype)
    _cmp(dx, ref["dx"][tok], w.dtype, "dx", sc["dx"][tok], bf16_out=True)
    exps = list(range(w.E)) if experts is None else list(experts)
    for name in ("dW1", "dW3", "dW2"):
        if ref[name] is None:
            continue
        got = np.stack([gu.from_dev(g[name][e]) for e in exps])
        _cmp(got, ref[name][exps], w.dtype, name, sc[name][exps])
    if with_w_gate:
        _cmp(gu.from_dev(g["dW_gate"]), ref["dW_gate"], w.dtype, "dW_gate", sc["dW_gate"])


@pytest.mark.parametrize("T,h,f,E,k,cf,act,dtype", [
    (64, 128, 256, 8, 2, 0.0, "swiglu", "f32"),
    (33, 256, 192, 6, 3, 0.0, "gelu", "bf16"),       # ragged T
    (65, 192, 320, 40, 3, 1.0, "swiglu", "bf16"),    # drops, many experts, some empty
    (200, 192, 256, 4, 1, 0.3, "gelu", "bf16"),      # heavy drops, k = 1
    (130, 64, 64, 1, 1, 0.0, "swiglu", "f32"),       # a single expert
    (300, 128, 128, 5, 5, 0.0, "swiglu", "bf16"),    # k = E
    (20, 1024, 2048, 8, 2, 0.0, "swiglu", "bf16"),   # K-split down projection: O in parts
    (500, 128, 256, 16, 2, 0.25, "gelu", "f32"),     # fp32 with drops
    (800, 768, 1024, 4, 2, 0.0, "swiglu", "bf16"),   # 256-row tiles: pipelined NT in two K parts, ragged segments
    (700, 512, 1024, 2, 1, 0.0, "gelu", "bf16"),     # 256-row tiles, GELU derivative in the pipelined NT
    (40, 256, 256, 16, 1, 0.0, "swiglu", "bf16"),    # pipelined TN with empty experts (zero gradients)
    (64, 128, 128, 256, 16, 0.0, "swiglu", "bf16"),  # the largest E and k the library takes
    (150, 320, 448, 4, 2, 0.0, "swiglu", "bf16"),    # pipelined TN with partial tiles in both weight dimensions
    (600, 320, 576, 3, 2, 0.5, "gelu", "bf16"),      # ... GELU with drops; 128-row NT tiles, partial in N
    (1400, 320, 576, 2, 1, 0.9, "gelu", "bf16"),     # 256-row NT tiles, partial in N, with drops
    (1090, 512, 256, 8, 2, 0.7, "swiglu", "bf16"),   # the forward's histogram in 16-token blocks (the
                                                     # logits kernel selects), ragged T, drops
])
def test_backward_edge_cases(T, h, f, E, k, cf, act, dtype):
    _say(f"backward edge T={T} h={h} f={f} E={E} k={k} cf={cf} {act} {dtype}")
    rng = np.random.default_rng(T + 3 * E)
    conv = (lambda a: mw.f32_to_bf16_bits(a)) if dtype == "bf16" else (lambda a: a)
    host = dict(x=conv(rng.standard_normal((T, h)).astype(np.float32)),
                W_gate=(rng.standard_normal((h, E)) / math.sqrt(h)).astype(np.float32),
                logit_bias=rng.standard_normal(E).astype(np.float32),
                W1=conv((rng.standard_normal((E, h, f)) / math.sqrt(h)).astype(np.float32)),
                W3=conv((rng.standard_normal((E, h, f)) / math.sqrt(h)).astype(np.float32)) if act == "swiglu" else None,
                W2=conv((rng.standard_normal((E, f, h)) / math.sqrt(f)).astype(np.float32)))
    dd = {kk: gu.to_dev(v, dtype if kk in ("x", "W1", "W3", "W2") else "f32") for kk, v in host.items()}
    w = mw.Workload("edge", T=T, h=h, f=f, E=E, k=k, act=act, dtype=dtype, cf=cf)
    dy = _dy(T, h, dtype)
    g, gl = _run(w, dd, dy)
    _check_all(w, host, g, gl, dy)


@pytest.mark.parametrize("h", [256, 2048])
def test_backward_skewed_experts(h):
    """The recomputing backward walks the forward's tile list, where a dominant expert in a
    launch of 128-row tiles takes 256-row tiles (with h >= 2048 every expert past 128 rows)."""
    T, f, E, k, cf, act, dtype = 1500, 512, 8, 1, 0.0, "swiglu", "bf16"
    _say(f"backward skewed T={T} h={h} f={f} E={E} k={k}")
    rng = np.random.default_rng(99)
    conv = mw.f32_to_bf16_bits
    bias = np.zeros(E, np.float32)
    bias[2] = 3.0
    host = dict(x=conv(rng.standard_normal((T, h)).astype(np.float32)),
                W_gate=(rng.standard_normal((h, E)) / math.sqrt(h)).astype(np.float32), logit_bias=bias,
                W1=conv((rng.standard_normal((E, h, f)) / math.sqrt(h)).astype(np.float32)),
                W3=conv((rng.standard_normal((E, h, f)) / math.sqrt(h)).astype(np.float32)),
                W2=conv((rng.standard_normal((E, f, h)) / math.sqrt(f)).astype(np.float32)))
    dd = {kk: gu.to_dev(v, dtype if kk in ("x", "W1", "W3", "W2") else "f32") for kk, v in host.items()}
    w = mw.Workload("skewed", T=T, h=h, f=f, E=E, k=k, act=act, dtype=dtype, cf=cf)
    dy = _dy(T, h, dtype)
    g, gl = _run(w, dd, dy)
    counts = o.histogram(o.select_topk(gl, k), E)
    _say(f"  rows per expert: {counts.tolist()}")
    assert counts.max() >= 512
    _check_all(w, host, g, gl, dy)


@pytest.mark.parametrize("name", ["tiny-fp32", "decode-mixtral", "capacity-e64"])
def test_backward_full_size(name):
    _say(f"backward {name}")
    w, host, dd = gu.workload(name)
    dy = _dy(w.T, w.h, w.dtype)
    g, gl = _run(w, dd, dy)
    _check_all(w, host, g, gl, dy)


@pytest.mark.parametrize("name", ["prefill-mixtral", "finegrained-e256"])
def test_backward_full_size_sampled(name):
    """dx on sampled tokens, dW_gate in full (it takes every token's logit gradient), and
    the weight gradients of the experts with the fewest and the most rows."""
    _say(f"backward {name} (sampled)")
    w, host, dd = gu.workload(name)
    dy = _dy(w.T, w.h, w.dtype)
    g, gl = _run(w, dd, dy)
    counts = o.histogram(o.select_topk(gl, w.k), w.E)
    live = np.nonzero(counts > 0)[0]
    e_small = int(live[np.argmin(counts[live])])
    e_big = int(np.argmax(counts))
    tokens = np.sort(np.random.default_rng(5).choice(w.T, 48, replace=False))
    _say(f"  experts checked: {e_small} ({int(counts[e_small])} rows), {e_big} ({int(counts[e_big])} rows); "
         f"tokens: {len(tokens)}; dW_gate in full")
    _check_all(w, host, g, gl, dy, tokens=tokens, experts=[e_small, e_big], with_w_gate=True)


def test_backward_deterministic():
    torch = gu.torch()
    w, host, dd = gu.workload("capacity-e64")
    dy = _dy(w.T, w.h, w.dtype)
    g1, _ = _run(w, dd, dy)
    first = {kk: gu.from_dev(v).copy() for kk, v in g1.items() if v is not None}
    g2, _ = _run(w, dd, dy)
    for kk, v in first.items():
        assert np.array_equal(v, gu.from_dev(g2[kk])), kk


def _fwd_bwd(w, dd, dy_host, saved):
    """Forward then backward; with `saved`, the training forward and the backward that reads
    its pre-activations."""
    torch = gu.torch()
    dev = dd["x"].device
    dt = moe.BF16 if w.dtype == "bf16" else moe.F32
    a = moe.SWIGLU if w.act == "swiglu" else moe.GELU
    fws = moe._ws(moe.workspace_bytes(w.T, w.h, w.f, w.E, w.k, w.cf, dt, a), dev)
    pre = moe._ws(moe.preact_bytes(w.T, w.h, w.f, w.E, w.k, w.cf, w.act), dev) if saved else None
    args = (dd["x"], dd["W_gate"], dd["logit_bias"], dd["W1"], dd["W3"], dd["W2"])
    fwd = moe.layer_forward(*args, k=w.k, capacity_factor=w.cf, act=w.act, ws=fws, preact=pre)
    g = moe.layer_backward(dd["x"], dd["W_gate"], dd["W1"], dd["W3"], dd["W2"], gu.to_dev(dy_host, w.dtype), k=w.k,
                           capacity_factor=w.cf, act=w.act, fwd_ws=fws, d_aux=D_AUX, preact=pre)
    torch.cuda.synchronize()
    return [gu.from_dev(t).copy() for t in fwd], {kk: gu.from_dev(v).copy() for kk, v in g.items() if v is not None}


@pytest.mark.parametrize("name", ["tiny-fp32", "decode-mixtral", "capacity-e64"])
def test_saved_preactivations_give_the_recomputed_gradients(name):
    """The training forward returns what the forward returns, and its saved a (| g) are the
    accumulators the recomputing backward would form (the same products, summed in the same
    order), so the gradients agree bit for bit."""
    _say(f"saved pre-activations {name}")
    w, host, dd = gu.workload(name)
    dy = _dy(w.T, w.h, w.dtype)
    f0, g0 = _fwd_bwd(w, dd, dy, saved=False)
    f1, g1 = _fwd_bwd(w, dd, dy, saved=True)
    for a, b in zip(f0, f1):
        assert np.array_equal(a, b)
    assert set(g0) == set(g1)
    for kk in g0:
        assert np.array_equal(g0[kk], g1[kk]), kk


@pytest.mark.parametrize("T,h,f,E,k,cf,act,dtype", [
    (20, 1024, 2048, 8, 2, 0.0, "swiglu", "bf16"),   # up projection in K parts: saved by the parts' sum
    (33, 256, 192, 6, 3, 0.0, "gelu", "bf16"),
    (500, 128, 256, 16, 2, 0.25, "gelu", "f32"),
])
def test_saved_preactivations_parity(T, h, f, E, k, cf, act, dtype):
    _say(f"saved pre-activations T={T} h={h} f={f} E={E} k={k} cf={cf} {act} {dtype}")
    rng = np.random.default_rng(T + 3 * E)
    conv = (lambda a: mw.f32_to_bf16_bits(a)) if dtype == "bf16" else (lambda a: a)
    host = dict(x=conv(rng.standard_normal((T, h)).astype(np.float32)),
                W_gate=(rng.standard_normal((h, E)) / math.sqrt(h)).astype(np.float32),
                logit_bias=rng.standard_normal(E).astype(np.float32),
                W1=conv((rng.standard_normal((E, h, f)) / math.sqrt(h)).astype(np.float32)),
                W3=conv((rng.standard_normal((E, h, f)) / math.sqrt(h)).astype(np.float32)) if act == "swiglu" else None,
                W2=conv((rng.standard_normal((E, f, h)) / math.sqrt(f)).astype(np.float32)))
    dd = {kk: gu.to_dev(v, dtype if kk in ("x", "W1", "W3", "W2") else "f32") for kk, v in host.items()}
    w = mw.Workload("edge", T=T, h=h, f=f, E=E, k=k, act=act, dtype=dtype, cf=cf)
    dy = _dy(T, h, dtype)
    torch = gu.torch()
    dev = dd["x"].device
    dt = moe.BF16 if dtype == "bf16" else moe.F32
    fws = moe._ws(moe.workspace_bytes(T, h, f, E, k, cf, dt, moe.SWIGLU if act == "swiglu" else moe.GELU), dev)
    pre = moe._ws(moe.preact_bytes(T, h, f, E, k, cf, act), dev)
    args = (dd["x"], dd["W_gate"], dd["logit_bias"], dd["W1"], dd["W3"], dd["W2"])
    moe.layer_forward(*args, k=k, capacity_factor=cf, act=act, ws=fws, preact=pre)
    logits, _, _, _ = moe.route(dd["x"], dd["W_gate"], dd["logit_bias"], k)
    g = moe.layer_backward(dd["x"], dd["W_gate"], dd["W1"], dd["W3"], dd["W2"], gu.to_dev(dy, dtype), k=k,
                           capacity_factor=cf, act=act, fwd_ws=fws, d_aux=D_AUX, preact=pre)
    torch.cuda.synchronize()
    _check_all(w, host, g, gu.from_dev(logits), dy)


VARIANTS = {
    "soft": dict(soft=True),
    "soft-temperature-0.6-noise": dict(soft=True, temperature=0.6, noise=True),
    "temperature-1.5-jitter": dict(temperature=1.5, jitter=True),
    "soft-noise-jitter": dict(soft=True, noise=True, jitter=True, temperature=0.8),
}


def _variant_case(w, host, dd, spec):
    vi = mw.router_variant_inputs(w)
    h_kw = dict(temperature=spec.get("temperature", 1.0), soft=spec.get("soft", False),
                noise=vi["noise"] if spec.get("noise") else None, jitter=vi["jitter"] if spec.get("jitter") else None)
    d_kw = dict(h_kw, noise=gu.to_dev(h_kw["noise"], "f32") if h_kw["noise"] is not None else None,
                jitter=gu.to_dev(h_kw["jitter"], w.dtype) if h_kw["jitter"] is not None else None)
    return h_kw, d_kw


def _run_variant(w, dd, dy_host, d_kw):
    torch = gu.torch()
    dt = moe.BF16 if w.dtype == "bf16" else moe.F32
    a = moe.SWIGLU if w.act == "swiglu" else moe.GELU
    opts = moe._opts(d_kw["jitter"], d_kw["noise"], d_kw["temperature"], False, dd["x"], w.T, w.E, d_kw["soft"])
    extra = moe.lib().moe_router_opts_workspace_bytes(w.T, w.h, dt, moe.ctypes.byref(opts))
    fws = moe._ws(moe.workspace_bytes(w.T, w.h, w.f, w.E, w.k, w.cf, dt, a) + extra, dd["x"].device)
    args = (dd["x"], dd["W_gate"], dd["logit_bias"], dd["W1"], dd["W3"], dd["W2"])
    moe.layer_forward(*args, k=w.k, capacity_factor=w.cf, act=w.act, ws=fws, **d_kw)
    logits, _, _, _ = moe.route(dd["x"], dd["W_gate"], dd["logit_bias"], w.k, jitter=d_kw["jitter"])
    g = moe.layer_backward(dd["x"], dd["W_gate"], dd["W1"], dd["W3"], dd["W2"], gu.to_dev(dy_host, w.dtype), k=w.k,
                           capacity_factor=w.cf, act=w.act, fwd_ws=fws, d_aux=D_AUX, **d_kw)
    torch.cuda.synchronize()
    return g, gu.from_dev(logits)


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("T,h,f,E,k,cf,act,dtype", [
    (200, 256, 512, 8, 2, 0.0, "swiglu", "bf16"),
    (130, 192, 256, 16, 3, 1.0, "gelu", "f32"),
    (64, 512, 1024, 8, 2, 0.6, "swiglu", "bf16"),      # one block of tokens, drops
])
def test_backward_router_variants(variant, T, h, f, E, k, cf, act, dtype):
    """moe_layer_backward_ex against the oracle's backward through the same variant router:
    soft top-K and temperature (the logit gradient reaches unselected experts, and with it
    every column of dW_gate), gate noise, jitter of the router input."""
    _say(f"backward variant {variant} T={T} h={h} f={f} E={E} k={k} cf={cf} {act} {dtype}")
    rng = np.random.default_rng(T + 5 * E)
    conv = (lambda a: mw.f32_to_bf16_bits(a)) if dtype == "bf16" else (lambda a: a)
    host = dict(x=conv(rng.standard_normal((T, h)).astype(np.float32)),
                W_gate=(rng.standard_normal((h, E)) / math.sqrt(h)).astype(np.float32),
                logit_bias=rng.standard_normal(E).astype(np.float32),
                W1=conv((rng.standard_normal((E, h, f)) / math.sqrt(h)).astype(np.float32)),
                W3=conv((rng.standard_normal((E, h, f)) / math.sqrt(h)).astype(np.float32)) if act == "swiglu" else None,
                W2=conv((rng.standard_normal((E, f, h)) / math.sqrt(f)).astype(np.float32)))
    dd = {kk: gu.to_dev(v, dtype if kk in ("x", "W1", "W3", "W2") else "f32") for kk, v in host.items()}
    w = mw.Workload("variant", T=T, h=h, f=f, E=E, k=k, act=act, dtype=dtype, cf=cf)
    h_kw, d_kw = _variant_case(w, host, dd, VARIANTS[variant])
    dy = _dy(T, h, dtype)
    g, gl = _run_variant(w, dd, dy, d_kw)
    _check_all(w, host, g, gl, dy, variants=h_kw)


@pytest.mark.parametrize("name,variant", [("decode-mixtral", "soft"), ("capacity-e64", "soft-noise-jitter")])
def test_backward_router_variants_full_size(name, variant):
    _say(f"backward variant {variant} {name}")
    w, host, dd = gu.workload(name)
    h_kw, d_kw = _variant_case(w, host, dd, VARIANTS[variant])
    dy = _dy(w.T, w.h, w.dtype)
    g, gl = _run_variant(w, dd, dy, d_kw)
    _check_all(w, host, g, gl, dy, variants=h_kw)
