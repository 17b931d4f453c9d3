"""Pins of the oracle's backward pass (layer_backward), on the CPU.

The hand-written adjoint is checked against things it does not share code with:
torch.autograd in float64 differentiating a torch forward (itself checked equal to
the oracle's forward), central finite differences of the oracle's forward, and
invariants of the softmax Jacobian and the aux-loss gradient.
"""
import math

import numpy as np
import pytest

import moe_workloads as mw
import oracle as o


def _case(T=24, h=16, f=20, E=5, k=2, act="swiglu", seed=0, bias=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, h)).astype(np.float32)
    Wg = (rng.standard_normal((h, E)) / math.sqrt(h)).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32) if bias else None
    W1 = (rng.standard_normal((E, h, f)) / math.sqrt(h)).astype(np.float32)
    W3 = (rng.standard_normal((E, h, f)) / math.sqrt(h)).astype(np.float32) if act == "swiglu" else None
    W2 = (rng.standard_normal((E, f, h)) / math.sqrt(f)).astype(np.float32)
    dy = rng.standard_normal((T, h)).astype(np.float32)
    return x, Wg, b, W1, W3, W2, dy


def _torch_grads(x, Wg, b, W1, W3, W2, dy, d_aux, k, cf, act, *, temperature=1.0, soft=False, noise=None,
                 jitter=None):
    """The layer in torch float64 with autograd; the selection and the capacity mask
    are taken from the oracle (they are piecewise constant).  Router variants: gate
    noise added to the logits, a softmax temperature, soft top-K weights (the
    temperature softmax over all experts at the selection, not renormalised), and a
    multiplicative jitter of the router's input."""
    torch = pytest.importorskip("torch")
    T, h = x.shape
    E = Wg.shape[1]
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True)
    X, G, A1, A2 = t(x), t(Wg), t(W1), t(W2)
    A3 = t(W3) if W3 is not None else None
    XR = X if jitter is None else X * torch.tensor(np.asarray(jitter, np.float64))
    logits = XR @ G + (torch.tensor(b, dtype=torch.float64) if b is not None else 0.0)
    if noise is not None:
        logits = logits + torch.tensor(np.asarray(noise, np.float64))
    xr = x if jitter is None else o.jitter_input(x, jitter, "f32")
    lf = o.noisy_logits(o.router_logits(xr, Wg, b, "f32"), noise)
    idx = o.select_topk(lf, k)
    C = o.expert_capacity(T, E, k, cf)
    counts, _, _, slot_pos = o.permute(idx, E, C)
    kept = torch.tensor(slot_pos.reshape(T, k) >= 0)
    I = torch.tensor(idx.astype(np.int64))
    p = torch.softmax(logits / temperature, dim=1)
    wsel = torch.gather(p, 1, I) if soft else torch.softmax(torch.gather(logits, 1, I) / temperature, dim=1)
    fe = torch.tensor(counts / (T * k), dtype=torch.float64)
    aux = E * torch.sum(fe * p.mean(0))
    y = torch.zeros((T, h), dtype=torch.float64)
    for j in range(k):
        for e in range(E):
            m = (I[:, j] == e) & kept[:, j]
            if not bool(m.any()):
                continue
            xe = X[m]
            a = xe @ A1[e]
            hm = torch.nn.functional.silu(a) * (xe @ A3[e]) if act == "swiglu" else \
                0.5 * a * (1 + torch.erf(a / math.sqrt(2)))
            out = hm @ A2[e]
            y = y.index_add(0, torch.nonzero(m).squeeze(1), wsel[m, j:j + 1] * out)
    L = torch.sum(torch.tensor(dy, dtype=torch.float64) * y) + d_aux * aux
    L.backward()
    return dict(y=y.detach().numpy(), aux=float(aux.detach()), dx=X.grad.numpy(), dW_gate=G.grad.numpy(),
                dW1=A1.grad.numpy(), dW3=None if A3 is None else A3.grad.numpy(), dW2=A2.grad.numpy())


def _close(a, b, rel, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    rms = float(np.sqrt(np.mean(b ** 2))) or 1.0
    err = float(np.abs(a - b).max())
    assert err <= rel * rms, f"{what}: max|d| {err:.3e} > {rel} * RMS {rms:.3e}"


@pytest.mark.parametrize("act,cf,d_aux,k,E", [("swiglu", 0.0, 0.0, 2, 5), ("gelu", 0.0, 0.7, 2, 5),
                                              ("swiglu", 0.6, 1.3, 2, 5), ("swiglu", 0.0, 0.5, 5, 5),
                                              ("gelu", 0.5, 0.0, 1, 4), ("swiglu", 1.0, 2.0, 3, 7)])
def test_backward_vs_torch_autograd(act, cf, d_aux, k, E):
    x, Wg, b, W1, W3, W2, dy = _case(E=E, act=act, seed=E + k)
    ref = _torch_grads(x, Wg, b, W1, W3, W2, dy, d_aux, k, cf, act)
    fwd = o.layer_forward(x, Wg, b, W1, W3, W2, k=k, capacity_factor=cf, act=act, dtype="f32")
    _close(fwd["y64"], ref["y"], 1e-6, "torch forward = oracle forward")   # weights in fp32 vs fp64
    assert abs(fwd["aux"] - ref["aux"]) <= 1e-6 * abs(ref["aux"])
    g = o.layer_backward(x, Wg, b, W1, W3, W2, dy, d_aux, k=k, capacity_factor=cf, act=act, dtype="f32")
    for key in ("dx", "dW_gate", "dW1", "dW2") + (("dW3",) if act == "swiglu" else ()):
        _close(g[key], ref[key], 2e-6, key)


def test_backward_vs_finite_differences():
    """Central differences of <dy, y> in the expert weights (the router is untouched,
    so the selection cannot move): fp64 forward, step 2^-12 (exact on the fp32 inputs
    the oracle reads)."""
    x, Wg, b, W1, W3, W2, dy = _case(T=10, h=8, f=6, E=3, k=2, seed=3)
    g = o.layer_backward(x, Wg, b, W1, W3, W2, dy, 0.0, k=2, capacity_factor=0.0, act="swiglu", dtype="f32")
    rng = np.random.default_rng(4)

    def loss(W1_, W3_, W2_):
        y = o.layer_forward(x, Wg, b, W1_, W3_, W2_, k=2, capacity_factor=0.0, act="swiglu", dtype="f32")["y64"]
        return float(np.sum(dy.astype(np.float64) * y))

    for name, arr in (("dW1", W1), ("dW3", W3), ("dW2", W2)):
        for _ in range(6):
            pos = tuple(int(rng.integers(0, s)) for s in arr.shape)
            eps = 2.0 ** -12
            up = arr.astype(np.float64).copy()
            dn = arr.astype(np.float64).copy()
            up[pos] += eps
            dn[pos] -= eps
            args_up = {"dW1": (up, W3, W2), "dW3": (W1, up, W2), "dW2": (W1, W3, up)}[name]
            args_dn = {"dW1": (dn, W3, W2), "dW3": (W1, dn, W2), "dW2": (W1, W3, dn)}[name]
            fd = (loss(*args_up) - loss(*args_dn)) / (2 * eps)
            assert abs(fd - g[name][pos]) <= 1e-6 * (1 + abs(fd)), (name, pos, fd, g[name][pos])


def test_router_gradient_invariants():
    """The softmax and the renormalisation are invariant to a shift of a token's logits,
    so every token's logit gradient sums to zero; balanced counts make the aux gradient
    vanish; with dy = 0 the aux term alone drives the router."""
    x, Wg, b, W1, W3, W2, dy = _case(T=40, E=8, k=2, seed=9)
    g = o.layer_backward(x, Wg, b, W1, W3, W2, dy, 1.5, k=2, capacity_factor=0.3, act="swiglu", dtype="f32")
    # (to the rounding of the stored fp32 weights, which sum to 1 within ~1e-7)
    assert np.abs(g["dlogits"].sum(1)).max() <= 1e-6 * np.abs(g["dlogits"]).sum(1).max()
    # unselected experts get only the aux term: with d_aux = 0 they get nothing
    g0 = o.layer_backward(x, Wg, b, W1, W3, W2, dy, 0.0, k=2, capacity_factor=0.3, act="swiglu", dtype="f32")
    sel = np.zeros(g0["dlogits"].shape, bool)
    np.put_along_axis(sel, g0["topk_idx"].astype(np.int64), True, axis=1)
    assert (g0["dlogits"][~sel] == 0).all()
    # dropped slots reach nothing
    dropped = g0["slot_pos"].reshape(40, 2) < 0
    assert dropped.any() and (g0["dw"][dropped] == 0).all()
    # balanced counts (T*k/E each): f_e = 1/E and the aux gradient is exactly zero
    T, E, k = 64, 8, 2
    l = np.random.default_rng(1).standard_normal((T, E)).astype(np.float32)
    idx = o.select_topk(l, k)
    counts = o.histogram(idx, E)
    if (counts == T * k // E).all():
        ga = o.layer_backward(*_case(T=T, E=E, k=k, seed=2)[:6], np.zeros((T, 16), np.float32), 1.0, k=k,
                              capacity_factor=0.0, act="swiglu", dtype="f32", logits=l)
        assert np.abs(ga["dlogits"]).max() < 1e-15
    # dy = 0: the aux gradient in closed form, d_aux (E/T) p (f - <f, p>)
    z = np.zeros_like(dy)
    gz = o.layer_backward(x, Wg, b, W1, W3, W2, z, 2.0, k=2, capacity_factor=0.0, act="swiglu", dtype="f32")
    p = o.softmax(gz["logits"])
    fe = gz["counts"] / (40 * 2)
    want = 2.0 * (8 / 40) * p * (fe[None, :] - (p * fe[None, :]).sum(1, keepdims=True))
    np.testing.assert_allclose(gz["dlogits"], want, rtol=1e-12, atol=1e-18)
    assert np.abs(gz["dW1"]).max() == 0 and np.abs(gz["dW2"]).max() == 0


def test_backward_bf16_uses_rounded_hidden_activation():
    """bf16: dW2 multiplies the rounded Hm the forward used; the other gradients treat
    the rounding as the identity.  Checked against the fp32 oracle on the same values:
    dW2 differs only by the rounding of Hm, the rest agree to rounding of nothing."""
    x, Wg, b, W1, W3, W2, dy = _case(T=16, h=16, f=12, E=4, k=2, seed=12)
    cv = mw.f32_to_bf16_bits
    xb, W1b, W3b, W2b, dyb = cv(x), cv(W1), cv(W3), cv(W2), cv(dy)
    back = lambda a: mw.bf16_bits_to_f32(a)
    gb = o.layer_backward(xb, Wg, b, W1b, W3b, W2b, dyb, 0.3, k=2, capacity_factor=0.0, act="swiglu", dtype="bf16")
    gf = o.layer_backward(back(xb), Wg, b, back(W1b), back(W3b), back(W2b), back(dyb), 0.3, k=2,
                          capacity_factor=0.0, act="swiglu", dtype="f32")
    # the hidden activation's rounding moves dw and hence the router part slightly; the
    # expert-weight gradients dW1/dW3 see it only through dw -> nothing (they use dHm)
    np.testing.assert_allclose(gb["dW1"], gf["dW1"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(gb["dW3"], gf["dW3"], rtol=0, atol=1e-12)
    _close(gb["dW2"], gf["dW2"], 2e-2, "dW2 with rounded Hm")
    assert np.abs(gb["dW2"] - gf["dW2"]).max() > 0


VARIANT_CASES = {
    "temperature": dict(temperature=0.6),
    "soft": dict(soft=True),
    "soft-temperature-noise": dict(soft=True, temperature=0.5, noise=True),
    "all": dict(soft=True, temperature=1.5, noise=True, jitter=True),
    "jitter-noise": dict(noise=True, jitter=True, temperature=0.8),
}


@pytest.mark.parametrize("variant", list(VARIANT_CASES))
@pytest.mark.parametrize("act,cf,d_aux", [("swiglu", 0.6, 0.8), ("gelu", 0.0, 0.0)])
def test_backward_router_variants_vs_torch_autograd(variant, act, cf, d_aux):
    spec = VARIANT_CASES[variant]
    T, E, k = 24, 6, 2
    x, Wg, b, W1, W3, W2, dy = _case(T=T, E=E, k=k, act=act, seed=31)
    rng = np.random.default_rng(32)
    noise = (rng.standard_normal((T, E)) / E).astype(np.float32) if spec.get("noise") else None
    jit = rng.uniform(0.9, 1.1, x.shape).astype(np.float32) if spec.get("jitter") else None
    kw = dict(temperature=spec.get("temperature", 1.0), soft=spec.get("soft", False), noise=noise, jitter=jit)
    ref = _torch_grads(x, Wg, b, W1, W3, W2, dy, d_aux, k, cf, act, **kw)
    fwd = o.layer_forward(x, Wg, b, W1, W3, W2, k=k, capacity_factor=cf, act=act, dtype="f32", **kw)
    _close(fwd["y64"], ref["y"], 1e-6, "torch forward = oracle forward")
    assert abs(fwd["aux"] - ref["aux"]) <= 1e-6 * abs(ref["aux"])
    g = o.layer_backward(x, Wg, b, W1, W3, W2, dy, d_aux, k=k, capacity_factor=cf, act=act, dtype="f32", **kw)
    for key in ("dx", "dW_gate", "dW1", "dW2") + (("dW3",) if act == "swiglu" else ()):
        _close(g[key], ref[key], 2e-6, key)


def test_soft_topk_reaches_unselected_experts():
    """The reason for the soft top-K ([OPS] "坑3"): with hard, renormalised weights an
    expert that was not selected gets no logit gradient (without the aux term); with
    soft weights it gets -p_b * sum_j w_j dw_j / tau, and every token's logit gradient
    still sums to zero (the softmax ignores a shift of all logits)."""
    T, E, k, tau = 32, 8, 2, 0.7
    x, Wg, b, W1, W3, W2, dy = _case(T=T, E=E, k=k, seed=33)
    kw = dict(k=k, capacity_factor=0.0, act="swiglu", dtype="f32", temperature=tau)
    hard = o.layer_backward(x, Wg, b, W1, W3, W2, dy, 0.0, **kw)
    soft = o.layer_backward(x, Wg, b, W1, W3, W2, dy, 0.0, soft=True, **kw)
    sel = np.zeros((T, E), bool)
    np.put_along_axis(sel, soft["topk_idx"].astype(np.int64), True, axis=1)
    assert (hard["dlogits"][~sel] == 0).all()
    assert (np.abs(soft["dlogits"][~sel]) > 0).all()
    p = o.softmax_t(soft["logits"], tau)
    s_wdw = np.sum(soft["topk_w"].astype(np.float64) * soft["dw"], axis=1, keepdims=True)
    want = -p * s_wdw / tau
    np.testing.assert_allclose(soft["dlogits"][~sel], want[~sel], rtol=1e-12)
    # (to the rounding of the stored fp32 weights against the fp64 probabilities)
    assert np.abs(soft["dlogits"].sum(1)).max() <= 1e-6 * np.abs(soft["dlogits"]).sum(1).max()
    # the soft weights are smaller than the renormalised ones, by the selected mass
    ratio = soft["topk_w"].astype(np.float64) / hard["topk_w"].astype(np.float64)
    mass = np.take_along_axis(p, soft["topk_idx"].astype(np.int64), 1).sum(1, keepdims=True)
    np.testing.assert_allclose(ratio, np.broadcast_to(mass, ratio.shape), rtol=1e-6)


# ----------------------------------------------------------------------------
# the magnitude scale (with_scale=True) that sets the bar for reduced-precision gradients

SCALE_KEYS = ("dx", "dW_gate", "dW1", "dW2", "dW3")


@pytest.mark.parametrize("act,cf,d_aux,k,variant", [("swiglu", 0.0, 0.0, 2, None), ("gelu", 0.5, 1.1, 2, None),
                                                    ("swiglu", 0.6, 0.7, 3, "soft"), ("gelu", 0.0, 0.4, 1, None),
                                                    ("swiglu", 0.0, 0.9, 2, "all")])
def test_grad_scale_bounds_every_gradient(act, cf, d_aux, k, variant):
    """Triangle inequality: the chain taken over absolute values bounds each gradient
    element, on random inputs of both signs."""
    T, E = 30, 6
    x, Wg, b, W1, W3, W2, dy = _case(T=T, E=E, k=k, act=act, seed=40 + k)
    kw = {}
    if variant:
        rng = np.random.default_rng(41)
        spec = VARIANT_CASES[variant]
        kw = dict(temperature=spec.get("temperature", 1.0), soft=spec.get("soft", False),
                  noise=(rng.standard_normal((T, E)) / E).astype(np.float32) if spec.get("noise") else None,
                  jitter=rng.uniform(0.9, 1.1, x.shape).astype(np.float32) if spec.get("jitter") else None)
    g = o.layer_backward(x, Wg, b, W1, W3, W2, dy, d_aux, k=k, capacity_factor=cf, act=act, dtype="f32",
                         with_scale=True, **kw)
    for key in SCALE_KEYS:
        if g[key] is None:
            continue
        sc = g["scale"][key]
        assert np.isfinite(sc).all() and (sc >= 0).all(), key
        assert (np.abs(g[key]) <= sc * (1 + 1e-12) + 1e-300).all(), key
        assert (sc > 0).any(), key


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_grad_scale_equals_gradient_without_cancellation(act):
    """With every operand non-negative no sum has terms of both signs, so the scale of
    each expert-side gradient is its magnitude exactly.  (k = 1 gives w = 1 and no
    renormalisation gradient; W_gate = 0 -- routing by the bias alone -- takes the
    router's share out of dx.)"""
    T, h, f, E = 20, 12, 10, 4
    rng = np.random.default_rng(42)
    x = rng.uniform(0.0, 1.0, (T, h)).astype(np.float32)
    W1 = rng.uniform(0.0, 0.3, (E, h, f)).astype(np.float32)
    W3 = rng.uniform(0.0, 0.3, (E, h, f)).astype(np.float32) if act == "swiglu" else None
    W2 = rng.uniform(0.0, 0.3, (E, f, h)).astype(np.float32)
    dy = rng.uniform(0.0, 1.0, (T, h)).astype(np.float32)
    Wg = np.zeros((h, E), np.float32)
    b = np.array([0.3, 0.1, -0.2, 0.0], np.float32)
    # the bias routes every token to expert 0; give each token its own top expert instead
    logits = rng.permutation(np.tile(np.arange(E, dtype=np.float32), (T, 1)).T).T.copy()
    g = o.layer_backward(x, Wg, b, W1, W3, W2, dy, 0.0, k=1, capacity_factor=0.0, act=act, dtype="f32",
                         logits=logits, with_scale=True)
    for key in ("dx", "dW1", "dW2") + (("dW3",) if act == "swiglu" else ()):
        np.testing.assert_allclose(g["scale"][key], np.abs(g[key]), rtol=1e-12, atol=0, err_msg=key)


def test_grad_scale_vs_brute_force_chain():
    """Every scale element recomputed with Python loops and math.fsum from the
    definition of the magnitude chain, on a tiny case with drops, the aux term and a
    soft router."""
    T, h, f, E, k, tau, d_aux = 7, 4, 3, 3, 2, 0.8, 0.6
    x, Wg, b, W1, W3, W2, dy = _case(T=T, h=h, f=f, E=E, k=k, seed=43)
    cf = 0.8
    g = o.layer_backward(x, Wg, b, W1, W3, W2, dy, d_aux, k=k, capacity_factor=cf, act="swiglu", dtype="f32",
                         with_scale=True, temperature=tau, soft=True)
    idx, w, sp = g["topk_idx"], g["topk_w"], g["slot_pos"].reshape(T, k)
    F = lambda v: float(v)
    sig = lambda z: 1.0 / (1.0 + math.exp(-z))
    dw_m = [[0.0] * k for _ in range(T)]
    sx = [[0.0] * h for _ in range(T)]
    s1 = [[[0.0] * f for _ in range(h)] for _ in range(E)]
    s3 = [[[0.0] * f for _ in range(h)] for _ in range(E)]
    s2 = [[[0.0] * h for _ in range(f)] for _ in range(E)]
    for t in range(T):
        for j in range(k):
            if sp[t, j] < 0:
                continue
            e = int(idx[t, j])
            a = [math.fsum(F(x[t, i]) * F(W1[e, i, c]) for i in range(h)) for c in range(f)]
            gg = [math.fsum(F(x[t, i]) * F(W3[e, i, c]) for i in range(h)) for c in range(f)]
            hm = [a[c] * sig(a[c]) * gg[c] for c in range(f)]
            O = [math.fsum(hm[c] * F(W2[e, c, i]) for c in range(f)) for i in range(h)]
            dw_m[t][j] = math.fsum(abs(F(dy[t, i])) * abs(O[i]) for i in range(h))
            dO = [abs(F(w[t, j])) * abs(F(dy[t, i])) for i in range(h)]
            dHm = [math.fsum(dO[i] * abs(F(W2[e, c, i])) for i in range(h)) for c in range(f)]
            sgrad = [sig(a[c]) * (1 + a[c] * (1 - sig(a[c]))) for c in range(f)]
            da = [dHm[c] * abs(gg[c] * sgrad[c]) for c in range(f)]
            dg = [dHm[c] * abs(a[c] * sig(a[c])) for c in range(f)]
            for i in range(h):
                sx[t][i] += math.fsum([da[c] * abs(F(W1[e, i, c])) for c in range(f)] +
                                      [dg[c] * abs(F(W3[e, i, c])) for c in range(f)])
                for c in range(f):
                    s1[e][i][c] += abs(F(x[t, i])) * da[c]
                    s3[e][i][c] += abs(F(x[t, i])) * dg[c]
            for c in range(f):
                for i in range(h):
                    s2[e][c][i] += abs(hm[c]) * dO[i]
    # router: soft weights p_b at the selection; |d/dl_b| <= p_b (dw_m_b + sum_j |w_j| dw_m_j) / tau
    # + |d_aux| (E/T) p_b (f_b + sum_e f_e p_e) / tau
    counts = [sum(1 for t in range(T) for j in range(k) if idx[t, j] == e) for e in range(E)]
    fe = [c / (T * k) for c in counts]
    l = g["logits"]
    dl_m = [[0.0] * E for _ in range(T)]
    for t in range(T):
        m = max(F(v) for v in l[t])
        ex = [math.exp((F(l[t, e]) - m) / tau) for e in range(E)]
        den = math.fsum(ex)
        p = [v / den for v in ex]
        s_m = math.fsum(abs(F(w[t, j])) * dw_m[t][j] for j in range(k))
        fp = math.fsum(fe[e] * p[e] for e in range(E))
        for e in range(E):
            own = math.fsum(dw_m[t][j] for j in range(k) if idx[t, j] == e)
            dl_m[t][e] = p[e] * (own + s_m) / tau + abs(d_aux) * (E / T) * p[e] * (fe[e] + fp) / tau
    for t in range(T):
        for i in range(h):
            sx[t][i] += math.fsum(dl_m[t][e] * abs(F(Wg[i, e])) for e in range(E))
    sg = [[math.fsum(abs(F(x[t, i])) * dl_m[t][e] for t in range(T)) for e in range(E)] for i in range(h)]
    for key, want in (("dx", sx), ("dW1", s1), ("dW3", s3), ("dW2", s2), ("dW_gate", sg)):
        np.testing.assert_allclose(g["scale"][key], np.array(want), rtol=1e-10, atol=1e-300, err_msg=key)


@pytest.mark.parametrize("with_w_gate", [True, False])
def test_restricted_backward_equals_the_full_one(with_w_gate):
    """Asking for some tokens' dx and some experts' weight gradients gives the full
    backward's values there (the oracle only skips the work nobody asked for; a matrix
    product over fewer rows may sum in another order, so to fp64 rounding)."""
    x, Wg, b, W1, W3, W2, dy = _case(T=40, E=6, k=2, seed=50)
    kw = dict(k=2, capacity_factor=0.7, act="swiglu", dtype="f32", with_scale=True, soft=True, temperature=0.8)
    full = o.layer_backward(x, Wg, b, W1, W3, W2, dy, 0.4, **kw)
    tokens, experts = [0, 7, 31, 39], [1, 4]
    part = o.layer_backward(x, Wg, b, W1, W3, W2, dy, 0.4, tokens=tokens, experts=experts, with_w_gate=with_w_gate,
                            **kw)
    same = lambda a, b_: np.testing.assert_allclose(a, b_, rtol=1e-12, atol=1e-15)
    same(part["dx"][tokens], full["dx"][tokens])
    same(part["scale"]["dx"][tokens], full["scale"]["dx"][tokens])
    for name in ("dW1", "dW3", "dW2"):
        same(part[name][experts], full[name][experts])
        same(part["scale"][name][experts], full["scale"][name][experts])
    if with_w_gate:
        same(part["dW_gate"], full["dW_gate"])
        same(part["scale"]["dW_gate"], full["scale"]["dW_gate"])
