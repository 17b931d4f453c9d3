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


def _torch_grads(x, Wg, b, W1, W3, W2, dy, d_aux, k, cf, act):
    """The layer in torch float64 with autograd; the selection and the capacity mask
    are taken from the oracle (they are piecewise constant)."""
    torch = pytest.importorskip("torch")
    T, h = x.shape
    E = Wg.shape[1]
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True)
    X, G, A1, A2 = t(x), t(Wg), t(W1), t(W2)
    A3 = t(W3) if W3 is not None else None
    logits = X @ G + (torch.tensor(b, dtype=torch.float64) if b is not None else 0.0)
    lf = o.router_logits(x, Wg, b, "f32")
    idx = o.select_topk(lf, k)
    C = o.expert_capacity(T, E, k, cf)
    counts, _, _, slot_pos = o.permute(idx, E, C)
    kept = torch.tensor(slot_pos.reshape(T, k) >= 0)
    I = torch.tensor(idx.astype(np.int64))
    wsel = torch.softmax(torch.gather(logits, 1, I), dim=1)
    p = torch.softmax(logits, dim=1)
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
