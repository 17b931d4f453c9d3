"""Pins of the CPU oracle to facts outside itself (CPU only).

Each test checks the oracle against something it does not compute itself: the
pages' worked examples (``tests/golden``), closed forms, library routines
(Python's stable sort, torch's bf16 cast, ``math.erf``), brute force in pure
Python on tiny inputs (``tests/brute.py``) and invariants of the method.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle as o
import moe_workloads as mw
from tests import brute

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as fh:
        return json.load(fh)


# ----------------------------------------------------------------------------
# worked examples printed on the pages

def test_top2_worked_example():
    g = _gold("ops_top2_example.json")
    l = np.array([g["scores"]], dtype=np.float32)
    idx = o.select_topk(l, g["k"])
    assert idx.tolist() == [g["topk_idx"]]
    w = o.topk_weights(l, idx)
    # the page feeds fp32-rounded scores (0.9f, 0.7f); the closed form is on the exact decimals
    np.testing.assert_allclose(w[0], g["topk_w"], rtol=2e-7)
    assert abs(float(w.astype(np.float64).sum()) - 1.0) < 1e-7


def test_histogram_worked_example_dropless():
    g = _gold("mb_histogram_example.json")
    idx = np.array(g["topk_idx"], dtype=np.int32).reshape(-1, 1)
    counts, offsets, sorted_slot, slot_pos = o.permute(idx, g["E"], None)
    assert counts.tolist() == g["counts"]
    assert o.histogram(idx, g["E"]).tolist() == g["counts"]
    assert offsets.tolist() == g["dropless"]["offsets"]
    assert sorted_slot.tolist() == g["dropless"]["sorted_slot"]
    assert slot_pos.tolist() == g["dropless"]["slot_pos"]


def test_histogram_worked_example_capacity():
    g = _gold("mb_histogram_example.json")
    idx = np.array(g["topk_idx"], dtype=np.int32).reshape(-1, 1)
    C = o.expert_capacity(len(idx), g["E"], g["k"], 1.0)
    assert C == g["cf_1"]["C"]
    counts, offsets, sorted_slot, slot_pos = o.permute(idx, g["E"], C)
    assert counts.tolist() == g["counts"]  # counts are taken before the drop
    assert offsets.tolist() == g["cf_1"]["offsets"]
    R = offsets[-1]
    assert sorted_slot[:R].tolist() == g["cf_1"]["sorted_slot_kept"]
    assert (sorted_slot[R:] == -1).all()
    assert slot_pos.tolist() == g["cf_1"]["slot_pos"]


# ----------------------------------------------------------------------------
# closed forms for the capacity

def test_capacity_closed_forms():
    w = mw.by_name("capacity-e64")
    assert o.expert_capacity(w.T, w.E, w.k, w.cf) == 320       # floor(1.25*8192*2/64)
    assert o.expert_capacity(4096, 8, 2, 0.0) is None          # factor 0: dropless
    assert o.expert_capacity(4096, 8, 2, -1.0) is None
    assert o.expert_capacity(8, 64, 1, 0.5) is None            # floor(0.5*8/64) = 0 -> dropless
    assert o.expert_capacity(8, 4, 1, 1.0) == 2
    assert o.expert_capacity(10, 4, 2, 1.0) == 5               # floor(1.0 * 20/4)
    assert o.expert_capacity(10, 4, 2, 0.3) == 1               # floor(0.3*5) = floor(1.5)
    with pytest.raises(ValueError):
        o.expert_capacity(8, 4, 1, float("nan"))


def test_capacity_zero_equals_dropless_bitwise():
    rng = np.random.default_rng(1)
    idx = np.stack([rng.permutation(16)[:3] for _ in range(50)]).astype(np.int32)
    a = o.permute(idx, 16, o.expert_capacity(50, 16, 3, 0.0))
    b = o.permute(idx, 16, None)
    big = o.permute(idx, 16, 10 ** 6)
    for u, v, z in zip(a, b, big):
        assert np.array_equal(u, v) and np.array_equal(u, z)


# ----------------------------------------------------------------------------
# the sort by expert id vs a library routine, and permutation invariants

@pytest.mark.parametrize("E,k,T,C", [(8, 2, 64, None), (64, 2, 300, 7), (256, 8, 40, 1),
                                     (4, 4, 9, 3), (3, 1, 1, None)])
def test_permute_vs_python_sorted(E, k, T, C):
    rng = np.random.default_rng(E * 1000 + T)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, sorted_slot, slot_pos = o.permute(idx, E, C)
    flat = idx.reshape(-1).tolist()
    order = sorted(range(T * k), key=flat.__getitem__)   # stable library sort
    rows = []
    for e in range(E):
        seg = [s for s in order if flat[s] == e]
        rows += seg if C is None else seg[:C]
    R = len(rows)
    assert offsets[-1] == R
    assert sorted_slot[:R].tolist() == rows
    assert np.bincount(idx.reshape(-1), minlength=E).tolist() == counts.tolist()


@pytest.mark.parametrize("name", ["tiny-fp32", "capacity-e64", "finegrained-e256"])
def test_permutation_invariants(name):
    w = mw.by_name(name)
    d = mw.make_inputs(w, with_weights=False)
    r = o.layer_forward(d["x"], d["W_gate"], d["logit_bias"], None, None, None, k=w.k,
                        capacity_factor=w.cf, act=w.act, dtype=w.dtype, with_y=False)
    idx, counts, offsets = r["topk_idx"], r["counts"], r["offsets"]
    sorted_slot, slot_pos, C = r["sorted_slot"], r["slot_pos"], r["C"]
    n = w.T * w.k
    assert counts.sum() == n                                   # histogram sums to T*k
    kept = counts if C is None else np.minimum(counts, C)
    assert np.array_equal(np.diff(offsets), kept)
    R = int(offsets[-1])
    # bijection between kept assignments and rows
    kept_s = np.nonzero(slot_pos >= 0)[0]
    assert len(kept_s) == R
    assert np.array_equal(sorted_slot[slot_pos[kept_s]], kept_s)
    assert np.array_equal(np.sort(slot_pos[kept_s]), np.arange(R))
    if C is None:
        assert np.array_equal(np.sort(sorted_slot), np.arange(n))
    for e in range(w.E):
        seg = sorted_slot[offsets[e]:offsets[e + 1]]
        assert (np.diff(seg) > 0).all()                       # stable: ascending assignment order
        assert (idx.reshape(-1)[seg] == e).all()              # rows of segment e chose e
    if name == "capacity-e64":
        assert C == 320 and R < n                              # the Zipf skew forces drops
        # every dropped assignment is later (in s) than all kept ones of its expert
        flat = idx.reshape(-1)
        for e in np.nonzero(counts > C)[0]:
            s_e = np.nonzero(flat == e)[0]
            assert (slot_pos[s_e[:C]] >= 0).all() and (slot_pos[s_e[C:]] == -1).all()


def test_uniform_assignment_counts():
    idx = mw.uniform_assignment(64, 8, 2)
    counts, offsets, _, _ = o.permute(idx, 8, None)
    assert (counts == 16).all()
    assert offsets.tolist() == list(range(0, 129, 16))


# ----------------------------------------------------------------------------
# top-k selection and weights

def test_topk_ties_and_signed_zero():
    l = np.array([[1.0, 2.0, 2.0, 0.5, 2.0],
                  [0.0, -0.0, 0.0, -1.0, -0.0],
                  [3.0, 3.0, 3.0, 3.0, 3.0]], dtype=np.float32)
    idx = o.select_topk(l, 3)
    assert idx.tolist() == [[1, 2, 4], [0, 1, 2], [0, 1, 2]]
    assert o.select_topk(l, 5)[1].tolist() == [0, 1, 2, 4, 3]
    w = o.topk_weights(l, idx)
    np.testing.assert_allclose(w[2], [1 / 3] * 3, rtol=1e-7)


def test_topk_weights_invariants():
    w = mw.by_name("finegrained-e256")
    d = mw.make_inputs(w, with_weights=False)
    l = o.router_logits(d["x"], d["W_gate"], d["logit_bias"], w.dtype)
    idx = o.select_topk(l, w.k)
    wt = o.topk_weights(l, idx).astype(np.float64)
    assert np.abs(wt.sum(1) - 1).max() < 1e-6                # renormalised to 1
    assert (np.diff(wt, axis=1) <= 0).all()                  # best first
    # closed form: the weights are a softmax over the selected logits alone
    sel = np.take_along_axis(l.astype(np.float64), idx.astype(np.int64), 1)
    ref = np.exp(sel - sel.max(1, keepdims=True))
    ref /= ref.sum(1, keepdims=True)
    np.testing.assert_allclose(wt, ref, rtol=1e-6, atol=1e-12)
    # the selected logits are the k largest
    top = -np.sort(-l, axis=1)[:, :w.k]
    assert np.array_equal(np.take_along_axis(l, idx.astype(np.int64), 1), top)


def test_k1_weight_is_one():
    l = np.random.default_rng(3).standard_normal((20, 6)).astype(np.float32)
    idx = o.select_topk(l, 1)
    assert (o.topk_weights(l, idx) == 1.0).all()
    assert np.array_equal(idx[:, 0], l.argmax(1))


# ----------------------------------------------------------------------------
# brute force on tiny inputs

def _tiny(T, h, f, E, seed, act, dtype, tie_cols=False, bias=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, h)).astype(np.float32)
    Wg = (rng.standard_normal((h, E)) / math.sqrt(h)).astype(np.float32)
    if tie_cols:
        Wg[:, 3] = Wg[:, 1]
    b = rng.standard_normal(E).astype(np.float32) if bias else None
    W1 = (rng.standard_normal((E, h, f)) / math.sqrt(h)).astype(np.float32)
    W3 = (rng.standard_normal((E, h, f)) / math.sqrt(h)).astype(np.float32) if act == "swiglu" else None
    W2 = (rng.standard_normal((E, f, h)) / math.sqrt(f)).astype(np.float32)
    if dtype == "bf16":
        cv = mw.f32_to_bf16_bits
        x, W1, W2 = cv(x), cv(W1), cv(W2)
        W3 = cv(W3) if W3 is not None else None
    return x, Wg, b, W1, W3, W2


def _to_list(a, dtype):
    if a is None:
        return None
    if dtype == "bf16" and a.dtype == np.uint16:
        a = mw.bf16_bits_to_f32(a)
    return np.asarray(a, dtype=np.float64).tolist()


@pytest.mark.parametrize("T,h,f,E,k,cf,act,dtype,tie,bias", [
    (6, 5, 7, 4, 2, 0.0, "gelu", "f32", False, False),
    (7, 4, 6, 6, 3, 0.0, "swiglu", "bf16", True, True),
    (9, 3, 4, 5, 1, 1.0, "gelu", "bf16", False, True),
    (8, 4, 5, 4, 4, 0.0, "swiglu", "f32", True, False),     # k = E
    (10, 6, 3, 3, 2, 0.7, "swiglu", "bf16", False, True),   # drops
])
def test_layer_vs_brute_force(T, h, f, E, k, cf, act, dtype, tie, bias):
    x, Wg, b, W1, W3, W2 = _tiny(T, h, f, E, seed=T * 31 + E, act=act, dtype=dtype,
                                  tie_cols=tie, bias=bias)
    r = o.layer_forward(x, Wg, b, W1, W3, W2, k=k, capacity_factor=cf, act=act, dtype=dtype)
    ref = brute.layer(_to_list(x, dtype), Wg.astype(np.float64).tolist(),
                      None if b is None else b.astype(np.float64).tolist(),
                      _to_list(W1, dtype), _to_list(W3, dtype), _to_list(W2, dtype),
                      k, cf, act, dtype)
    assert r["logits"].astype(np.float64).tolist() == ref["logits"]
    assert r["topk_idx"].tolist() == ref["topk_idx"]
    np.testing.assert_allclose(r["topk_w"], ref["topk_w"], rtol=2e-7)
    assert r["C"] == ref["C"]
    assert r["counts"].tolist() == ref["counts"]
    assert r["offsets"].tolist() == ref["offsets"]
    R = r["offsets"][-1]
    assert r["sorted_slot"][:R].tolist() == ref["sorted_slot"]
    assert r["slot_pos"].tolist() == ref["slot_pos"]
    np.testing.assert_allclose(r["y64"], ref["y64"], rtol=1e-10, atol=1e-12)
    assert abs(r["aux"] - ref["aux"]) < 1e-12


# ----------------------------------------------------------------------------
# special cases that reduce to a dense computation

def _dense_ffn(x64, W1e, W3e, W2e, act):
    z = np.einsum("th,hf->tf", x64, W1e)
    if act == "swiglu":
        hm = z / (1 + np.exp(-z)) * np.einsum("th,hf->tf", x64, W3e)
    else:
        hm = np.array([[0.5 * v * (1 + math.erf(v / math.sqrt(2))) for v in row] for row in z])
    return np.einsum("tf,fh->th", hm, W2e)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_k_equals_E_is_dense_softmax_mixture(act):
    T, h, f, E = 12, 16, 24, 5
    x, Wg, b, W1, W3, W2 = _tiny(T, h, f, E, seed=7, act=act, dtype="f32", bias=True)
    r = o.layer_forward(x, Wg, b, W1, W3, W2, k=E, capacity_factor=0.0, act=act, dtype="f32")
    l = (x.astype(np.float64) @ Wg.astype(np.float64) + b.astype(np.float64)).astype(np.float32)
    p = np.exp(l.astype(np.float64) - l.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    x64 = x.astype(np.float64)
    dense = sum(p[:, e:e + 1] * _dense_ffn(x64, W1[e].astype(np.float64),
                                           None if W3 is None else W3[e].astype(np.float64),
                                           W2[e].astype(np.float64), act) for e in range(E))
    # weights pass through fp32 once (topk_w), hence the relative 1e-7 level
    np.testing.assert_allclose(r["y64"], dense, rtol=2e-6, atol=1e-7)


def test_single_expert_is_plain_ffn():
    T, h, f = 9, 8, 12
    x, Wg, b, W1, W3, W2 = _tiny(T, h, f, 1, seed=11, act="swiglu", dtype="f32")
    r = o.layer_forward(x, Wg, b, W1, W3, W2, k=1, capacity_factor=0.0, act="swiglu", dtype="f32")
    dense = _dense_ffn(x.astype(np.float64), W1[0].astype(np.float64), W3[0].astype(np.float64),
                       W2[0].astype(np.float64), "swiglu")
    np.testing.assert_allclose(r["y64"], dense, rtol=1e-12, atol=1e-14)


def test_k1_dropless_is_argmax_expert():
    T, h, f, E = 15, 8, 6, 4
    x, Wg, b, W1, W3, W2 = _tiny(T, h, f, E, seed=5, act="gelu", dtype="f32")
    r = o.layer_forward(x, Wg, b, W1, W3, W2, k=1, capacity_factor=0.0, act="gelu", dtype="f32")
    for t in range(T):
        e = int(r["logits"][t].argmax())
        ref = _dense_ffn(x[t:t + 1].astype(np.float64), W1[e].astype(np.float64), None,
                         W2[e].astype(np.float64), "gelu")
        np.testing.assert_allclose(r["y64"][t], ref[0], rtol=1e-12, atol=1e-14)


def test_all_dropped_token_outputs_zero():
    # every token prefers expert 0 (large bias); C = floor(1*4*1/2) = 2 -> tokens 2, 3 dropped
    T, h, f, E = 4, 8, 6, 2
    x, Wg, _, W1, W3, W2 = _tiny(T, h, f, E, seed=2, act="gelu", dtype="f32")
    b = np.array([30.0, 0.0], dtype=np.float32)
    r = o.layer_forward(x, Wg, b, W1, W3, W2, k=1, capacity_factor=1.0, act="gelu", dtype="f32")
    assert r["C"] == 2 and r["slot_pos"].tolist() == [0, 1, -1, -1]
    assert (r["y"][2:] == 0).all() and (np.abs(r["y"][:2]) > 0).any()


# ----------------------------------------------------------------------------
# aux loss closed forms

def test_aux_equal_logits_is_one():
    T, h, E, k = 32, 8, 6, 2
    x = np.random.default_rng(0).standard_normal((T, h)).astype(np.float32)
    Wg = np.zeros((h, E), dtype=np.float32)
    r = o.layer_forward(x, Wg, None, None, None, None, k=k, capacity_factor=0.0, act="gelu",
                        dtype="f32", with_y=False)
    assert r["topk_idx"].tolist() == [[0, 1]] * T              # ties -> lower index
    assert abs(r["aux"] - 1.0) < 1e-15


def test_aux_uniform_counts_is_one_and_collapse_is_E():
    rng = np.random.default_rng(4)
    E, T, k = 8, 64, 2
    probs = rng.dirichlet(np.ones(E), size=T)
    counts = np.bincount(mw.uniform_assignment(T, E, k).reshape(-1), minlength=E)
    assert abs(o.aux_loss(counts, probs, T, k, E) - 1.0) < 1e-14
    # routing collapse: k = 1, one expert takes every token with probability -> 1
    l = np.zeros((T, E), dtype=np.float32)
    l[:, 5] = 60.0
    idx = o.select_topk(l, 1)
    c = o.histogram(idx, E)
    assert c.tolist() == [0, 0, 0, 0, 0, T, 0, 0]
    aux = o.aux_loss(c, o.softmax(l), T, 1, E)
    assert abs(aux - E) < 1e-20 * E + E * 1e-24 + 1e-12


# ----------------------------------------------------------------------------
# elementwise pieces vs library routines

def test_gelu_silu_vs_math():
    z = np.linspace(-8, 8, 101)
    np.testing.assert_allclose(o.gelu(z), [0.5 * v * (1 + math.erf(v / math.sqrt(2))) for v in z],
                               rtol=1e-15, atol=1e-300)
    np.testing.assert_allclose(o.silu(z), [v / (1 + math.exp(-v)) for v in z], rtol=1e-15)
    assert o.gelu(np.array([0.0]))[0] == 0.0
    assert abs(o.gelu(np.array([10.0]))[0] - 10.0) < 1e-15


def test_round_to_bf16_vs_torch_and_ties():
    torch = pytest.importorskip("torch")
    v = np.random.default_rng(9).standard_normal(200000).astype(np.float32) * 10
    ours = o.round_to_bf16(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    one = 1.0
    cases = {one: 0x3F80,
             one + 2 ** -8: 0x3F80,                 # tie -> even (1.0)
             one + 3 * 2 ** -8: 0x3F82,             # tie -> even (1 + 2^-6)
             one + 2 ** -8 + 2 ** -40: 0x3F81,      # just above the tie: needs fp64, not fp32
             -2.5: 0xC020, 0.0: 0x0000}
    for val, bits in cases.items():
        assert int(o.round_to_bf16(np.array([val]))[0]) == bits, val
    # agrees with the brute-force neighbour search
    for val in np.random.default_rng(1).standard_normal(2000) * 3:
        b = o.bf16_to_f64(o.round_to_bf16(np.array([val])))[0]
        assert b == brute.bf16(float(val))


def test_bf16_roundtrip_exact():
    bits = np.arange(0, 0x7F80, 7, dtype=np.uint16)  # positive finite patterns
    assert np.array_equal(o.round_to_bf16(o.bf16_to_f64(bits)), bits)


def test_expert_ffn_vs_loops_bf16():
    rng = np.random.default_rng(12)
    h, f, n = 6, 5, 4
    a = mw.bf16_bits_to_f32(mw.f32_to_bf16_bits(rng.standard_normal((n, h)).astype(np.float32))).astype(np.float64)
    W1 = mw.f32_to_bf16_bits(rng.standard_normal((h, f)).astype(np.float32))
    W3 = mw.f32_to_bf16_bits(rng.standard_normal((h, f)).astype(np.float32))
    W2 = mw.f32_to_bf16_bits(rng.standard_normal((f, h)).astype(np.float32))
    out = o.expert_ffn(a, W1, W3, W2, "swiglu", "bf16")
    w1, w3, w2 = (mw.bf16_bits_to_f32(m).astype(np.float64) for m in (W1, W3, W2))
    for r in range(n):
        hm = []
        for c in range(f):
            z1 = math.fsum(a[r, i] * w1[i, c] for i in range(h))
            z3 = math.fsum(a[r, i] * w3[i, c] for i in range(h))
            hm.append(brute.bf16(z1 / (1 + math.exp(-z1)) * z3))
        ref = [math.fsum(hm[c] * w2[c, q] for c in range(f)) for q in range(h)]
        np.testing.assert_allclose(out[r], ref, rtol=1e-12, atol=1e-13)


def test_generator_is_seeded_and_sliceable():
    w = mw.by_name("tiny-fp32")
    a = mw.make_inputs(w)
    b = mw.make_inputs(w)
    for key in ("x", "W_gate", "W1", "W2"):
        assert np.array_equal(a[key], b[key])
    assert np.array_equal(a["W1"][3], mw.expert_slice(w, "W1", 3))
    assert a["W3"] is None and a["logit_bias"] is None
    # distributions: N(0,1) x, N(0,1/h) gate
    assert abs(a["x"].std() - 1) < 0.05 and abs(a["W_gate"].std() * math.sqrt(w.h) - 1) < 0.1


# ----------------------------------------------------------------------------
# fixed-capacity ("binned") layout

def test_binned_worked_example():
    g = _gold("mb_histogram_example.json")
    idx = np.array(g["topk_idx"], dtype=np.int32).reshape(-1, 1)
    counts = o.histogram(idx, g["E"])
    for key, cf, mn in (("cf_1", 1.0, 0), ("cf_0", 0.0, 0), ("cf_0.5_min_3", 0.5, 3)):
        ref = g["binned"][key]
        C = o.binned_capacity(idx.shape[0], g["E"], 1, cf, mn, counts)
        assert C == ref["C"], key
        bins, slot_pos = o.binned_layout(idx, g["E"], C)
        assert bins.tolist() == ref["bins"], key
        assert slot_pos.tolist() == ref["slot_pos"], key


def test_binned_capacity_rules():
    counts = [5, 1, 0, 9]
    assert o.binned_capacity(8, 4, 2, 0.0, 4, counts) == 9          # factor 0: the largest count
    assert o.binned_capacity(8, 4, 2, -1.0, 0, counts) == 9
    assert o.binned_capacity(8, 4, 2, 1.25, 0, counts) == 5         # floor(1.25 * 16 / 4)
    assert o.binned_capacity(8, 4, 2, 0.1, 4, counts) == 4          # the minimum capacity
    assert o.binned_capacity(8, 4, 2, 0.1, 0, counts) == 9          # computed zero: the largest count
    with pytest.raises(ValueError):
        o.binned_capacity(8, 4, 2, float("nan"), 0, counts)


def test_binned_keeps_what_the_compact_layout_keeps():
    # the same stable ranks decide both layouts: row e*C + i holds the assignment that the
    # compact layout puts at offsets[e] + i
    rng = np.random.default_rng(21)
    for E, k, T, C in [(5, 2, 40, 7), (8, 3, 33, 2), (3, 1, 50, 30)]:
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        counts, offsets, sorted_slot, _ = o.permute(idx, E, C)
        bins, slot_pos = o.binned_layout(idx, E, C)
        for e in range(E):
            kept = sorted_slot[offsets[e]:offsets[e + 1]].tolist()
            assert bins[e, :len(kept)].tolist() == kept
            assert (bins[e, len(kept):] == -1).all()
        assert ((slot_pos >= 0) == (o.permute(idx, E, C)[3] >= 0)).all()


@pytest.mark.parametrize("T,h,f,E,k,cf,act,dtype", [
    (7, 4, 6, 6, 3, 0.0, "swiglu", "bf16"),   # factor 0: buckets of the largest count, nothing dropped
    (10, 6, 3, 3, 2, 0.7, "swiglu", "bf16"),  # drops
    (9, 3, 4, 5, 1, 1.0, "gelu", "f32"),
])
def test_binned_layer_vs_brute_force(T, h, f, E, k, cf, act, dtype):
    x, Wg, b, W1, W3, W2 = _tiny(T, h, f, E, seed=T * 17 + E, act=act, dtype=dtype, bias=True)
    r = o.layer_forward_binned(x, Wg, b, W1, W3, W2, k=k, capacity_factor=cf, min_capacity=0, act=act,
                               dtype=dtype)
    ref = brute.layer(_to_list(x, dtype), Wg.astype(np.float64).tolist(), b.astype(np.float64).tolist(),
                      _to_list(W1, dtype), _to_list(W3, dtype), _to_list(W2, dtype), k, cf, act, dtype)
    np.testing.assert_allclose(r["y64"], ref["y64"], rtol=1e-10, atol=1e-12)
    assert abs(r["aux"] - ref["aux"]) < 1e-12
    # the buckets: token rows where a slot is filled, zero rows elsewhere
    C = r["C"]
    for e in range(E):
        for i in range(C):
            s = r["bins"][e, i]
            want = x[s // k] if s >= 0 else np.zeros_like(x[0])
            assert np.array_equal(r["x_bins"][e, i], want)


# ----------------------------------------------------------------------------
# router variants: temperature, gate noise, uniform assignment, jitter

def test_temperature_one_is_the_plain_router():
    rng = np.random.default_rng(5)
    l = rng.standard_normal((40, 16)).astype(np.float32)
    r = o.route(l, 4)
    idx = o.select_topk(l, 4)
    assert np.array_equal(r["topk_idx"], idx)
    assert np.array_equal(r["topk_w"], o.topk_weights(l, idx))
    assert np.array_equal(r["probs"], o.softmax(l))


def test_temperature_closed_form_on_the_worked_example():
    """k = 2 on the [OPS] worked example (experts 0 and 6, scores 0.9 and 0.7): the
    renormalised pair is a logistic of the score gap over the temperature,
    w0 = 1 / (1 + exp(-(0.9 - 0.7) / tau))."""
    g = _gold("ops_top2_example.json")
    l = np.array([g["scores"]], dtype=np.float32)
    for tau in (0.5, 2.0, 0.1):
        r = o.route(l, 2, temperature=tau)
        assert r["topk_idx"].tolist() == [g["topk_idx"]]   # selection does not move with tau
        gap = float(np.float32(0.9)) - float(np.float32(0.7))
        w0 = 1.0 / (1.0 + math.exp(-gap / tau))
        np.testing.assert_allclose(r["topk_w"][0], [w0, 1.0 - w0], rtol=3e-7)
        # the full probabilities are the plain softmax of the scores over tau
        z = np.exp((np.array(g["scores"], np.float32).astype(np.float64) - 0.9) / tau)
        np.testing.assert_allclose(r["probs"][0], z / z.sum(), rtol=1e-6)


def test_soft_topk_closed_form_on_the_worked_example():
    """Soft top-K ([OPS] "坑3") on the worked example, k = 2 (experts 0 and 6): the
    weights are the temperature softmax over all eight scores taken at the two selected
    experts, not renormalised -- w_j = exp(s_j / tau) / sum_e exp(s_e / tau), written
    out with math.exp and math.fsum.  The unselected experts keep the rest of the mass."""
    g = _gold("ops_top2_example.json")
    s32 = [float(np.float32(v)) for v in g["scores"]]
    l = np.array([g["scores"]], dtype=np.float32)
    for tau in (1.0, 0.5, 2.0, 0.1):
        r = o.route(l, 2, temperature=tau, soft=True)
        assert r["topk_idx"].tolist() == [g["topk_idx"]]   # the selection is the hard top-k's
        den = math.fsum(math.exp(v / tau) for v in s32)
        want = [math.exp(s32[e] / tau) / den for e in g["topk_idx"]]
        np.testing.assert_allclose(r["topk_w"][0], want, rtol=3e-7)
        rest = math.fsum(math.exp(s32[e] / tau) / den for e in range(8) if e not in g["topk_idx"])
        assert abs(math.fsum(map(float, r["topk_w"][0])) + rest - 1.0) < 1e-6
        assert float(r["topk_w"][0].sum()) < 1.0 - 0.5 * rest        # mass left to the other six
    # tau = 1: exactly the plain softmax probabilities of the selected pair
    w1 = o.route(l, 2, soft=True)["topk_w"][0]
    p = o.softmax(l)[0]
    assert w1.tolist() == [np.float32(p[0]), np.float32(p[6])]


def test_soft_topk_limits_and_special_cases():
    rng = np.random.default_rng(16)
    l = (rng.permutation(64).reshape(8, 8) / 8.0).astype(np.float32)  # distinct logits, gaps >= 1/8
    cold = o.route(l, 3, temperature=1e-3, soft=True)["topk_w"]
    np.testing.assert_allclose(cold[:, 0], 1.0, atol=1e-30)             # all mass on the best expert
    assert np.abs(cold[:, 1:]).max() < 1e-30
    hot = o.route(l, 3, temperature=1e9, soft=True)["topk_w"]
    np.testing.assert_allclose(hot, 1.0 / 8.0, rtol=1e-6)               # spread over all E experts
    # k = E: nothing is left unselected, so the soft weights are the renormalised ones
    full_s = o.route(l, 8, temperature=0.7, soft=True)["topk_w"]
    full_r = o.route(l, 8, temperature=0.7)["topk_w"]
    np.testing.assert_allclose(full_s, full_r, rtol=1e-6)
    # the ratios between the selected weights do not depend on the renormalisation
    ws = o.route(l, 3, temperature=0.7, soft=True)["topk_w"].astype(np.float64)
    wr = o.route(l, 3, temperature=0.7)["topk_w"].astype(np.float64)
    np.testing.assert_allclose(ws / ws.sum(1, keepdims=True), wr, rtol=1e-6)
    assert (ws.sum(1) < 1.0).all()


def test_temperature_limits():
    rng = np.random.default_rng(6)
    l = (rng.permutation(64).reshape(8, 8) / 8.0).astype(np.float32)  # distinct logits, gaps >= 1/8
    hot = o.route(l, 3, temperature=1e9)["topk_w"]
    np.testing.assert_allclose(hot, 1.0 / 3.0, rtol=1e-6)               # flat: uniform weights
    cold = o.route(l, 3, temperature=1e-3)["topk_w"]
    np.testing.assert_allclose(cold[:, 0], 1.0, atol=1e-30)             # sharp: all weight on the best
    with pytest.raises(ValueError):
        o.route(l, 3, temperature=0.0)


def test_noise_shift_per_token_changes_nothing():
    """Softmax and top-k are invariant to adding one constant to all logits of a token.
    Logits on a 2^-10 grid plus whole-number shifts are exact in fp32, so the noisy
    selection is bit-identical and the weights equal to fp64 rounding."""
    rng = np.random.default_rng(7)
    l = (rng.integers(-2048, 2048, size=(32, 12)) / 1024.0).astype(np.float32)
    shift = rng.integers(-8, 9, size=(32, 1)).astype(np.float32) * np.ones((1, 12), np.float32)
    a, b = o.route(l, 3), o.route(l, 3, noise=shift)
    assert np.array_equal(a["topk_idx"], b["topk_idx"])
    np.testing.assert_allclose(b["topk_w"], a["topk_w"], rtol=1e-6)
    np.testing.assert_allclose(b["probs"], a["probs"], rtol=1e-12)


def test_noise_decides_the_selection():
    l = np.zeros((6, 5), np.float32)
    noise = np.zeros((6, 5), np.float32)
    for t in range(6):
        noise[t, (t * 2) % 5] = 4.0
    r = o.route(l, 2, noise=noise)
    assert r["topk_idx"][:, 0].tolist() == [(t * 2) % 5 for t in range(6)]
    # second place: the equal zeros, lowest expert first
    assert r["topk_idx"][:, 1].tolist() == [1 if (t * 2) % 5 == 0 else 0 for t in range(6)]
    # noise equal to minus the logits leaves all-equal scores: experts 0..k-1, equal weights
    l2 = np.random.default_rng(8).standard_normal((4, 6)).astype(np.float32)
    r2 = o.route(l2, 3, noise=-l2)
    assert r2["topk_idx"].tolist() == [[0, 1, 2]] * 4
    np.testing.assert_allclose(r2["topk_w"], 1.0 / 3.0, rtol=1e-7)


def test_uniform_assignment_ids_counts_and_aux():
    # ids of slot j of token t: (t*k + j) % E, written out for T = 3, k = 2, E = 4
    assert o.uniform_assignment(3, 2, 4).tolist() == [[0, 1], [2, 3], [0, 1]]
    rng = np.random.default_rng(9)
    l = rng.standard_normal((48, 8)).astype(np.float32)
    r = o.route(l, 2, uniform=True)
    counts = o.histogram(r["topk_idx"], 8)
    assert (counts == 12).all()
    # the weights are those of the real top-k
    assert np.array_equal(r["topk_w"], o.topk_weights(l, o.select_topk(l, 2)))
    # perfectly balanced counts: the aux loss is sum_e P_e = 1 whatever the router says
    assert abs(o.aux_loss(counts, r["probs"], 48, 2, 8) - 1.0) < 1e-12


def test_jitter_input_vs_torch_and_identity():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(10)
    x = mw.f32_to_bf16_bits(rng.standard_normal((16, 64)).astype(np.float32))
    u = mw.f32_to_bf16_bits(rng.uniform(0.99, 1.01, size=(16, 64)).astype(np.float32))
    got = o.jitter_input(x, u, "bf16")
    tx = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
    tu = torch.from_numpy(u.view(np.int16)).view(torch.bfloat16)
    want = (tx * tu).view(torch.int16).numpy().view(np.uint16)   # torch: fp32 product, RNE to bf16
    assert np.array_equal(got, want)
    one = mw.f32_to_bf16_bits(np.ones((16, 64), np.float32))
    assert np.array_equal(o.jitter_input(x, one, "bf16"), x)
    xf = rng.standard_normal((4, 8)).astype(np.float32)
    uf = rng.uniform(0.9, 1.1, (4, 8)).astype(np.float32)
    assert np.array_equal(o.jitter_input(xf, uf, "f32"), xf * uf)   # fp32: one rounding of the product


def test_layer_router_variants_vs_brute_force():
    """The layer with jitter, noise, a temperature, the uniform assignment and the soft
    top-K against a brute force fed the same variant routing."""
    rng = np.random.default_rng(11)
    T, h, f, E, k = 12, 16, 24, 5, 2
    x = rng.standard_normal((T, h)).astype(np.float32)
    Wg = (rng.standard_normal((h, E)) / 4).astype(np.float32)
    W1 = (rng.standard_normal((E, h, f)) / 4).astype(np.float32)
    W2 = (rng.standard_normal((E, f, h)) / 5).astype(np.float32)
    u = rng.uniform(0.9, 1.1, (T, h)).astype(np.float32)
    noise = (rng.standard_normal((T, E)) / E).astype(np.float32)
    for uniform, soft in ((False, False), (True, False), (False, True)):
        ref = o.layer_forward(x, Wg, None, W1, None, W2, k=k, capacity_factor=0.0, act="gelu", dtype="f32",
                              jitter=u, noise=noise, temperature=0.7, uniform=uniform, soft=soft)
        # routing of the variant, recomputed step by step from its definitions
        xr = x * u
        lg = (xr.astype(np.float64) @ Wg.astype(np.float64)).astype(np.float32)
        ln = (lg + noise).astype(np.float32)
        idx = np.argsort(-ln.astype(np.float64), axis=1, kind="stable")[:, :k]
        p = np.exp((ln.astype(np.float64) - ln.max(1, keepdims=True)) / 0.7)
        ps = np.take_along_axis(p, idx, 1)
        w = ps / (p.sum(1, keepdims=True) if soft else ps.sum(1, keepdims=True))
        if uniform:
            idx = (np.arange(T * k) % E).reshape(T, k)
        y = np.zeros((T, h))
        for t in range(T):
            for j in range(k):
                e = idx[t, j]
                a = np.array([math.fsum(float(x[t, i]) * float(W1[e, i, c]) for i in range(h)) for c in range(f)])
                hm = 0.5 * a * (1 + np.array([math.erf(v / math.sqrt(2)) for v in a]))
                y[t] += w[t, j] * np.array([math.fsum(hm[c] * float(W2[e, c, i]) for c in range(f))
                                            for i in range(h)])
        assert np.array_equal(ref["topk_idx"], idx)
        np.testing.assert_allclose(ref["y64"], y, rtol=1e-5, atol=1e-6)
