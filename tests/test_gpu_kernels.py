"""GPU parity of each entry point against the CPU oracle (through the C ABI).

Integer results (indices, counts, offsets, the permutation, drops) must be
bit-identical when both sides route on the same fp32 logits; floats within the
stated tolerances: fp32 relative 1e-5 (with an RMS floor), bf16 outputs
max |d| <= 2e-2 * RMS(ref).
"""
import math

import numpy as np
import pytest

import moe_workloads as mw
import oracle as o
import top_routing_expert_moe_amd as moe
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------- router

@pytest.mark.parametrize("name", [w.name for w in mw.WORKLOADS])
def test_route_parity(name):
    torch = gu.torch()
    w = mw.by_name(name)
    _say(f"route {name}")
    d = mw.make_inputs(w, with_weights=False)
    x = gu.to_dev(d["x"], w.dtype)
    Wg = gu.to_dev(d["W_gate"], "f32")
    b = gu.to_dev(d["logit_bias"], "f32")
    logits, idx, wt, ps = moe.route(x, Wg, b, w.k, with_prob_sum=True)
    torch.cuda.synchronize()
    gl = gu.from_dev(logits)
    # logits vs the oracle's fp64-accumulated logits
    ref_l = o.router_logits(d["x"], d["W_gate"], d["logit_bias"], w.dtype)
    gu.check_rel_rms(gl, ref_l, 1e-5, "logits")
    # Mode A: the oracle routes on the GPU's logits -> bit-identical selection
    ridx = o.select_topk(gl, w.k)
    assert np.array_equal(gu.from_dev(idx), ridx)
    gu.check_rel_rms(gu.from_dev(wt), o.topk_weights(gl, ridx), 1e-5, "topk_w")
    gu.check_rel_rms(gu.from_dev(ps), o.softmax(gl).sum(0), 1e-5, "prob_sum")
    # how many tokens would route differently on the oracle's own logits (near ties only)
    own = o.select_topk(ref_l, w.k)
    diff = int((np.sort(own, 1) != np.sort(ridx, 1)).any(1).sum())
    _say(f"  tokens whose top-k set differs on oracle logits: {diff}")
    assert diff <= max(2, w.T // 500)


def test_route_ties_signed_zero_and_k_equals_E():
    torch = gu.torch()
    rng = np.random.default_rng(5)
    for E, k in [(8, 2), (6, 6), (100, 7), (256, 16), (64, 1), (3, 2)]:
        T = 70
        l = rng.standard_normal((T, E)).astype(np.float32)
        l[0] = 1.5                                   # all equal
        l[1, : min(E, 4)] = 2.0                      # a tie at the top
        l[2] = 0.0
        l[2, ::2] = -0.0                             # signed zeros are equal
        l[3] = l[4]                                  # equal rows
        l[5, -1] = 50.0                              # collapse onto the last expert
        l = np.round(l * 4) / 4                      # many exact ties
        dl = gu.to_dev(l.copy(), "f32")
        _, idx, wt, ps = moe.route(None, None, None, k, logits=dl, with_prob_sum=True)
        torch.cuda.synchronize()
        ridx = o.select_topk(l, k)
        assert np.array_equal(gu.from_dev(idx), ridx), (E, k)
        gu.check_rel_rms(gu.from_dev(wt), o.topk_weights(l, ridx), 1e-5, f"w E={E}")
        gu.check_rel_rms(gu.from_dev(ps), o.softmax(l).sum(0), 1e-5, f"prob_sum E={E}")
        assert np.abs(gu.from_dev(wt).astype(np.float64).sum(1) - 1).max() < 1e-6


@pytest.mark.parametrize("T,h,E,k", [(65, 192, 8, 2), (100, 64, 40, 3), (1, 256, 256, 8), (130, 320, 96, 4),
                                     (70, 128, 32, 1), (3, 192, 16, 16), (257, 512, 64, 2), (64, 1024, 200, 6),
                                     (1100, 256, 64, 2), (1030, 384, 256, 8),  # 64 tokens per router wave
                                     (1030, 512, 128, 4), (1100, 768, 192, 3)])  # ... eight waves, 8-way k split
def test_route_bf16_shapes(T, h, E, k):
    """The MFMA router's code paths: k split across waves (h % 128), 1/2/4 expert blocks, ragged T and E."""
    torch = gu.torch()
    rng = np.random.default_rng(T * 7 + E)
    x = mw.f32_to_bf16_bits(rng.standard_normal((T, h)).astype(np.float32))
    Wg = (rng.standard_normal((h, E)) / np.sqrt(h)).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    logits, idx, wt, ps = moe.route(gu.to_dev(x, "bf16"), gu.to_dev(Wg, "f32"), gu.to_dev(b, "f32"), k,
                                    with_prob_sum=True)
    torch.cuda.synchronize()
    gl = gu.from_dev(logits)
    gu.check_rel_rms(gl, o.router_logits(x, Wg, b, "bf16"), 1e-5, "logits")
    ridx = o.select_topk(gl, k)
    assert np.array_equal(gu.from_dev(idx), ridx)
    gu.check_rel_rms(gu.from_dev(wt), o.topk_weights(gl, ridx), 1e-5, "topk_w")
    gu.check_rel_rms(gu.from_dev(ps), o.softmax(gl).sum(0), 1e-5, "prob_sum")


def test_route_fp32_input_small_T():
    torch = gu.torch()
    rng = np.random.default_rng(8)
    for T in (1, 31, 33):
        x = rng.standard_normal((T, 128)).astype(np.float32)
        Wg = (rng.standard_normal((128, 16)) / 11).astype(np.float32)
        logits, idx, wt, _ = moe.route(gu.to_dev(x, "f32"), gu.to_dev(Wg, "f32"), None, 3)
        torch.cuda.synchronize()
        gl = gu.from_dev(logits)
        gu.check_rel_rms(gl, o.router_logits(x, Wg, None, "f32"), 1e-5, f"logits T={T}")
        assert np.array_equal(gu.from_dev(idx), o.select_topk(gl, 3))


# ---------------------------------------------------------------- permutation

def _perm_cases():
    rng = np.random.default_rng(11)
    cases = []
    cases.append(("uniform", mw.uniform_assignment(4096, 8, 2), 8, 0.0))
    cases.append(("uniform-e256", mw.uniform_assignment(4096, 256, 8), 256, 0.0))
    cases.append(("e256-k16-cap", mw.uniform_assignment(1000, 256, 16), 256, 0.5))  # largest E and k
    one = np.zeros((3000, 1), dtype=np.int32)
    cases.append(("all-to-one", one, 16, 0.0))
    cases.append(("all-to-one-cap", one, 16, 1.0))          # C = 187: almost all dropped
    idx = np.stack([rng.permutation(64)[:2] for _ in range(8192)]).astype(np.int32)
    idx[idx % 8 == 3] = 0                                    # empty experts, one hot expert
    cases.append(("empty-experts-cap", idx, 64, 1.25))
    cases.append(("C=1", np.stack([rng.permutation(8)[:2] for _ in range(40)]).astype(np.int32), 8, 0.1))
    zipf = np.minimum(rng.zipf(1.3, size=(5000, 1)) - 1, 99).astype(np.int32)
    cases.append(("zipf-k1-E100", zipf, 100, 0.9))
    cases.append(("ragged", np.stack([rng.permutation(5)[:3] for _ in range(777)]).astype(np.int32), 5, 0.0))
    return cases


@pytest.mark.parametrize("case", _perm_cases(), ids=lambda c: c[0])
def test_permute_parity(case):
    torch = gu.torch()
    name, idx, E, cf = case
    T, k = idx.shape
    _say(f"permute {name} T={T} k={k} E={E} cf={cf}")
    h = 64
    x = mw.f32_to_bf16_bits(np.random.default_rng(T).standard_normal((T, h)).astype(np.float32))
    probs = np.random.default_rng(1).dirichlet(np.ones(E), size=T).astype(np.float32)
    ps = probs.astype(np.float64).sum(0).astype(np.float32)
    xps = gu.sentinel_like((T * k, h), "bf16")
    r = moe.permute(torch.from_numpy(idx).to(gu.dev()), gu.to_dev(x, "bf16"), E, cf,
                    prob_sum=gu.to_dev(ps, "f32"), x_perm=xps)
    torch.cuda.synchronize()
    C = o.expert_capacity(T, E, k, cf)
    counts, offsets, sorted_slot, slot_pos = o.permute(idx, E, C)
    R = int(offsets[-1])
    assert np.array_equal(gu.from_dev(r["counts"]), counts)
    assert np.array_equal(gu.from_dev(r["offsets"]), offsets)
    assert np.array_equal(gu.from_dev(r["slot_pos"]), slot_pos)
    assert np.array_equal(gu.from_dev(r["sorted_slot"])[:R], sorted_slot[:R])
    xp_all = gu.from_dev(r["x_perm"])
    xp = xp_all[:R]
    assert np.array_equal(xp, x[sorted_slot[:R] // k])
    assert gu.is_sentinel(xp_all[R:], "bf16").all()   # only the kept rows are written
    aux = float(gu.from_dev(r["aux"]))
    ref = E * float(np.sum(counts / (T * k) * (ps.astype(np.float64) / T)))
    assert abs(aux - ref) <= 1e-5 * abs(ref)


# ---------------------------------------------------------------- combine

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_unpermute_parity(dtype):
    torch = gu.torch()
    rng = np.random.default_rng(3)
    T, k, E, h = 300, 3, 7, 192
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    C = o.expert_capacity(T, E, k, 0.8)
    _, offsets, sorted_slot, slot_pos = o.permute(idx, E, C)
    R = int(offsets[-1])
    O = _rand((R, h), 1.0, rng, dtype)
    w = rng.dirichlet(np.ones(k), size=T).astype(np.float32)
    y = moe.unpermute(gu.to_dev(O, dtype), torch.from_numpy(slot_pos).to(gu.dev()), gu.to_dev(w, "f32"))
    torch.cuda.synchronize()
    O64 = gu.as_f64(O, dtype)
    ref = np.zeros((T, h))
    sp = slot_pos.reshape(T, k)
    for j in range(k):
        m = sp[:, j] >= 0
        ref[m] += w[m, j:j + 1].astype(np.float64) * O64[sp[m, j]]
    got = gu.as_f64(gu.from_dev(y), dtype)
    assert (sp < 0).all(1).any()                # some tokens lost every slot ...
    assert (got[(sp < 0).all(1)] == 0).all()    # ... and output exactly zero
    if dtype == "bf16":
        gu.check_bf16_out(got, ref, "y", frac=1e-2)
    else:
        gu.check_rel_rms(got, ref, 1e-6, "y")


# ---------------------------------------------------------------- expert FFN (grouped GEMM)

def _rand(shape, scale, rng, dtype):
    a = (rng.standard_normal(shape) * scale).astype(np.float32)
    return mw.f32_to_bf16_bits(a) if dtype == "bf16" else a


def _ffn_case(E, h, f, seg, act, dtype, seed):
    rng = np.random.default_rng(seed)
    R = int(sum(seg))
    R_max = R + 7  # rows beyond offsets[E] must stay untouched (checked with a sentinel)
    xp = _rand((R_max, h), 1.0, rng, dtype)
    W1 = _rand((E, h, f), 1 / math.sqrt(h), rng, dtype)
    W3 = _rand((E, h, f), 1 / math.sqrt(h), rng, dtype) if act == "swiglu" else None
    W2 = _rand((E, f, h), 1 / math.sqrt(f), rng, dtype)
    offsets = np.concatenate([[0], np.cumsum(seg)]).astype(np.int32)
    return xp, W1, W3, W2, offsets, R


@pytest.mark.parametrize("act,dtype,E,h,f,seg", [
    ("swiglu", "bf16", 5, 256, 512, [0, 1, 300, 257, 37]),       # empty, single row, >1 tile, ragged
    ("gelu", "bf16", 4, 192, 320, [256, 0, 513, 2]),              # N tails in both projections
    ("swiglu", "bf16", 3, 512, 384, [31, 64, 700]),
    ("swiglu", "bf16", 8, 256, 512, [16, 0, 3, 40, 16, 1, 33, 17]),  # few rows per expert: 32-row tiles
    ("gelu", "bf16", 2, 256, 320, [600, 700]),                     # many rows per expert: 256-row tiles
    ("swiglu", "bf16", 2, 192, 320, [300, 530]),                   # 256-row tiles with k and N tails
    ("swiglu", "bf16", 4, 1024, 2048, [5, 20, 0, 9]),              # 32-row tiles, K split 2 (up) and 4 (down)
    ("gelu", "bf16", 3, 2048, 1024, [12, 3, 30]),                  # K split 4 (up) and 2 (down), GELU parts
    ("swiglu", "bf16", 8, 256, 512, [700, 20, 5, 40, 60, 0, 100, 90]),  # 128-row launch, one big expert: 256-row tiles
    ("gelu", "bf16", 6, 192, 320, [512, 511, 3, 0, 40, 33]),           # ... at the threshold (512 rows) and just below
    ("swiglu", "bf16", 4, 2048, 256, [200, 129, 0, 60]),               # h >= 2048: 256-row tiles from 129 rows
    ("swiglu", "f32", 5, 128, 256, [0, 1, 70, 129, 37]),
    ("gelu", "f32", 3, 192, 320, [65, 0, 64]),
])
def test_expert_ffn_parity(act, dtype, E, h, f, seg):
    torch = gu.torch()
    _say(f"expert_ffn {act} {dtype} E={E} h={h} f={f} seg={seg}")
    xp, W1, W3, W2, offsets, R = _ffn_case(E, h, f, seg, act, dtype, seed=E * 7 + h)
    dx = gu.to_dev(xp, dtype)
    out = moe.expert_ffn(dx, torch.from_numpy(offsets).to(gu.dev()), gu.to_dev(W1, dtype), gu.to_dev(W3, dtype),
                         gu.to_dev(W2, dtype), act, out=gu.sentinel_like(tuple(dx.shape), dtype))
    torch.cuda.synchronize()
    raw = gu.from_dev(out)
    assert gu.is_sentinel(raw[R:], dtype).all(), "rows past offsets[E] were written"
    assert not gu.is_sentinel(raw[:R], dtype).any(), "a kept row was not written"
    got = gu.as_f64(raw[:R], dtype)
    a64 = gu.as_f64(xp, dtype)
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if hi == lo:
            continue
        ref = o.expert_ffn(a64[lo:hi], W1[e], None if W3 is None else W3[e], W2[e], act, dtype)
        if dtype == "bf16":
            gu.check_bf16_out(got[lo:hi], ref, f"expert {e}")
        else:
            gu.check_rel_rms(got[lo:hi], ref, 1e-5, f"expert {e}")
