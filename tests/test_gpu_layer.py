"""GPU parity of the whole layer (moe_layer_forward) against the CPU oracle, at the
workloads' full sizes, in the launch configuration the benchmark times.

Mode A: the oracle routes on the GPU router's fp32 logits (obtained from
moe_route, the same kernel the layer runs), so every integer decision is
shared and must agree bit for bit (counts).  Mode B: the layer output y is
compared with the oracle's y on that routing -- all tokens for the small
workloads, a seeded sample of 256 tokens (each one exact, independent of the
others) for the large ones.
"""
import numpy as np
import pytest

import moe_workloads as mw
import oracle as o
import top_routing_expert_moe_amd as moe
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

SAMPLE = 256


def _say(*a):
    print(*a, flush=True)


def _run_layer(w, d_host, d_dev):
    """The layer on a sentinel-filled y, with its workspace kept: returns y, aux, counts,
    the router's logits (from moe_route, the same kernel) and the routing the layer left
    in its workspace (moe_layer_routing)."""
    torch = gu.torch()
    dt = moe.BF16 if w.dtype == "bf16" else moe.F32
    ws = moe._ws(moe.workspace_bytes(w.T, w.h, w.f, w.E, w.k, w.cf, dt, moe.SWIGLU if w.act == "swiglu" else moe.GELU),
                 d_dev["x"].device)
    y = gu.sentinel_like(tuple(d_dev["x"].shape), w.dtype)
    y, aux, counts = moe.layer_forward(d_dev["x"], d_dev["W_gate"], d_dev["logit_bias"], d_dev["W1"], d_dev["W3"],
                                       d_dev["W2"], k=w.k, capacity_factor=w.cf, act=w.act, ws=ws, y=y)
    logits, idx, _, _ = moe.route(d_dev["x"], d_dev["W_gate"], d_dev["logit_bias"], w.k)
    torch.cuda.synchronize()
    routing = moe.layer_routing(ws, T=w.T, h=w.h, f=w.f, E=w.E, k=w.k, capacity_factor=w.cf, dtype=dt, act=w.act)
    routing = {kk: gu.from_dev(v).copy() for kk, v in routing.items()}
    return y, aux, counts, logits, routing


def _check_layer(w, host, y, aux, counts, logits, tokens, routing=None):
    gl = gu.from_dev(logits)
    ref = o.layer_forward(host["x"], host["W_gate"], host["logit_bias"], host["W1"], host["W3"], host["W2"],
                          k=w.k, capacity_factor=w.cf, act=w.act, dtype=w.dtype, logits=gl, tokens=tokens)
    assert np.array_equal(gu.from_dev(counts), ref["counts"])
    assert not gu.is_sentinel(gu.from_dev(y), w.dtype).any(), "a row of y was not written"
    if routing is not None:
        # the layer's own routing, bit for bit: the same logits, selection, permutation and drops
        R = int(ref["offsets"][-1])
        assert np.array_equal(routing["logits"], gl)
        assert np.array_equal(routing["topk_idx"], ref["topk_idx"])
        assert np.array_equal(routing["offsets"], ref["offsets"])
        assert np.array_equal(routing["slot_pos"], ref["slot_pos"])
        assert np.array_equal(routing["slot_pos"] < 0, ref["slot_pos"] < 0)      # the drop mask
        assert np.array_equal(routing["sorted_slot"][:R], ref["sorted_slot"][:R])
        gu.check_rel_rms(routing["topk_w"], ref["topk_w"], 1e-5, "topk_w")
    R = int(ref["offsets"][-1])
    _say(f"  rows kept {R} of {w.T * w.k}; active experts {int((ref['counts'] > 0).sum())}; C={ref['C']}")
    a = float(gu.from_dev(aux))
    assert abs(a - ref["aux"]) <= 1e-5 * abs(ref["aux"]), (a, ref["aux"])
    got = gu.as_f64(gu.from_dev(y)[tokens], w.dtype)
    if w.dtype == "bf16":
        raw, beyond = gu.check_bf16_out(got, ref["y64"], "y")
        _say(f"  y max|d|/RMS = {raw:.4f} (beyond the output's own bf16 rounding: {beyond:.4f})")
    else:
        gu.check_rel_rms(got, ref["y64"], 1e-5, "y")
    return ref


@pytest.mark.parametrize("name", [w.name for w in mw.WORKLOADS])
def test_layer_forward_parity(name):
    _say(f"layer {name}")
    w, host, dd = gu.workload(name)
    y, aux, counts, logits, routing = _run_layer(w, host, dd)
    if w.T <= 64:
        tokens = np.arange(w.T)
    else:
        tokens = np.sort(np.random.default_rng(123).choice(w.T, SAMPLE, replace=False))
        tokens[0], tokens[-1] = 0, w.T - 1  # include both ends of the batch
    _check_layer(w, host, y, aux, counts, logits, tokens, routing)


def test_layer_forward_deterministic():
    torch = gu.torch()
    for name in ("tiny-fp32", "capacity-e64"):
        w, host, dd = gu.workload(name)
        outs = []
        for _ in range(2):
            y, aux, counts = moe.layer_forward(dd["x"], dd["W_gate"], dd["logit_bias"], dd["W1"], dd["W3"], dd["W2"],
                                               k=w.k, capacity_factor=w.cf, act=w.act)
            torch.cuda.synchronize()
            outs.append((gu.from_dev(y).copy(), float(gu.from_dev(aux)), gu.from_dev(counts).copy()))
        assert np.array_equal(outs[0][0], outs[1][0]) and outs[0][1] == outs[1][1]
        assert np.array_equal(outs[0][2], outs[1][2])


@pytest.mark.parametrize("T,h,f,E,k,cf,act,dtype", [
    (1, 128, 256, 8, 2, 0.0, "swiglu", "bf16"),      # one token
    (33, 256, 192, 6, 3, 0.0, "gelu", "bf16"),       # ragged against the 64-token router blocks
    (65, 192, 320, 40, 3, 1.0, "swiglu", "bf16"),    # one full block + 1 token, h % 128 != 0, drops
    (300, 128, 128, 5, 5, 0.0, "swiglu", "bf16"),    # k = E: every expert, dense mixture
    (200, 192, 256, 4, 1, 0.3, "gelu", "bf16"),      # heavy drops, k = 1
    (130, 64, 64, 1, 1, 0.0, "swiglu", "f32"),       # a single expert: the plain FFN
    (500, 128, 256, 16, 2, 0.25, "swiglu", "f32"),   # drops in fp32
    (20, 1024, 2048, 8, 2, 0.0, "swiglu", "bf16"),   # few rows per expert: K-split GEMMs, parts added in combine
    (40, 2048, 1024, 6, 2, 0.5, "gelu", "bf16"),     # K-split GEMMs with drops
    (64, 128, 128, 256, 16, 0.0, "swiglu", "bf16"),  # the largest E and k the library takes
    (96, 64, 128, 256, 16, 1.0, "gelu", "f32"),      # ... in fp32, with drops
    (64, 256, 512, 8, 2, 0.5, "swiglu", "bf16"),     # one block of tokens (fused scan and scatter), drops
    (50, 128, 256, 16, 3, 0.4, "gelu", "bf16"),      # ... ragged, heavy drops
    (64, 128, 128, 64, 4, 0.7, "swiglu", "f32"),     # ... 64 experts, fp32
])
def test_layer_edge_cases(T, h, f, E, k, cf, act, dtype):
    import math
    _say(f"layer edge T={T} h={h} f={f} E={E} k={k} cf={cf} {act} {dtype}")
    rng = np.random.default_rng(T + E)
    conv = (lambda a: mw.f32_to_bf16_bits(a)) if dtype == "bf16" else (lambda a: a)
    host = dict(x=conv(rng.standard_normal((T, h)).astype(np.float32)),
                W_gate=(rng.standard_normal((h, E)) / math.sqrt(h)).astype(np.float32),
                logit_bias=rng.standard_normal(E).astype(np.float32),
                W1=conv((rng.standard_normal((E, h, f)) / math.sqrt(h)).astype(np.float32)),
                W3=conv((rng.standard_normal((E, h, f)) / math.sqrt(h)).astype(np.float32)) if act == "swiglu" else None,
                W2=conv((rng.standard_normal((E, f, h)) / math.sqrt(f)).astype(np.float32)))
    dd = {kk: gu.to_dev(v, dtype if kk in ("x", "W1", "W3", "W2") else "f32") for kk, v in host.items()}
    w = mw.Workload("edge", T=T, h=h, f=f, E=E, k=k, act=act, dtype=dtype, cf=cf)
    y, aux, counts, logits, routing = _run_layer(w, host, dd)
    ref = _check_layer(w, host, y, aux, counts, logits, np.arange(T), routing)
    if cf > 0:
        dropped = (ref["slot_pos"].reshape(T, k) < 0).all(1)
        if dropped.any():
            assert (gu.from_dev(y)[dropped] == 0).all()


@pytest.mark.parametrize("T,h,f,E,k,cf,act,dtype", [
    (1500, 256, 512, 8, 1, 0.0, "swiglu", "bf16"),   # 128-row tiles; the dominant expert takes 256-row tiles
    (2000, 192, 320, 16, 2, 0.0, "gelu", "bf16"),    # ... two big experts, the rest small
    (3000, 128, 256, 8, 1, 0.8, "swiglu", "bf16"),   # capacity 300 keeps every expert below the threshold
    (600, 2048, 256, 8, 2, 0.0, "gelu", "bf16"),     # h >= 2048: every expert past 128 rows takes 256-row tiles
])
def test_layer_skewed_experts(T, h, f, E, k, cf, act, dtype):
    """Launches of 128-row tiles in which some experts have 512 rows or more: those experts'
    m-tiles are 256 rows high (the tile list and the GEMMs agree on the height)."""
    import math
    _say(f"layer skewed T={T} h={h} f={f} E={E} k={k} cf={cf} {act} {dtype}")
    rng = np.random.default_rng(T + 7 * E)
    conv = (lambda a: mw.f32_to_bf16_bits(a)) if dtype == "bf16" else (lambda a: a)
    bias = np.zeros(E, np.float32)
    bias[0] = 3.0
    if E > 8:
        bias[5] = 2.5
    if h >= 2048:
        bias[1] = 1.5    # an expert between 129 and 511 rows as well
    host = dict(x=conv(rng.standard_normal((T, h)).astype(np.float32)),
                W_gate=(rng.standard_normal((h, E)) / math.sqrt(h)).astype(np.float32), logit_bias=bias,
                W1=conv((rng.standard_normal((E, h, f)) / math.sqrt(h)).astype(np.float32)),
                W3=conv((rng.standard_normal((E, h, f)) / math.sqrt(h)).astype(np.float32)) if act == "swiglu" else None,
                W2=conv((rng.standard_normal((E, f, h)) / math.sqrt(f)).astype(np.float32)))
    dd = {kk: gu.to_dev(v, dtype if kk in ("x", "W1", "W3", "W2") else "f32") for kk, v in host.items()}
    w = mw.Workload("skewed", T=T, h=h, f=f, E=E, k=k, act=act, dtype=dtype, cf=cf)
    y, aux, counts, logits, routing = _run_layer(w, host, dd)
    ref = _check_layer(w, host, y, aux, counts, logits, np.arange(T), routing)
    kept = np.diff(ref["offsets"])
    _say(f"  rows per expert: {kept.tolist()}")
    if cf <= 0:
        assert kept.max() >= 512       # the case this test is for


@pytest.mark.parametrize("T,E,k,cf", [
    (1025, 8, 2, 0.0),      # 64 blocks of 16 tokens + 1 token
    (2001, 5, 3, 0.6),      # five experts (four per lane group), ragged, drops
    (1100, 16, 16, 0.0),    # k = E = 16: every expert
    (1040, 16, 1, 1.0),     # k = 1, drops
    (4097, 8, 2, 1.25),     # 257 blocks of 16 tokens, 65 scatter blocks
])
def test_layer_selection_in_logits_kernel(T, E, k, cf):
    """bf16, at most 16 experts, h a multiple of 512 and many tokens: the logits kernel
    selects each 16-token group's experts itself and counts the histogram per 16 tokens,
    and the fused scan + scatter reads four histogram blocks per 64-token block.  Everything
    the layer decides is bit-exact against the oracle."""
    import math
    h, f = 512, 256
    _say(f"layer selection in the logits kernel E={E} T={T} k={k} cf={cf}")
    rng = np.random.default_rng(T + 5 * k)
    conv = mw.f32_to_bf16_bits
    host = dict(x=conv(rng.standard_normal((T, h)).astype(np.float32)),
                W_gate=(rng.standard_normal((h, E)) / math.sqrt(h)).astype(np.float32),
                logit_bias=(0.5 * rng.standard_normal(E)).astype(np.float32),
                W1=conv((rng.standard_normal((E, h, f)) / math.sqrt(h)).astype(np.float32)),
                W3=conv((rng.standard_normal((E, h, f)) / math.sqrt(h)).astype(np.float32)),
                W2=conv((rng.standard_normal((E, f, h)) / math.sqrt(f)).astype(np.float32)))
    dd = {kk: gu.to_dev(v, "bf16" if kk in ("x", "W1", "W3", "W2") else "f32") for kk, v in host.items()}
    w = mw.Workload("select-in-logits", T=T, h=h, f=f, E=E, k=k, act="swiglu", dtype="bf16", cf=cf)
    y, aux, counts, logits, routing = _run_layer(w, host, dd)
    tokens = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 300, replace=False)]))
    _check_layer(w, host, y, aux, counts, logits, tokens, routing)


@pytest.mark.parametrize("T,E,k,cf", [
    (1024, 64, 2, 1.25),    # the fused scan + scatter: 16 blocks
    (1500, 64, 4, 0.0),     # ... with a ragged last block (24 blocks, 28 tokens in the last)
    (8256, 64, 2, 1.0),     # 129 blocks: the largest fused scan at 64 experts (64 blocks per thread)
    (16448, 64, 1, 1.0),    # 257 blocks are too many for it: the separate scan and scatter kernels
    (8256, 256, 1, 2.0),    # ... and 129 blocks of 256 experts too
])
def test_layer_many_tokens_routing_paths(T, E, k, cf):
    """Many tokens, many experts: the fused scan + scatter up to the sizes whose histograms
    one workgroup reads, the separate scan and scatter kernels past them.  Everything the
    layer decides is bit-exact against the oracle, as for the other shapes."""
    import math
    h, f = 256, 256 if E == 64 else 128
    _say(f"layer E={E} T={T} k={k} cf={cf}")
    rng = np.random.default_rng(T + k)
    conv = mw.f32_to_bf16_bits
    host = dict(x=conv(rng.standard_normal((T, h)).astype(np.float32)),
                W_gate=(rng.standard_normal((h, E)) / math.sqrt(h)).astype(np.float32),
                logit_bias=(0.5 * rng.standard_normal(E)).astype(np.float32),
                W1=conv((rng.standard_normal((E, h, f)) / math.sqrt(h)).astype(np.float32)), W3=None,
                W2=conv((rng.standard_normal((E, f, h)) / math.sqrt(f)).astype(np.float32)))
    dd = {kk: gu.to_dev(v, "bf16" if kk in ("x", "W1", "W2") else "f32") for kk, v in host.items()
          if v is not None}
    dd["W3"] = None
    w = mw.Workload("many-tokens", T=T, h=h, f=f, E=E, k=k, act="gelu", dtype="bf16", cf=cf)
    y, aux, counts, logits, routing = _run_layer(w, host, dd)
    _check_layer(w, host, y, aux, counts, logits, np.sort(rng.choice(T, 300, replace=False)), routing)


def test_layer_forward_timed_matches_untimed():
    """The measurement entry point runs the same kernels: identical outputs, and the
    stage events are ordered and add up to the whole layer."""
    import bench
    torch = gu.torch()
    w, host, dd = gu.workload("tiny-fp32")
    args = (dd["x"], dd["W_gate"], dd["logit_bias"], dd["W1"], dd["W3"], dd["W2"])
    kw = dict(k=w.k, capacity_factor=w.cf, act=w.act)
    y0, aux0, c0 = moe.layer_forward(*args, **kw)
    hip = bench.Hip()
    ev = hip.events(len(moe.LAYER_STAGES) + 1)
    y1, aux1, c1 = moe.layer_forward(*args, **kw, events=ev)
    torch.cuda.synchronize()
    assert np.array_equal(gu.from_dev(y0), gu.from_dev(y1))
    assert float(gu.from_dev(aux0)) == float(gu.from_dev(aux1))
    assert np.array_equal(gu.from_dev(c0), gu.from_dev(c1))
    stages = [hip.elapsed_ms(ev[i], ev[i + 1]) for i in range(len(moe.LAYER_STAGES))]
    total = hip.elapsed_ms(ev[0], ev[len(moe.LAYER_STAGES)])
    hip.destroy(ev)
    assert all(s >= 0 for s in stages)
    assert abs(sum(stages) - total) <= 1e-3 * max(total, 1e-3) + 1e-3
    # null entries record nothing: two events around the up-projection only
    import ctypes
    pair = hip.events(2)
    j = moe.LAYER_STAGES.index("expert_up")
    part = (ctypes.c_void_p * (len(moe.LAYER_STAGES) + 1))()
    part[j], part[j + 1] = pair[0], pair[1]
    y2, aux2, c2 = moe.layer_forward(*args, **kw, events=part)
    torch.cuda.synchronize()
    assert np.array_equal(gu.from_dev(y0), gu.from_dev(y2))
    assert np.array_equal(gu.from_dev(c0), gu.from_dev(c2))
    assert hip.elapsed_ms(pair[0], pair[1]) > 0
    hip.destroy(pair)


@pytest.mark.parametrize("layout,backward", [("compact", False), ("binned", False), ("compact", True)])
def test_bench_json_contract(layout, backward):
    """bench.py on the small fp32 workload prints one JSON line with the fields the
    benchmark contract names."""
    import json
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--steps", "3", "--warmup", "1",
                        "--workload", "tiny-fp32", "--cpu-sample", "64", "--layout", layout,
                        "--min-capacity", "3"] + (["--backward"] if backward else []), capture_output=True, text=True,
                       timeout=300, cwd=root)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["value"] > 0
    assert d["config"]["workload"] == "tiny-fp32" and d["dtype"] == "f32" and d["config"]["layout"] == layout
    assert d["extra"]["gemm_rows"] >= d["extra"]["rows_kept"]
    rf = d["roofline"]
    assert rf["bound"] in ("hbm", "mfma", "alu") and rf["peak"] > 0 and rf["achieved"] > 0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    if backward:
        assert d["config"]["step"] == "forward + backward" and d["extra"]["backward_ms"] > 0
        assert set(d["extra"]["backward_stage_ms"]) == set(moe.BACKWARD_STAGES)
    else:
        assert d["extra"]["parity_vs_oracle"]["routing_differs"] <= 1  # a near-tie may route differently
