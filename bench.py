"""Benchmark: one MoE layer forward per step on one MI355X.

A step is one call of the whole hot path (router -> histogram -> scan ->
stable scatter -> expert up-projection -> expert down-projection -> combine)
over the Mixtral-shaped prefill batch (T = 4096 tokens, h = 4096, f = 14336,
E = 8, k = 2, SwiGLU, bf16, fp32 router), inputs resident in HBM.  Prints one
JSON line with tokens/s, a roofline entry for the dominant kernel (the
SwiGLU up-projection GEMM, timed with HIP events recorded around it on the
library's stream inside the timed loop), and the CPU oracle timed on a
bounded sample of the same workload.  The per-stage times under ``extra``
come from a separate instrumented pass with an event between every two
stages (each record idles the GPU for a few microseconds); the timed loop
records only the two events around the dominant kernel.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload prefill-mixtral]
                    [--layout compact|binned] [--capacity-factor CF] [--min-capacity N]

``--layout binned`` times the fixed-capacity variant instead: every expert gets a
bucket of C rows (zero padding past its count), the expert GEMMs run over all E*C
bucket rows, so the padding cost shows against the compact layout.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s at Mixtral shape (T=4096); % bf16 MFMA peak; route GB/s"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 vector
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Hip:
    """Minimal HIP event API through ctypes (events on the library's stream).  The events
    are only read for elapsed times after a device-wide synchronisation, so they are
    created without the system-scope fence that a record otherwise performs (a cache
    write-back and invalidate that slows the kernels around it: about 2 us per record
    between the small kernels of the decode layer)."""

    DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence

    def __init__(self):
        self.l = ctypes.CDLL("libamdhip64.so")
        self.l.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.l.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.l.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def events(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            if self.l.hipEventCreateWithFlags(ctypes.byref(ev), self.DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            arr[i] = ev
        return arr

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        if self.l.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def destroy(self, arr):
        for ev in arr:
            self.l.hipEventDestroy(ev)


# the sources the expert GEMM kernels (the dominant forward kernel) are compiled from
GEMM_SOURCES = ("common.h", "gemm.hip", "kernels.h")
# the oracle's timed sample is repeated until it has run this long (or this many passes)
CPU_MIN_SECONDS, CPU_MAX_PASSES = 10.0, 5
# the backward stages that are grouped GEMMs (candidates for the dominant backward kernel)
BWD_GEMMS = ("recompute_up", "down_dgrad", "down_wgrad", "up_dgrad", "up_wgrad")


def kernel_source_hash() -> str:
    """sha256 prefix over the expert GEMM's sources: counters taken on other sources are stale."""
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(ROOT, "top_routing_expert_moe_amd", "csrc", name), "rb") as fh:
            h.update(name.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_entry(workload: str):
    """HBM bytes per launch of the dominant kernel from committed rocprofv3 counters, if they
    were taken on the current kernel sources."""
    try:
        with open(TRAFFIC_JSON) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    e = t.get(workload)
    if not e or e.get("source_hash") != kernel_source_hash():
        return None
    return e.get("bytes_per_launch")


# the other configurations whose fractions the default run also records (timed in the same
# process after the headline workload)
OTHER_WORKLOADS = ("decode-mixtral", "capacity-e64", "finegrained-e256")


def measure_other(name: str, steps: int, warmup: int) -> dict:
    """One more workload's layer forward, timed like the headline: an instrumented pass for the
    stage times, then `steps` calls with events only around the up projection.  Returns the
    figures the roofline needs (ms per layer, the layer's roofline fraction, the up and down
    projections' HBM or MFMA fractions)."""
    import numpy as np
    import torch

    import moe_workloads as mw
    import top_routing_expert_moe_amd as moe

    dev = torch.device("cuda:0")
    w = mw.by_name(name)
    t = time.time()
    host = mw.make_inputs(w)
    bf = w.dtype == "bf16"

    def to_dev(a, low):
        if a is None:
            return None
        if low and bf:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    d = {k: to_dev(v, k in ("x", "W1", "W3", "W2")) for k, v in host.items()}
    del host
    torch.cuda.synchronize()
    log(f"[bench] {name}: inputs drawn and resident in {time.time() - t:.1f}s")
    T, h, f, E, k = w.T, w.h, w.f, w.E, w.k
    act = moe.SWIGLU if w.act == "swiglu" else moe.GELU
    dt = moe.BF16 if bf else moe.F32
    y = torch.empty((T, h), dtype=d["x"].dtype, device=dev)
    aux = torch.empty((), dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    ws = torch.empty(moe.workspace_bytes(T, h, f, E, k, w.cf, dt, act), dtype=torch.uint8, device=dev)

    def step(events=None):
        moe.layer_forward(d["x"], d["W_gate"], d["logit_bias"], d["W1"], d["W3"], d["W2"], k=k,
                          capacity_factor=w.cf, act=w.act, ws=ws, y=y, aux=aux, counts=counts, events=events)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    hip = Hip()
    stages = moe.LAYER_STAGES
    nst = len(stages)
    n_inst = max(1, min(steps, 10))
    ev = [hip.events(nst + 1) for _ in range(n_inst)]
    for i in range(n_inst):
        step(ev[i])
    torch.cuda.synchronize()
    stage_ms = {s: sum(hip.elapsed_ms(ev[i][j], ev[i][j + 1]) for i in range(n_inst)) / n_inst
                for j, s in enumerate(stages)}
    for e_ in ev:
        hip.destroy(e_)
    jd = stages.index("expert_up")
    # events before the router and around the up projection (the one before it closes the
    # routing + permutation region, which so carries no event gaps inside)
    live = [hip.events(3) for _ in range(steps)]
    arrs = []
    for i in range(steps):
        a_ = (ctypes.c_void_p * (nst + 1))()
        a_[0] = live[i][2]
        a_[jd], a_[jd + 1] = live[i][0], live[i][1]
        arrs.append(a_)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(arrs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    up_ms = sum(hip.elapsed_ms(live[i][0], live[i][1]) for i in range(steps)) / steps
    route_ms = sum(hip.elapsed_ms(live[i][2], live[i][0]) for i in range(steps)) / steps
    for e_ in live:
        hip.destroy(e_)
    cnt = counts.cpu().numpy().astype(np.int64)
    C = moe.capacity(T, E, k, w.cf)
    kept = cnt if C is None else np.minimum(cnt, C)
    R = int(kept.sum())
    active = int((kept > 0).sum())
    es = 2 if bf else 4
    n_up = 2 if w.act == "swiglu" else 1
    ms = wall / steps * 1e3
    flops_up, flops_down = 2.0 * n_up * R * h * f, 2.0 * R * f * h
    bytes_up = active * n_up * h * f * es + R * h * es + R * f * es
    bytes_down = active * f * h * es + R * f * es + R * h * 4
    layer_bytes = T * h * es + h * E * 4 + active * (n_up + 1) * h * f * es + T * h * es + T * k * 12
    t_roof = max((flops_up + flops_down) / (PEAK_BF16_TFLOPS * 1e12), layer_bytes / (PEAK_HBM_GBS * 1e9))
    route_bytes = T * h * es + h * E * 4 + T * E * 4 + T * k * 16
    down_s = stage_ms["expert_down"] / 1e3
    out = {"ms_per_layer": round(ms, 5), "tokens_per_s": round(T / (ms / 1e3), 1),
           "layer_roofline_frac": round(t_roof / (ms / 1e3), 4),
           "layer_bound": "mfma" if (flops_up + flops_down) / PEAK_BF16_TFLOPS / 1e12 >= layer_bytes / PEAK_HBM_GBS / 1e9
           else "hbm",
           "up_ms": round(up_ms, 5), "up_hbm_frac": round(bytes_up / (up_ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
           "up_mfma_frac": round(flops_up / (up_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "down_ms": round(stage_ms["expert_down"], 5),
           "down_hbm_frac": round(bytes_down / down_s / 1e9 / PEAK_HBM_GBS, 4),
           "down_mfma_frac": round(flops_down / down_s / 1e12 / PEAK_BF16_TFLOPS, 4),
           "route_permute_ms": round(route_ms, 5), "route_gbps": round(route_bytes / (route_ms / 1e3) / 1e9, 1),
           "combine_ms": round(stage_ms["combine"], 5), "rows_kept": R, "active_experts": active,
           "steps": steps, "stage_ms": {s_: round(v, 5) for s_, v in stage_ms.items()}}
    del d, ws, y
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill-mixtral")
    ap.add_argument("--cpu-sample", type=int, default=4096,
                    help="tokens in the oracle's timed sample (capped at the workload's T)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layout", choices=("compact", "binned"), default="compact")
    ap.add_argument("--capacity-factor", type=float, default=None, help="override the workload's factor")
    ap.add_argument("--min-capacity", type=int, default=0, help="binned layout: the smallest bucket size")
    ap.add_argument("--backward", action="store_true",
                    help="time a training step: the training forward (which saves the up projection's "
                         "pre-activations), then the backward pass (dy ~ N(0,1), aux weight 0.01), with per-stage "
                         "times of both")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the other configurations (decode-mixtral, capacity-e64, finegrained-e256) that the "
                         "default prefill run also times, in the same process, for extra.others")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before warm-up, run a plain elementwise copy (y = x + 1, fp32) over this many MiB three "
                         "times: a kernel of known traffic for calibrating rocprofv3's FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}); the layer's sharding plan is design-only.", flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import moe_workloads as mw
    import top_routing_expert_moe_amd as moe

    w = mw.by_name(args.workload)
    if args.capacity_factor is not None:
        import dataclasses
        w = dataclasses.replace(w, cf=args.capacity_factor)
    binned = args.layout == "binned"
    if args.backward and binned:
        print("bench.py: the backward pass is built for the compact layout only", flush=True)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    moe.lib()  # fail loudly if the HIP library is missing

    t = time.time()
    host = mw.make_inputs(w)
    bf = w.dtype == "bf16"

    def to_dev(a, low):
        if a is None:
            return None
        if low and bf:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    d = {k: to_dev(v, k in ("x", "W1", "W3", "W2")) for k, v in host.items()}
    torch.cuda.synchronize()
    log(f"[bench] {w.name}: inputs drawn and resident in {time.time() - t:.1f}s")

    T, h, f, E, k = w.T, w.h, w.f, w.E, w.k
    act = moe.SWIGLU if w.act == "swiglu" else moe.GELU
    dt = moe.BF16 if bf else moe.F32
    y = torch.empty((T, h), dtype=d["x"].dtype, device=dev)
    aux = torch.empty((), dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    if binned:
        mc = args.min_capacity
        ws = torch.empty(moe.binned_workspace_bytes(T, h, f, E, k, w.cf, mc, dt, act), dtype=torch.uint8,
                         device=dev)
        cap = torch.empty((), dtype=torch.int32, device=dev)
        x_bins = torch.empty((E * moe.binned_capacity_max(T, E, k, w.cf, mc), h), dtype=d["x"].dtype, device=dev)
        stages = moe.BINNED_STAGES

        def step(events=None):
            moe.layer_forward_binned(d["x"], d["W_gate"], d["logit_bias"], d["W1"], d["W3"], d["W2"], k=k,
                                     capacity_factor=w.cf, min_capacity=mc, act=w.act, ws=ws, y=y, aux=aux,
                                     counts=counts, capacity=cap, x_bins=x_bins, events=events)
    else:
        ws = torch.empty(moe.workspace_bytes(T, h, f, E, k, w.cf, dt, act), dtype=torch.uint8, device=dev)
        stages = moe.LAYER_STAGES

        def step(events=None):
            moe.layer_forward(d["x"], d["W_gate"], d["logit_bias"], d["W1"], d["W3"], d["W2"], k=k,
                              capacity_factor=w.cf, act=w.act, ws=ws, y=y, aux=aux, counts=counts, events=events)
    if args.backward:
        g = torch.Generator(device="cpu").manual_seed(1)
        dy = torch.randn((T, h), generator=g, dtype=torch.float32).to(d["x"].dtype).to(dev)
        bws = torch.empty(moe.lib().moe_layer_backward_workspace_bytes(T, h, f, E, k, w.cf, dt, act), dtype=torch.uint8,
                          device=dev)
        grads = {}
        nf = len(moe.LAYER_STAGES)
        stages = tuple(moe.LAYER_STAGES) + ("forward_to_backward",) + tuple("bwd_" + s for s in moe.BACKWARD_STAGES)
        # the training forward saves the up projection's pre-activations for the backward
        pre = torch.empty(moe.preact_bytes(T, h, f, E, k, w.cf, w.act), dtype=torch.uint8, device=dev)

        def step(events=None):
            evf = evb = None
            if events is not None:
                evf = (ctypes.c_void_p * (nf + 1))(*events[:nf + 1])
                evb = (ctypes.c_void_p * (len(moe.BACKWARD_STAGES) + 1))(*events[nf + 1:])
            moe.layer_forward(d["x"], d["W_gate"], d["logit_bias"], d["W1"], d["W3"], d["W2"], k=k,
                              capacity_factor=w.cf, act=w.act, ws=ws, y=y, aux=aux, counts=counts, events=evf,
                              preact=pre)
            out = moe.layer_backward(d["x"], d["W_gate"], d["W1"], d["W3"], d["W2"], dy, k=k, capacity_factor=w.cf,
                                     act=w.act, fwd_ws=ws, d_aux=0.01, ws=bws, out=grads or None, events=evb,
                                     preact=pre)
            grads.update(out)

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.zeros(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.add(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
        log(f"[bench] copy probe: 3 x {args.copy_probe_mib} MiB read + {args.copy_probe_mib} MiB written")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    hip = Hip()
    nst = len(stages)
    # Per-stage breakdown: an instrumented pass with an event between every two stages.  Each
    # event record leaves the GPU idle for a few microseconds between the kernels around it,
    # so this pass is reported but not the timed one.
    n_inst = max(1, min(args.steps, 20))
    ev = [hip.events(nst + 1) for _ in range(n_inst)]
    torch.cuda.synchronize()
    for i in range(n_inst):
        step(ev[i])
    torch.cuda.synchronize()
    stage_ms = {s: 0.0 for s in stages}
    step_ms = []  # per instrumented step, from the first to the last event
    for i in range(n_inst):
        for j, s in enumerate(stages):
            stage_ms[s] += hip.elapsed_ms(ev[i][j], ev[i][j + 1]) / n_inst
        step_ms.append(hip.elapsed_ms(ev[i][0], ev[i][nst]))
    for e_ in ev:
        hip.destroy(e_)

    # The timed steps: events only around the dominant kernel (the up-projection GEMM of the
    # forward; in a training step the slowest backward GEMM of the instrumented pass), null
    # entries everywhere else, so the whole-step wall time carries two event records.
    if args.backward:
        dom_stage = "bwd_" + max(BWD_GEMMS, key=lambda s_: stage_ms["bwd_" + s_])
    else:
        dom_stage = "expert_up"
    jd = stages.index(dom_stage)
    # one more pair of events brackets routing + permutation (before the router, after the
    # scatter), with no event inside it; where the scatter's end is the dominant kernel's
    # start the same event serves both
    ir = stages.index("scatter") + 1
    live = [hip.events(4) for _ in range(args.steps)]
    arrs = []
    for i in range(args.steps):
        a_ = (ctypes.c_void_p * (nst + 1))()
        a_[jd], a_[jd + 1] = live[i][0], live[i][1]
        a_[0] = live[i][2]
        if ir != jd:
            a_[ir] = live[i][3]
        arrs.append(a_)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(arrs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    dom_ms = sum(hip.elapsed_ms(live[i][0], live[i][1]) for i in range(args.steps)) / args.steps
    route_ms = sum(hip.elapsed_ms(live[i][2], live[i][0] if ir == jd else live[i][3])
                   for i in range(args.steps)) / args.steps
    for e_ in live:
        hip.destroy(e_)
    log("[bench] stage ms: " + ", ".join(f"{s}={v:.4f}" for s, v in stage_ms.items()))

    cnt = counts.cpu().numpy().astype(np.int64)
    if binned:
        C = int(cap.cpu())
        kept = np.minimum(cnt, C)
        R = E * C  # the GEMMs run over every bucket row, padding included
    else:
        C = moe.capacity(T, E, k, w.cf)
        kept = cnt if C is None else np.minimum(cnt, C)
        R = int(kept.sum())
    n_up = 2 if w.act == "swiglu" else 1
    flops_up = 2.0 * n_up * R * h * f
    flops_down = 2.0 * R * f * h
    flops_router = 2.0 * T * h * E
    up_s = (dom_ms if dom_stage == "expert_up" else stage_ms["expert_up"]) / 1e3
    ms_per_step = wall / args.steps * 1e3
    es = 2 if bf else 4
    active = E if binned else int((kept > 0).sum())
    # algorithmic bytes of the up-projection: each active expert's W1 (and W3) once, the R
    # gathered activation rows read, the R hidden rows written
    bytes_up = active * n_up * h * f * es + R * h * es + R * f * es
    bytes_down = active * f * h * es + R * f * es + R * h * 4
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    # the library's tile choice: 32-row tiles when the planned rows per expert are <= 48
    # (T*k/E, at most C; the bucket size in the binned layout with a positive factor); with
    # SwiGLU those write the raw a and g (512-column tiles of W1 or W3 alone) and a second
    # pass applies the activation
    rpe = T * k / E
    if binned and w.cf > 0:
        rpe = float(moe.binned_capacity_max(T, E, k, w.cf, args.min_capacity))
    elif not binned and moe.capacity(T, E, k, w.cf) is not None:
        rpe = min(rpe, float(moe.capacity(T, E, k, w.cf)))
    if bf and w.act == "swiglu" and rpe <= 48:
        kname = "expert up-projection (grouped bf16 MFMA GEMM writing raw a and g, then the SwiGLU pass, "
    else:
        kname = ("expert up-projection (grouped bf16 MFMA GEMM, SwiGLU epilogue, " if w.act == "swiglu"
                 else "expert up-projection (grouped bf16 MFMA GEMM, GELU epilogue, ")
    kname += "over the E x C buckets)" if binned else "gather fused)"
    if not bf:  # the fp32 GEMM runs on the vector ALUs
        achieved = flops_up / up_s / 1e12
        roofline = {"bound": "alu", "achieved": round(achieved, 3), "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / PEAK_FP32_TFLOPS, 5)}
    elif flops_up / bytes_up >= ridge:
        achieved = flops_up / up_s / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    else:
        achieved = bytes_up / up_s / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roofline.update({"traffic": None if binned else traffic_entry(w.name), "kernel": kname,
                     "flops_per_launch": flops_up,
                     "algorithmic_bytes_per_launch": bytes_up, "avg_launch_ms": round(up_s * 1e3, 5)})
    # compulsory bytes of routing + permutation metadata: x and W_gate read once, logits written,
    # topk idx/w, slot_pos and the sorted order (4 B each per assignment)
    route_bytes = T * h * es + h * E * 4 + T * E * 4 + T * k * 16
    route_stage_ms = sum(stage_ms[s] for s in ("logits", "select", "scan", "scatter"))
    # the layer's own roof: compulsory bytes (x, W_gate, active weights, y, routing metadata) against
    # its MFMA work
    layer_bytes = T * h * es + h * E * 4 + active * (n_up + 1) * h * f * es + T * h * es + T * k * 12
    # (on the kept rows only: bucket padding is work the layer's own roof does not count)
    flops_kept = 2.0 * (n_up + 1) * int(kept.sum()) * h * f
    t_roof = max(flops_kept / (PEAK_BF16_TFLOPS * 1e12), layer_bytes / (PEAK_HBM_GBS * 1e9))
    # combine: one fp32 expert-output row per kept assignment and the routing weights read,
    # y written (a lower bound: a K-split down projection leaves two or four parts to add)
    combine_bytes = int(kept.sum()) * h * 4 + T * h * es + T * k * 8
    q = np.percentile(np.array(step_ms), [10, 50, 90])
    extra = {
        "instrumented_steps": n_inst,
        "layer_ms_p10_p50_p90": [round(float(v), 5) for v in q],
        "combine_gbps_min": round(combine_bytes / (stage_ms["combine"] / 1e3) / 1e9, 1),
        "stage_ms": {s: round(v, 5) for s, v in stage_ms.items()},
        "rows_kept": int(kept.sum()), "gemm_rows": R, "active_experts": active,
        "layer_mfma_frac": round(flops_kept / (ms_per_step / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "layer_roofline_frac": round(t_roof / (ms_per_step / 1e3), 4),
        "expert_down_frac": round(flops_down / (stage_ms["expert_down"] / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "expert_up_hbm_gbs": round(bytes_up / up_s / 1e9, 1),
        "expert_down_hbm_gbs": round(bytes_down / (stage_ms["expert_down"] / 1e3) / 1e9, 1),
        "route_permute_ms": round(route_ms, 5),
        "route_gbps": round(route_bytes / (route_ms / 1e3) / 1e9, 1),
        "route_stage_sum_ms": round(route_stage_ms, 5),
        "router_flops": flops_router,
        "aux_loss": float(aux.cpu()),
    }

    if args.backward:
        # the backward GEMMs: FLOPs and algorithmic bytes (operands read once, outputs written once;
        # the weight gradients are fp32)
        bw = {s_: stage_ms["bwd_" + s_] for s_ in moe.BACKWARD_STAGES}
        Rk = int(kept.sum())
        # (the pre-activations are saved by the training forward: no recompute)
        fl = {"recompute_up": 0.0, "down_dgrad": 2.0 * Rk * h * f, "down_wgrad": 2.0 * Rk * f * h,
              "up_dgrad": 2.0 * n_up * Rk * f * h, "up_wgrad": 2.0 * n_up * Rk * h * f}
        by = {"recompute_up": 0,
              "down_dgrad": active * f * h * es + Rk * h * es + Rk * n_up * f * 4 + Rk * n_up * f * es,
              "down_wgrad": Rk * f * es + Rk * h * es + active * f * h * 4,
              "up_dgrad": active * n_up * h * f * es + Rk * n_up * f * es + Rk * h * 4,
              "up_wgrad": Rk * h * es + Rk * n_up * f * es + active * n_up * h * f * 4}
        dom = dom_stage[len("bwd_"):]
        assert set(fl) == set(BWD_GEMMS)
        t_dom = dom_ms / 1e3
        if not bf:
            ach = fl[dom] / t_dom / 1e12
            roofline = {"bound": "alu", "achieved": round(ach, 3), "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(ach / PEAK_FP32_TFLOPS, 5)}
        elif fl[dom] / by[dom] >= ridge:
            ach = fl[dom] / t_dom / 1e12
            roofline = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(ach / PEAK_BF16_TFLOPS, 4)}
        else:
            ach = by[dom] / t_dom / 1e9
            roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(ach / PEAK_HBM_GBS, 4)}
        roofline.update({"traffic": None, "kernel": f"backward {dom} (grouped GEMM)", "flops_per_launch": fl[dom],
                         "algorithmic_bytes_per_launch": by[dom], "avg_launch_ms": round(dom_ms, 5)})
        bwd_ms = sum(bw.values())
        extra["backward_stage_ms"] = {s_: round(v, 5) for s_, v in bw.items()}
        extra["backward_ms"] = round(bwd_ms, 5)
        extra["backward_gemm_tflops"] = round(sum(fl.values()) / (sum(bw[s_] for s_ in fl) / 1e3) / 1e12, 2)
        extra["train_step_mfma_frac"] = round((flops_up + flops_down + sum(fl.values())) / (ms_per_step / 1e3) / 1e12
                                              / PEAK_BF16_TFLOPS, 4)

    cpu = None
    if not args.no_cpu_baseline and args.backward:
        import oracle as o
        try:
            import threadpoolctl
            threads = max(p_["num_threads"] for p_ in threadpoolctl.threadpool_info()) or 1
        except Exception:  # pragma: no cover
            threads = os.cpu_count() or 1
        ns = min(args.cpu_sample, T)
        tokens = np.arange(ns) * (T // ns)
        dyh = dy.cpu()
        dyh = dyh.view(torch.int16).numpy().view(np.uint16) if bf else dyh.numpy()
        reps, el = 0, 0.0
        while reps < CPU_MAX_PASSES and el < CPU_MIN_SECONDS:
            tc = time.perf_counter()
            o.layer_backward(host["x"], host["W_gate"], host["logit_bias"], host["W1"], host["W3"], host["W2"], dyh,
                             0.01, k=k, capacity_factor=w.cf, act=w.act, dtype=w.dtype, tokens=tokens, experts=[],
                             with_w_gate=False)
            el += time.perf_counter() - tc
            reps += 1
        cpu = {"value": round(ns * reps / el, 3), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
               "sample": f"backward: full routing of all {T} tokens + dx of {ns} evenly spaced tokens through their "
                         f"experts, no weight gradients; {reps} pass(es), fp64 numpy, {el:.1f} s"}
    elif not args.no_cpu_baseline:
        import oracle as o
        try:
            import threadpoolctl
            threads = max(p["num_threads"] for p in threadpoolctl.threadpool_info()) or 1
        except Exception:  # pragma: no cover
            threads = os.cpu_count() or 1
        ns = min(args.cpu_sample, T)
        tokens = np.arange(ns) * (T // ns)
        reps, el = 0, 0.0
        while reps < CPU_MAX_PASSES and el < CPU_MIN_SECONDS:
            tc = time.perf_counter()
            if binned:
                ref = o.layer_forward_binned(host["x"], host["W_gate"], host["logit_bias"], host["W1"], host["W3"],
                                             host["W2"], k=k, capacity_factor=w.cf, min_capacity=args.min_capacity,
                                             act=w.act, dtype=w.dtype, tokens=tokens)
            else:
                ref = o.layer_forward(host["x"], host["W_gate"], host["logit_bias"], host["W1"], host["W3"],
                                      host["W2"], k=k, capacity_factor=w.cf, act=w.act, dtype=w.dtype, tokens=tokens)
            el += time.perf_counter() - tc
            reps += 1
        cpu = {"value": round(ns * reps / el, 3), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
               "sample": f"full routing of all {T} tokens + expert outputs of {ns} evenly spaced tokens; {reps} "
                         f"pass(es), fp64 numpy, {el:.1f} s"}
        # the bench's own output against the same oracle run, on tokens routed identically
        _, gidx, _, _ = moe.route(d["x"], d["W_gate"], d["logit_bias"], k)
        same = (np.sort(gidx.cpu().numpy()[tokens], 1) == np.sort(ref["topk_idx"][tokens], 1)).all(1)
        gy = y.cpu()
        gy = (gy.view(torch.int16).numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32) \
            if bf else gy.numpy()
        got = gy[tokens][same].astype(np.float64)
        ry = ref["y64"][same]
        rms = float(np.sqrt(np.mean(ry ** 2)))
        extra["parity_vs_oracle"] = {"tokens": int(same.sum()), "routing_differs": int((~same).sum()),
                                     "max_abs_over_rms": round(float(np.abs(got - ry).max()) / rms, 5),
                                     "aux_rel_err": abs(extra["aux_loss"] - ref["aux"]) / abs(ref["aux"])}

    if not args.no_others and not args.backward and not binned and args.capacity_factor is None and \
            w.name == "prefill-mixtral":
        del d, ws
        torch.cuda.empty_cache()
        others = {}
        for name in OTHER_WORKLOADS:
            others[name] = measure_other(name, steps=max(args.steps, 20) if name == "decode-mixtral" else
                                         max(args.steps // 2, 10), warmup=3)
            log(f"[bench] {name}: {json.dumps(others[name])}")
        extra["others"] = others

    out = {
        "metric": METRIC if not args.backward else "MoE layer training step (forward + backward) tokens/s",
        "value": round(T * args.steps / wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf else "f32",
        "data": "synthetic (seeded N(0,1) activations, N(0,1/fan_in) random weights of the layer's shape)",
        "config": {"workload": w.name, "T": T, "h": h, "f": f, "E": E, "k": k, "act": w.act,
                   "capacity_factor": w.cf, "router": "fp32", "logit_bias": w.bias, "layout": args.layout,
                   "step": "forward + backward" if args.backward else "forward"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
