"""Seeded synthetic workloads for the MoE layer forward.

This module only *draws* inputs.  It holds none of the layer's arithmetic: no
routing, no permutation, no expert math.  Both the CPU oracle's tests and the
HIP path's tests/bench take their inputs from here, so that the two sides see
the same bytes.

Shapes and distributions
------------------------
Every workload is one MoE layer forward over ``T`` tokens of width ``h``, with
``E`` experts of inner width ``f`` and top-``k`` routing:

* ``x[T,h]``            ~ N(0, 1)
* ``W_gate[h,E]``       ~ N(0, 1/h)   (kept in fp32: the router runs in fp32)
* ``W1[E,h,f]``, ``W3[E,h,f]`` ~ N(0, 1/h)   (``W3`` only for SwiGLU experts)
* ``W2[E,f,h]``         ~ N(0, 1/f)
* ``logit_bias[E]``     per workload (see ``WORKLOADS``), fp32

``N(0, v)`` names the *variance* ``v``.  Values are drawn in fp32 and, for bf16
workloads, rounded to bf16 (round-to-nearest-even) and handed over as raw
``uint16`` bit patterns.  Each tensor -- and each expert's slice of a weight
tensor -- draws from its own PCG64 stream seeded by ``(seed, tensor id,
expert)``, so any slice can be regenerated alone and generation parallelises.

The Mixtral-shaped workloads stand in for the Mixtral-8x7B layer that the
pages measure (random weights of that architecture; trained weights are not
used).
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import os

import numpy as np

__all__ = ["Workload", "WORKLOADS", "by_name", "make_inputs", "f32_to_bf16_bits",
           "bf16_bits_to_f32", "uniform_assignment", "router_variant_inputs"]


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    h: int
    f: int
    E: int
    k: int
    act: str            # "gelu" or "swiglu"
    dtype: str          # "f32" or "bf16": dtype of x, W1/W3/W2 and y
    cf: float = 0.0     # capacity factor; <= 0 means dropless
    bias: str = "none"  # "none" | "normal:<variance>" | "zipf:<s>"
    seed: int = 0
    note: str = field(default="", compare=False)


WORKLOADS = (
    Workload("tiny-fp32", T=64, h=128, f=256, E=8, k=2, act="gelu", dtype="f32",
             note="tiny layer, fp32 throughout"),
    Workload("decode-mixtral", T=64, h=4096, f=14336, E=8, k=2, act="swiglu", dtype="bf16",
             note="decode-shaped Mixtral-8x7B layer, weight-streaming bound"),
    Workload("prefill-mixtral", T=4096, h=4096, f=14336, E=8, k=2, act="swiglu", dtype="bf16",
             bias="normal:0.5", note="prefill-shaped Mixtral-8x7B layer (batch 2 x seq 2048)"),
    Workload("capacity-e64", T=8192, h=1024, f=4096, E=64, k=2, act="gelu", dtype="bf16",
             cf=1.25, bias="zipf:1.1", note="Switch/GShard-style capacity factor, C=320"),
    Workload("finegrained-e256", T=4096, h=4096, f=2048, E=256, k=8, act="swiglu", dtype="bf16",
             bias="normal:1.0", note="fine-grained many-expert layer"),
)


def by_name(name: str) -> Workload:
    for w in WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)


# ----------------------------------------------------------------------------
# dtype helpers (plain casts, used to hand the drawn values to either side)

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern (uint16), round-to-nearest-even.  Finite input only."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# generators

_TENSOR_ID = {"x": 1, "W_gate": 2, "logit_bias": 3, "W1": 4, "W3": 5, "W2": 6, "jitter": 7, "noise": 8}


def _stream(seed: int, name: str, e: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _TENSOR_ID[name], e])))


def _normal(seed: int, name: str, e: int, shape, std: float) -> np.ndarray:
    a = _stream(seed, name, e).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def expert_slice(w: Workload, name: str, e: int) -> np.ndarray:
    """One expert's slice of W1/W3 ([h,f]) or W2 ([f,h]) in the workload's storage dtype."""
    if name in ("W1", "W3"):
        a = _normal(w.seed, name, e, (w.h, w.f), 1.0 / math.sqrt(w.h))
    elif name == "W2":
        a = _normal(w.seed, name, e, (w.f, w.h), 1.0 / math.sqrt(w.f))
    else:
        raise KeyError(name)
    return f32_to_bf16_bits(a) if w.dtype == "bf16" else a


def logit_bias(w: Workload) -> np.ndarray | None:
    kind, _, arg = w.bias.partition(":")
    if kind == "none":
        return None
    if kind == "normal":
        return _normal(w.seed, "logit_bias", 0, (w.E,), math.sqrt(float(arg)))
    if kind == "zipf":
        s = float(arg)
        pop = (np.arange(1, w.E + 1, dtype=np.float64)) ** (-s)
        pop /= pop.sum()
        return np.log(pop).astype(np.float32)
    raise ValueError(w.bias)


def make_inputs(w: Workload, with_weights: bool = True, experts=None) -> dict:
    """Draw one workload's tensors.

    Returns a dict of numpy arrays: ``x`` (fp32, or bf16 bits as uint16),
    ``W_gate`` (fp32 [h,E]), ``logit_bias`` (fp32 [E] or None) and, when
    ``with_weights``, ``W1``/``W3``/``W2`` ([E,h,f]/[E,h,f]/[E,f,h], bf16 bits or
    fp32; ``W3`` is None for GELU experts).  ``experts`` restricts weight
    generation to a subset (other slices are left zero) -- useful when only a
    few experts are needed.
    """
    out = {}
    x = _normal(w.seed, "x", 0, (w.T, w.h), 1.0)
    out["x"] = f32_to_bf16_bits(x) if w.dtype == "bf16" else x
    out["W_gate"] = _normal(w.seed, "W_gate", 0, (w.h, w.E), 1.0 / math.sqrt(w.h))
    out["logit_bias"] = logit_bias(w)
    if not with_weights:
        return out
    st = np.uint16 if w.dtype == "bf16" else np.float32
    names = ["W1", "W2"] + (["W3"] if w.act == "swiglu" else [])
    ex = range(w.E) if experts is None else sorted(set(int(e) for e in experts))
    for n in names:
        shape = (w.E, w.h, w.f) if n != "W2" else (w.E, w.f, w.h)
        out[n] = np.zeros(shape, dtype=st) if experts is not None else np.empty(shape, dtype=st)
    out.setdefault("W3", None)

    def fill(job):
        n, e = job
        out[n][e] = expert_slice(w, n, e)

    jobs = [(n, e) for n in names for e in ex]
    with ThreadPoolExecutor(_threads()) as pool:
        list(pool.map(fill, jobs))
    return out


def uniform_assignment(T: int, E: int, k: int) -> np.ndarray:
    """Benchmark-mode expert ids ``(t*k + j) % E`` as int32 [T,k] (every expert equally loaded
    when E divides T*k).  The MegaBlocks chapter describes this mode for its router."""
    return (np.arange(T * k, dtype=np.int64) % E).astype(np.int32).reshape(T, k)


def router_variant_inputs(w: Workload, eps: float = 0.01, noise_std: float | None = None, seed: int = 0) -> dict:
    """Random draws of the router variants, seeded like the other inputs:
    ``jitter`` [T,h] ~ U[1 - eps, 1 + eps] in the workload's dtype (bf16 bit patterns or
    fp32), and gate ``noise`` [T,E] fp32 ~ N(0, noise_std^2), noise_std = 1/E by default
    (noise scaled by the expert count)."""
    std = 1.0 / w.E if noise_std is None else noise_std
    u = _stream(seed, "jitter").uniform(1.0 - eps, 1.0 + eps, size=(w.T, w.h)).astype(np.float32)
    noise = _normal(seed, "noise", 0, (w.T, w.E), std)
    return dict(jitter=f32_to_bf16_bits(u) if w.dtype == "bf16" else u, noise=noise)
