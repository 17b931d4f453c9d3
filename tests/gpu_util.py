"""Helpers for the GPU parity tests: moving the seeded numpy inputs to the device,
caching full-size workloads, and the tolerances the parity checks use."""
from __future__ import annotations

import numpy as np

import moe_workloads as mw

_CACHE: dict = {}


def torch():
    import torch as _t
    return _t


def dev():
    t = torch()
    if not t.cuda.is_available():
        raise RuntimeError("GPU tests need a GPU")
    return t.device("cuda:0")


def to_dev(a, dtype: str):
    """numpy fp32 array or bf16 bit pattern array -> device tensor (None passes through)."""
    if a is None:
        return None
    t = torch()
    if dtype == "bf16" and a.dtype == np.uint16:
        return t.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(t.bfloat16).to(dev())
    return t.from_numpy(np.ascontiguousarray(a)).to(dev())


def from_dev(x) -> np.ndarray:
    t = torch()
    x = x.detach()
    if x.dtype == t.bfloat16:
        return x.view(t.int16).cpu().numpy().view(np.uint16)
    return x.cpu().numpy()


def as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16" and a.dtype == np.uint16:
        return mw.bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def workload(name: str):
    """(Workload, host inputs, device inputs), cached for the test session."""
    if name not in _CACHE:
        w = mw.by_name(name)
        host = mw.make_inputs(w)
        devd = {}
        for key in ("x", "W1", "W3", "W2"):
            devd[key] = to_dev(host[key], w.dtype)
        devd["W_gate"] = to_dev(host["W_gate"], "f32")
        devd["logit_bias"] = to_dev(host["logit_bias"], "f32")
        _CACHE.clear()  # keep at most one full-size workload resident
        _CACHE[name] = (w, host, devd)
        torch().cuda.synchronize()
    return _CACHE[name]


# ---------------------------------------------------------------- tolerances

def check_rel_rms(got, ref, rel: float, what: str):
    """|got - ref| <= rel * (|ref| + RMS(ref)) elementwise (relative error with an RMS floor)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    err = np.abs(got - ref)
    bound = rel * (np.abs(ref) + rms)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {ref.size} outside rel {rel}; worst "
                           f"|d|={float(err.max()):.3e} at {np.unravel_index(int(np.argmax(err - bound)), err.shape)}, "
                           f"rms={rms:.3e}")


def half_ulp_bf16(v):
    """Half the spacing of bf16 values at |v|: for |v| in [2^e, 2^(e+1)) the spacing is 2^(e-7)."""
    _, e = np.frexp(np.abs(np.asarray(v, dtype=np.float64)))  # |v| = m 2^e, m in [0.5, 1)
    return np.ldexp(1.0, e - 9)


def check_bf16_out(got, ref, what: str, frac: float = 2e-2):
    """bf16 output bar: |got - ref| <= frac * RMS(ref) + half a bf16 ulp of ref, elementwise.

    ``ref`` is the exact (fp64) result.  The half-ulp term is the rounding of the
    output into bf16 itself, which no bf16-storing implementation avoids; the
    frac * RMS term bounds everything else.  Returns (max|d|/RMS, max(|d| - half_ulp)/RMS).
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    d = np.abs(got - ref)
    hu = half_ulp_bf16(ref)
    bad = d > frac * rms + hu
    raw = float(d.max()) / rms if rms else 0.0
    beyond = float(np.maximum(d - hu, 0).max()) / rms if rms else 0.0
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements beyond {frac}*RMS + half-ulp; "
                           f"max|d|/RMS {raw:.4f}, beyond-rounding {beyond:.4f}")
    return raw, beyond


# ---------------------------------------------------------------- sentinels

SENTINEL = {"bf16": 0x5A5A, "f32": 0x5A5A5A5A}   # finite bit patterns no kernel writes by chance


def sentinel_like(shape, dtype: str):
    """A device tensor of ``shape`` filled with the sentinel bit pattern of ``dtype``."""
    t = torch()
    if dtype == "bf16":
        return t.full(shape, SENTINEL["bf16"], dtype=t.int16, device=dev()).view(t.bfloat16)
    return t.full(shape, SENTINEL["f32"], dtype=t.int32, device=dev()).view(t.float32)


def is_sentinel(a: np.ndarray, dtype: str) -> np.ndarray:
    """Elementwise: does the host copy (bf16 bits or fp32 values) still hold the sentinel?"""
    if dtype == "bf16":
        return np.asarray(a).view(np.uint16) == SENTINEL["bf16"]
    return np.asarray(a, dtype=np.float32).view(np.uint32) == SENTINEL["f32"]
