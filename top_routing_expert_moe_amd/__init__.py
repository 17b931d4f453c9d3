"""MI355X (gfx950) MoE layer forward: a thin ctypes binding over ``libmoe_mi355x.so``.

Only argument marshalling happens here: every step of the layer runs in the
library's HIP kernels.  PyTorch supplies device memory (tensors are passed by
``data_ptr()``) and the stream (``torch.cuda.current_stream()``).  There is no
fallback: if the library is missing or no GPU is present, calls raise.

Entry points mirror the C ABI in ``include/moe.h``: ``route``, ``permute``,
``expert_ffn``, ``unpermute``, ``layer_forward`` plus ``capacity`` and
``workspace_bytes``.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

__all__ = ["MoEError", "lib", "lib_path", "capacity", "workspace_bytes", "status_string", "route",
           "permute", "expert_ffn", "unpermute", "layer_forward", "LAYER_STAGES", "F32", "BF16", "GELU", "SWIGLU",
           "ROUTE_LOGITS_IN", "layer_backward", "layer_forward_binned", "preact_bytes", "BACKWARD_STAGES",
           "BINNED_STAGES", "binned_capacity_max", "binned_workspace_bytes", "CapacityConfig", "RouterOpts",
           "layer_routing", "LayerRouting"]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libmoe_mi355x.so")

F32, BF16 = 0, 1
GELU, SWIGLU = 0, 1
ROUTE_LOGITS_IN = 1
_ACT = {"gelu": GELU, "swiglu": SWIGLU}

_c_void_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_f32 = ctypes.c_float
_sz = ctypes.c_size_t

class RouterOpts(ctypes.Structure):
    """moe_router_opts_t: router-input jitter, gate noise, softmax temperature, uniform
    expert assignment, soft top-K weights (device pointers as integers, or None)."""
    _fields_ = [("jitter", ctypes.c_void_p), ("logit_noise", ctypes.c_void_p), ("temperature", ctypes.c_float),
                ("uniform_assignment", ctypes.c_int32), ("soft_topk", ctypes.c_int32)]


_opts_p = ctypes.POINTER(RouterOpts)


class LayerRouting(ctypes.Structure):
    """moe_layer_routing_t: device pointers into a layer call's workspace."""
    _fields_ = [(n, ctypes.c_void_p) for n in ("logits", "topk_idx", "topk_w", "counts", "offsets", "slot_pos",
                                              "sorted_slot")]

_SIGS = {
    "moe_capacity": (_i32, [_i32, _i32, _i32, _f32]),
    "moe_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _f32, ctypes.c_int, ctypes.c_int]),
    "moe_expert_ffn_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, ctypes.c_int, ctypes.c_int]),
    "moe_route_workspace_bytes": (_sz, [_i32, _i32, _i32, ctypes.c_int, ctypes.c_uint32, _i32]),
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_route": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _i32, _i32, _i32, _i32, ctypes.c_int,
                                 ctypes.c_uint32, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _sz,
                                 _c_void_p]),
    "moe_permute_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "moe_permute": (ctypes.c_int, [_c_void_p, _c_void_p, _i32, _i32, _i32, _i32, _f32, ctypes.c_int,
                                   _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                   _c_void_p, _c_void_p, _sz, _c_void_p]),
    "moe_expert_ffn": (ctypes.c_int, [_c_void_p, _c_void_p, _i32, _i32, _i32, _i32, _c_void_p, _c_void_p,
                                      _c_void_p, ctypes.c_int, ctypes.c_int, _c_void_p, _c_void_p, _sz,
                                      _c_void_p]),
    "moe_unpermute": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _i32, _i32, _i32, ctypes.c_int,
                                     _c_void_p, _c_void_p]),
    "moe_layer_forward": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                         _i32, _i32, _i32, _i32, _i32, _f32, ctypes.c_int, ctypes.c_int,
                                         _c_void_p, _c_void_p, _c_void_p, _c_void_p, _sz, _c_void_p]),
    "moe_layer_forward_timed": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                               _i32, _i32, _i32, _i32, _i32, _f32, ctypes.c_int, ctypes.c_int,
                                               _c_void_p, _c_void_p, _c_void_p, _c_void_p, _sz, _c_void_p,
                                               _c_void_p]),
    "moe_layer_routing": (ctypes.c_int, [_c_void_p, _sz, _i32, _i32, _i32, _i32, _i32, _f32, ctypes.c_int,
                                         ctypes.c_int, ctypes.POINTER(LayerRouting)]),
    "moe_router_opts_workspace_bytes": (_sz, [_i32, _i32, ctypes.c_int, _opts_p]),
    "moe_route_ex": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _i32, _i32, _i32, _i32, ctypes.c_int,
                                    ctypes.c_uint32, _opts_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                    _c_void_p, _sz, _c_void_p]),
    "moe_layer_forward_ex": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                            _i32, _i32, _i32, _i32, _i32, _f32, ctypes.c_int, ctypes.c_int,
                                            _opts_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _sz,
                                            _c_void_p]),
    "moe_layer_backward_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _f32, ctypes.c_int, ctypes.c_int]),
    "moe_layer_backward": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i32, _i32,
                                          _i32, _i32, _f32, ctypes.c_int, ctypes.c_int, _c_void_p, _f32, _c_void_p,
                                          _sz, _c_void_p, _sz, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                          _c_void_p, _c_void_p, _sz, _c_void_p]),
    "moe_layer_backward_ex": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i32,
                                             _i32, _i32, _i32, _f32, ctypes.c_int, ctypes.c_int, _opts_p, _c_void_p,
                                             _f32, _c_void_p, _sz, _c_void_p, _sz, _c_void_p, _c_void_p, _c_void_p,
                                             _c_void_p, _c_void_p, _c_void_p, _sz, _c_void_p]),
    "moe_layer_backward_timed": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i32,
                                                _i32, _i32, _i32, _f32, ctypes.c_int, ctypes.c_int, _c_void_p, _f32,
                                                _c_void_p, _sz, _c_void_p, _sz, _c_void_p, _c_void_p, _c_void_p,
                                                _c_void_p, _c_void_p, _c_void_p, _sz, _c_void_p, _c_void_p]),
    "moe_layer_preact_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _f32, ctypes.c_int]),
    "moe_layer_forward_train": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                               _i32, _i32, _i32, _i32, _i32, _f32, ctypes.c_int, ctypes.c_int,
                                               _c_void_p, _c_void_p, _c_void_p, _c_void_p, _sz, _c_void_p, _sz,
                                               _c_void_p, _c_void_p]),
    "moe_binned_capacity_max": (_i32, [_i32, _i32, _i32, _f32, _i32]),
    "moe_binned_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _f32, _i32, ctypes.c_int, ctypes.c_int]),
    "moe_layer_forward_binned": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                                _i32, _i32, _i32, _i32, _i32, _f32, _i32, ctypes.c_int,
                                                ctypes.c_int, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                                _c_void_p, _c_void_p, _sz, _c_void_p]),
    "moe_layer_forward_binned_timed": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                                      _c_void_p, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                                                      ctypes.c_int, ctypes.c_int, _c_void_p, _c_void_p, _c_void_p,
                                                      _c_void_p, _c_void_p, _c_void_p, _sz, _c_void_p, _c_void_p]),
}

LAYER_STAGES = ("logits", "select", "scan", "scatter", "expert_up", "expert_down", "combine")
BACKWARD_STAGES = ("combine_bwd", "router_bwd", "recompute_up", "down_dgrad", "down_wgrad", "up_dgrad", "up_wgrad",
                   "router_gemms", "dx")
BINNED_STAGES = ("logits", "select", "scan", "scatter", "gather", "expert_up", "expert_down", "combine")

_lib = None


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise RuntimeError(f"{lib_path} is not built: run `python -m top_routing_expert_moe_amd.build`")
        l = ctypes.CDLL(lib_path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != 0:
        raise MoEError(status, where)


def capacity(T: int, E: int, k: int, capacity_factor: float) -> int | None:
    """Per-expert capacity as the library computes it; None = never drop."""
    c = lib().moe_capacity(T, E, k, capacity_factor)
    if c < 0:
        raise ValueError("invalid capacity arguments")
    return None if c == 2 ** 31 - 1 else c


def workspace_bytes(T, h, f, E, k, capacity_factor, dtype: int, act: int) -> int:
    return int(lib().moe_workspace_bytes(T, h, f, E, k, capacity_factor, dtype, act))


@dataclasses.dataclass(frozen=True)
class CapacityConfig:
    """Capacity settings of a fixed-capacity layer, after the SparseMLP parameters of the
    Colossal-AI MoE page: one factor for training and one for evaluation, a minimum bucket
    size, and whether assignments past the capacity are dropped.  Without dropping, the
    bucket is the largest expert count of the call (factor 0), so nothing is dropped."""
    train: float = 1.25
    eval: float = 2.0
    min_capacity: int = 4
    drop_tokens: bool = True

    def factor(self, training: bool) -> float:
        if not self.drop_tokens:
            return 0.0
        return float(self.train if training else self.eval)


def binned_capacity_max(T, E, k, capacity_factor, min_capacity) -> int:
    return int(lib().moe_binned_capacity_max(T, E, k, capacity_factor, min_capacity))


def binned_workspace_bytes(T, h, f, E, k, capacity_factor, min_capacity, dtype: int, act: int) -> int:
    return int(lib().moe_binned_workspace_bytes(T, h, f, E, k, capacity_factor, min_capacity, dtype, act))


# ----------------------------------------------------------------------------
# torch marshalling

def _torch():
    import torch
    return torch


def _dt(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _p(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(dev):
    return _torch().cuda.current_stream(dev).cuda_stream


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _ws(nbytes: int, dev):
    return _torch().empty(max(int(nbytes), 1), dtype=_torch().uint8, device=dev)


def _opts(jitter, noise, temperature, uniform, x=None, T=None, E=None, soft=False):
    """A RouterOpts for the given variants, or None when all are at their defaults."""
    if jitter is None and noise is None and float(temperature) == 1.0 and not uniform and not soft:
        return None
    torch = _torch()
    if jitter is not None and (x is None or jitter.shape != x.shape or jitter.dtype != x.dtype):
        raise ValueError("jitter must have x's shape and dtype")
    if noise is not None and (tuple(noise.shape) != (T, E) or noise.dtype != torch.float32):
        raise ValueError("noise must be fp32 [T, E]")
    return RouterOpts(_p(jitter), _p(noise), float(temperature), 1 if uniform else 0, 1 if soft else 0)


def route(x, W_gate, logit_bias, k: int, *, logits=None, with_prob_sum: bool = False, jitter=None, noise=None,
          temperature: float = 1.0, uniform: bool = False, soft: bool = False):
    """Router on ``x[T,h]`` (or on given fp32 ``logits[T,E]``), optionally with the
    router variants (``jitter`` [T,h] in x's dtype, gate ``noise`` [T,E] fp32, softmax
    ``temperature``, ``uniform`` expert assignment, ``soft`` top-K weights).

    Returns ``(logits, topk_idx, topk_w, prob_sum)`` (prob_sum is None unless
    requested)."""
    torch = _torch()
    ref = logits if logits is not None else x
    dev = ref.device
    T = ref.shape[0]
    E = (logits if logits is not None else W_gate).shape[-1]
    opts = _opts(jitter, noise, temperature, uniform, x, T, E, soft)
    h = 0 if x is None else x.shape[1]
    dt = F32 if x is None else _dt(x)
    flags = ROUTE_LOGITS_IN if logits is not None else 0
    out_logits = logits if logits is not None else torch.empty((T, E), dtype=torch.float32, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    ps = torch.empty(E, dtype=torch.float32, device=dev) if with_prob_sum else None
    need = lib().moe_route_workspace_bytes(T, h, E, dt, flags, 1 if with_prob_sum else 0)
    if opts is not None:
        need += lib().moe_router_opts_workspace_bytes(T, h, dt, ctypes.byref(opts))
    ws = _ws(need, dev) if need else None
    args = (None if logits is not None else _p(x), None if logits is not None else _p(W_gate),
            None if (logits is not None or logit_bias is None) else _p(logit_bias), T, h, E, k, dt, flags)
    tail = (_p(out_logits), _p(idx), _p(w), _p(ps), _p(ws), 0 if ws is None else ws.numel(), _stream(dev))
    if opts is None:
        _check(lib().moe_route(*args, *tail), "moe_route")
    else:
        _check(lib().moe_route_ex(*args, ctypes.byref(opts), *tail), "moe_route_ex")
    return out_logits, idx, w, ps


def permute(topk_idx, x, E: int, capacity_factor: float, *, with_x_perm: bool = True, prob_sum=None,
            x_perm=None):
    """Histogram, capacity, stable sort by expert id and gather.

    Returns a dict with ``counts``, ``offsets``, ``sorted_slot``, ``slot_pos``,
    ``x_perm`` (or None) and ``aux`` (0-d tensor, or None without prob_sum).
    ``x_perm``: a preallocated ``[T*k, h]`` output (rows past the kept count are left
    as they are)."""
    torch = _torch()
    dev = topk_idx.device
    T, k = topk_idx.shape
    h = 0 if x is None else x.shape[1]
    dt = F32 if x is None else _dt(x)
    n = T * k
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sorted_slot = torch.full((n,), -1, dtype=torch.int32, device=dev)
    slot_pos = torch.empty(n, dtype=torch.int32, device=dev)
    if x_perm is None and with_x_perm and x is not None:
        x_perm = torch.empty((n, h), dtype=x.dtype, device=dev)
    aux = torch.empty((), dtype=torch.float32, device=dev) if prob_sum is not None else None
    ws = _ws(lib().moe_permute_workspace_bytes(T, E, k), dev)
    st = lib().moe_permute(_p(topk_idx), _p(x) if x_perm is not None else None, T, h, E, k,
                           float(capacity_factor), dt, _p(counts), _p(offsets), _p(sorted_slot), _p(slot_pos),
                           _p(x_perm), _p(prob_sum), _p(aux), _p(ws), ws.numel(), _stream(dev))
    _check(st, "moe_permute")
    return dict(counts=counts, offsets=offsets, sorted_slot=sorted_slot, slot_pos=slot_pos, x_perm=x_perm,
                aux=aux)


def expert_ffn(x_perm, offsets, W1, W3, W2, act: str, out=None):
    """Grouped expert MLP over the segments of ``x_perm``; returns ``out_perm[R_max,h]``
    (``out``: a preallocated one; rows from ``offsets[E]`` on are not written)."""
    torch = _torch()
    dev = x_perm.device
    R_max, h = x_perm.shape
    E, _, f = W1.shape
    dt = _dt(x_perm)
    if out is None:
        out = torch.empty_like(x_perm)
    elif out.shape != x_perm.shape or out.dtype != x_perm.dtype:
        raise ValueError("out must have x_perm's shape and dtype")
    ws = _ws(lib().moe_expert_ffn_workspace_bytes(R_max, h, f, E, dt, _ACT[act]), dev)
    st = lib().moe_expert_ffn(_p(x_perm), _p(offsets), R_max, h, f, E, _p(W1), _p(W3), _p(W2), _ACT[act], dt,
                              _p(out), _p(ws), ws.numel(), _stream(dev))
    _check(st, "moe_expert_ffn")
    return out


def unpermute(out_perm, slot_pos, topk_w):
    """Weighted combine back to token order; returns ``y[T,h]``."""
    torch = _torch()
    T, k = topk_w.shape
    h = out_perm.shape[1]
    y = torch.empty((T, h), dtype=out_perm.dtype, device=out_perm.device)
    st = lib().moe_unpermute(_p(out_perm), _p(slot_pos), _p(topk_w), T, h, k, _dt(out_perm), _p(y),
                             _stream(out_perm.device))
    _check(st, "moe_unpermute")
    return y


def preact_bytes(T: int, h: int, f: int, E: int, k: int, capacity_factor: float, act: str) -> int:
    """Bytes of the pre-activation context that the training forward writes."""
    return lib().moe_layer_preact_bytes(T, h, f, E, k, float(capacity_factor), _ACT[act])


def layer_forward(x, W_gate, logit_bias, W1, W3, W2, *, k: int, capacity_factor: float, act: str,
                  ws=None, y=None, aux=None, counts=None, events=None, jitter=None, noise=None,
                  temperature: float = 1.0, uniform: bool = False, soft: bool = False, preact=None):
    """The whole layer.  Returns ``(y, aux_loss, counts)``.  Pass preallocated
    ``ws``/``y``/``aux``/``counts`` to avoid allocations in a timed loop.
    ``events``: a ctypes array of ``len(LAYER_STAGES) + 1`` hipEvent_t handles to
    record between the stages (the measurement variant of the entry point).
    ``jitter``/``noise``/``temperature``/``uniform``/``soft``: the router variants (see route).
    ``preact``: a uint8 device tensor of ``preact_bytes(...)`` bytes: the training forward,
    which also saves the up projection's pre-activations there for layer_backward."""
    torch = _torch()
    dev = x.device
    T, h = x.shape
    E, _, f = W1.shape
    opts = _opts(jitter, noise, temperature, uniform, x, T, E, soft)
    if opts is not None and events is not None:
        raise ValueError("the measurement entry point takes no router variants")
    if opts is not None and preact is not None:
        raise ValueError("the training forward takes no router variants")
    dt = _dt(x)
    a = _ACT[act]
    if ws is None:
        extra = 0 if opts is None else lib().moe_router_opts_workspace_bytes(T, h, dt, ctypes.byref(opts))
        ws = _ws(workspace_bytes(T, h, f, E, k, capacity_factor, dt, a) + extra, dev)
    if y is None:
        y = torch.empty_like(x)
    if aux is None:
        aux = torch.empty((), dtype=torch.float32, device=dev)
    if counts is None:
        counts = torch.empty(E, dtype=torch.int32, device=dev)
    if opts is not None:
        _check(lib().moe_layer_forward_ex(_p(x), _p(W_gate), _p(logit_bias), _p(W1), _p(W3), _p(W2), T, h, f, E, k,
                                          float(capacity_factor), a, dt, ctypes.byref(opts), _p(y), _p(aux),
                                          _p(counts), _p(ws), ws.numel(), _stream(dev)), "moe_layer_forward_ex")
        return y, aux, counts
    args = (_p(x), _p(W_gate), _p(logit_bias), _p(W1), _p(W3), _p(W2), T, h, f, E, k, float(capacity_factor), a,
            dt, _p(y), _p(aux), _p(counts), _p(ws), ws.numel(), _stream(dev))
    if preact is not None:
        _check(lib().moe_layer_forward_train(*args[:-1], _p(preact), _nbytes(preact), _stream(dev),
                                             None if events is None else ctypes.cast(events, _c_void_p)),
               "moe_layer_forward_train")
    elif events is None:
        _check(lib().moe_layer_forward(*args), "moe_layer_forward")
    else:
        _check(lib().moe_layer_forward_timed(*args, ctypes.cast(events, _c_void_p)), "moe_layer_forward_timed")
    return y, aux, counts


def layer_routing(ws, *, T: int, h: int, f: int, E: int, k: int, capacity_factor: float, dtype, act: str) -> dict:
    """The routing that the layer call using workspace ``ws`` left there (moe_layer_routing):
    torch views (no copies) of ``logits``, ``topk_idx``, ``topk_w``, ``counts`` (valid when
    the call got no counts buffer of its own), ``offsets``, ``slot_pos`` and
    ``sorted_slot`` (first ``offsets[E]`` valid)."""
    torch = _torch()
    dt = dtype if isinstance(dtype, int) else _dt(torch.empty(0, dtype=dtype))
    r = LayerRouting()
    _check(lib().moe_layer_routing(_p(ws), ws.numel(), T, h, f, E, k, float(capacity_factor), dt, _ACT[act],
                                   ctypes.byref(r)), "moe_layer_routing")
    base = ws.data_ptr()

    def view(name, n, tdtype):
        off = getattr(r, name) - base
        esz = torch.empty(0, dtype=tdtype).element_size()
        return ws[off:off + n * esz].view(tdtype)
    n = T * k
    return dict(logits=view("logits", T * E, torch.float32).view(T, E),
                topk_idx=view("topk_idx", n, torch.int32).view(T, k),
                topk_w=view("topk_w", n, torch.float32).view(T, k), counts=view("counts", E, torch.int32),
                offsets=view("offsets", E + 1, torch.int32), slot_pos=view("slot_pos", n, torch.int32),
                sorted_slot=view("sorted_slot", n, torch.int32))


def layer_forward_binned(x, W_gate, logit_bias, W1, W3, W2, *, k: int, capacity_factor: float,
                         min_capacity: int = 0, act: str, ws=None, y=None, aux=None, counts=None,
                         capacity=None, x_bins=None, events=None):
    """The layer with fixed-capacity buckets of C rows per expert.  Returns
    ``(y, aux_loss, counts, capacity, x_bins)``; ``x_bins`` is ``[E * Cmax, h]`` with
    bucket e in rows ``[e*C, (e+1)*C)``, C = ``capacity`` (a device scalar).
    ``events``: ``len(BINNED_STAGES) + 1`` hipEvent_t handles recorded between the stages."""
    torch = _torch()
    dev = x.device
    T, h = x.shape
    E, _, f = W1.shape
    dt = _dt(x)
    a = _ACT[act]
    cmax = binned_capacity_max(T, E, k, capacity_factor, min_capacity)
    if cmax < 0:
        raise MoEError(1, "moe_binned_capacity_max")
    if ws is None:
        ws = _ws(binned_workspace_bytes(T, h, f, E, k, capacity_factor, min_capacity, dt, a), dev)
    if y is None:
        y = torch.empty_like(x)
    if aux is None:
        aux = torch.empty((), dtype=torch.float32, device=dev)
    if counts is None:
        counts = torch.empty(E, dtype=torch.int32, device=dev)
    if capacity is None:
        capacity = torch.empty((), dtype=torch.int32, device=dev)
    if x_bins is None:
        x_bins = torch.empty((E * cmax, h), dtype=x.dtype, device=dev)
    args = (_p(x), _p(W_gate), _p(logit_bias), _p(W1), _p(W3), _p(W2), T, h, f, E, k, float(capacity_factor),
            int(min_capacity), a, dt, _p(y), _p(aux), _p(counts), _p(capacity), _p(x_bins), _p(ws), ws.numel(),
            _stream(dev))
    if events is None:
        _check(lib().moe_layer_forward_binned(*args), "moe_layer_forward_binned")
    else:
        _check(lib().moe_layer_forward_binned_timed(*args, ctypes.cast(events, _c_void_p)),
               "moe_layer_forward_binned_timed")
    return y, aux, counts, capacity, x_bins


def layer_backward(x, W_gate, W1, W3, W2, dy, *, k: int, capacity_factor: float, act: str, fwd_ws,
                   d_aux: float = 0.0, with_w_gate: bool = True, ws=None, out=None, events=None, preact=None,
                   jitter=None, noise=None, temperature: float = 1.0, soft: bool = False):
    """Gradients of ``<dy, y> + d_aux * aux`` for the layer_forward call that used the
    workspace ``fwd_ws`` (pass the same inputs).  Returns a dict with ``dx`` (x's dtype)
    and fp32 ``dW_gate`` (or None), ``dW1``, ``dW3`` (None for GELU), ``dW2``.  ``out``:
    preallocated tensors under those names.  ``events``: ``len(BACKWARD_STAGES) + 1``
    hipEvent_t handles recorded between the stages.  ``preact``: the pre-activations that
    the training forward (layer_forward with ``preact``) saved; None = recompute them.
    ``jitter``/``noise``/``temperature``/``soft``: the router variants of the forward call
    (the same tensors), differentiated through ``moe_layer_backward_ex``."""
    torch = _torch()
    dev = x.device
    T, h = x.shape
    E, _, f = W1.shape
    dt = _dt(x)
    a = _ACT[act]
    if ws is None:
        ws = _ws(lib().moe_layer_backward_workspace_bytes(T, h, f, E, k, float(capacity_factor), dt, a), dev)
    o = dict(out or {})
    o.setdefault("dx", torch.empty_like(x))
    o.setdefault("dW_gate", torch.empty((h, E), dtype=torch.float32, device=dev) if with_w_gate else None)
    o.setdefault("dW1", torch.empty((E, h, f), dtype=torch.float32, device=dev))
    o.setdefault("dW3", torch.empty((E, h, f), dtype=torch.float32, device=dev) if act == "swiglu" else None)
    o.setdefault("dW2", torch.empty((E, f, h), dtype=torch.float32, device=dev))
    args = (_p(x), _p(W_gate), _p(W1), _p(W3), _p(W2), T, h, f, E, k, float(capacity_factor), a, dt, _p(dy),
            float(d_aux), _p(fwd_ws), fwd_ws.numel(), _p(preact), 0 if preact is None else _nbytes(preact),
            _p(o["dx"]), _p(o["dW_gate"]), _p(o["dW1"]), _p(o["dW3"]), _p(o["dW2"]), _p(ws), ws.numel(),
            _stream(dev))
    opts = _opts(jitter, noise, temperature, False, x, T, E, soft)
    if opts is not None:
        if events is not None:
            raise ValueError("the measurement entry point takes no router variants")
        _check(lib().moe_layer_backward_ex(*args[:13], ctypes.byref(opts), *args[13:]), "moe_layer_backward_ex")
    elif events is None:
        _check(lib().moe_layer_backward(*args), "moe_layer_backward")
    else:
        _check(lib().moe_layer_backward_timed(*args, ctypes.cast(events, _c_void_p)), "moe_layer_backward_timed")
    return o
