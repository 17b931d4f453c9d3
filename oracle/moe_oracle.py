"""CPU oracle for the top-k-routed MoE layer forward -- TEST INFRASTRUCTURE ONLY.

This is the plain, slow, obviously-correct definition that the HIP path is
checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product path never
does, and it imports nothing from the product package.  It shares no code with
the HIP kernels or their host library.

Arithmetic is fp64 throughout (numpy), with exactly the rounding points the
method fixes:

* router logits are formed in fp64 from the exact input values and rounded
  once to fp32 -- the pages keep routing in fp32;
* in bf16 workloads the expert's hidden activation ``Hm`` is rounded to bf16
  (round-to-nearest-even) before the down projection, because the down
  projection's left operand is a bf16 tensor;
* the layer output is rounded once to its storage dtype.

Sources (the pages' titles; the sections named in each docstring):

* [OPS]  aicoding.csdn.net article on the ops-transformer MoE operators
  (sections "原理：MoE的稀疏路由是怎么工作的" Steps 1-4, "坑1：负载均衡",
  "实现：ops-transformer里面的MoE算子" with the ``MoEGatingForward`` sketch).
* [CANN] "MoE 路由算子到底在做什么？一次拆透 ops-transformer 的核心机制"
  (sections 2.1-2.3, 3).
* [RTR]  "MoE Router：谁来决定 Token 去哪个 Expert" (router passage, the
  ``MoERouter`` snippet, the load-balancing passage, the capacity-limit passage).
* [MB]   "01 · MoE 为什么难算：变长专家输入" (MegaBlocks chapter 1; sections 1,
  2, 3, 4.1-4.6, 5).
* [CAI]  "在 Colossal-AI 中为你的模型集成混合专家（MoE）..." (SparseMLP forward
  data flow, ``MoeLoss`` passage).

Readings taken where the pages are silent or disagree are listed beside the
function that takes them.  Every function here is pinned by ``tests/`` against
worked examples, closed forms, brute force or library routines.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf as _erf

__all__ = [
    "bf16_to_f64", "round_to_bf16", "router_logits", "softmax", "select_topk",
    "topk_weights", "expert_capacity", "histogram", "permute", "silu", "gelu",
    "expert_ffn", "combine", "aux_loss", "layer_forward",
    "binned_capacity", "binned_layout", "layer_forward_binned",
    "jitter_input", "noisy_logits", "softmax_t", "topk_weights_t", "uniform_assignment", "route",
    "silu_grad", "gelu_grad", "router_logit_grad", "router_logit_grad_scale", "expert_grad_scale",
    "layer_backward",
]


# ----------------------------------------------------------------------------
# number formats

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp64 values (a bf16 is the top half of an fp32)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """fp64 -> nearest bf16, ties to even, returned as uint16 bit patterns.

    bf16 keeps 8 significant bits.  With v = m * 2**e (0.5 <= |m| < 1), the
    spacing of bf16 values around v is q = 2**(e-8); rounding v/q to the
    nearest integer with ties to even (numpy's ``rint``) and scaling back is an
    exact, single rounding.  The result is representable in fp32, whose top 16
    bits are the bf16 pattern.  Finite inputs in the normal range only.
    """
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    q = np.ldexp(1.0, e - 8)
    r = np.rint(v / q) * q
    r = np.where(v == 0.0, v, r)
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_to_f64(a) if dtype == "bf16" else np.asarray(a, dtype=np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# routing: router linear, softmax, top-k, renormalisation

def router_logits(x: np.ndarray, W_gate: np.ndarray, logit_bias, dtype: str) -> np.ndarray:
    """``logits[t,e] = sum_i x[t,i] * W_gate[i,e] (+ logit_bias[e])`` as fp32 [T,E].

    The router is one bias-free linear map from the hidden width to the expert
    count ([RTR] ``MoERouter``: ``Linear(hidden_dim, num_experts, bias=False)``;
    [OPS] Step 1; [MB] section 1, LearnedRouter).  Routing runs in fp32 ([CAI]
    SparseMLP data flow, step 2: gate logits are cast to fp32 before the
    router).  Reading: formed in fp64 from the exact inputs, rounded once to
    fp32.  ``logit_bias`` is not a learned parameter of the method: it only
    skews the synthetic workloads' expert popularity.
    """
    l = _as_f64(x, dtype) @ np.asarray(W_gate, dtype=np.float32).astype(np.float64)
    if logit_bias is not None:
        l = l + np.asarray(logit_bias, dtype=np.float32).astype(np.float64)[None, :]
    return l.astype(np.float32)


def softmax(logits: np.ndarray) -> np.ndarray:
    """Row softmax over the E experts, fp64, with the row maximum subtracted
    ([OPS] ``MoEGatingForward`` step 1; [RTR] ``F.softmax(logits, dim=-1)``)."""
    l = np.asarray(logits, dtype=np.float32).astype(np.float64)
    z = np.exp(l - l.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def select_topk(logits: np.ndarray, k: int) -> np.ndarray:
    """The k experts with the largest scores per token, best first, as int32 [T,k].

    [OPS] Step 2 and ``MoEGatingForward`` step 2 (a selection of the K best);
    [RTR] ``torch.topk`` (sorted output).  Readings: the ranking is on the fp32
    *logits* (softmax is monotone, so this is the same set, and it avoids ties
    created by rounding of exp); equal logits rank the lower expert index
    first; -0.0 equals +0.0 (IEEE comparison).  Slot j holds the j-th best.
    """
    l = np.asarray(logits, dtype=np.float32)
    T, E = l.shape
    expert = np.broadcast_to(np.arange(E), (T, E))
    # lexsort: the last key is the primary one -> (logit descending, expert ascending)
    order = np.lexsort((expert, -l), axis=1)
    return order[:, :k].astype(np.int32)


def topk_weights(logits: np.ndarray, topk_idx: np.ndarray) -> np.ndarray:
    """Renormalised gate weights of the selected experts, fp32 [T,k].

    ``w[t,j] = p[t,S_j] / sum_j' p[t,S_j']`` with p the full softmax
    ([OPS] ``MoEGatingForward`` step 3: the chosen weights are scaled to sum
    to one; [RTR] ``topk_weights / topk_weights.sum(-1)``).  Always applied,
    also for k = 1 (then w = 1).  fp64, rounded once to fp32.
    """
    p = softmax(logits)
    sel = np.take_along_axis(p, np.asarray(topk_idx, dtype=np.int64), axis=1)
    return (sel / sel.sum(axis=1, keepdims=True)).astype(np.float32)


# ----------------------------------------------------------------------------
# router variants: jitter, gate noise, softmax temperature, uniform assignment

def jitter_input(x: np.ndarray, u: np.ndarray, dtype: str) -> np.ndarray:
    """The router's input under multiplicative jitter: ``x * u`` elementwise, stored in
    the input's dtype ([MB] section 5: during training the router input may be
    multiplied by uniform noise in [1 - eps, 1 + eps], an exploration aid from Switch).
    Readings: the noise ``u`` is drawn by the caller in x's dtype (it is an input
    here); the product is rounded once to that dtype (bf16: round to nearest even);
    only the router sees the jittered input -- the experts get x.  Returns bf16 bit
    patterns or fp32 values."""
    prod = _as_f64(x, dtype) * _as_f64(u, dtype)
    return round_to_bf16(prod) if dtype == "bf16" else prod.astype(np.float32)


def noisy_logits(logits: np.ndarray, noise) -> np.ndarray:
    """Gate logits with additive noise ([CAI] Top2Router with a NormalNoiseGenerator:
    Gaussian noise scaled by the expert count is added to the router scores during
    training).  Readings: the noise [T,E] is an input (the caller draws it); it is
    added in fp32, so selection sees exactly the fp32 sum; every later step (softmax,
    top-k, weights, aux loss) uses the noisy logits."""
    l = np.asarray(logits, dtype=np.float32)
    if noise is None:
        return l
    return (l + np.asarray(noise, dtype=np.float32)).astype(np.float32)


def softmax_t(logits: np.ndarray, temperature: float) -> np.ndarray:
    """Row softmax of ``logits / temperature`` in fp64, with the row maximum subtracted
    ([OPS] "坑3：数值稳定性": the soft top-K remedy uses a softmax with a temperature).
    temperature = 1 is :func:`softmax`."""
    l = np.asarray(logits, dtype=np.float32).astype(np.float64)
    z = np.exp((l - l.max(axis=1, keepdims=True)) / float(temperature))
    return z / z.sum(axis=1, keepdims=True)


def topk_weights_t(logits: np.ndarray, topk_idx: np.ndarray, temperature: float,
                   soft: bool = False) -> np.ndarray:
    """Gate weights of the selected experts under ``p = softmax(l / temperature)``, fp32 [T,k].

    ``soft=False``: renormalised over the k selected experts, ``w[t,j] = p[t,S_j] /
    sum_j' p[t,S_j']`` -- the plain router's weights ([OPS] Step 4) with a temperature.

    ``soft=True``: the soft top-K of [OPS] "坑3：数值稳定性".  The page contrasts it with
    a hard top-K: a softmax with a temperature over all experts, so that experts that
    are not selected keep a little probability (and with it a gradient).  Reading: the
    k best experts are still the ones that run (the selection is unchanged), and their
    weights are the temperature softmax over all E experts taken at the selection,
    ``w[t,j] = p[t,S_j]``, *without* renormalising over the k.  The weights then sum to
    less than one; the rest of the mass, ``sum over unselected e of p[t,e]``, belongs to
    the experts that did not run.  Each weight depends on every expert's logit through
    the softmax's denominator, so unselected experts receive gradient (see
    :func:`layer_backward`).  The temperature sets how much mass they keep: a small one
    concentrates it on the best expert, a large one spreads it towards 1/E each.
    """
    p = softmax_t(logits, temperature)
    sel = np.take_along_axis(p, np.asarray(topk_idx, dtype=np.int64), axis=1)
    if soft:
        return sel.astype(np.float32)
    return (sel / sel.sum(axis=1, keepdims=True)).astype(np.float32)


def uniform_assignment(T: int, k: int, E: int) -> np.ndarray:
    """Benchmark mode of [MB] section 5: the expert ids are replaced by
    ``arange(T*k) % E`` laid out as [T,k] (slot j of token t gets ``(t*k + j) % E``),
    a perfectly balanced assignment for measuring speed without a trained router.
    Reading: only the ids are replaced; the weights stay those of the real top-k."""
    return (np.arange(T * k, dtype=np.int64) % E).astype(np.int32).reshape(T, k)


def route(logits: np.ndarray, k: int, *, noise=None, temperature: float = 1.0,
          uniform: bool = False, soft: bool = False) -> dict:
    """Selection with the router variants applied in the pages' order: noise on the
    logits, top-k on the (noisy) logits, temperature-softmax weights (renormalised over
    the selection, or not with the soft top-K), ids optionally replaced by the uniform
    assignment.  Returns ``topk_idx``, ``topk_w``, ``probs`` (the temperature softmax
    over all experts, for the aux loss) and the logits used."""
    if not (float(temperature) > 0.0 and math.isfinite(float(temperature))):
        raise ValueError("temperature must be finite and > 0")
    l = noisy_logits(logits, noise)
    idx = select_topk(l, k)
    w = topk_weights_t(l, idx, temperature, soft)
    if uniform:
        idx = uniform_assignment(l.shape[0], k, l.shape[1])
    return dict(logits=l, topk_idx=idx, topk_w=w, probs=softmax_t(l, temperature))


# ----------------------------------------------------------------------------
# capacity, histogram, stable sort by expert

def expert_capacity(T: int, E: int, k: int, capacity_factor: float):
    """Per-expert capacity ``C = floor(cf * (k*T/E))``; ``None`` means unlimited.

    [MB] section 3 (``C = capacity_factor * tokens * top_k / num_experts``)
    and section 4.2 (``expert_capacity``: tokens-per-expert first, then the
    factor, then truncation to int).  [RTR]'s capacity passage drops the k;
    the MegaBlocks form with k is taken.  Section 4.6: a computed capacity of
    zero means "never drop" -- taken here also for a factor <= 0.  The factor
    enters as an fp32 value (that is how the library receives it) and the
    product is formed in fp64.
    """
    cf = float(np.float32(capacity_factor))
    if not math.isfinite(cf):
        raise ValueError("capacity factor must be finite")
    if cf <= 0.0:
        return None
    tokens_per_expert = (k * T) / E
    C = int(math.floor(cf * tokens_per_expert))
    return None if C == 0 else C


def histogram(topk_idx: np.ndarray, E: int) -> np.ndarray:
    """``tokens_per_expert``: how many (token, slot) assignments chose each expert, before
    any capacity drop ([MB] section 4.1 table)."""
    counts = np.zeros(E, dtype=np.int64)
    for e in np.asarray(topk_idx).reshape(-1).tolist():
        counts[e] += 1
    return counts.astype(np.int32)


def permute(topk_idx: np.ndarray, E: int, C):
    """Sort the flattened assignments by expert id, stably, and apply the capacity.

    Assignment ``s = t*k + j`` (token t, slot j).  [MB] section 4.1 sorts the
    flattened expert ids and takes the running end positions of each expert
    (``bins``); section 4.5: an expert keeps only its first C rows, later ones
    are dropped silently and contribute zero.  Readings: the sort is stable,
    so "first" means ascending s; offsets are exclusive starts over the
    *kept* rows, ``offsets[E] = R`` the total kept.

    Returns ``counts[E]`` (pre-drop), ``offsets[E+1]``, ``sorted_slot[T*k]``
    (row r of the expert-sorted order -> its assignment s; rows >= R are -1) and
    ``slot_pos[T*k]`` (assignment s -> its row, -1 if dropped).
    """
    flat = np.asarray(topk_idx).reshape(-1).tolist()
    n = len(flat)
    counts = [0] * E
    for e in flat:
        counts[e] += 1
    kept = [c if C is None else min(c, C) for c in counts]
    offsets = [0]
    for e in range(E):
        offsets.append(offsets[-1] + kept[e])
    seen = [0] * E
    sorted_slot = [-1] * n
    slot_pos = [-1] * n
    for s, e in enumerate(flat):
        r = seen[e]
        seen[e] += 1
        if C is None or r < C:
            slot_pos[s] = offsets[e] + r
            sorted_slot[offsets[e] + r] = s
    i32 = lambda a: np.asarray(a, dtype=np.int32)
    return i32(counts), i32(offsets), i32(sorted_slot), i32(slot_pos)


# ----------------------------------------------------------------------------
# experts

def silu(z: np.ndarray) -> np.ndarray:
    """``silu(z) = z / (1 + exp(-z))`` (the gate of SwiGLU, [CANN] section 7)."""
    return z / (1.0 + np.exp(-z))


def gelu(z: np.ndarray) -> np.ndarray:
    """GELU in its exact form ``z/2 * (1 + erf(z/sqrt(2)))`` ([MB] section 4.4 sketch names
    gelu without a variant; the exact erf form is taken)."""
    return 0.5 * z * (1.0 + _erf(z / math.sqrt(2.0)))


def expert_ffn(a: np.ndarray, W1e, W3e, W2e, act: str, dtype: str) -> np.ndarray:
    """One expert's MLP on fp64 rows ``a[n,h]``, returned in fp64 [n,h].

    [MB] section 4.3: ``MLP.forward`` is matmul, activation, matmul on the
    expert's ``[hs, ffn]`` weights.  SwiGLU experts gate the up projection:
    ``(silu(a @ W1) * (a @ W3)) @ W2``; GELU experts: ``gelu(a @ W1) @ W2``.
    In bf16 workloads the hidden activation is rounded to bf16 before the
    down projection.
    """
    z1 = a @ _as_f64(W1e, dtype)
    if act == "swiglu":
        hm = silu(z1) * (a @ _as_f64(W3e, dtype))
    elif act == "gelu":
        hm = gelu(z1)
    else:
        raise ValueError(act)
    if dtype == "bf16":
        hm = bf16_to_f64(round_to_bf16(hm))
    return hm @ _as_f64(W2e, dtype)


def combine(x: np.ndarray, topk_idx, topk_w, slot_pos, W1, W3, W2, act: str, dtype: str,
            tokens=None) -> np.ndarray:
    """Layer output, token by token from the definition, fp64 [len(tokens), h].

    ``y[t] = sum_j w[t,j] * FFN_{S_j}(x[t])`` over the slots that were kept
    ([OPS] Step 4; [MB] section 4.3 ``binned_scatter``: scale by the routing
    weight, then sum over the top-k slots).  A dropped slot adds nothing and the
    surviving weights are *not* renormalised ([MB] section 3 item 2 and
    section 4.5; [RTR] capacity passage: dropped tokens bypass the experts).
    It does not use the permuted layout, so it checks the permutation rather
    than trusting it.  Contributions are summed in ascending j.
    """
    T, k = np.asarray(topk_idx).shape
    tokens = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    xs = _as_f64(np.asarray(x)[tokens], dtype)
    h = xs.shape[1]
    contrib = np.zeros((len(tokens), k, h), dtype=np.float64)
    idx = np.asarray(topk_idx)[tokens]
    w = np.asarray(topk_w, dtype=np.float32)[tokens].astype(np.float64)
    kept = np.asarray(slot_pos).reshape(T, k)[tokens] >= 0
    for e in np.unique(idx[kept]):
        rows, slots = np.nonzero((idx == e) & kept)
        out = expert_ffn(xs[rows], W1[e], None if W3 is None else W3[e], W2[e], act, dtype)
        contrib[rows, slots] = w[rows, slots][:, None] * out
    y = np.zeros((len(tokens), h), dtype=np.float64)
    for j in range(k):
        y += contrib[:, j]
    return y


def aux_loss(counts: np.ndarray, probs: np.ndarray, T: int, k: int, E: int) -> float:
    """Switch-style load-balance loss ``E * sum_e f_e * P_e``, unscaled.

    [OPS] "坑1：负载均衡" and the ``MoELoadBalance`` call, [RTR] load-balancing
    passage (each expert should get about 1/E of the assignments), [CAI]
    ``MoeLoss`` (the 0.01 weight is applied by the caller).  Readings:
    ``f_e = counts_e / (T*k)`` with the pre-drop counts (the loss is a function
    of the router alone), ``P_e`` = mean over tokens of the full softmax.
    """
    f = np.asarray(counts, dtype=np.float64) / float(T * k)
    P = np.asarray(probs, dtype=np.float64).sum(axis=0) / float(T)
    return float(E * np.sum(f * P))


# ----------------------------------------------------------------------------
# the whole layer

def layer_forward(x, W_gate, logit_bias, W1, W3, W2, *, k: int, capacity_factor: float,
                  act: str, dtype: str, logits=None, tokens=None, with_y: bool = True,
                  jitter=None, noise=None, temperature: float = 1.0, uniform: bool = False,
                  soft: bool = False) -> dict:
    """Router -> top-k -> permute (with capacity) -> experts -> weighted combine, plus aux.

    ``logits`` may be given (fp32 [T,E]) to route on another implementation's
    logits, so that integer routing results can be compared bit for bit.
    ``tokens`` restricts the expensive output ``y`` to a subset of tokens
    (routing, capacity and aux always cover all tokens).  ``y`` is returned in
    the storage dtype: fp32 values, or bf16 bit patterns.  ``jitter``, ``noise``,
    ``temperature``, ``uniform`` and ``soft`` are the router variants
    (:func:`jitter_input`, :func:`route`); the experts always read the unjittered x.
    """
    x = np.asarray(x)
    T = x.shape[0]
    E = np.asarray(W_gate).shape[1]
    if logits is None:
        xr = x if jitter is None else jitter_input(x, jitter, dtype)
        logits = router_logits(xr, W_gate, logit_bias, dtype)
    logits = np.asarray(logits, dtype=np.float32)
    r = route(logits, k, noise=noise, temperature=temperature, uniform=uniform, soft=soft)
    idx, w = r["topk_idx"], r["topk_w"]
    C = expert_capacity(T, E, k, capacity_factor)
    counts, offsets, sorted_slot, slot_pos = permute(idx, E, C)
    out = dict(logits=logits, topk_idx=idx, topk_w=w, C=C, counts=counts, offsets=offsets,
               sorted_slot=sorted_slot, slot_pos=slot_pos,
               aux=aux_loss(counts, r["probs"], T, k, E))
    if with_y:
        tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
        y64 = combine(x, idx, w, slot_pos, W1, W3, W2, act, dtype, tokens=tok)
        out["y_tokens"] = tok
        out["y64"] = y64
        out["y"] = round_to_bf16(y64) if dtype == "bf16" else y64.astype(np.float32)
    return out


# ----------------------------------------------------------------------------
# backward pass: the adjoint of layer_forward

def silu_grad(z: np.ndarray) -> np.ndarray:
    """d silu / dz = s (1 + z (1 - s)), s = 1 / (1 + exp(-z))."""
    s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def gelu_grad(z: np.ndarray) -> np.ndarray:
    """d gelu / dz for the exact form: Phi(z) + z phi(z)."""
    return 0.5 * (1.0 + _erf(z / math.sqrt(2.0))) + z * np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)


def router_logit_grad(l: np.ndarray, idx: np.ndarray, w: np.ndarray, dw: np.ndarray, counts: np.ndarray,
                      d_aux: float, k: int, temperature: float = 1.0, soft: bool = False) -> np.ndarray:
    """Gradient of ``L`` with respect to the (noisy) logits ``l`` [T,E], fp64, given the
    gradient ``dw`` [T,k] of the selected experts' weights.

    With ``p = softmax(l / tau)`` the softmax's Jacobian is ``dp_a/dl_b = p_a (delta_ab -
    p_b) / tau``:

    * renormalised weights (the plain router; ``w = softmax(l_S / tau)`` over the k
      selected): ``dl[t,S_j] = w_j (dw_j - sum_j' w_j' dw_j') / tau``, zero for experts
      that were not selected;
    * soft top-K (``w_j = p[S_j]``, no renormalisation, [OPS] "坑3"): ``dl[t,b] = p_b
      (dw_b - sum_j w_j dw_j) / tau`` for every expert b, with ``dw_b`` the weight
      gradient of b's slot if b was selected and 0 otherwise -- experts that did not run
      still get ``-p_b sum_j w_j dw_j / tau``;
    * the aux loss ``E sum_e f_e P_e`` with ``P_e`` the mean of p adds ``d_aux (E/T) p_b
      (f_b - sum_e f_e p_e) / tau``; the counts ``f = counts / (T k)`` are piecewise
      constant in the logits (no gradient).

    The stored fp32 weights ``w`` are used where the weights appear.
    """
    T, E = l.shape
    tau = float(temperature)
    p = softmax_t(l, tau)
    wk = np.asarray(w, dtype=np.float32).astype(np.float64)
    s_dw = np.sum(wk * dw, axis=1, keepdims=True)
    rows = np.repeat(np.arange(T), k)
    dl = np.zeros((T, E))
    if soft:
        g = np.zeros((T, E))
        np.add.at(g, (rows, np.asarray(idx).reshape(-1)), dw.reshape(-1))
        dl += p * (g - s_dw) / tau
    else:
        np.add.at(dl, (rows, np.asarray(idx).reshape(-1)), (wk * (dw - s_dw) / tau).reshape(-1))
    fe = np.asarray(counts, dtype=np.float64) / float(T * k)
    dl += float(d_aux) * (E / float(T)) * p * (fe[None, :] - np.sum(p * fe[None, :], axis=1, keepdims=True)) / tau
    return dl


def router_logit_grad_scale(l: np.ndarray, idx: np.ndarray, w: np.ndarray, dw_m: np.ndarray, counts: np.ndarray,
                            d_aux: float, k: int, temperature: float = 1.0, soft: bool = False) -> np.ndarray:
    """Magnitude scale of :func:`router_logit_grad`: the same sums with every term taken
    by absolute value (differences become sums of the absolute terms), from the
    magnitude ``dw_m`` of the weight gradients.  ``|router_logit_grad| <= this`` for
    ``|dw| <= dw_m``; equality when no two terms cancel."""
    T, E = l.shape
    tau = float(temperature)
    p = softmax_t(l, tau)
    wk = np.abs(np.asarray(w, dtype=np.float32).astype(np.float64))
    s_m = np.sum(wk * dw_m, axis=1, keepdims=True)
    rows = np.repeat(np.arange(T), k)
    dl_m = np.zeros((T, E))
    if soft:
        g = np.zeros((T, E))
        np.add.at(g, (rows, np.asarray(idx).reshape(-1)), dw_m.reshape(-1))
        dl_m += p * (g + s_m) / tau
    else:
        np.add.at(dl_m, (rows, np.asarray(idx).reshape(-1)), (wk * (dw_m + s_m) / tau).reshape(-1))
    fe = np.asarray(counts, dtype=np.float64) / float(T * k)
    dl_m += abs(float(d_aux)) * (E / float(T)) * p * (fe[None, :] + np.sum(p * fe[None, :], axis=1,
                                                                            keepdims=True)) / tau
    return dl_m


def expert_grad_scale(X: np.ndarray, dy_rows: np.ndarray, w_rows: np.ndarray, a: np.ndarray, g, hm_r: np.ndarray,
                      W1e: np.ndarray, W3e, W2e: np.ndarray, act: str) -> dict:
    """Magnitude scales of one expert's gradients (rows X of that expert, fp64): the
    chain of products of :func:`layer_backward` taken over absolute values,

      ``|dO| = |w| |dy|``, ``dHm_m = |dO| |W2|^T``; SwiGLU ``da_m = dHm_m |g silu'(a)|``,
      ``dg_m = dHm_m |silu(a)|``; GELU ``da_m = dHm_m |gelu'(a)|``;
      ``dW2_m = |Hm|^T |dO|``, ``dW1_m = |X|^T da_m``, ``dW3_m = |X|^T dg_m``,
      ``dX_m = da_m |W1|^T (+ dg_m |W3|^T)``.

    Each is at least the magnitude of the matching gradient (triangle inequality), and
    equals it when no sum has terms of both signs.  A computation that rounds its
    operands with relative error u moves the gradient, to first order, by at most a
    small multiple of u times this scale -- which is what makes it a bound for a
    reduced-precision implementation."""
    dO_m = np.abs(w_rows)[:, None] * np.abs(dy_rows)
    dHm_m = dO_m @ np.abs(W2e).T
    out = dict(dW2=np.abs(hm_r).T @ dO_m)
    if act == "swiglu":
        da_m = dHm_m * np.abs(g * silu_grad(a))
        dg_m = dHm_m * np.abs(silu(a))
        out["dW3"] = np.abs(X).T @ dg_m
        out["dX"] = da_m @ np.abs(W1e).T + dg_m @ np.abs(W3e).T
    else:
        da_m = dHm_m * np.abs(gelu_grad(a))
        out["dX"] = da_m @ np.abs(W1e).T
    out["dW1"] = np.abs(X).T @ da_m
    return out


def layer_backward(x, W_gate, logit_bias, W1, W3, W2, dy, d_aux: float, *, k: int, capacity_factor: float,
                   act: str, dtype: str, logits=None, tokens=None, experts=None,
                   with_w_gate: bool = True, with_scale: bool = False, jitter=None, noise=None,
                   temperature: float = 1.0, soft: bool = False) -> dict:
    """Gradients of ``L = <dy, y> + d_aux * aux`` for the layer of :func:`layer_forward`,
    fp64, as the adjoint of each forward step in reverse order (chain rule).

    The pages name a backward pass for the gating operator ([OPS] operator list:
    moe_gating holds the router's forward and backward) and autograd wrappers around
    the gather / scatter of the permutation ([MB] section 5 file map) without writing
    them out, so this is the plain derivative of the forward as defined here:

    * combine: ``dw[t,j] = <dy[t], O[r]>`` and ``dO[r] = w[t,j] dy[t]`` for kept slots
      ``r = slot_pos[t*k+j]``; dropped slots get ``dw = 0`` (they do not reach y);
    * expert e on its rows X: ``dHm = dO W2^T``, ``dW2 = Hm^T dO``; SwiGLU
      ``da = dHm * g * silu'(a)``, ``dg = dHm * silu(a)``; GELU ``da = dHm * gelu'(a)``;
      ``dW1 = X^T da``, ``dW3 = X^T dg``, ``dX = da W1^T (+ dg W3^T)``;
    * the permutation's adjoint: ``dx[t] += sum_j dX[slot_pos[t*k+j]]``;
    * the router: :func:`router_logit_grad` (the weights and the aux loss);
    * ``dW_gate = xr^T dl``, ``dx += (dl W_gate^T) * u`` where ``xr`` is the router's
      input: x, or with jitter ``u`` the rounded product ``x * u``.

    Router variants: ``noise`` (added to the logits: the gradient with respect to the
    noisy logits is the one with respect to the logits), ``temperature`` and ``soft``
    (:func:`topk_weights_t`), ``jitter`` (:func:`jitter_input`; the rounding of the
    product passes gradients unchanged).  The uniform assignment is a benchmarking
    mode with no gradient of its own and is not differentiated here.

    Readings: top-k selection and the capacity drop are piecewise constant (no
    gradient); in bf16 workloads the rounding of Hm passes gradients unchanged while
    ``dW2`` uses the rounded Hm that the forward multiplied; ``logit_bias`` gets no
    gradient (it is not a parameter of the method).  ``tokens`` limits ``dx`` to those
    tokens, ``experts`` limits the weight gradients (and the expert work) to those
    experts, and ``with_w_gate=False`` skips ``dW_gate`` (which needs every token);
    the returned arrays are full-sized, with zeros where nothing was computed.

    ``with_scale`` also returns, for each gradient, its magnitude scale: the same chain
    of products taken over absolute values (:func:`expert_grad_scale`,
    :func:`router_logit_grad_scale`), carried through ``|dl| |W_gate|^T |u|`` and
    ``|xr|^T |dl|`` for the router's share of dx and for dW_gate.
    """
    x = np.asarray(x)
    T = x.shape[0]
    E = np.asarray(W_gate).shape[1]
    x64 = _as_f64(x, dtype)
    h = x64.shape[1]
    f = np.asarray(W1).shape[2]
    Wg = np.asarray(W_gate, dtype=np.float32).astype(np.float64)
    xr = x if jitter is None else jitter_input(x, jitter, dtype)
    xr64 = _as_f64(xr, dtype)
    u64 = None if jitter is None else _as_f64(jitter, dtype)
    if logits is None:
        logits = router_logits(xr, W_gate, logit_bias, dtype)
    r = route(np.asarray(logits, dtype=np.float32), k, noise=noise, temperature=temperature, soft=soft)
    l, idx, w = r["logits"], r["topk_idx"], r["topk_w"]
    C = expert_capacity(T, E, k, capacity_factor)
    counts, offsets, sorted_slot, slot_pos = permute(idx, E, C)
    dy64 = _as_f64(dy, dtype)
    kept = slot_pos.reshape(T, k) >= 0
    wk = w.astype(np.float64)
    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    want_dx = np.zeros(T, dtype=bool)
    want_dx[tok] = True
    want_e = set(range(E)) if experts is None else set(int(e) for e in experts)

    dx = np.zeros((T, h))
    dW1 = np.zeros((E, h, f))
    dW3 = np.zeros((E, h, f)) if act == "swiglu" else None
    dW2 = np.zeros((E, f, h))
    dw = np.zeros((T, k))
    sc = {}
    if with_scale:
        sc = dict(dx=np.zeros((T, h)), dW1=np.zeros((E, h, f)), dW2=np.zeros((E, f, h)),
                  dW3=np.zeros((E, h, f)) if act == "swiglu" else None)
        dw_m = np.zeros((T, k))
    for e in range(E):
        rows, slots = np.nonzero((idx == e) & kept)
        # the expert's forward for the rows whose dw is needed: every row when dW_gate (which
        # takes dl of every token) or this expert's weight gradients are asked for, else the
        # rows of the tokens whose dx is (dl of a token needs the dw of all its slots)
        fwd = np.ones(rows.shape, dtype=bool) if (e in want_e or with_w_gate) else want_dx[rows]
        rows, slots = rows[fwd], slots[fwd]
        if rows.size == 0:
            continue
        X = x64[rows]
        W1e = _as_f64(W1[e], dtype)
        W2e = _as_f64(W2[e], dtype)
        W3e = _as_f64(W3[e], dtype) if act == "swiglu" else None
        a = X @ W1e
        if act == "swiglu":
            g = X @ W3e
            hm = silu(a) * g
        else:
            g = None
            hm = gelu(a)
        hm_r = bf16_to_f64(round_to_bf16(hm)) if dtype == "bf16" else hm
        O = hm_r @ W2e
        dw[rows, slots] = np.sum(dy64[rows] * O, axis=1)
        if with_scale:
            dw_m[rows, slots] = np.sum(np.abs(dy64[rows]) * np.abs(O), axis=1)
        # the chain through the expert for every row of a wanted expert, else for the rows
        # of the tokens whose dx is asked for
        back = np.ones(rows.shape, dtype=bool) if e in want_e else want_dx[rows]
        if not back.any():
            continue
        rows, slots, X, a, hm_r = rows[back], slots[back], X[back], a[back], hm_r[back]
        g = None if g is None else g[back]
        dO = wk[rows, slots][:, None] * dy64[rows]
        dHm = dO @ W2e.T
        if act == "swiglu":
            da = dHm * g * silu_grad(a)
            dg = dHm * silu(a)
            dX = da @ W1e.T + dg @ W3e.T
        else:
            da = dHm * gelu_grad(a)
            dX = da @ W1e.T
        if e in want_e:
            dW2[e] = hm_r.T @ dO
            dW1[e] = X.T @ da
            if act == "swiglu":
                dW3[e] = X.T @ dg
        if with_scale:
            m = expert_grad_scale(X, dy64[rows], wk[rows, slots], a, g, hm_r, W1e, W3e, W2e, act)
            if e in want_e:
                sc["dW2"][e] = m["dW2"]
                sc["dW1"][e] = m["dW1"]
                if act == "swiglu":
                    sc["dW3"][e] = m["dW3"]
            np.add.at(sc["dx"], rows, m["dX"])
        np.add.at(dx, rows, dX)
    dl = router_logit_grad(l, idx, w, dw, counts, d_aux, k, temperature, soft)
    dxr = dl @ Wg.T
    dx += dxr if u64 is None else dxr * u64
    dWg = xr64.T @ dl if with_w_gate else None
    out = dict(dx=dx, dW_gate=dWg, dW1=dW1, dW3=dW3, dW2=dW2, dlogits=dl, dw=dw, topk_idx=idx, topk_w=w,
               counts=counts, slot_pos=slot_pos, logits=l)
    if with_scale:
        dl_m = router_logit_grad_scale(l, idx, w, dw_m, counts, d_aux, k, temperature, soft)
        dxr_m = dl_m @ np.abs(Wg).T
        sc["dx"] += dxr_m if u64 is None else dxr_m * np.abs(u64)
        sc["dW_gate"] = np.abs(xr64).T @ dl_m if with_w_gate else None
        out["scale"] = sc
    return out


# ----------------------------------------------------------------------------
# fixed-capacity ("binned") layout

def binned_capacity(T: int, E: int, k: int, capacity_factor: float, min_capacity: int, counts) -> int:
    """Bucket size C of the fixed-capacity layout.

    [MB] section 3: every expert gets C = capacity_factor * tokens * top_k / num_experts
    rows; section 4.2 truncates to int; section 4.6: a computed capacity of zero means
    "the largest expert count of this step" (nothing dropped, buckets padded to the worst
    case).  [CAI] SparseMLP parameters: a minimum capacity (router_min_capacity) applies
    on top of the formula.  Readings: the minimum is applied to the formula's value
    (cf > 0); a factor <= 0, or a capacity that is still zero, takes the largest count.
    """
    cf = float(np.float32(capacity_factor))
    if not math.isfinite(cf) or min_capacity < 0:
        raise ValueError("capacity factor must be finite, minimum capacity >= 0")
    cmax = int(max(np.asarray(counts).tolist() or [0]))
    if cf <= 0.0:
        return cmax
    C = max(int(math.floor(cf * ((k * T) / E))), int(min_capacity))
    return cmax if C == 0 else C


def binned_layout(topk_idx: np.ndarray, E: int, C: int):
    """The [E, C] buckets of the fixed-capacity layout, from the page's slot semantics.

    [MB] section 4.5: slot i of expert e holds the i-th assignment routed to e when e has
    more than i of them; otherwise it stays zero (padding); assignments past the C-th are
    not read by any slot (dropped).  Assignments are taken in ascending s = t*k + j (the
    stable order).  Returns ``bins[E, C]`` (assignment s, or -1 for padding) and
    ``slot_pos[T*k]`` (assignment -> bucket row e*C + i, or -1 if dropped).
    """
    flat = np.asarray(topk_idx).reshape(-1).tolist()
    bins = [[-1] * C for _ in range(E)]
    seen = [0] * E
    slot_pos = [-1] * len(flat)
    for s, e in enumerate(flat):
        i = seen[e]
        seen[e] += 1
        if i < C:
            bins[e][i] = s
            slot_pos[s] = e * C + i
    return np.asarray(bins, dtype=np.int32).reshape(E, C), np.asarray(slot_pos, dtype=np.int32)


def layer_forward_binned(x, W_gate, logit_bias, W1, W3, W2, *, k: int, capacity_factor: float,
                         min_capacity: int, act: str, dtype: str, logits=None, tokens=None) -> dict:
    """The layer with fixed-capacity buckets ([MB] sections 3 and 4.3: gather into
    [E, C, h], the expert MLPs on every bucket row, weighted scatter back; [CAI] SparseMLP
    data flow step 4).  Padding rows are zero and are never read back, so the output is
    the compact layer's output for the same capacity; the bucket tensor ``x_bins`` is
    returned as well (bf16 bit patterns or fp32, zero rows for padding)."""
    x = np.asarray(x)
    T = x.shape[0]
    E = np.asarray(W_gate).shape[1]
    if logits is None:
        logits = router_logits(x, W_gate, logit_bias, dtype)
    logits = np.asarray(logits, dtype=np.float32)
    idx = select_topk(logits, k)
    w = topk_weights(logits, idx)
    counts = histogram(idx, E)
    C = binned_capacity(T, E, k, capacity_factor, min_capacity, counts)
    bins, slot_pos = binned_layout(idx, E, C)
    x_bins = np.zeros((E, C) + x.shape[1:], dtype=x.dtype)
    for e in range(E):
        for i in range(C):
            if bins[e, i] >= 0:
                x_bins[e, i] = x[bins[e, i] // k]
    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    y64 = combine(x, idx, w, slot_pos, W1, W3, W2, act, dtype, tokens=tok)
    return dict(logits=logits, topk_idx=idx, topk_w=w, C=C, counts=counts, bins=bins, slot_pos=slot_pos,
                x_bins=x_bins, aux=aux_loss(counts, softmax(logits), T, k, E), y_tokens=tok, y64=y64,
                y=round_to_bf16(y64) if dtype == "bf16" else y64.astype(np.float32))
