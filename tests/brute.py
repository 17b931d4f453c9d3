"""Brute-force MoE layer forward in pure Python (math module only), for tiny inputs.

An independent second reading of the layer, written with different means than
the oracle: Python loops, ``math.fsum`` for exactly rounded dot products,
Python's stable ``sorted`` for the ranking and for the sort by expert id.  It
pins the oracle (the oracle must agree with it) and shares no code with it.
"""
from __future__ import annotations

import math
import struct


def f32(v: float) -> float:
    """Round a Python float to the nearest fp32 value."""
    return struct.unpack("<f", struct.pack("<f", v))[0]


def bf16(v: float) -> float:
    """Round to the nearest bf16 value, ties to even, by brute search over the two
    neighbouring bf16 values (bit patterns of the fp32 truncation and the next one)."""
    if v == 0.0:
        return v
    lo_bits = struct.unpack("<I", struct.pack("<f", v))[0] & 0xFFFF0000
    lo = struct.unpack("<f", struct.pack("<I", lo_bits))[0]
    # the fp32 truncation may be above |v| after fp32 rounding of v; step down if so
    cands = []
    for b in (lo_bits - 0x10000, lo_bits, lo_bits + 0x10000):
        if 0 <= b <= 0xFFFFFFFF:
            c = struct.unpack("<f", struct.pack("<I", b))[0]
            if math.isfinite(c):
                cands.append((abs(c - v), (b >> 16) & 1, c))
    cands.sort(key=lambda t: (t[0], t[1]))  # nearest; on a tie the even pattern
    return cands[0][2]


def layer(x, W_gate, bias, W1, W3, W2, k, cf, act, dtype):
    """Everything as nested Python lists / floats.  Returns a dict like the oracle's."""
    T, h = len(x), len(x[0])
    E = len(W_gate[0])
    f = len(W1[0][0])
    logits = [[f32(math.fsum([x[t][i] * W_gate[i][e] for i in range(h)] + ([bias[e]] if bias else [])))
               for e in range(E)] for t in range(T)]
    probs = []
    idx = []
    wts = []
    for t in range(T):
        m = max(logits[t])
        ex = [math.exp(l - m) for l in logits[t]]
        s = math.fsum(ex)
        p = [v / s for v in ex]
        probs.append(p)
        order = sorted(range(E), key=lambda e: (-logits[t][e], e))[:k]
        idx.append(order)
        ps = math.fsum(p[e] for e in order)
        wts.append([f32(p[e] / ps) for e in order])
    # capacity
    if cf <= 0:
        C = None
    else:
        C = int(math.floor(f32(cf) * (k * T / E)))
        C = None if C == 0 else C
    flat = [idx[t][j] for t in range(T) for j in range(k)]
    counts = [flat.count(e) for e in range(E)]
    order = sorted(range(T * k), key=flat.__getitem__)  # Python's sort is stable
    kept_rows = []
    for e in range(E):
        rows = [s for s in order if flat[s] == e]
        kept_rows.append(rows if C is None else rows[:C])
    offsets = [0]
    for e in range(E):
        offsets.append(offsets[-1] + len(kept_rows[e]))
    sorted_slot = [s for e in range(E) for s in kept_rows[e]]
    slot_pos = [-1] * (T * k)
    for r, s in enumerate(sorted_slot):
        slot_pos[s] = r

    def ffn(e, a):
        z1 = [math.fsum(a[i] * W1[e][i][c] for i in range(h)) for c in range(f)]
        if act == "swiglu":
            z3 = [math.fsum(a[i] * W3[e][i][c] for i in range(h)) for c in range(f)]
            hm = [z1[c] / (1.0 + math.exp(-z1[c])) * z3[c] for c in range(f)]
        else:
            hm = [0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in z1]
        if dtype == "bf16":
            hm = [bf16(v) for v in hm]
        return [math.fsum(hm[c] * W2[e][c][o] for c in range(f)) for o in range(h)]

    y = []
    for t in range(T):
        acc = [0.0] * h
        for j in range(k):
            if slot_pos[t * k + j] < 0:
                continue
            out = ffn(idx[t][j], x[t])
            acc = [acc[o] + wts[t][j] * out[o] for o in range(h)]
        y.append(acc)
    aux = E * math.fsum((counts[e] / (T * k)) * (math.fsum(probs[t][e] for t in range(T)) / T)
                        for e in range(E))
    return dict(logits=logits, topk_idx=idx, topk_w=wts, C=C, counts=counts, offsets=offsets,
                sorted_slot=sorted_slot, slot_pos=slot_pos, y64=y, aux=aux)
