"""The grouped GEMMs' workgroup schedule does not change their results.

The schedule has two knobs, environment variables read at each launch:
MOE_GEMM_ORDER picks which workgroup runs which tile, and MOE_GEMM_WORKGROUPS sets
the number of workgroups.  A bf16 GEMM launch of short tiles has at most one
workgroup per CU; each runs its share of the tile list in turn, and a tile followed by
one of the same shape copies that tile's first stages during its own last ones.  With
few workgroups every workgroup runs many tiles in a row,
so the hand-over between tiles (including the gathered activation rows of the up
projection) runs at every tile boundary.  Every tile's arithmetic is the same whoever
runs it, so the outputs must be bit-identical to the default schedule's, and they are
also checked against the oracle.
"""
import math
import os

import numpy as np
import pytest

import moe_workloads as mw
import oracle as o
import top_routing_expert_moe_amd as moe
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

ENV = "MOE_GEMM_WORKGROUPS"


def _say(*a):
    print(*a, flush=True)


class _Env:
    """Environment variable `var` set to n (None: unset) inside the block."""

    def __init__(self, var, n):
        self.var, self.n = var, n

    def __enter__(self):
        self.old = os.environ.get(self.var)
        if self.n is None:
            os.environ.pop(self.var, None)
        else:
            os.environ[self.var] = str(self.n)

    def __exit__(self, *exc):
        if self.old is None:
            os.environ.pop(self.var, None)
        else:
            os.environ[self.var] = self.old


def _Workgroups(n):
    """MOE_GEMM_WORKGROUPS set to n (None: unset) inside the block."""
    return _Env(ENV, n)


def _rand(shape, scale, rng, dtype):
    a = (rng.standard_normal(shape) * scale).astype(np.float32)
    return mw.f32_to_bf16_bits(a) if dtype == "bf16" else a


@pytest.mark.parametrize("act,E,h,f,seg", [
    ("swiglu", 8, 256, 512, [16, 0, 3, 40, 16, 1, 33, 17]),         # 32-row tiles, wide tiles
    ("gelu", 6, 512, 1024, [700, 20, 5, 300, 60, 0]),              # 256-, 128- and 32-row tiles in one launch
    ("swiglu", 5, 256, 1024, [0, 1, 300, 257, 37]),                # 128-row tiles, ragged segments
    ("swiglu", 4, 1024, 2048, [5, 20, 0, 9]),                      # 32-row tiles, K parts
    ("gelu", 3, 2048, 1024, [12, 3, 30]),                          # K parts in both projections
    ("swiglu", 4, 2048, 768, [200, 129, 0, 60]),                   # h >= 2048: 256-row tiles from 129 rows
    ("gelu", 4, 384, 768, [100, 90, 120, 70]),                     # 128-row tiles, stage counts 6 and 12:
                                                                   # multiples of their three buffers
])
@pytest.mark.parametrize("wgs", [8, 24])
def test_expert_ffn_schedule_invariant(act, E, h, f, seg, wgs):
    torch = gu.torch()
    _say(f"expert_ffn schedule {act} E={E} h={h} f={f} seg={seg} workgroups={wgs}")
    rng = np.random.default_rng(E * 11 + h + f)
    R = int(sum(seg))
    R_max = R + 5
    xp = _rand((R_max, h), 1.0, rng, "bf16")
    W1 = _rand((E, h, f), 1 / math.sqrt(h), rng, "bf16")
    W3 = _rand((E, h, f), 1 / math.sqrt(h), rng, "bf16") if act == "swiglu" else None
    W2 = _rand((E, f, h), 1 / math.sqrt(f), rng, "bf16")
    offsets = np.concatenate([[0], np.cumsum(seg)]).astype(np.int32)
    d = dict(x=gu.to_dev(xp, "bf16"), off=torch.from_numpy(offsets).to(gu.dev()), W1=gu.to_dev(W1, "bf16"),
             W3=None if W3 is None else gu.to_dev(W3, "bf16"), W2=gu.to_dev(W2, "bf16"))
    outs = []
    for n in (None, wgs):
        with _Workgroups(n):
            out = moe.expert_ffn(d["x"], d["off"], d["W1"], d["W3"], d["W2"], act,
                                 out=gu.sentinel_like((R_max, h), "bf16"))
            torch.cuda.synchronize()
        outs.append(gu.from_dev(out).copy())
    assert gu.is_sentinel(outs[1][R:], "bf16").all(), "rows past offsets[E] were written"
    assert np.array_equal(outs[0], outs[1]), "the schedule changed the result"
    got = gu.as_f64(outs[1][:R], "bf16")
    a64 = gu.as_f64(xp, "bf16")
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            ref = o.expert_ffn(a64[lo:hi], W1[e], None if W3 is None else W3[e], W2[e], act, "bf16")
            gu.check_bf16_out(got[lo:hi], ref, f"expert {e}")


@pytest.mark.parametrize("T,h,f,E,k,cf,act", [
    (1500, 256, 512, 8, 1, 0.0, "swiglu"),    # gathered up projection: 256- and 128-row tiles
    (2000, 192, 320, 16, 2, 0.0, "gelu"),     # N tails, mixed tile heights
    (3000, 128, 256, 64, 2, 1.25, "gelu"),    # many experts, capacity drops
    (40, 1024, 2048, 8, 2, 0.0, "swiglu"),    # wide tiles, K parts
    (1600, 384, 768, 16, 1, 0.0, "swiglu"),   # gathered 128-row tiles whose stage count (6) fills
                                              # the three buffers: handed over with their row indices
])
def test_layer_schedule_invariant(T, h, f, E, k, cf, act):
    torch = gu.torch()
    _say(f"layer schedule T={T} h={h} f={f} E={E} k={k} cf={cf} {act}")
    rng = np.random.default_rng(T + 3 * E)
    conv = mw.f32_to_bf16_bits
    bias = (0.7 * rng.standard_normal(E)).astype(np.float32)
    host = dict(x=conv(rng.standard_normal((T, h)).astype(np.float32)),
                W_gate=(rng.standard_normal((h, E)) / math.sqrt(h)).astype(np.float32), logit_bias=bias,
                W1=conv((rng.standard_normal((E, h, f)) / math.sqrt(h)).astype(np.float32)),
                W3=conv((rng.standard_normal((E, h, f)) / math.sqrt(h)).astype(np.float32)) if act == "swiglu" else None,
                W2=conv((rng.standard_normal((E, f, h)) / math.sqrt(f)).astype(np.float32)))
    dd = {kk: (None if v is None else gu.to_dev(v, "bf16" if kk in ("x", "W1", "W3", "W2") else "f32"))
          for kk, v in host.items()}
    outs = []
    for n in (None, 8):
        with _Workgroups(n):
            y, aux, counts = moe.layer_forward(dd["x"], dd["W_gate"], dd["logit_bias"], dd["W1"], dd["W3"], dd["W2"],
                                               k=k, capacity_factor=cf, act=act)
            torch.cuda.synchronize()
        outs.append((gu.from_dev(y).copy(), float(gu.from_dev(aux)), gu.from_dev(counts).copy()))
    assert np.array_equal(outs[0][0], outs[1][0]), "the schedule changed y"
    assert outs[0][1] == outs[1][1] and np.array_equal(outs[0][2], outs[1][2])
    logits, _, _, _ = moe.route(dd["x"], dd["W_gate"], dd["logit_bias"], k)
    torch.cuda.synchronize()
    tokens = np.sort(rng.choice(T, min(T, 200), replace=False))
    ref = o.layer_forward(host["x"], host["W_gate"], host["logit_bias"], host["W1"], host["W3"], host["W2"],
                          k=k, capacity_factor=cf, act=act, dtype="bf16", logits=gu.from_dev(logits), tokens=tokens)
    assert np.array_equal(outs[1][2], ref["counts"])
    gu.check_bf16_out(gu.as_f64(outs[1][0][tokens], "bf16"), ref["y64"], "y")


@pytest.mark.parametrize("act,E,h,f,seg", [
    ("swiglu", 4, 256, 512, [1100, 20, 700, 300]),                  # 256-row launches: 256-, 128- and
                                                                     # 32-row tiles, NT a multiple of 8
    ("gelu", 8, 512, 768, [104, 1300, 557, 0, 800, 734, 699, 134]),  # skewed, one expert empty, NT = 3 / 2
    ("swiglu", 16, 256, 256, [400] * 3 + [33] * 5 + [2000, 0, 257, 5, 1900, 128, 129, 700]),
    ("gelu", 6, 512, 1024, [700, 20, 5, 300, 60, 0]),               # 128-row launches
    ("swiglu", 3, 2048, 512, [12, 3, 30]),                           # K parts (down projection)
])
@pytest.mark.parametrize("order", [0, 1, 2])
@pytest.mark.parametrize("wgs", [None, 16])
def test_expert_ffn_tile_order_invariant(act, E, h, f, seg, order, wgs):
    """MOE_GEMM_ORDER picks which workgroup runs which tile (XCD ranges of the list, launch
    order, or n-tile ranges per XCD): the outputs are bit-identical to the default
    schedule's, with one workgroup per tile slot and with few workgroups running many
    tiles each."""
    torch = gu.torch()
    _say(f"expert_ffn tile order {order} {act} E={E} h={h} f={f} seg={seg} workgroups={wgs}")
    rng = np.random.default_rng(E * 7 + h + f)
    R = int(sum(seg))
    R_max = R + 3
    xp = _rand((R_max, h), 1.0, rng, "bf16")
    W1 = _rand((E, h, f), 1 / math.sqrt(h), rng, "bf16")
    W3 = _rand((E, h, f), 1 / math.sqrt(h), rng, "bf16") if act == "swiglu" else None
    W2 = _rand((E, f, h), 1 / math.sqrt(f), rng, "bf16")
    offsets = np.concatenate([[0], np.cumsum(seg)]).astype(np.int32)
    d = dict(x=gu.to_dev(xp, "bf16"), off=torch.from_numpy(offsets).to(gu.dev()), W1=gu.to_dev(W1, "bf16"),
             W3=None if W3 is None else gu.to_dev(W3, "bf16"), W2=gu.to_dev(W2, "bf16"))
    outs = []
    for ordr, n in ((None, None), (order, wgs)):
        with _Env("MOE_GEMM_ORDER", ordr), _Workgroups(n):
            out = moe.expert_ffn(d["x"], d["off"], d["W1"], d["W3"], d["W2"], act,
                                 out=gu.sentinel_like((R_max, h), "bf16"))
            torch.cuda.synchronize()
        outs.append(gu.from_dev(out).copy())
    assert gu.is_sentinel(outs[1][R:], "bf16").all(), "rows past offsets[E] were written"
    assert np.array_equal(outs[0], outs[1]), "the tile order changed the result"
    got = gu.as_f64(outs[1][:R], "bf16")
    a64 = gu.as_f64(xp, "bf16")
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            ref = o.expert_ffn(a64[lo:hi], W1[e], None if W3 is None else W3[e], W2[e], act, "bf16")
            gu.check_bf16_out(got[lo:hi], ref, f"expert {e}")
