"""Build ``libmoe_mi355x.so`` (all HIP sources, gfx950 only) in-tree with hipcc.

``python -m top_routing_expert_moe_amd.build`` compiles every time it is run.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmoe_mi355x.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed-fp32 VALU forms anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature name; that warning is harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
