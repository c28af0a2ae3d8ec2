"""Build ``libmoe_route.so`` (the gfx950 HIP library) in-tree with hipcc.

    python -m permutation_group_limited_amd.build

Flags: gfx950 only, -O3, no FP contraction (every fused multiply-add in the
kernels is an explicit fmaf), packed-fp32 instruction selection disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmoe_route.so")
SOURCES = ["api.hip", "router.hip", "indices.hip", "finalize.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-I", INCLUDE, "-I", CSRC] + \
        [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature and says so
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (r.stderr or "").splitlines() if noise not in l and "(ignoring feature)" not in l]
    if r.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError("hipcc failed building %s" % LIB)
    if verbose and msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
