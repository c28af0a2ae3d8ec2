"""Build ``libmoe_route.so`` (the gfx950 HIP library) and ``libmoe_probe.so``
(bandwidth probes for the benchmark) in-tree with hipcc.

    python -m permutation_group_limited_amd.build

Flags: gfx950 only, -O3, no FP contraction (every fused multiply-add in the
kernels is an explicit fmaf), packed-fp32 instruction selection disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmoe_route.so")
# bandwidth probes timed by the benchmark beside the routing path
PROBE_LIB = os.path.join(HERE, "libmoe_probe.so")
PROBE_SOURCES = ["probe.hip"]
SOURCES = ["api.hip", "router.hip", "indices.hip", "finalize.hip", "route_index.hip",
           "route_index_f32.hip", "route_index_bf16.hip", "route_index_f16.hip",
           "no_alloc.hip", "plan.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature and says so
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (r.stderr or "").splitlines()
            if noise not in l and "(ignoring feature)" not in l]
    return r.returncode, msgs


def _compile_all(jobs_list, verbose):
    jobs = max(1, min(len(jobs_list), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda c: _run(c[0], verbose), jobs_list))
    for (rc, msgs), (_, src) in zip(results, jobs_list):
        if rc != 0:
            sys.stderr.write("\n".join(msgs) + "\n")
            raise RuntimeError("hipcc failed compiling %s" % src)
        if verbose and msgs:
            sys.stderr.write("\n".join(msgs) + "\n")


def _link(objs, lib, verbose):
    tmp = lib + ".tmp%d" % os.getpid()
    rc, msgs = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp],
                    verbose)
    if rc != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError("hipcc failed linking %s" % lib)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link the routing
    library and the probe library."""
    tmpdir = tempfile.mkdtemp(prefix="moe_build_")
    try:
        groups = [(LIB, SOURCES), (PROBE_LIB, PROBE_SOURCES)]
        jobs, objs = [], {}
        for lib, srcs in groups:
            objs[lib] = []
            for s in srcs:
                o = os.path.join(tmpdir, s.replace(".hip", ".o"))
                objs[lib].append(o)
                jobs.append(([HIPCC] + FLAGS + ["-I", INCLUDE, "-I", CSRC, "-c",
                                                os.path.join(CSRC, s), "-o", o], s))
        _compile_all(jobs, verbose)
        for lib, _ in groups:
            _link(objs[lib], lib, verbose)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
