"""Benchmark of the routing path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dsv3]

One step = one pass of the whole path over one batch: router and index
creation through moe_route_and_index (two kernels: the router, which also
fills the index step's per-chunk histogram, then the scatter), then
moe_finalize, all through the C ABI on torch's current stream, with every
input already resident in HBM. W untimed steps, then K timed steps between
a synchronize and HIP events; prints ONE JSON line.

Headline workload: DeepSeek-V3-shaped, T=8192 tokens, E=256 experts in 8
groups (4 kept), K=8, hidden 7168, bf16 expert outputs and output. One
routed token-slot is one (token, k) pair, i.e. one row of `down`.

Reported beside the throughput:
  * per-stage mean durations: each entry point (router, create_indices,
    route_and_index, finalize) K times back to back on the launch stream
    between two HIP events;
  * roofline of the dominant kernel (finalize): algorithmic bytes per launch
    (T*K*H*2 read + T*K*(4+4) restore and weights + T*H*2 written) divided by
    its mean duration above, against 8 TB/s; plus the HBM bytes measured by
    rocprofv3 counters when the committed counter summary matches the
    current kernel source;
  * protocol: the step and each stage captured in HIP graphs, replayed with
    a cold cache (1 GiB written before each replay, outside the events) and
    warm, median / minimum; a 1 GiB device-copy bandwidth probe;
  * cpu_baseline: the CPU oracle (plain C, OpenMP over tokens) timed on the
    host cores over whole steps of the same workload, per stage on all
    threads and on one thread, and a parity check of the GPU step against
    it.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time
from dataclasses import replace

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, vendor figure
COUNTER_FILE = os.path.join(ROOT, "profiles", "finalize_dsv3_counters.txt")
FINALIZE_SOURCES = [os.path.join(ROOT, "permutation_group_limited_amd", "csrc", f)
                    for f in ("finalize.hip", "common.hpp")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="approximate CPU time for the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the side measurements (logits router, decode latency)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="after the run, copy BYTES with torch's plain copy kernel (3 times): "
                         "the reference dispatch for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE")
    return ap.parse_args()


def finalize_source_hash() -> str:
    """sha256 of the finalize kernel's sources with comments and layout
    removed: any change to the code itself changes it, an edited comment
    does not."""
    h = hashlib.sha256()
    for p in FINALIZE_SOURCES:
        with open(p) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()


def counter_traffic():
    """HBM bytes per finalize launch from the committed rocprofv3 counter
    summary, or None if it is missing or was taken on other kernel source."""
    try:
        with open(COUNTER_FILE) as f:
            kv = dict(l.split(":", 1) for l in f if ":" in l and not l.startswith("#"))
        kv = {k.strip(): v.strip() for k, v in kv.items()}
        if kv.get("kernel_source_sha256") != finalize_source_hash():
            return None
        return int(float(kv["hbm_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the routing path "
              "shards by token with no exchange; run one process per GPU). --gpus %d refused."
              % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from permutation_group_limited_amd import binding
    from permutation_group_limited_amd import workloads as wl

    binding.load_library()  # raises if the HIP library is not built
    wk = wl.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    T, E, K, H = wk.T, wk.E, wk.K, wk.H
    N = T * K
    db = 2 if wk.down_dtype == torch.bfloat16 else 4
    ob = 2 if wk.out_dtype == torch.bfloat16 else 4

    scores_h, bias_h = wl.make_scores(wk), wl.make_bias(wk)
    scores, bias = scores_h.to(dev), bias_h.to(dev)
    down = wl.make_down(wk, device=dev)
    idx = torch.empty(T, K, dtype=torch.int32, device=dev)
    wts = torch.empty(T, K, dtype=torch.float32, device=dev)
    order = torch.empty(N, dtype=torch.int32, device=dev)
    restore = torch.empty(N, dtype=torch.int32, device=dev)
    starts = torch.empty(E + 1, dtype=torch.int32, device=dev)
    eids = torch.empty(E, dtype=torch.int32, device=dev)
    stats = torch.empty(2, dtype=torch.int32, device=dev)
    ws = torch.empty(max(binding.moe_create_indices_workspace_size(N, E), 4) // 4,
                     dtype=torch.int32, device=dev)
    # moe_route_and_index's workspace: zero once here, left zero by every call
    ws_ri = torch.zeros(binding.moe_route_and_index_workspace_size(T, K, E) // 4,
                        dtype=torch.int32, device=dev)
    out = torch.empty(T, H, dtype=wk.out_dtype, device=dev)

    def router():
        binding.moe_router_group_limited(idx, wts, scores, bias, wk.n_groups, wk.topk_group,
                                         wk.norm_weights, wk.scale)

    def indices():
        binding.moe_create_indices(order, starts, restore, eids, stats, idx, ws)

    def route_and_index():
        binding.moe_route_and_index(idx, wts, order, starts, restore, eids, stats, scores, bias,
                                    ws_ri, wk.n_groups, wk.topk_group, wk.norm_weights, wk.scale)

    def finalize():
        binding.moe_finalize(out, down, restore, wts)

    # One step = the whole path on one batch: router and index creation
    # through moe_route_and_index (the router also fills the index step's
    # histogram), then finalize. The separate entry points are timed below.
    def step():
        route_and_index()
        finalize()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region 1 (headline): K back-to-back steps between two events
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t_start.record()
    for _ in range(args.steps):
        step()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    elapsed_ms = t_start.elapsed_time(t_end)
    ms_per_step = elapsed_ms / args.steps

    # timed region 2: each stage K times back to back on the launch stream
    # (every stage is idempotent on its inputs), bracketed by events, for
    # per-stage mean durations; finalize's is the roofline's denominator
    for f in (router, indices, route_and_index, finalize):  # first launches load code
        for _ in range(2):
            f()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(args.steps):
        router()
    ev[1].record()
    for _ in range(args.steps):
        indices()
    ev[2].record()
    for _ in range(args.steps):
        route_and_index()
    ev[3].record()
    for _ in range(args.steps):
        finalize()
    ev[4].record()
    torch.cuda.synchronize()
    stage_ms = {name: ev[j].elapsed_time(ev[j + 1]) / args.steps
                for j, name in enumerate(("router", "create_indices", "route_and_index",
                                          "finalize"))}
    fin_avg_ms = stage_ms["finalize"]

    bytes_router = T * E * 4 + E * 4 + N * (4 + 4)
    bytes_indices = N * 4 + 2 * N * 4 + (2 * E + 1) * 4 + 8
    bytes_finalize = N * H * db + N * (4 + 4) + T * H * ob
    bytes_total = bytes_router + bytes_indices + bytes_finalize
    step_s = ms_per_step * 1e-3
    fin_gbps = bytes_finalize / (fin_avg_ms * 1e-3) / 1e9
    traffic = counter_traffic()

    result = {
        "metric": "routed token-slots/s + HBM GB/s (% of peak), DSv3 shape T=8192 E=256 K=8",
        "value": N / step_s,
        "unit": "token-slots/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; sigmoid/softmax scores, N(0,1) expert outputs)",
        "config": {"workload": wk.describe(), "tokens": T, "experts": E, "n_groups": wk.n_groups,
                   "topk_group": wk.topk_group, "top_k": K, "hidden": H,
                   "storage": "bf16" if db == 2 else "f32", "accumulate": "f32"},
        "hbm_gbps": bytes_total / step_s / 1e9,
        "hbm_pct_of_peak": 100.0 * bytes_total / step_s / 1e9 / PEAK_HBM_GBPS,
        "algorithmic_bytes_per_step": bytes_total,
        "stage_bytes": {"router": bytes_router, "create_indices": bytes_indices,
                        "finalize": bytes_finalize},
        "step": "moe_route_and_index (router filling the index histogram, then the scatter) "
                "+ moe_finalize: 3 kernels",
        "stage_ms": stage_ms,
        "wall_s": wall,
        "roofline": {"kernel": "finalize_kernel", "bound": "hbm", "achieved": fin_gbps,
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": fin_gbps / PEAK_HBM_GBPS,
                     "traffic": traffic},
    }

    if not args.no_extras:
        # 100 replays per setting (20 for the multi-GB Skewed workload)
        result["protocol"] = timing_protocol(
            step, {"router": router, "create_indices": indices,
                   "route_and_index": route_and_index, "finalize": finalize},
            replays=20 if wk.T * wk.K * wk.H > (1 << 31) else 100)
        result["extras"] = extras(wk, scores_h, bias_h, idx, wts, args.steps)
        result["extras"]["two_batches_in_flight"] = two_batches_in_flight(
            wk, scores, bias, down, args.steps)
        result["extras"]["finalize_rotating_outputs"] = finalize_rotating_outputs(
            wk, down, restore, wts, bytes_finalize, args.steps)

    if args.copy_probe > 0:
        src = torch.ones(args.copy_probe // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_probe_bytes"] = args.copy_probe
        del src, dst

    if not args.no_cpu_baseline:
        result["cpu_baseline"], result["parity"] = cpu_leg(
            wk, scores_h, bias_h, down, idx, wts, order, restore, starts, eids, stats, out,
            args.cpu_seconds)
    print(json.dumps(result), flush=True)


def graph_replay_us(fn, per_graph=20, reps=50):
    """Mean GPU time of one fn() call: per_graph calls captured back to back
    in one HIP graph, the graph replayed reps times (a graph of one call
    would mostly time the graph launch itself)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            fn()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (reps * per_graph) * 1e3


def extras(wk, scores_h, bias_h, idx, wts, steps):
    """Side measurements of the widened entry points:
      * the router on logits (sigmoid computed in the kernel) against the
        router on precomputed scores, same workload, K back-to-back launches;
      * router + index creation through the two entry points against
        moe_route_and_index (router filling the index histogram), same
        workload;
      * the decode-shaped workload (T=128, and T=16, which
        moe_route_and_index routes in one launch): whole steps captured 20
        to a HIP graph (decode_latency; eager launches would measure the
        host, not the GPU)."""
    import torch

    from permutation_group_limited_amd import binding
    from permutation_group_limited_amd import workloads as wl

    dev = torch.device("cuda:0")
    res = {}
    fn = binding.SCORE_SIGMOID if wk.score_fn == "sigmoid" else binding.SCORE_SOFTMAX
    logits = wl.make_logits(wk).to(dev)
    bias = bias_h.to(dev)

    def run(f):
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            f()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    res["router_logits_ms"] = run(lambda: binding.moe_router_group_limited_logits(
        idx, wts, logits, bias, fn, wk.n_groups, wk.topk_group, wk.norm_weights, wk.scale))
    scores = scores_h.to(dev)
    res["router_scores_ms"] = run(lambda: binding.moe_router_group_limited(
        idx, wts, scores, bias, wk.n_groups, wk.topk_group, wk.norm_weights, wk.scale))

    # router + index creation: two entry points vs moe_route_and_index
    T, E, K = wk.T, wk.E, wk.K
    o1, r1 = (torch.empty(T * K, dtype=torch.int32, device=dev) for _ in range(2))
    st1 = torch.empty(E + 1, dtype=torch.int32, device=dev)
    e1 = torch.empty(E, dtype=torch.int32, device=dev)
    u1 = torch.empty(2, dtype=torch.int32, device=dev)
    ws1 = torch.empty(max(binding.moe_create_indices_workspace_size(T * K, E), 4) // 4,
                      dtype=torch.int32, device=dev)
    tk1 = torch.zeros(binding.moe_route_and_index_workspace_size(T, K, E) // 4,
                      dtype=torch.int32, device=dev)

    def route_then_index():
        binding.moe_router_group_limited(idx, wts, scores, bias, wk.n_groups, wk.topk_group,
                                         wk.norm_weights, wk.scale)
        binding.moe_create_indices(o1, st1, r1, e1, u1, idx, ws1)

    res["route_then_index_ms"] = run(route_then_index)
    res["route_and_index_ms"] = run(lambda: binding.moe_route_and_index(
        idx, wts, o1, st1, r1, e1, u1, scores, bias, tk1, wk.n_groups, wk.topk_group,
        wk.norm_weights, wk.scale))

    dk = wl.WORKLOADS["decode"]
    res["decode"] = decode_latency(dk)
    # a batch small enough for moe_route_and_index's one-launch form
    res["decode_t16"] = decode_latency(replace(dk, T=16))
    return res


def decode_latency(dk):
    """Decode-sized steps (router -> create_indices -> finalize) captured 20
    to a HIP graph: mean GPU time per step through the separate entry points
    and with moe_route_and_index, and router + index creation alone both
    ways."""
    import torch

    from permutation_group_limited_amd import binding
    from permutation_group_limited_amd import workloads as wl

    dev = torch.device("cuda:0")
    T, E, K = dk.T, dk.E, dk.K
    s = wl.make_scores(dk).to(dev)
    b = wl.make_bias(dk).to(dev)
    down = wl.make_down(dk, device=dev)
    i2 = torch.empty(T, K, dtype=torch.int32, device=dev)
    w2 = torch.empty(T, K, dtype=torch.float32, device=dev)
    o2, r2 = (torch.empty(T * K, dtype=torch.int32, device=dev) for _ in range(2))
    st2 = torch.empty(E + 1, dtype=torch.int32, device=dev)
    e2 = torch.empty(E, dtype=torch.int32, device=dev)
    u2 = torch.empty(2, dtype=torch.int32, device=dev)
    ws2 = torch.empty(max(binding.moe_create_indices_workspace_size(T * K, E), 4) // 4,
                      dtype=torch.int32, device=dev)
    out2 = torch.empty(T, dk.H, dtype=dk.out_dtype, device=dev)

    def decode_step():
        binding.moe_router_group_limited(i2, w2, s, b, dk.n_groups, dk.topk_group,
                                         dk.norm_weights, dk.scale)
        binding.moe_create_indices(o2, st2, r2, e2, u2, i2, ws2)
        binding.moe_finalize(out2, down, r2, w2)

    us = graph_replay_us(decode_step)
    tk = torch.zeros(binding.moe_route_and_index_workspace_size(T, K, E) // 4,
                     dtype=torch.int32, device=dev)

    def decode_step_fused():
        binding.moe_route_and_index(i2, w2, o2, st2, r2, e2, u2, s, b, tk, dk.n_groups,
                                    dk.topk_group, dk.norm_weights, dk.scale)
        binding.moe_finalize(out2, down, r2, w2)

    us_fused = graph_replay_us(decode_step_fused)
    us_ri_sep = graph_replay_us(lambda: (
        binding.moe_router_group_limited(i2, w2, s, b, dk.n_groups, dk.topk_group,
                                         dk.norm_weights, dk.scale),
        binding.moe_create_indices(o2, st2, r2, e2, u2, i2, ws2)))
    us_ri_fused = graph_replay_us(lambda: binding.moe_route_and_index(
        i2, w2, o2, st2, r2, e2, u2, s, b, tk, dk.n_groups, dk.topk_group, dk.norm_weights,
        dk.scale))
    db = T * E * 4 + E * 4 + T * K * 8 + T * K * 12 + (2 * E + 1) * 4 + 8 + \
        T * K * dk.H * 2 + T * K * 8 + T * dk.H * 2
    return {"workload": dk.describe(), "us_per_step_graph": us,
            "us_per_step_graph_fused": us_fused,
            "us_route_index_graph": us_ri_sep,
            "us_route_index_graph_fused": us_ri_fused,
            "token_slots_per_s": T * K / (us * 1e-6),
            "token_slots_per_s_fused": T * K / (us_fused * 1e-6),
            "hbm_gbps": db / (us * 1e-6) / 1e9}


def finalize_rotating_outputs(wk, down, restore, wts, bytes_finalize, steps, n_out=8):
    """finalize writing a different output buffer on each call (n_out of
    them, used in turn), so that no output row is still held in the
    memory-side cache from the call before, as it is when one output
    buffer is rewritten back to back: mean time per call and the
    algorithmic bandwidth, against 8 TB/s."""
    import torch

    from permutation_group_limited_amd import binding

    outs = [torch.empty(wk.T, wk.H, dtype=wk.out_dtype, device="cuda:0") for _ in range(n_out)]
    for o in outs:
        binding.moe_finalize(o, down, restore, wts)
    torch.cuda.synchronize()
    n = max(n_out, (steps // n_out) * n_out)
    a = torch.cuda.Event(enable_timing=True)
    z = torch.cuda.Event(enable_timing=True)
    a.record()
    for k in range(n):
        binding.moe_finalize(outs[k % n_out], down, restore, wts)
    z.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(z) / n * 1e3
    gbps = bytes_finalize / (us * 1e-6) / 1e9
    return {"buffers": n_out, "us_per_call": us, "achieved_gbps": gbps,
            "frac": gbps / PEAK_HBM_GBPS}


def two_batches_in_flight(wk, scores, bias, down, steps):
    """Throughput with two batches in flight, as micro-batch overlap in
    serving runs them: the same step on two sets of output buffers on two
    streams, alternating, so that one batch's routing and index creation
    (latency-bound, few waves) runs beside the other batch's finalize
    (HBM-bound). Every step is still the whole path on one batch; the
    steps of one buffer set stay in order on its stream. Mean GPU time per
    step over `steps` steps, and whether both sets end with the
    single-stream output."""
    import torch

    from permutation_group_limited_amd import binding

    dev = torch.device("cuda:0")
    T, E, K, H = wk.T, wk.E, wk.K, wk.H
    N = T * K

    def buffers():
        i32 = lambda *shape: torch.empty(shape, dtype=torch.int32, device=dev)  # noqa: E731
        return {"idx": i32(T, K), "w": torch.empty(T, K, device=dev), "order": i32(N),
                "restore": i32(N), "starts": i32(E + 1), "eids": i32(E), "stats": i32(2),
                "ws": torch.zeros(binding.moe_route_and_index_workspace_size(T, K, E) // 4,
                                  dtype=torch.int32, device=dev),
                "out": torch.empty(T, H, dtype=wk.out_dtype, device=dev)}

    sets = [buffers(), buffers()]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority

    def step(b, st):
        binding.moe_route_and_index(b["idx"], b["w"], b["order"], b["starts"], b["restore"],
                                    b["eids"], b["stats"], scores, bias, b["ws"], wk.n_groups,
                                    wk.topk_group, wk.norm_weights, wk.scale, stream=st)
        binding.moe_finalize(b["out"], down, b["restore"], b["w"], stream=st)

    def run(n, two):
        cur = torch.cuda.current_stream()
        a = torch.cuda.Event(enable_timing=True)
        z = torch.cuda.Event(enable_timing=True)
        a.record(cur)
        for st in streams:
            st.wait_event(a)
        for k in range(n):
            j = k % 2 if two else 0
            step(sets[j], streams[j])
        for st in streams:
            cur.wait_stream(st)
        z.record(cur)
        torch.cuda.synchronize()
        return a.elapsed_time(z) / n * 1e3

    run(4, False)
    single = run(steps, False)
    ref = sets[0]["out"].clone()
    run(4, True)
    two = run(steps, True)
    same = all(torch.equal(b["out"].view(torch.int16), ref.view(torch.int16)) for b in sets)
    return {"us_per_step_one_stream": single, "us_per_step_two_streams": two,
            "token_slots_per_s_two_streams": N / (two * 1e-6), "outputs_equal": bool(same)}


def timing_protocol(step, stages, flush_bytes=1 << 30, replays=100):
    """The step and each stage captured in HIP graphs and replayed (one step
    per graph, and 20 steps per graph for the GPU time per step with the
    graph launch amortised): `replays` times with a cold cache (a read of
    flush_bytes from a scratch buffer before each replay, outside the timed
    events: more than the 256 MB memory-side cache and the L2s together; a
    read, so that no write-back of the flush itself overlaps the replay)
    and as many times warm; median
    and minimum in microseconds. Also a plain device copy of flush_bytes as
    the achievable-bandwidth probe (read + write bytes / time)."""
    import torch
    scratch = torch.ones(flush_bytes // 8, dtype=torch.int64, device="cuda:0")
    sink = torch.empty((), dtype=torch.int64, device="cuda:0")

    def capture(fn):
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            fn()
        torch.cuda.current_stream().wait_stream(st)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        for _ in range(5):
            g.replay()
        torch.cuda.synchronize()
        return g

    def replay_times(g, cold):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(replays)]
        for a, b in evs:
            if cold:
                torch.sum(scratch, dim=0, out=sink)
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        us = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
        return {"median_us": us[len(us) // 2], "min_us": us[0], "replays": replays}

    res = {}
    g = capture(step)
    res["step_graph_cold"] = replay_times(g, True)
    res["step_graph_warm"] = replay_times(g, False)
    # 20 steps per graph: the graph launch amortised, GPU time per step
    many = 20

    def steps():
        for _ in range(many):
            step()

    g20 = capture(steps)
    w20 = replay_times(g20, False)
    res["steps_per_graph_20_warm_us_per_step"] = {"median": w20["median_us"] / many,
                                                   "min": w20["min_us"] / many}
    res["stage_graph_cold_median_us"] = {
        name: replay_times(capture(fn), True)["median_us"] for name, fn in stages.items()}
    dst = torch.empty_like(scratch)
    dst.copy_(scratch)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(5):
        dst.copy_(scratch)
    b.record()
    torch.cuda.synchronize()
    res["copy_probe_gbps"] = 2 * flush_bytes * 5 / (a.elapsed_time(b) * 1e-3) / 1e9
    del scratch, dst
    return res


def cpu_leg(wk, scores_h, bias_h, down, idx, wts, order, restore, starts, eids, stats, out,
            budget_s):
    """Time the CPU oracle over whole steps of the same workload and check the
    GPU step against it."""
    import numpy as np
    import torch

    import oracle

    T, E, K = wk.T, wk.E, wk.K
    N = T * K
    s = scores_h.numpy()
    b = bias_h.numpy()
    if wk.down_dtype == torch.bfloat16:
        d = down.cpu().view(torch.int16).numpy().view(np.uint16)
        dcode = oracle.BF16
    else:
        d = down.cpu().numpy()
        dcode = oracle.F32
    ocode = oracle.BF16 if wk.out_dtype == torch.bfloat16 else oracle.F32

    def oracle_step():
        oi, ow = oracle.router(s, b, K, wk.n_groups, wk.topk_group, wk.norm_weights, wk.scale)
        ind = oracle.create_indices(oi, E)
        o = oracle.finalize(d, dcode, ind["restore_token_order"], ow, oracle.F32, ocode)
        return oi, ow, ind, o

    steps = 0
    t0 = time.perf_counter()
    res = None
    while True:
        res = oracle_step()
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or steps >= 200:
            break
    oi, ow, ind, o = res
    baseline = {"value": N * steps / el, "unit": "token-slots/s", "cores": oracle.num_threads(),
                "kind": "oracle",
                "sample": "%d whole steps of the %s workload (router + create_indices + "
                          "finalize), %.1f s" % (steps, wk.name, el)}

    # per stage, once each, on all threads and on one thread
    def stage_times():
        t = {}
        a = time.perf_counter()
        r_i, r_w = oracle.router(s, b, K, wk.n_groups, wk.topk_group, wk.norm_weights, wk.scale)
        t["router"] = time.perf_counter() - a
        a = time.perf_counter()
        r_ind = oracle.create_indices(r_i, E)
        t["create_indices"] = time.perf_counter() - a
        a = time.perf_counter()
        oracle.finalize(d, dcode, r_ind["restore_token_order"], r_w, oracle.F32, ocode)
        t["finalize"] = time.perf_counter() - a
        return {k: v * 1e3 for k, v in t.items()}

    threads = oracle.num_threads()
    baseline["stage_ms"] = stage_times()
    oracle.set_num_threads(1)
    try:
        baseline["single_thread_stage_ms"] = stage_times()
    finally:
        oracle.set_num_threads(threads)

    u32 = lambda t: t.cpu().numpy().view(np.uint32)
    gi = idx.cpu().numpy()
    gw = wts.cpu().numpy()
    parity = {
        "router_indices": bool(np.array_equal(gi, oi)),
        "router_weights": bool(np.array_equal(gw.view(np.uint32), ow.view(np.uint32))),
        "create_indices": bool(np.array_equal(u32(order), ind["token_expert_order"]) and
                               np.array_equal(u32(restore), ind["restore_token_order"]) and
                               np.array_equal(u32(starts), ind["expert_start_indices"]) and
                               np.array_equal(eids.cpu().numpy(), ind["expert_ids"]) and
                               np.array_equal(u32(stats), ind["expert_usage_stats"])),
    }
    # finalize ran on the GPU's own weights, equal to the oracle's bit for
    # bit: every output within 1 bf16 ulp
    if ocode == oracle.BF16:
        gb = out.cpu().view(torch.int16).numpy().view(np.uint16)
        ordg = np.where(gb & 0x8000, -(gb.astype(np.int64) & 0x7FFF), gb & 0x7FFF)
        orde = np.where(o & 0x8000, -(o.astype(np.int64) & 0x7FFF), o & 0x7FFF)
        ulp = np.abs(ordg - orde)
        parity["finalize_max_ulp"] = int(ulp.max(initial=0))
        parity["finalize"] = bool(ulp.max(initial=0) <= 1)
    else:
        parity["finalize"] = bool(np.allclose(out.cpu().numpy(), o, rtol=1e-5, atol=1e-6))
    return baseline, parity


if __name__ == "__main__":
    main()
