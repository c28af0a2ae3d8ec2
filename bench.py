"""Benchmark of the routing path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dsv3]

One step = one pass of the whole path over one batch: router and index
creation through moe_route_and_index, then moe_finalize, all through the C
ABI on torch's current stream, with every input already resident in HBM.
Each step writes its output into the next of 8 output buffers in turn, so
that no output row is still held in the 256 MB memory-side cache from the
step before (a layer that rewrote one buffer back to back would be
flattered by that cache). W untimed steps, then K timed steps between a
synchronize and HIP events; prints ONE JSON line.

Headline workload: DeepSeek-V3-shaped, T=8192 tokens, E=256 experts in 8
groups (4 kept), K=8, hidden 7168, bf16 expert outputs and output. One
routed token-slot is one (token, k) pair, i.e. one row of `down`.

Reported beside the throughput:
  * per-stage mean durations: each entry point (router, create_indices,
    route_and_index, finalize) K times back to back on the launch stream
    between two HIP events (finalize with rotating outputs);
  * roofline of the dominant kernel (finalize): algorithmic bytes per launch
    (T*K*H*2 read + T*K*(4+4) restore and weights + T*H*2 written) divided
    by its mean duration above, against 8 TB/s; plus the HBM bytes measured
    by rocprofv3 counters when the committed counter summary matches the
    current kernel source;
  * protocol: the step and each stage captured in HIP graphs (one per
    output buffer, replayed in turn), replayed with a cold cache (1 GiB
    written before each replay, outside the events; a 1 GiB read instead
    reported beside it) and warm, median / minimum;
  * extras.configs: all five workloads (tiny, mixtral, dsv3, decode, skewed)
    with 20 steps per HIP graph: GPU time per step, per stage, algorithmic
    bandwidth and fraction of 8 TB/s, finalize's fraction, and parity of
    the step's outputs against the CPU oracle on the same inputs;
  * extras.probes: the achievable rates of finalize's own access patterns
    (libmoe_probe.so): streaming read, streaming write, and the gather
    without the stores, at the headline shape;
  * cpu_baseline: the CPU oracle (plain C, OpenMP over tokens) timed on the
    host cores over whole steps of the headline workload, per stage on all
    threads and on one thread, and a parity check of the GPU step against
    it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, vendor figure
N_OUT = 8  # output buffers written in turn
COUNTER_FILE = os.path.join(ROOT, "profiles", "finalize_dsv3_counters.txt")
FINALIZE_SOURCES = [os.path.join(ROOT, "permutation_group_limited_amd", "csrc", f)
                    for f in ("finalize.hip", "common.hpp")]
CONFIG_ORDER = ("tiny", "mixtral", "dsv3", "decode", "skewed")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU time for the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the side measurements (protocol, configs, probes, ...)")
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


def stage_bytes(wk):
    """Algorithmic bytes of each stage (what the method must move)."""
    import torch
    T, E, K, H = wk.T, wk.E, wk.K, wk.H
    N = T * K
    db = 2 if wk.down_dtype == torch.bfloat16 else 4
    ob = 2 if wk.out_dtype == torch.bfloat16 else 4
    return {"router": T * E * 4 + E * 4 + N * (4 + 4),
            "create_indices": N * 4 + 2 * N * 4 + (2 * E + 1) * 4 + 8,
            "finalize": N * H * db + N * (4 + 4) + T * H * ob}


class Path:
    """Device buffers of one workload and the calls of one step. finalize
    writes the next of n_out output buffers on each call."""

    def __init__(self, wk, n_out=N_OUT):
        import torch

        from permutation_group_limited_amd import binding
        from permutation_group_limited_amd import workloads as wl

        self.b = binding
        self.wk = wk
        dev = torch.device("cuda:0")
        T, E, K, H = wk.T, wk.E, wk.K, wk.H
        N = T * K
        i32 = lambda *shape: torch.empty(shape, dtype=torch.int32, device=dev)  # noqa: E731
        self.scores_h, self.bias_h = wl.make_scores(wk), wl.make_bias(wk)
        self.scores, self.bias = self.scores_h.to(dev), self.bias_h.to(dev)
        self.down = wl.make_down(wk, device=dev)
        self.idx, self.wts = i32(T, K), torch.empty(T, K, dtype=torch.float32, device=dev)
        self.order, self.restore = i32(N), i32(N)
        self.starts, self.eids, self.stats = i32(E + 1), i32(E), i32(2)
        self.ws = i32(max(binding.moe_create_indices_workspace_size(N, E), 4) // 4)
        # moe_route_and_index's workspace: zero once here, left zero by every call
        self.ws_ri = torch.zeros(binding.moe_route_and_index_workspace_size(T, K, E) // 4,
                                 dtype=torch.int32, device=dev)
        self.outs = [torch.empty(T, H, dtype=wk.out_dtype, device=dev) for _ in range(n_out)]
        self.k = 0
        self.last_out = self.outs[0]
        self.bytes = stage_bytes(wk)

    def router(self):
        wk = self.wk
        self.b.moe_router_group_limited(self.idx, self.wts, self.scores, self.bias, wk.n_groups,
                                        wk.topk_group, wk.norm_weights, wk.scale)

    def indices(self):
        self.b.moe_create_indices(self.order, self.starts, self.restore, self.eids, self.stats,
                                  self.idx, self.ws)

    def route_and_index(self):
        wk = self.wk
        self.b.moe_route_and_index(self.idx, self.wts, self.order, self.starts, self.restore,
                                   self.eids, self.stats, self.scores, self.bias, self.ws_ri,
                                   wk.n_groups, wk.topk_group, wk.norm_weights, wk.scale)

    def finalize(self):
        out = self.outs[self.k % len(self.outs)]
        self.k += 1
        self.b.moe_finalize(out, self.down, self.restore, self.wts)
        self.last_out = out

    def finalize_one_buffer(self):
        self.b.moe_finalize(self.outs[0], self.down, self.restore, self.wts)
        self.last_out = self.outs[0]

    def step(self):
        self.route_and_index()
        self.finalize()

    def step_separate(self):
        self.router()
        self.indices()
        self.finalize()


def event_loop_ms(fn, n):
    """Mean duration of fn() over n back-to-back calls between two events."""
    import torch
    a = torch.cuda.Event(enable_timing=True)
    z = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(n):
        fn()
    z.record()
    torch.cuda.synchronize()
    return a.elapsed_time(z) / n


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the routing path "
              "shards by token with no exchange; run one process per GPU). --gpus %d refused."
              % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    from permutation_group_limited_amd import binding
    from permutation_group_limited_amd import workloads as wl

    binding.load_library()  # raises if the HIP library is not built
    wk = wl.WORKLOADS[args.workload]
    P = Path(wk)
    N = wk.T * wk.K

    for _ in range(args.warmup):
        P.step()
    torch.cuda.synchronize()

    # timed region 1 (headline): K back-to-back steps between two events
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t_start.record()
    for _ in range(args.steps):
        P.step()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    # the step's outputs, kept for the parity check
    last_out = P.last_out.clone()

    # timed region 2: each stage K times back to back on the launch stream
    # (every stage is idempotent on its inputs); finalize's mean duration,
    # with rotating outputs, is the roofline's denominator
    stages = (("router", P.router), ("create_indices", P.indices),
              ("route_and_index", P.route_and_index), ("finalize", P.finalize))
    for _, f in stages:  # first launches load code
        for _ in range(2):
            f()
    stage_ms = {name: event_loop_ms(f, args.steps) for name, f in stages}
    P.route_and_index()  # leave the step's index outputs in place for parity
    torch.cuda.synchronize()

    by = P.bytes
    bytes_total = sum(by.values())
    step_s = ms_per_step * 1e-3
    fin_gbps = by["finalize"] / (stage_ms["finalize"] * 1e-3) / 1e9

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
        "config": {"workload": wk.describe(), "tokens": wk.T, "experts": wk.E,
                   "n_groups": wk.n_groups, "topk_group": wk.topk_group, "top_k": wk.K,
                   "hidden": wk.H,
                   "storage": "bf16" if wk.down_dtype == torch.bfloat16 else "f32",
                   "accumulate": "f32", "output_buffers": N_OUT},
        "hbm_gbps": bytes_total / step_s / 1e9,
        "hbm_pct_of_peak": 100.0 * bytes_total / step_s / 1e9 / PEAK_HBM_GBPS,
        "algorithmic_bytes_per_step": bytes_total,
        "stage_bytes": by,
        "step": "moe_route_and_index (router filling the index histogram, then the scatter) "
                "+ moe_finalize into the next of %d output buffers: 3 kernels" % N_OUT,
        "stage_ms": stage_ms,
        "wall_s": wall,
        "roofline": {"kernel": "finalize_kernel", "bound": "hbm", "achieved": fin_gbps,
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": fin_gbps / PEAK_HBM_GBPS,
                     "traffic": counter_traffic(),
                     "outputs": "rotating over %d buffers (no output row cached from the "
                                "call before)" % N_OUT},
    }

    if not args.no_extras:
        reps = 20 if N * wk.H > (1 << 31) else 100
        result["protocol"] = timing_protocol(P, replays=reps)
        P.route_and_index()
        torch.cuda.synchronize()
        ex = {}
        ms_one = event_loop_ms(P.finalize_one_buffer, args.steps)
        g_one = by["finalize"] / (ms_one * 1e-3) / 1e9
        ex["finalize_one_output_buffer"] = {
            "us_per_call": ms_one * 1e3, "achieved_gbps": g_one, "frac": g_one / PEAK_HBM_GBPS,
            "note": "the same output buffer rewritten call after call: its rows stay in the "
                    "memory-side cache, so part of the write cost never reaches HBM"}
        ex["probes"] = probes(P, args.steps)
        ex["launch_probes"] = launch_probes()
        ex["router_on_logits"] = router_on_logits(P, args.steps)
        ex["two_batches_in_flight"] = two_batches_in_flight(P, args.steps)
        del P
        torch.cuda.empty_cache()
        ex["configs"] = {}
        for name in CONFIG_ORDER:
            ex["configs"][name] = config_report(wl.WORKLOADS[name])
            torch.cuda.empty_cache()
        ex["decode_t16"] = config_report(wl.WORKLOADS["decode"].with_tokens(16), parity=False)
        result["extras"] = ex
        P = None

    if args.copy_probe > 0:
        src = torch.ones(args.copy_probe // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_probe_bytes"] = args.copy_probe
        del src, dst

    if not args.no_cpu_baseline:
        if P is None:  # the extras released the headline buffers: rebuild them
            P = Path(wk)
            P.step()
            torch.cuda.synchronize()
            last_out = P.last_out.clone()
        result["cpu_baseline"], result["parity"] = cpu_leg(P, last_out, args.cpu_seconds)
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
    del g
    return a.elapsed_time(b) / (reps * per_graph) * 1e3


def config_report(wk, parity=True):
    """One workload with 20 calls per HIP graph (the graph launch amortised):
    GPU time per step (moe_route_and_index + moe_finalize, and the three
    separate entry points), per stage, algorithmic bandwidth against 8 TB/s,
    and parity of one step's outputs against the CPU oracle."""
    import torch
    P = Path(wk)
    by = P.bytes
    total = sum(by.values())
    reps = 10 if wk.T * wk.K * wk.H > (1 << 31) else 50
    us = graph_replay_us(P.step, reps=reps)
    us_sep = graph_replay_us(P.step_separate, reps=reps)
    us_ri = graph_replay_us(P.route_and_index, reps=reps)
    us_fin = graph_replay_us(P.finalize, reps=reps)
    us_router = graph_replay_us(P.router, reps=reps)
    us_idx = graph_replay_us(P.indices, reps=reps)
    rep = {"workload": wk.describe(), "token_slots": wk.T * wk.K,
           "algorithmic_bytes": total, "stage_bytes": by,
           "us_per_step_graph": us, "us_per_step_graph_separate_calls": us_sep,
           "token_slots_per_s": wk.T * wk.K / (us * 1e-6),
           "hbm_gbps": total / (us * 1e-6) / 1e9,
           "pct_of_peak": 100.0 * total / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS,
           "us_route_and_index": us_ri, "us_router": us_router,
           "us_create_indices": us_idx, "us_finalize": us_fin,
           "finalize_frac": by["finalize"] / (us_fin * 1e-6) / 1e9 / PEAK_HBM_GBPS,
           "output_buffers": N_OUT}
    if parity:
        P.step()
        torch.cuda.synchronize()
        rep["parity"] = oracle_parity(P, P.last_out)
    del P
    return rep


def oracle_parity(P, out):
    """The step's outputs against the CPU oracle on the same inputs: router
    indices and weights, every index output and the finalize output
    bit-exact (the largest difference is reported beside it)."""
    import numpy as np
    import torch

    import oracle

    wk = P.wk
    T, E, K = wk.T, wk.E, wk.K
    oi, ow = oracle.router(P.scores_h.numpy(), P.bias_h.numpy(), K, wk.n_groups,
                           wk.topk_group, wk.norm_weights, wk.scale)
    ind = oracle.create_indices(oi, E)
    u32 = lambda t: t.cpu().numpy().view(np.uint32)  # noqa: E731
    res = {
        "router_indices": bool(np.array_equal(P.idx.cpu().numpy(), oi)),
        "router_weights_bit_exact": bool(np.array_equal(P.wts.cpu().numpy().view(np.uint32),
                                                        ow.view(np.uint32))),
        "create_indices": bool(np.array_equal(u32(P.order), ind["token_expert_order"]) and
                               np.array_equal(u32(P.restore), ind["restore_token_order"]) and
                               np.array_equal(u32(P.starts), ind["expert_start_indices"]) and
                               np.array_equal(P.eids.cpu().numpy(), ind["expert_ids"]) and
                               np.array_equal(u32(P.stats), ind["expert_usage_stats"])),
    }
    if wk.down_dtype == torch.bfloat16:
        d = P.down.cpu().view(torch.int16).numpy().view(np.uint16)
        dcode = oracle.BF16
    else:
        d = P.down.cpu().numpy()
        dcode = oracle.F32
    if wk.out_dtype == torch.bfloat16:
        o = oracle.finalize(d, dcode, ind["restore_token_order"], ow, oracle.F32, oracle.BF16)
        gb = out.cpu().view(torch.int16).numpy().view(np.uint16)
        ordg = np.where(gb & 0x8000, -(gb.astype(np.int64) & 0x7FFF), gb & 0x7FFF)
        orde = np.where(o & 0x8000, -(o.astype(np.int64) & 0x7FFF), o & 0x7FFF)
        ulp = np.abs(ordg - orde)
        res["finalize_max_ulp"] = int(ulp.max(initial=0))
        res["finalize"] = bool(np.array_equal(gb, o))
    else:
        o = oracle.finalize(d, dcode, ind["restore_token_order"], ow, oracle.F32, oracle.F32)
        rows = d[ind["restore_token_order"].astype(np.int64)].astype(np.float64)
        mag = (np.abs(ow.astype(np.float64))[:, :, None] *
               np.abs(rows.reshape(T, K, -1))).sum(1)
        g = out.cpu().numpy()
        err = np.abs(g.astype(np.float64) - o.astype(np.float64))
        res["finalize_max_abs_err"] = float(err.max(initial=0.0))
        res["finalize_within_1e-5_of_terms"] = bool(np.all(err <= 1e-5 * mag))
        res["finalize"] = bool(np.array_equal(g.view(np.uint32), o.view(np.uint32)))
    return res


def probes(P, steps):
    """Rates of finalize's own access patterns on their own, at the headline
    shape (libmoe_probe.so): a streaming read of `down` (8 KiB per wave of
    non-temporal 16-byte loads), a 1 GiB streaming read, the output written
    alone (finalize's 16-byte stores) into the rotating output buffers, and the
    gather of finalize without its stores. read-phase + write-phase is what
    finalize would take if its reads and writes did not share the memory at
    the same time."""
    import torch

    from permutation_group_limited_amd import probe

    wk = P.wk
    T, K, H = wk.T, wk.K, wk.H
    sink = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    big = torch.ones(1 << 28, dtype=torch.int32, device="cuda:0")
    down_bytes = P.down.numel() * P.down.element_size()
    out_bytes = T * H * P.outs[0].element_size()
    k = [0]

    # finalize streams its output (nt stores) when its gathered rows exceed
    # the 256 MiB memory-side cache, and keeps it there (sc1) otherwise
    streaming = down_bytes > (256 << 20)

    def write_next():
        probe.write(P.outs[k[0] % len(P.outs)], streaming=streaming)
        k[0] += 1

    for f in (lambda: probe.read(big, sink), lambda: probe.read(P.down, sink), write_next,
              lambda: probe.gather(P.down, P.restore, T, K, sink)):
        f()
    res = {}
    ms = event_loop_ms(lambda: probe.read(big, sink), max(10, steps // 2))
    res["read_1GiB"] = {"us": ms * 1e3, "gbps": (1 << 30) / (ms * 1e-3) / 1e9}
    ms = event_loop_ms(lambda: probe.read(P.down, sink), steps)
    res["read_down"] = {"us": ms * 1e3, "gbps": down_bytes / (ms * 1e-3) / 1e9}
    ms_w = event_loop_ms(write_next, steps)
    res["write_output_rotating"] = {"us": ms_w * 1e3, "gbps": out_bytes / (ms_w * 1e-3) / 1e9}
    ms_g = event_loop_ms(lambda: probe.gather(P.down, P.restore, T, K, sink), steps)
    gb = down_bytes + T * K * 4
    res["gather_without_stores"] = {"us": ms_g * 1e3, "gbps": gb / (ms_g * 1e-3) / 1e9}
    bound_us = (ms_g + ms_w) * 1e3
    res["read_phase_plus_write_phase_us"] = bound_us
    res["read_phase_plus_write_phase_frac"] = \
        P.bytes["finalize"] / (bound_us * 1e-6) / 1e9 / PEAK_HBM_GBPS
    del big
    return res


def launch_probes():
    """Fixed costs that bound the small batches, each as GPU time per call
    with 20 calls per HIP graph (libmoe_probe.so): a launch of one workgroup
    that does nothing, the same with 1,024 workgroups, one workgroup reading
    64 KiB, and that read right after a kernel (1,024 waves of 16-byte
    stores) wrote the 64 KiB. The last minus the write alone is what one
    launch costs when it reads what the launch before it wrote, as the
    index step reads the router's counts."""
    import torch

    from permutation_group_limited_amd import probe

    buf = torch.zeros(1 << 14, dtype=torch.int32, device="cuda:0")  # 64 KiB
    sink = torch.zeros(4, dtype=torch.int32, device="cuda:0")

    def pair():
        probe.write(buf)
        probe.consume(buf, sink)

    cases = {"empty_1_workgroup": lambda: probe.empty(1),
             "empty_1024_workgroups": lambda: probe.empty(1024),
             "write_64KiB": lambda: probe.write(buf),
             "read_64KiB_one_workgroup": lambda: probe.consume(buf, sink),
             "write_then_read_64KiB": pair}
    res = {}
    for name, f in cases.items():
        f()
        torch.cuda.synchronize()
        res[name + "_us"] = graph_replay_us(f)
    res["read_after_write_us"] = res["write_then_read_64KiB_us"] - res["write_64KiB_us"]
    return res


def router_on_logits(P, steps):
    """The router on logits (sigmoid or softmax computed in the kernel)
    against the router on precomputed scores, same workload."""
    from permutation_group_limited_amd import binding
    from permutation_group_limited_amd import workloads as wl

    wk = P.wk
    fn = binding.SCORE_SIGMOID if wk.score_fn == "sigmoid" else binding.SCORE_SOFTMAX
    logits = wl.make_logits(wk).to("cuda:0")

    def on_logits():
        binding.moe_router_group_limited_logits(P.idx, P.wts, logits, P.bias, fn, wk.n_groups,
                                                wk.topk_group, wk.norm_weights, wk.scale)

    for f in (on_logits, P.router):
        f()
    res = {"router_logits_ms": event_loop_ms(on_logits, steps),
           "router_scores_ms": event_loop_ms(P.router, steps)}
    P.router()
    return res


def two_batches_in_flight(P, steps):
    """Throughput with two batches in flight, as micro-batch overlap in
    serving runs them: the same step on two sets of index / output buffers
    on two streams, alternating, so that one batch's routing and index
    creation (latency-bound, few waves) runs beside the other batch's
    finalize (HBM-bound). Every step is still the whole path on one batch;
    the steps of one buffer set stay in order on its stream. Mean GPU time
    per step, and whether both sets end with the single-stream output."""
    import torch

    from permutation_group_limited_amd import binding

    wk = P.wk
    dev = torch.device("cuda:0")
    T, E, K, H = wk.T, wk.E, wk.K, wk.H
    N = T * K

    def buffers():
        i32 = lambda *shape: torch.empty(shape, dtype=torch.int32, device=dev)  # noqa: E731
        return {"idx": i32(T, K), "w": torch.empty(T, K, device=dev), "order": i32(N),
                "restore": i32(N), "starts": i32(E + 1), "eids": i32(E), "stats": i32(2),
                "ws": torch.zeros(binding.moe_route_and_index_workspace_size(T, K, E) // 4,
                                  dtype=torch.int32, device=dev),
                "outs": [torch.empty(T, H, dtype=wk.out_dtype, device=dev)
                         for _ in range(N_OUT // 2)], "k": 0}

    sets = [buffers(), buffers()]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority

    def step(b, st):
        binding.moe_route_and_index(b["idx"], b["w"], b["order"], b["starts"], b["restore"],
                                    b["eids"], b["stats"], P.scores, P.bias, b["ws"],
                                    wk.n_groups, wk.topk_group, wk.norm_weights, wk.scale,
                                    stream=st)
        out = b["outs"][b["k"] % len(b["outs"])]
        b["k"] += 1
        binding.moe_finalize(out, P.down, b["restore"], b["w"], stream=st)
        b["last"] = out

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
    ref = sets[0]["last"].clone()
    run(4, True)
    two = run(steps, True)
    same = all(torch.equal(b["last"].view(torch.int16), ref.view(torch.int16)) for b in sets)
    return {"us_per_step_one_stream": single, "us_per_step_two_streams": two,
            "token_slots_per_s_two_streams": N / (two * 1e-6), "outputs_equal": bool(same)}


def timing_protocol(P, flush_bytes=1 << 30, replays=100):
    """The step and each stage captured in HIP graphs and replayed. Output
    buffers rotate as in the eager loop: one graph per output buffer,
    replayed in turn (a graph that rewrote one buffer would find part of
    its previous output still in the memory-side cache). Cold: flush_bytes
    written to a scratch buffer before each replay, outside the timed
    events (more than the 256 MB memory-side cache and the L2s together,
    which it leaves full of dirty lines, as the kernels before a step
    would); the same with a read of flush_bytes instead is reported beside
    it ("read_flush": a clean cache then absorbs the replay's stores and
    writes them back after the timed events). Warm: no flush. Median and
    minimum in microseconds; 20 steps per graph for the GPU time per step
    with the graph launch amortised; and a plain device copy of
    flush_bytes (read + write bytes / time)."""
    import torch
    scratch = torch.ones(flush_bytes // 8, dtype=torch.int64, device="cuda:0")
    sink = torch.empty((), dtype=torch.int64, device="cuda:0")

    def finalize_into(k):
        return lambda: P.b.moe_finalize(P.outs[k], P.down, P.restore, P.wts)

    def step_into(k):
        fin = finalize_into(k)

        def step():
            P.route_and_index()
            fin()
        return step

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

    def replay_times(graphs, flush):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(replays)]
        for i, (a, b) in enumerate(evs):
            if flush == "write":
                scratch.fill_(i)
            elif flush == "read":
                torch.sum(scratch, dim=0, out=sink)
            a.record()
            graphs[i % len(graphs)].replay()
            b.record()
        torch.cuda.synchronize()
        us = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
        return {"median_us": us[len(us) // 2], "min_us": us[0], "replays": replays}

    n_out = len(P.outs)
    res = {"outputs": "one graph per output buffer (%d), replayed in turn" % n_out,
           "cold_flush": "%d-byte write before each replay" % flush_bytes}
    graphs = [capture(step_into(k)) for k in range(n_out)]
    res["step_graph_cold"] = replay_times(graphs, "write")
    res["step_graph_cold_read_flush"] = replay_times(graphs, "read")
    res["step_graph_warm"] = replay_times(graphs, None)
    del graphs
    many = 20

    def steps():
        for i in range(many):
            step_into(i % n_out)()

    w20 = replay_times([capture(steps)], None)
    res["steps_per_graph_20_warm_us_per_step"] = {"median": w20["median_us"] / many,
                                                   "min": w20["min_us"] / many}
    stages = {"router": [P.router], "create_indices": [P.indices],
              "route_and_index": [P.route_and_index],
              "finalize": [finalize_into(k) for k in range(n_out)]}
    res["stage_graph_cold_median_us"] = {}
    res["stage_graph_cold_read_flush_median_us"] = {}
    for name, fns in stages.items():
        graphs = [capture(fn) for fn in fns]
        res["stage_graph_cold_median_us"][name] = replay_times(graphs, "write")["median_us"]
        res["stage_graph_cold_read_flush_median_us"][name] = \
            replay_times(graphs, "read")["median_us"]
        del graphs
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


def cpu_leg(P, out, budget_s):
    """Time the CPU oracle over whole steps of the same workload and check the
    GPU step against it."""
    import numpy as np
    import torch

    import oracle

    wk = P.wk
    T, E, K = wk.T, wk.E, wk.K
    N = T * K
    s = P.scores_h.numpy()
    b = P.bias_h.numpy()
    if wk.down_dtype == torch.bfloat16:
        d = P.down.cpu().view(torch.int16).numpy().view(np.uint16)
        dcode = oracle.BF16
    else:
        d = P.down.cpu().numpy()
        dcode = oracle.F32
    ocode = oracle.BF16 if wk.out_dtype == torch.bfloat16 else oracle.F32

    def oracle_step():
        oi, ow = oracle.router(s, b, K, wk.n_groups, wk.topk_group, wk.norm_weights, wk.scale)
        ind = oracle.create_indices(oi, E)
        o = oracle.finalize(d, dcode, ind["restore_token_order"], ow, oracle.F32, ocode)
        return oi, ow, ind, o

    steps = 0
    t0 = time.perf_counter()
    while True:
        oracle_step()
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or steps >= 400:
            break
    baseline = {"value": N * steps / el, "unit": "token-slots/s", "cores": oracle.num_threads(),
                "kind": "oracle",
                "sample": "%d whole steps of the %s workload (router + create_indices + "
                          "finalize), %.1f s" % (steps, wk.name, el)}

    # per stage, median of 3 runs, on all threads and on one thread
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

    def median_stage_times(runs=3):
        ts = [stage_times() for _ in range(runs)]
        return {k: sorted(t[k] for t in ts)[runs // 2] for k in ts[0]}

    threads = oracle.num_threads()
    baseline["stage_ms"] = median_stage_times()
    oracle.set_num_threads(1)
    try:
        baseline["single_thread_stage_ms"] = median_stage_times()
    finally:
        oracle.set_num_threads(threads)
    baseline["host_cpus"] = {"cpu_count": os.cpu_count(),
                             "affinity": len(os.sched_getaffinity(0))}
    return baseline, oracle_parity(P, out)


if __name__ == "__main__":
    main()
