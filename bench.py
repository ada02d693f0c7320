"""Benchmark of one tensor-parallel rank's routed-MoE call on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config c1] [--also c2,c3,c4] [--no-cpu]

One step = one complete call (route, align, gate/up, mid quant, down, combine
[, shared expert]) on one batch of synthetic inputs already resident in HBM.
Protocol: before every timed call a 1 GiB buffer is read (a reduction) so the
weights are not in the 256 MB MALL (cold, the regime of a model whose 75
layers of experts never fit in it) and the MALL holds only clean lines (a
flush that writes would leave dirty lines whose write-back competes with the
measured call). value = mean cold device span per call: from the start of
the call's first kernel to the end of its last kernel, read from events the
library binds to those two launches (the host's launch latency is outside
it, as it is for a layer inside a captured model step). The same calls as
hipGraph replays bracketed by stream events are reported beside it
(us_per_call_graph_replay: adds the runtime's graph launch latency). The
stage durations come from events the library binds to each stage's first
and last launch (eager calls, same cold protocol).

Prints one JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
FP4_PEAK_TFLOPS = 10100.0  # dense MXFP4 MFMA
BF16_PEAK_TFLOPS = 2500.0


def per_expert_bytes(shape):
    H, I = shape.H, shape.I
    w13 = 2 * I * H // 2 + 2 * I * H // 32
    w2 = H * I // 2 + H * I // 32
    return w13, w2


def call_bytes(shape, n_act):
    """Algorithmic HBM bytes of one call: active experts' weights read once,
    x, logits and out, plus the shared expert's weights."""
    w13, w2 = per_expert_bytes(shape)
    b = n_act * (w13 + w2) + shape.M * shape.H * 2 + shape.M * shape.E * 4 + shape.M * shape.H * 2
    if shape.shared_I:
        Is, H = shape.shared_I, shape.H
        b += 2 * Is * H + 4 * (2 * Is // 128) * (H // 128) + H * Is + 4 * (H // 128) * (Is // 128)
    return b


def gate_up_bytes(shape, n_act):
    """Algorithmic bytes of the gate/up launch: active experts' w13 (values +
    scales), the tokens' MXFP4 x (values + scales) and the fp32 h it writes."""
    w13, _ = per_expert_bytes(shape)
    M, H, k, I = shape.M, shape.H, shape.top_k, shape.I
    return n_act * w13 + M * (H // 2 + H // 32) + M * k * I * 4


def call_flops(shape):
    f = 2 * shape.M * shape.top_k * 3 * shape.H * shape.I
    if shape.shared_I:
        f += 2 * shape.M * 3 * shape.H * shape.shared_I
    return f


def kernel_source_hash():
    h = hashlib.sha256()
    d = os.path.join(ROOT, "quantized_moe_expert_route_amd", "csrc")
    for f in sorted(os.listdir(d)):
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


_WEIGHTS = {}


def _weights(shape, seed):
    """The routed experts' weights of a workload: drawn once per (E, I, H,
    seed) and kept for the other workloads that share them (one at a time)."""
    from quantized_moe_expert_route_amd import fixtures as X

    key = (shape.E, shape.I, shape.H, seed)
    if key not in _WEIGHTS:
        _WEIGHTS.clear()
        _WEIGHTS[key] = X.make_weights(shape, seed)
    return _WEIGHTS[key]


def measure(name, steps, warmup, n_sets, mid_fmt=0, tp_loopback=0):
    """Time `name`'s calls. tp_loopback = T > 0 runs them with the
    tensor-parallel exchange epilogue as rank 0 of T alone: the peers'
    partials zeros tagged with the epoch, the pushes into scratch sinks."""
    import torch

    from quantized_moe_expert_route_amd import fixtures as X
    from quantized_moe_expert_route_amd.binding import HipEvents, Plan, layout_for, pack_w13, pack_w2, stage_names

    wl = X.WORKLOADS[name]
    s = wl.shape
    dev = torch.device("cuda", 0)
    base = X.make_inputs(name, with_weights=False)
    base["w13"], base["s13"], base["w2"], base["s2"] = _weights(s, wl.seed)
    t = {k: torch.from_numpy(base[k]).to(dev) for k in ("w13", "s13", "w2", "s2")}
    t["w13"], t["s13"] = pack_w13(t["w13"], t["s13"])  # load-time packing, outside the timed calls
    if mid_fmt:
        t["w2"], t["s2"] = pack_w2(t["w2"], t["s2"])  # the MXFP4-mid down reads packed down weights
    torch.cuda.synchronize()
    sets = []
    for i in range(n_sets):
        d = (X.make_inputs(X.Shape(**vars(s)), wl.logits, wl.seed * 1000 + i, with_weights=False,
                           shared_slot=wl.shared_slot) if i else base)
        sets.append((torch.from_numpy(d["x"].view(np.int16)).to(dev), torch.from_numpy(d["logits"]).to(dev)))
    plan = Plan(s.M, s.H, s.E, s.I, s.top_k, s.routed_scaling, s.shared_I)
    if s.shared_I:
        sh = [torch.from_numpy(base[k]).to(dev) for k in ("ws13", "ss13", "ws2", "ss2")]
        plan.set_shared(*sh)
    plan.set_mid_format(mid_fmt)
    plan.set_weight_layout(layout_for(mid_fmt))
    plan.set_shared_slot(wl.shared_slot)
    if tp_loopback:
        T = tp_loopback
        inbox = torch.zeros((T, s.M, s.H), dtype=torch.float64, device=dev)
        tags = torch.ones((T, s.M, s.H // 512), dtype=torch.int32, device=dev)
        sinks = [None] + [torch.empty((s.M, s.H), dtype=torch.float64, device=dev) for _ in range(T - 1)]
        sink_tags = [None] + [torch.empty((s.M, s.H // 512), dtype=torch.int32, device=dev) for _ in range(T - 1)]
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        plan.set_tp_exchange(T, 0, 1, inbox, tags, sinks, sink_tags, status)
    x = torch.empty_like(sets[0][0])
    logits = torch.empty_like(sets[0][1])
    out = torch.empty((s.M, s.H), dtype=torch.int16, device=dev)
    flush = torch.ones(256 * 1024 * 1024, dtype=torch.float32, device=dev)  # 1 GiB, read before each timed call
    sink = torch.empty((), dtype=torch.float32, device=dev)

    def call():
        plan.forward(x, logits, t["w13"], t["s13"], t["w2"], t["s2"], out)

    # active experts of every input set, read from the library's own counts
    n_act = []
    for xs_, lg in sets:
        x.copy_(xs_)
        logits.copy_(lg)
        call()
        torch.cuda.synchronize()
        cnt = plan.view("count", torch.int32, (s.E,))
        n_act.append(int((cnt > 0).sum().item()))

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        call()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()

    # timed region: K cold calls; each call's device span (its first kernel's
    # start to its last kernel's end) comes from events the library records
    # with those two launches, so host launch latency is not in it
    cev = HipEvents(2 * steps)
    for i in range(warmup):
        x.copy_(sets[i % n_sets][0])
        logits.copy_(sets[i % n_sets][1])
        torch.sum(flush, 0, out=sink)
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        x.copy_(sets[i % n_sets][0])
        logits.copy_(sets[i % n_sets][1])
        torch.sum(flush, 0, out=sink)
        plan.set_call_events(cev.handles[2 * i], cev.handles[2 * i + 1])
        call()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    plan.set_call_events(None, None)
    cold_us = np.array([cev.elapsed_ms(2 * i, 2 * i + 1) * 1000.0 for i in range(steps)])
    cev.close()

    # the same calls as graph replays, timed by stream events around each
    # replay (adds the graph launch latency of the host runtime)
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        x.copy_(sets[i % n_sets][0])
        logits.copy_(sets[i % n_sets][1])
        torch.sum(flush, 0, out=sink)
        ev0[i].record()
        graph.replay()
        ev1[i].record()
    torch.cuda.synchronize()
    graph_us = np.array([a.elapsed_time(b) * 1000.0 for a, b in zip(ev0, ev1)])

    # cold calls as a difference of two graphs (the protocol's cross-check):
    # R x [flush, call] against R x [flush], each replayed whole and timed by
    # events around the replay; no host launch gaps and no event packets
    # between the call's kernels (one input set)
    R = 16
    x.copy_(sets[0][0])
    logits.copy_(sets[0][1])
    torch.cuda.synchronize()
    g_f, g_fc = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_f):
        for _ in range(R):
            torch.sum(flush, 0, out=sink)
    with torch.cuda.graph(g_fc):
        for _ in range(R):
            torch.sum(flush, 0, out=sink)
            call()
    torch.cuda.synchronize()
    t_f, t_fc = [], []
    for rep in range(6):
        for gr, acc in ((g_f, t_f), (g_fc, t_fc)):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            gr.replay()
            b.record()
            torch.cuda.synchronize()
            if rep:  # the first replay of each warms up
                acc.append(a.elapsed_time(b) * 1000.0)
    graph_delta_us = (float(np.median(t_fc)) - float(np.median(t_f))) / R
    del g_f, g_fc

    # warm: the same inputs back to back (weights partly MALL-resident)
    x.copy_(sets[0][0])
    logits.copy_(sets[0][1])
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    warm_us = e0.elapsed_time(e1) * 1000.0 / steps

    # per-stage durations (eager calls, cold), on the stream the kernels run on
    names = stage_names()
    hev = HipEvents(2 * len(names))
    plan.set_stage_events(hev.handles)
    stage_us = np.zeros((steps, len(names)))
    for i in range(steps):
        x.copy_(sets[i % n_sets][0])
        logits.copy_(sets[i % n_sets][1])
        torch.sum(flush, 0, out=sink)
        call()
        torch.cuda.synchronize()
        for j in range(len(names)):
            stage_us[i, j] = hev.elapsed_ms(2 * j, 2 * j + 1) * 1000.0
    plan.set_stage_events(None)
    hev.close()
    # stages folded into another one for this M record an empty pair of events
    launches = np.array(plan.stage_launches(s.M))
    kern_us = np.where(launches[None, :] > 0, stage_us, 0.0)
    if tp_loopback:
        assert int(status.item()) == 0, "an exchange wait gave up"
    per_set_act = [n_act[i % n_sets] for i in range(steps)]
    mean_act = float(np.mean(per_set_act))
    res = {
        "name": name, "shape": s, "cold_us": cold_us, "graph_us": graph_us, "warm_us": warm_us, "wall_s": wall,
        "graph_delta_us": graph_delta_us,
        "stage_us": dict(zip(names, kern_us.mean(0).tolist())), "n_act": mean_act, "launches": launches.tolist(),
        "n_act_sets": n_act, "bytes": float(np.mean([call_bytes(s, a) for a in per_set_act])),
        "gate_up_bytes": float(np.mean([gate_up_bytes(s, a) for a in per_set_act])),
        "flops": call_flops(s), "base": base,
    }
    del graph, flush
    torch.cuda.synchronize()
    return res


def _time_oracle(d, n_max, budget_s):
    from oracle import moe as O

    s = d["shape"]
    shared = (d["ws13"], d["ss13"], d["ws2"], d["ss2"]) if s.shared_I else None
    times = []
    t_start = time.perf_counter()
    while len(times) < n_max:
        t0 = time.perf_counter()
        O.moe_forward(d["x"], d["logits"], d["w13"], d["s13"], d["w2"], d["s2"], s.top_k, s.routed_scaling, shared)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s:
            break
    return float(np.median(times) * 1e6), len(times)


def cpu_baseline(res, budget_s=12.0):
    """The oracle, as it stands, on the host: whole calls on the headline
    workload's inputs (median of up to 5, within ~budget_s of CPU work), with
    every BLAS thread and with one; and the tiny c0 call likewise."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from quantized_moe_expert_route_amd import fixtures as X

    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    d = res["base"]
    multi, n_multi = _time_oracle(d, 5, budget_s)
    with threadpool_limits(1):
        single, n_single = _time_oracle(d, 5, budget_s / 2)
    d0 = X.make_inputs("c0")
    c0_multi, _ = _time_oracle(d0, 5, 2.0)
    with threadpool_limits(1):
        c0_single, _ = _time_oracle(d0, 5, 2.0)
    return {"value": round(multi, 1), "unit": "us per call", "cores": int(threads), "kind": "oracle",
            "sample": f"whole calls of the {res['name']} workload (M={d['shape'].M}): median of {n_multi} with "
                      f"{threads} BLAS threads; host os.cpu_count()={os.cpu_count()}, "
                      f"affinity={len(os.sched_getaffinity(0))}",
            "single_thread_us": round(single, 1), "single_thread_calls": n_single,
            "c0_us": round(c0_multi, 1), "c0_single_thread_us": round(c0_single, 1)}


def cpu_full():
    """The oracle on every configuration: c0-c2 median of 5 with all BLAS
    threads and with one, c3/c4 once with all threads (minutes of CPU work;
    not part of the default run)."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from quantized_moe_expert_route_amd import fixtures as X

    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    out = {"cores": int(threads), "cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)),
           "unit": "us per call", "configs": {}}
    for name in ("c0", "c1", "c2", "c3", "c4"):
        d = X.make_inputs(name)
        reps = 5 if name in ("c0", "c1", "c2") else 1
        multi, n = _time_oracle(d, reps, 1e9)
        row = {"multi_thread_us": round(multi, 1), "runs": n}
        if reps == 5:
            with threadpool_limits(1):
                row["single_thread_us"] = round(_time_oracle(d, reps, 1e9)[0], 1)
        out["configs"][name] = row
        print(f"[cpu] {name}: {row}", file=sys.stderr, flush=True)
    return out


def traffic_for(name, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 PMC
    summary, if it was taken on the current kernel sources."""
    p = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(p):
        return None
    try:
        j = json.load(open(p))
    except Exception:
        return None
    if j.get("kernel_source_hash") != kernel_source_hash():
        return None
    e = j.get("workloads", {}).get(name, {}).get(kernel)
    return None if e is None else e.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c1", help="headline workload (c1..c4)")
    ap.add_argument("--also", default="c2,c3,c4,c1s,c2s,c1b,c2b,m256_hot,m256_mixed,t4_m4096_spread,t4_m4096_hot",
                    help="more workloads reported in the same line ('' for none); mid-range batches are "
                         "m{32,64,128,256}_{hot,mixed,spread}; c1s/c2s add the shared expert as expert 256, top-9")
    ap.add_argument("--mxfp4", default="m256_hot,m256_mixed,t4_m4096_spread,t4_m4096_hot",
                    help="workloads also timed with the MXFP4 mid hand-off (the pages' stock MXFP4 comparison "
                         "arm), reported as '<name>/mxfp4' ('' for none)")
    ap.add_argument("--sets", type=int, default=8, help="distinct input batches cycled through the steps")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-full", action="store_true",
                    help="only time the CPU oracle on c0..c4 (c0-c2 median of 5, all threads and one; c3/c4 once) "
                         "and print it as JSON; needs no GPU")
    ap.add_argument("--tp-loopback", default="c1",
                    help="workloads also timed with the tensor-parallel exchange epilogue as rank 0 of TP8 alone "
                         "(zero peer partials tagged with the epoch, pushes into scratch sinks), reported as "
                         "'<name>/tp8_loopback' ('' for none)")
    ap.add_argument("--torch-read", type=int, default=0, metavar="MIB",
                    help="only time torch's reduction over a cold MIB MiB buffer (the same 1 GiB flush before "
                         "each) and print its rate: a library baseline for reading that many bytes once")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 plain device-to-device copies of MIB MiB (the known-size kernel that "
                         "scales the HBM byte counters of a profiler run), then exit")
    args = ap.parse_args()
    if args.cpu_full:
        print(json.dumps(cpu_full()))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the path is one tensor-parallel rank's call on one MI355X)", file=sys.stderr)
        sys.exit(2)
    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.torch_read:
        n = args.torch_read * 1024 * 1024 // 4
        buf = torch.ones(n, dtype=torch.float32, device="cuda")
        flush = torch.ones(256 * 1024 * 1024, dtype=torch.float32, device="cuda")
        sink = torch.empty((), dtype=torch.float32, device="cuda")
        us = []
        for i in range(25):
            torch.sum(flush, 0, out=sink)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            torch.sum(buf, 0, out=sink)
            e1.record()
            torch.cuda.synchronize()
            if i >= 5:
                us.append(e0.elapsed_time(e1) * 1000.0)
        med = float(np.median(us))
        print(json.dumps({"torch_read_bytes": 4 * n, "us_median": round(med, 2),
                          "GBps": round(4 * n / (med * 1e-6) / 1e9, 1), "reads": len(us)}))
        return
    if args.copy_calibration:
        n = args.copy_calibration * 1024 * 1024 // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": 4 * n, "copy_calibration_bytes_written": 4 * n, "copies": 5}))
        return
    from quantized_moe_expert_route_amd import fixtures as X

    head = measure(args.config, args.steps, args.warmup, args.sets)
    print(f"[bench] {args.config}: cold {head['cold_us'].mean():.1f} us (graph replay {head['graph_us'].mean():.1f}, "
          f"graph difference {head['graph_delta_us']:.1f}), "
          f"warm {head['warm_us']:.1f} us, "
          f"stages {json.dumps({k: round(v, 1) for k, v in head['stage_us'].items()})}", file=sys.stderr, flush=True)
    others = {}
    runs = [(c, 0) for c in args.also.split(",") if c and c != args.config]
    runs += [(c, 1) for c in args.mxfp4.split(",") if c]
    runs += [(c, 8) for c in args.tp_loopback.split(",") if c]
    for name, mode in runs:
        fmt, tp = (mode, 0) if mode < 2 else (0, mode)
        r = measure(name, max(10, args.steps // 2), max(3, args.warmup // 2), min(args.sets, 4), mid_fmt=fmt,
                    tp_loopback=tp)
        mu = r["cold_us"].mean()
        name = f"{name}/mxfp4" if fmt else f"{name}/tp{tp}_loopback" if tp else name
        others[name] = {
            "us_per_call_cold": round(mu, 2), "us_per_call_graph_replay": round(float(r["graph_us"].mean()), 2),
            "us_per_call_graph_difference": round(r["graph_delta_us"], 2),
            "us_per_call_warm": round(r["warm_us"], 2),
            "n_active_experts": round(r["n_act"], 1),
            "hbm_frac": round(r["bytes"] / (mu * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "fp4_mfma_frac": round(r["flops"] / (mu * 1e-6) / 1e12 / FP4_PEAK_TFLOPS, 4),
            "stage_us": {k: round(v, 2) for k, v in r["stage_us"].items()},
        }
        print(f"[bench] {name}: {others[name]}", file=sys.stderr, flush=True)
        del r
    mu = float(head["cold_us"].mean())
    s = head["shape"]
    gu_us = head["stage_us"]["gate_up"]
    routes = head["launches"][0] == 0  # gate/up also ranks the logits and quantizes x (no routing launch)
    gu_bytes = head["gate_up_bytes"] + (s.M * s.H * 2 + s.M * s.E * 4 if routes else 0)
    achieved = gu_bytes / (gu_us * 1e-6) / 1e9
    line = {
        "metric": "us per local MoE call (cold MALL, device span of the call's kernels)",
        "value": round(mu, 3),
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(mu / 1000.0, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {
            "workload": f"{args.config}: {X.WORKLOAD_TITLES[args.config]}",
            "M": s.M, "H": s.H, "E": s.E, "I": s.I, "top_k": s.top_k, "routed_scaling": s.routed_scaling,
            "shared_I": s.shared_I, "n_active_experts": round(head["n_act"], 2),
            "protocol": "cold: a 1 GiB read before each call; value = device span of the call (its first "
                        "kernel's start to its last kernel's end, events bound to those launches)",
        },
        "us_per_call_p50": round(float(np.median(head["cold_us"])), 3),
        "us_per_call_graph_replay": round(float(head["graph_us"].mean()), 3),
        "us_per_call_graph_difference": round(head["graph_delta_us"], 3),
        "us_per_call_warm": round(head["warm_us"], 3),
        "hbm_frac_call": round(head["bytes"] / (mu * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "fp4_mfma_frac_call": round(head["flops"] / (mu * 1e-6) / 1e12 / FP4_PEAK_TFLOPS, 6),
        "stage_us": {k: round(v, 3) for k, v in head["stage_us"].items()},
        "stage_timing": "events recorded by the launches of each stage (start of its first kernel, end "
                        "of its last); 0 for a stage folded into another; cold, eager",
        "timed_region_s": round(head["wall_s"], 4),
        "roofline_call": {"bound": "hbm", "frac": round(head["bytes"] / (mu * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                          "note": "the whole call's algorithmic bytes over its device span, against 8 TB/s"},
        "roofline": {
            "kernel": "gate_up",
            "note": "the dominant kernel of the call (gate/up weight streaming), not the whole call"
                    + ("; on this path the same launch also ranks the logits, sorts the entries and quantizes x "
                       "(the call has no routing launch)" if routes else ""),
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_for(args.config, "gate_up"),
            "algorithmic_bytes_per_launch": round(gu_bytes),
            "avg_launch_us": round(gu_us, 3),
        },
        "others": others,
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(head)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
