"""Benchmark of the decode-batch attention front on one MI355X.

One step is one qkvf_run call: the projection, norm, rotation, y store and
K|V insert of M tokens, on weight set (step mod S) of S rotated sets so the
weights come from HBM rather than the 256 MB MALL.  Prints ONE JSON line.

Default workload: M = 8 tokens, 8 KV heads, N = 9216 (151 MB of bf16
weights per set, 4 sets).  `value` is achieved GB/s of algorithmic bytes
(W + x + y + cos|sin rows + indices + K|V slots) per call, inputs resident
in HBM.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import kv_insert_amd as qf  # noqa: E402
from kv_insert_amd import workloads as wl  # noqa: E402

HBM_PEAK_GBS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "kv_insert_amd", "csrc", "qkvf_kernels.hip")
COUNTERS = os.path.join(ROOT, "profiles", "front_fused_counters.json")


ATTN2_SRC = os.path.join(ROOT, "kv_insert_amd", "csrc", "qkvf_attn2.hip")
ATTN2_COUNTERS = os.path.join(ROOT, "profiles", "attn2_counters.json")
LF_SRC = os.path.join(ROOT, "kv_insert_amd", "csrc", "qkvf_layer_front.hip")
LF_COUNTERS = os.path.join(ROOT, "profiles", "layer_front_counters.json")


def kernel_hash(path: str = KERNEL_SRC) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def measured_traffic(w, counters: str = COUNTERS, src: str = KERNEL_SRC) -> float | None:
    """HBM bytes per call from the rocprofv3 FETCH_SIZE / WRITE_SIZE runs
    recorded in profiles/, if they were taken on the kernel as it is now."""
    try:
        rec = json.load(open(counters))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sha256_16") != kernel_hash(src):
        return None
    entry = rec.get("workloads", {}).get(w.name)
    if entry is None:
        return None
    return entry.get("hbm_bytes_per_launch", entry.get("hbm_bytes_per_call"))


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=wl.C3.name,
                    help="one of " + ", ".join(wl.WORKLOADS) + " or sweep_m<M>_nkv<K>")
    ap.add_argument("--wsets", type=int, default=0, help="override rotated weight sets")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=12.0,
                    help="CPU time budget of the oracle baseline (0 = skip)")
    ap.add_argument("--repeats", type=int, default=3, help="timed repeats; the median is kept")
    ap.add_argument("--all", action="store_true",
                    help="also time every workload and sweep point; one JSON line each on stderr")
    ap.add_argument("--attn2-lines", action="store_true",
                    help="only the attn2 lines of --all (stderr), then exit")
    ap.add_argument("--attn2", default="", metavar="WORKLOAD",
                    help="time attn2 instead of the front: one of " + ", ".join(wl.ATTN2_WORKLOADS))
    ap.add_argument("--attn2-batch-invariant", action="store_true",
                    help="with --attn2: prepare the layer with batch-invariant splits")
    ap.add_argument("--layer-front", default="", metavar="WORKLOAD",
                    help="time LayerFront instead of the front: one of "
                         + ", ".join(wl.LAYER_FRONT_WORKLOADS))
    ap.add_argument("--route", default="", metavar="WORKLOAD",
                    help="time MuseRouting instead of the front: one of "
                         + ", ".join(wl.ROUTE_WORKLOADS))
    ap.add_argument("--eager", action="store_true",
                    help="time LayerFront and routing calls issued one by one instead of "
                         "replaying a HIP graph (for profiler runs)")
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="MB",
                    help="instead of the front, time device-to-device copies of MB megabytes "
                         "(a plain copy kernel of known size, for scaling memory counters)")
    ap.add_argument("--all-cpu-seconds", type=float, default=2.0,
                    help="CPU time budget of the oracle baseline of each --all line (0 = skip)")
    ap.add_argument("--profile-workloads", default="", metavar="W1,W2,...",
                    help="instead of timing, issue warmup + steps front calls of each workload "
                         "in turn on one stream (for a rocprofv3 run); one JSON line per "
                         "workload on stdout names its calls, in order")
    ap.add_argument("--summarize-attn2-profiles", default="", metavar="DIR",
                    help="summarize attn2 kernel traces and counters under DIR/a2/<workload>/ "
                         "into profiles/attn2_counters.json and print a table")
    ap.add_argument("--summarize-profiles", default="", metavar="DIR",
                    help="no GPU: read the rocprofv3 output of a --profile-workloads run under "
                         "DIR (order.jsonl, trace/, fetch/, write/, calib_fetch/, calib_write/, "
                         "optionally all.jsonl from --all), write the per-workload counter "
                         "record to profiles/front_fused_counters.json and print a table")
    return ap.parse_args()


def workload_by_name(name: str) -> wl.Workload:
    if name in wl.WORKLOADS:
        return wl.WORKLOADS[name]
    if name.startswith("sweep_m"):
        m, k = name[len("sweep_m"):].split("_nkv")
        return wl.sweep(int(m), int(k))
    raise SystemExit(f"unknown workload {name}")


class Pool:
    """Device-resident inputs of S calls, rotated per step."""

    def __init__(self, w: wl.Workload, sets: int):
        dev = "cuda"
        self.w = w
        self.sets = sets
        self.W = [wl.make_weights_on_device(w, s, dev) for s in range(sets)]
        toks = [wl.make_tokens(w, s) for s in range(sets)]
        self.x = [t[0].to(dev) for t in toks]
        self.pos = [t[1].to(dev) for t in toks]
        self.slots = [t[2].to(dev) for t in toks]
        self.cos_sin = wl.rope_table(w.table_rows).to(dev)
        self.cache = wl.make_cache(w).to(dev)
        self.y = [torch.empty(w.M, w.N, dtype=torch.bfloat16, device=dev) for _ in range(sets)]

    def call(self, i: int, stream) -> None:
        s = i % self.sets
        qf.run(self.x[s], self.W[s], self.pos[s], self.slots[s], self.cos_sin, self.y[s],
               self.cache, M=self.w.M, stream=stream)


def host_threads() -> tuple[int, int]:
    """(threads the oracle uses, cores this process may run on).  All the
    cores the process may run on, unless OMP_NUM_THREADS sets the machine's
    share for one GPU lower."""
    host = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    limit = os.environ.get("OMP_NUM_THREADS", "")
    threads = min(host, int(limit)) if limit.isdigit() and int(limit) > 0 else host
    return max(1, threads), host


def cpu_baseline(w: wl.Workload, budget_s: float, single_core: bool = True) -> dict | None:
    """The oracle, as it stands, on full calls of the same workload (set 0),
    timed on this host's cores; as many calls as fit the budget (>= 1)."""
    if budget_s <= 0:
        return None
    import numpy as np

    import oracle
    threads, host = host_threads()
    x, pos, slots = wl.make_tokens(w, 0)
    W = wl.bits(wl.make_weights(w, 0))
    xb = wl.bits(x)
    table = wl.rope_table(w.table_rows).numpy()
    cache = np.zeros((w.pages, w.nkv, wl.PAGE_SLOTS, wl.SLOT_WIDTH), np.uint16)
    def timed(nthreads: int, budget: float):
        calls, t0 = 0, time.perf_counter()
        while True:
            oracle.front(xb, W, pos.numpy(), slots.numpy(), table, w.nkv, wl.EPS, cache,
                         nthreads=nthreads)
            calls += 1
            el = time.perf_counter() - t0
            if el >= budget or (el / calls) * (calls + 1) > 2 * budget:
                return el / calls, calls

    per_call, calls = timed(threads, budget_s)
    out = {"value": round(w.algorithmic_bytes() / per_call / 1e9, 4), "unit": "GB/s",
           "us_per_call": round(per_call * 1e6, 1), "cores": threads, "host_cores": host,
           "kind": "oracle",
           "sample": f"{calls} full oracle calls of {w.name} (weight set 0), {threads} OpenMP "
                     f"threads on a host whose process may run on {host} cores"}
    if single_core:
        # The same oracle on one core, for a third of the budget (>= 1 call).
        one, one_calls = timed(1, budget_s / 3)
        out["single_core"] = {"value": round(w.algorithmic_bytes() / one / 1e9, 4), "unit": "GB/s",
                              "us_per_call": round(one * 1e6, 1), "cores": 1,
                              "sample": f"{one_calls} full oracle calls of {w.name} (weight set 0), "
                                        "1 thread"}
    return out


def stream_context(w: wl.Workload, sets: int, steps: int, repeats: int) -> dict:
    """For context: qkvf_stream_read (a plain streaming read with the front's
    launch and load shape) over buffers the size of one weight set, rotated
    over as many sets as the front's timing, timed the same way."""
    nbytes = w.N * wl.HIDDEN * 2
    bufs = [torch.empty(nbytes // 4, dtype=torch.int32, device="cuda") for _ in range(sets)]
    sink = torch.empty(256 * 512, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for i in range(2 * sets):
            qf.stream_read(bufs[i % sets], sink, stream)
    torch.cuda.synchronize()
    times = []
    for _ in range(repeats):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for i in range(steps):
            qf.stream_read(bufs[i % sets], sink, stream)
        end.record(stream)
        torch.cuda.synchronize()
        times.append(start.elapsed_time(end) / steps)
    ms = sorted(times)[len(times) // 2]
    gbs = nbytes / (ms * 1e-3) / 1e9
    del bufs
    torch.cuda.empty_cache()
    return {"kernel": "qkvf_stream_read (plain streaming read, 256 x 512 threads, "
                      "16 x 16-byte non-temporal loads in flight per lane)",
            "bytes_per_call": nbytes, "buffers_rotated": sets,
            "us_per_call": round(ms * 1e3, 3), "GB_per_s": round(gbs, 1),
            "frac_of_8TBs": round(gbs / HBM_PEAK_GBS, 4)}


def time_front(w: wl.Workload, sets: int, steps: int, warmup: int, repeats: int):
    pool = Pool(w, sets)
    qf.prepare(w.N, w.nkv, w.M)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for i in range(warmup):
            pool.call(i, stream)
    torch.cuda.synchronize()
    times = []
    for _ in range(repeats):
        # HIP events on the stream the kernel is launched on: one launch per
        # call, so elapsed / steps is the average launch duration.
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(steps):
            pool.call(warmup + i, stream)
        end.record(stream)
        torch.cuda.synchronize()
        times.append(start.elapsed_time(end) / steps)  # ms per call
    fault = qf.device_fault()
    if fault != 0:
        raise RuntimeError(f"a timed call gave up waiting for a partial: {qf.strerror(fault)}")
    del pool
    torch.cuda.empty_cache()
    return sorted(times)[len(times) // 2], times


class Attn2Pool:
    """Device-resident inputs of S attn2 calls: request sets on disjoint
    pages of one cache (so a call's K|V is not left in the MALL by the
    previous one), each with its own q | gate rows, table and output."""

    def __init__(self, a: wl.Attn2Workload, sets: int):
        dev = "cuda"
        self.a = a = dataclasses.replace(a, sets=sets)
        self.sets = sets
        self.cache = wl.make_attn2_cache(a, device=dev)
        self.y = [wl.make_attn2_y(a, s, device=dev) for s in range(sets)]
        tables = [wl.make_attn2_table(a, s) for s in range(sets)]
        need = a.pages_per_req
        for t in tables:   # every page a call can read is inside the cache
            assert int(t[:, :need].min()) >= 0 and int(t[:, :need].max()) < a.pages
        self.table = [t.to(dev) for t in tables]
        self.lens = wl.make_attn2_lens(a).to(dev)
        width = wl.QHEADS_PER_KV * a.nkv * wl.HEAD_DIM
        self.out = [torch.empty(8 * a.R, width, dtype=torch.bfloat16, device=dev)
                    for _ in range(sets)]

    def call(self, i: int, stream) -> None:
        s = i % self.sets
        q, g = wl.attn2_views(self.y[s], self.a.nkv)
        qf.attn2_run(q, g, self.cache, self.table[s], self.lens, self.out[s], stream=stream)


def attn2_sets(a: wl.Attn2Workload) -> int:
    kv = a.algorithmic_bytes()
    return max(a.sets, int(600e6 // kv) + 1)


def time_attn2(a: wl.Attn2Workload, steps: int, warmup: int, repeats: int,
               invariant: bool = False):
    sets = attn2_sets(a)
    pool = Attn2Pool(a, sets)
    qf.attn2_prepare(a.nkv, a.max_model_len, a.R, a.window, batch_invariant=invariant)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for i in range(warmup):
            pool.call(i, stream)
    torch.cuda.synchronize()
    times = []
    for _ in range(repeats):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(steps):
            pool.call(warmup + i, stream)
        end.record(stream)
        torch.cuda.synchronize()
        times.append(start.elapsed_time(end) / steps)
    del pool
    torch.cuda.empty_cache()
    return sorted(times)[len(times) // 2], times, sets


def attn2_cpu_baseline(a: wl.Attn2Workload, budget_s: float) -> dict | None:
    """The attn2 oracle on full calls of the same workload (set 0)."""
    if budget_s <= 0:
        return None
    import oracle
    threads, host = host_threads()   # the OpenMP default team: OMP_NUM_THREADS, else every core
    a1 = dataclasses.replace(a, sets=1)
    y = wl.make_attn2_y(a1, 0)
    q, g = wl.attn2_views(y, a.nkv)
    qb, gb = wl.bits(q), wl.bits(g)
    cache = wl.bits(wl.make_attn2_cache(a1))
    table = wl.make_attn2_table(a1, 0).numpy()
    lens = wl.make_attn2_lens(a1).numpy()
    calls, t0 = 0, time.perf_counter()
    while True:
        oracle.attn2(qb, gb, cache, a.nkv, table, lens, a.eff_window)
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s or (el / calls) * (calls + 1) > 2 * budget_s:
            break
    per_call = el / calls
    return {"value": round(a.algorithmic_bytes() / per_call / 1e9, 4), "unit": "GB/s",
            "us_per_call": round(per_call * 1e6, 1), "cores": threads, "host_cores": host,
            "kind": "oracle",
            "sample": f"{calls} full oracle calls of {a.name} (request set 0), "
                      f"OpenMP over (row, head) pairs, {threads} threads"}


def attn2_line(a: wl.Attn2Workload, args) -> dict:
    invariant = bool(getattr(args, "attn2_batch_invariant", False))
    ms, times, sets = time_attn2(a, args.steps, args.warmup, args.repeats, invariant)
    nbytes = a.algorithmic_bytes()
    gbs = nbytes / (ms * 1e-3) / 1e9
    z = qf.attn2_plan(a.nkv, a.max_model_len, a.window, 1 if invariant else a.R)
    kernels = "attn2_split" + (" + attn2_merge" if z > 1 else "")
    return {
        "metric": "attn2 achieved HBM GB/s (algorithmic bytes per call / time per call)",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "us_per_call": round(ms * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": dict(wl.describe_attn2(a), splits=z, batch_invariant_splits=invariant,
                       request_sets_rotated=sets, algorithmic_bytes_per_call=nbytes),
        "roofline": {"bound": "hbm", "kernel": f"{kernels} (the whole call)",
                     "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(a, ATTN2_COUNTERS, ATTN2_SRC)},
        "repeats_ms": [round(t, 6) for t in times],
    }


def eager_time(call, steps: int, warmup: int, repeats: int, stream):
    """Per-call time of `steps` calls issued one by one after `warmup`."""
    with torch.cuda.stream(stream):
        for i in range(warmup):
            call(i)
    torch.cuda.synchronize()
    times = []
    for _ in range(repeats):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        with torch.cuda.stream(stream):
            for i in range(steps):
                call(warmup + i)
        end.record(stream)
        torch.cuda.synchronize()
        times.append(start.elapsed_time(end) / steps)
    return sorted(times)[len(times) // 2], times


def graph_rotation_time(call, sets: int, steps: int, warmup: int, repeats: int, stream,
                        eager: bool = False):
    """Per-call time of a launch-bound kernel: one rotation of `sets` calls
    is captured in a HIP graph and replayed until about `steps` calls have
    run (the way such calls run in a decode step; issued one by one from
    Python, the host's enqueue rate would be measured instead).  Also
    returns the eager per-call time of 500 calls, for context.  With
    eager=True only `warmup` + `steps` calls are issued one by one (for
    profiler runs, where each dispatch is slow)."""
    if eager:
        ms, times = eager_time(call, steps, warmup, repeats, stream)
        return ms, times, steps, ms
    with torch.cuda.stream(stream):
        for i in range(max(warmup, sets)):
            call(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    with torch.cuda.stream(stream):
        for i in range(500):
            call(i)
    end.record(stream)
    torch.cuda.synchronize()
    eager_ms = start.elapsed_time(end) / 500
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(sets):
            call(i)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    replays = max(1, steps // sets)
    times = []
    for _ in range(repeats):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for _ in range(replays):
            graph.replay()
        end.record()
        torch.cuda.synchronize()
        times.append(start.elapsed_time(end) / (replays * sets))
    return sorted(times)[len(times) // 2], times, replays * sets, eager_ms


def time_layer_front(w: wl.LayerFrontWorkload, steps: int, warmup: int, repeats: int,
                     eager: bool = False):
    """Calls rotate over input/output sets of >= 600 MB in total, so every
    call's rows come from HBM."""
    dev = "cuda"
    per_set = w.algorithmic_bytes()
    sets = max(2, int(600e6 // per_set) + 1)
    xs = [wl.make_lf_x(w, s, device=dev) for s in range(min(sets, 64))]
    # beyond 64 distinct inputs, further sets reuse their x (only the
    # buffers differ, which keeps generation fast)
    xs = [xs[s % len(xs)].clone() if s >= len(xs) else xs[s] for s in range(sets)]
    weight = wl.make_lf_weight(w, device=dev)
    st = [torch.empty(w.rows, wl.HIDDEN, device=dev) for _ in range(sets)]
    ax = [torch.empty(w.rows, wl.HIDDEN, device=dev) for _ in range(sets)] if w.aux else None
    out = [torch.empty(w.rows, wl.HIDDEN, dtype=torch.bfloat16, device=dev) for _ in range(sets)]
    stream = torch.cuda.Stream()

    def call(i):
        s = i % sets
        qf.layer_front(xs[s], st[s], out[s], aux=None if ax is None else ax[s], weight=weight,
                       stream=stream)

    ms, times, calls, eager_ms = graph_rotation_time(call, sets, steps, warmup, repeats, stream,
                                                     eager)
    return ms, times, sets, calls, eager_ms


def layer_front_cpu_baseline(w: wl.LayerFrontWorkload, budget_s: float) -> dict | None:
    if budget_s <= 0:
        return None
    import oracle
    threads, host = host_threads()   # the OpenMP default team: OMP_NUM_THREADS, else every core
    x = wl.make_lf_x(w, 0)
    xn = x.numpy() if w.fp32_input else wl.bits(x)
    weight = wl.make_lf_weight(w)
    wn = None if weight is None else wl.bits(weight)
    calls, t0 = 0, time.perf_counter()
    while True:
        oracle.layer_front(xn, wn, aux=w.aux)
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s or (el / calls) * (calls + 1) > 2 * budget_s:
            break
    per_call = el / calls
    return {"value": round(w.algorithmic_bytes() / per_call / 1e9, 4), "unit": "GB/s",
            "us_per_call": round(per_call * 1e6, 1), "cores": threads, "host_cores": host,
            "kind": "oracle",
            "sample": f"{calls} full oracle calls of {w.name} (input set 0), OpenMP over rows, "
                      f"{threads} threads"}


def layer_front_line(w: wl.LayerFrontWorkload, args) -> dict:
    ms, times, sets, calls, eager_ms = time_layer_front(w, args.steps, args.warmup, args.repeats,
                                                        args.eager)
    nbytes = w.algorithmic_bytes()
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {
        "metric": "LayerFront achieved HBM GB/s (algorithmic bytes per call / time per call)",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": calls,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "us_per_call": round(ms * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32" if w.fp32_input else "bf16", "data": "synthetic",
        "config": dict(wl.describe_layer_front(w), sets_rotated=sets,
                       algorithmic_bytes_per_call=nbytes,
                       timing="calls issued one by one" if args.eager else
                       f"one rotation of {sets} calls captured in a HIP graph and replayed",
                       eager_us_per_call=round(eager_ms * 1e3, 3)),
        "roofline": {"bound": "hbm", "kernel": "layer_front (the whole call)",
                     "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(w, LF_COUNTERS, LF_SRC)},
        "repeats_ms": [round(t, 6) for t in times],
    }


def route_line(w: wl.RouteWorkload, args) -> dict:
    """MuseRouting calls rotate over 64 input sets (the data are a few KB),
    timed by graph replay like LayerFront's."""
    dev = "cuda"
    sets = 64
    inputs = [wl.make_route_inputs(w, s, device=dev) for s in range(sets)]
    ids = [torch.empty(w.tokens, 8, dtype=torch.int32, device=dev) for _ in range(sets)]
    wts = [torch.empty(w.tokens, 8, device=dev) for _ in range(sets)]
    stream = torch.cuda.Stream()

    def call(i):
        s = i % sets
        qf.route(inputs[s][0], inputs[s][1], w.route_scale, ids[s], wts[s], stream=stream)

    ms, times, calls, eager_ms = graph_rotation_time(call, sets, args.steps, args.warmup,
                                                     args.repeats, stream, args.eager)
    nbytes = w.algorithmic_bytes()
    gbs = nbytes / (ms * 1e-3) / 1e9
    base = None
    if args.cpu_baseline_seconds > 0:
        import oracle
        lg, bs = wl.make_route_inputs(w, 0)
        lg, bs = lg.numpy(), bs.numpy()
        ncalls, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < min(args.cpu_baseline_seconds, 2.0):
            oracle.route(lg, bs, w.route_scale)
            ncalls += 1
        per = (time.perf_counter() - t0) / ncalls
        base = {"value": round(nbytes / per / 1e9, 4), "unit": "GB/s",
                "us_per_call": round(per * 1e6, 2), "cores": 1, "kind": "oracle",
                "sample": f"{ncalls} full oracle calls of {w.name} (input set 0), one thread"}
    return {
        "metric": "MuseRouting us per call (and algorithmic GB/s)",
        "value": round(gbs, 3), "unit": "GB/s", "n_gpus": 1, "steps": calls,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "us_per_call": round(ms * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.tokens, "experts": 256, "top_k": 8,
                   "route_scale": w.route_scale, "algorithmic_bytes_per_call": nbytes,
                   "timing": "calls issued one by one" if args.eager else
                   f"one rotation of {sets} calls captured in a HIP graph and replayed",
                   "eager_us_per_call": round(eager_ms * 1e3, 3)},
        "roofline": {"bound": "hbm", "kernel": "route (the whole call)", "achieved": round(gbs, 3),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 6),
                     "traffic": None},
        "cpu_baseline": base,
        "repeats_ms": [round(t, 6) for t in times],
    }


def rotated_sets(w: wl.Workload, requested: int) -> int:
    sets = requested or w.wsets
    # enough weight sets that the rotation exceeds the 256 MB MALL
    return max(sets, int(600e6 // (w.N * wl.HIDDEN * 2)) + 1)


def copy_calibration(mb: float, steps: int) -> None:
    n = int(mb * 1e6) // 2
    src = torch.empty(n, dtype=torch.bfloat16, device="cuda").normal_()
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        dst.copy_(src)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    print(json.dumps({"copy_bytes_read": 2 * n, "copy_bytes_written": 2 * n, "steps": steps,
                      "ms_per_copy": round(ms, 6)}), flush=True)


def profile_workloads(names: list[str], steps: int, warmup: int) -> None:
    """warmup + steps eager calls per workload, announced before they are
    issued, for a profiler to attribute its per-dispatch records."""
    for name in names:
        w = workload_by_name(name)
        sets = rotated_sets(w, 0)
        pool = Pool(w, sets)
        qf.prepare(w.N, w.nkv, w.M)
        stream = torch.cuda.Stream()
        torch.cuda.synchronize()
        print(json.dumps({"profile_workload": w.name, "M": w.M, "num_kv_heads": w.nkv, "N": w.N,
                          "front_dispatches": warmup + steps, "warmup": warmup,
                          "weight_sets_rotated": sets,
                          "algorithmic_bytes": w.algorithmic_bytes()}), flush=True)
        with torch.cuda.stream(stream):
            for i in range(warmup + steps):
                pool.call(i, stream)
        torch.cuda.synchronize()
        del pool
        torch.cuda.empty_cache()
    fault = qf.device_fault()
    if fault != 0:
        raise RuntimeError(f"a profiled call gave up waiting: {qf.strerror(fault)}")


def _csv_rows(directory: str, suffix: str) -> list[dict]:
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {directory}")
    rows = []
    for f in files:
        rows += list(csv.DictReader(open(f)))
    return rows


def _front_rows(rows: list[dict], counter: str | None = None) -> list[dict]:
    out = [r for r in rows if "front_fused" in r["Kernel_Name"]
           and (counter is None or r.get("Counter_Name") == counter)]
    return sorted(out, key=lambda r: int(r["Dispatch_Id"]))


def _nkv_of(kernel_name: str) -> int:
    import re
    m = re.search(r"front_fusedILi(\d+)E", kernel_name) or re.search(r"front_fused<(\d+)>", kernel_name)
    return int(m.group(1)) if m else -1


def _split(rows: list[dict], order: list[dict]) -> dict:
    """Per workload, its post-warmup rows (dispatches come in the order the
    workloads were run, each workload's count announced beforehand)."""
    need = sum(o["front_dispatches"] for o in order)
    if len(rows) != need:
        raise SystemExit(f"{len(rows)} front dispatches recorded, {need} announced")
    out, i = {}, 0
    for o in order:
        part = rows[i:i + o["front_dispatches"]]
        i += o["front_dispatches"]
        bad = {_nkv_of(r["Kernel_Name"]) for r in part} - {o["num_kv_heads"]}
        if bad:
            raise SystemExit(f"{o['profile_workload']}: dispatches of front_fused<{bad}>")
        out[o["profile_workload"]] = part[o["warmup"]:]
    return out


def summarize_profiles(d: str, out: str | None = None) -> str:
    import statistics
    order = [json.loads(l) for l in open(os.path.join(d, "order.jsonl"))
             if l.startswith("{") and "profile_workload" in l]
    trace = _split(_front_rows(_csv_rows(os.path.join(d, "trace"), "kernel_trace.csv")), order)
    fetch = _split(_front_rows(_csv_rows(os.path.join(d, "fetch"), "counter_collection.csv"),
                               "FETCH_SIZE"), order)
    write = _split(_front_rows(_csv_rows(os.path.join(d, "write"), "counter_collection.csv"),
                               "WRITE_SIZE"), order)

    def copy_median(sub: str, counter: str) -> float:
        rows = [float(r["Counter_Value"]) for r in _csv_rows(os.path.join(d, sub),
                                                               "counter_collection.csv")
                if "copyBuffer" in r["Kernel_Name"] and r["Counter_Name"] == counter]
        return statistics.median(rows)

    calib = json.load(open(os.path.join(d, "calibration.json")))
    copy_fetch, copy_write = copy_median("calib_fetch", "FETCH_SIZE"), copy_median("calib_write",
                                                                                 "WRITE_SIZE")
    fetch_factor = calib["copy_bytes_read"] / (copy_fetch * 1024)
    write_factor = calib["copy_bytes_written"] / (copy_write * 1024)
    events = {}
    all_path = os.path.join(d, "all.jsonl")
    if os.path.exists(all_path):
        for l in open(all_path):
            if l.startswith("{") and '"workload"' in l:
                rec = json.loads(l)
                events[rec["workload"]] = rec
    record = {"kernel": "front_fused<nkv>", "kernel_sha256_16": kernel_hash(),
              "calibration": {"copy_bytes_read": calib["copy_bytes_read"],
                              "copy_bytes_written": calib["copy_bytes_written"],
                              "copy_FETCH_SIZE_KiB": copy_fetch, "copy_WRITE_SIZE_KiB": copy_write,
                              "fetch_factor": round(fetch_factor, 5),
                              "write_factor": round(write_factor, 5)},
              "workloads": {}}
    lines = ["| Workload | M | KV heads | N | bench.py us/call | trace avg us (min / max) | "
             "algorithmic GB/s | frac of 8 TB/s | FETCH KiB | WRITE KiB | HBM bytes (scaled) | "
             "traffic / algorithmic | counter GB/s | oracle us/call (threads / host cores) |",
             "|" + "---|" * 14]
    for o in order:
        name = o["profile_workload"]
        dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace[name]]
        f_kib = statistics.median(float(r["Counter_Value"]) for r in fetch[name])
        w_kib = statistics.median(float(r["Counter_Value"]) for r in write[name])
        hbm = f_kib * 1024 * fetch_factor + w_kib * 1024 * write_factor
        alg = o["algorithmic_bytes"]
        avg = sum(dur) / len(dur)
        record["workloads"][name] = {
            "FETCH_SIZE_KiB": f_kib, "WRITE_SIZE_KiB": w_kib,
            "hbm_bytes_per_launch": int(round(hbm)), "algorithmic_bytes_per_launch": alg,
            "trace_avg_us": round(avg, 3), "trace_min_us": round(min(dur), 3),
            "trace_max_us": round(max(dur), 3), "trace_dispatches": len(dur),
            "counter_dispatches": len(fetch[name])}
        ev = events.get(name, {})
        us = ev.get("us_per_call")
        base = ev.get("cpu_baseline") or {}
        gbs = alg / (us * 1e-6) / 1e9 if us else None
        cell = lambda v, f: "n/a" if v is None else f.format(v)
        lines.append(
            f"| {name} | {o['M']} | {o['num_kv_heads']} | {o['N']} | {cell(us, '{:.2f}')} | "
            f"{avg:.2f} ({min(dur):.2f} / {max(dur):.2f}) | {cell(gbs, '{:.0f}')} | "
            f"{cell(gbs and gbs / HBM_PEAK_GBS, '{:.3f}')} | {f_kib:.1f} | {w_kib:.1f} | "
            f"{hbm:,.0f} | {hbm / alg:.3f} | {hbm / (avg * 1e-6) / 1e9:.0f} | "
            f"{cell(base.get('us_per_call'), '{:,.0f}')} ({base.get('cores', '-')} / "
            f"{base.get('host_cores', '-')}) |")
    out = out or os.path.join(ROOT, "profiles", "front_fused_counters.json")
    with open(out, "w") as fh:
        json.dump(record, fh, indent=1)
        fh.write("\n")
    table = "\n".join(lines)
    print(table)
    print(f"\nwrote {out}", file=sys.stderr)
    return table


def summarize_attn2_profiles(d: str, out: str | None = None) -> str:
    """attn2 summary from a profiling directory: per workload W, the kernel
    trace under a2/W/trace and, where taken, FETCH_SIZE / WRITE_SIZE under
    a2/W/fetch and a2/W/write (each a `bench.py --attn2 W` run); the copy
    calibration and the --all event lines (all.jsonl) of the front's run in
    the same directory.  The first `skip` dispatches of each kernel are the
    run's warm-up."""
    import statistics
    skip = 20
    calib = json.load(open(os.path.join(d, "calibration.json")))

    def copy_median(sub: str, counter: str) -> float:
        return statistics.median(float(r["Counter_Value"]) for r in
                                 _csv_rows(os.path.join(d, sub), "counter_collection.csv")
                                 if "copyBuffer" in r["Kernel_Name"] and r["Counter_Name"] == counter)

    fetch_factor = calib["copy_bytes_read"] / (copy_median("calib_fetch", "FETCH_SIZE") * 1024)
    write_factor = calib["copy_bytes_written"] / (copy_median("calib_write", "WRITE_SIZE") * 1024)
    events = {}
    all_path = os.path.join(d, "all.jsonl")
    if os.path.exists(all_path):
        for l in open(all_path):
            if l.startswith("{") and '"workload"' in l:
                rec = json.loads(l)
                events[rec["workload"]] = rec
    record = {"kernel_source": os.path.relpath(ATTN2_SRC, ROOT),
              "kernel_sha256_16": kernel_hash(ATTN2_SRC),
              "fetch_scale": round(fetch_factor, 5), "write_scale": round(write_factor, 5),
              "calibration": "device-to-device copy of "
                             f"{calib['copy_bytes_read'] / 1e6:.0f} MB (torch copy_)",
              "workloads": {}}
    lines = ["| Workload | splits | bench.py us/call | trace attn2_split avg (min / max) us | "
             "trace attn2_merge avg (min / max) us | algorithmic bytes | GB/s | frac of 8 TB/s | "
             "HBM bytes per call (counters, scaled) | traffic / algorithmic | "
             "oracle us/call (threads / host cores) |", "|" + "---|" * 11]

    def stats(rows):
        dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows][skip:]
        return (sum(dur) / len(dur), min(dur), max(dur), len(dur)) if dur else None

    for name in sorted(os.listdir(os.path.join(d, "a2")),
                       key=lambda n: list(wl.ATTN2_WORKLOADS).index(n)):
        w = wl.ATTN2_WORKLOADS[name]
        base = os.path.join(d, "a2", name)
        tr = _csv_rows(os.path.join(base, "trace"), "kernel_trace.csv")
        sp = stats(sorted((r for r in tr if "attn2_split" in r["Kernel_Name"]),
                          key=lambda r: int(r["Dispatch_Id"])))
        mg = stats(sorted((r for r in tr if "attn2_merge" in r["Kernel_Name"]),
                          key=lambda r: int(r["Dispatch_Id"])))
        entry = {"trace_split_avg_us": round(sp[0], 3), "trace_split_min_us": round(sp[1], 3),
                 "trace_split_max_us": round(sp[2], 3), "trace_dispatches": sp[3]}
        if mg:
            entry.update(trace_merge_avg_us=round(mg[0], 3), trace_merge_min_us=round(mg[1], 3),
                         trace_merge_max_us=round(mg[2], 3))
        hbm = None
        if os.path.isdir(os.path.join(base, "fetch")):
            kib = {}
            for sub, counter in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
                rows = _csv_rows(os.path.join(base, sub), "counter_collection.csv")
                for kern in ("split", "merge"):
                    v = [float(r["Counter_Value"]) for r in rows
                         if f"attn2_{kern}" in r["Kernel_Name"] and r["Counter_Name"] == counter]
                    kib[f"{kern}_{sub}_kib"] = statistics.median(v) if v else 0.0
            hbm = ((kib["split_fetch_kib"] + kib["merge_fetch_kib"]) * fetch_factor +
                   (kib["split_write_kib"] + kib["merge_write_kib"]) * write_factor) * 1024
            entry.update(kib, hbm_bytes_per_call=int(round(hbm)))
        record["workloads"][name] = entry
        alg = w.algorithmic_bytes()
        ev = events.get(name, {})
        us = ev.get("us_per_call")
        gbs = alg / (us * 1e-6) / 1e9 if us else None
        cb = ev.get("cpu_baseline") or {}
        cell = lambda v, f: "n/a" if v is None else f.format(v)
        merge_cell = f"{mg[0]:.2f} ({mg[1]:.2f} / {mg[2]:.2f})" if mg else "-"
        lines.append(
            f"| {name} | {qf.attn2_plan(w.nkv, w.max_model_len, w.window, w.R)} | "
            f"{cell(us, '{:.2f}')} | {sp[0]:.2f} ({sp[1]:.2f} / {sp[2]:.2f}) | {merge_cell} | "
            f"{alg:,} | {cell(gbs, '{:.0f}')} | {cell(gbs and gbs / HBM_PEAK_GBS, '{:.3f}')} | "
            f"{cell(hbm, '{:,.0f}')} | {cell(hbm and hbm / alg, '{:.3f}')} | "
            f"{cell(cb.get('us_per_call'), '{:,.0f}')} ({cb.get('cores', '-')} / "
            f"{cb.get('host_cores', '-')}) |")
    out = out or ATTN2_COUNTERS
    with open(out, "w") as fh:
        json.dump(record, fh, indent=1)
        fh.write("\n")
    table = "\n".join(lines)
    print(table)
    print(f"\nwrote {out}", file=sys.stderr)
    return table


def attn2_all_lines(a) -> None:
    """The attn2 part of the --all lines: one JSON line per timing workload on
    stderr, with the oracle on this host."""
    for aw in wl.ATTN2_WORKLOADS.values():
        if aw is wl.A0:   # the small parity case, not a timing workload
            continue
        line = attn2_line(aw, a)
        line["cpu_baseline"] = attn2_cpu_baseline(aw, a.all_cpu_seconds)
        print(json.dumps({"workload": aw.name, "splits": line["config"]["splits"],
                          "us_per_call": line["us_per_call"], "GB_per_s": line["value"],
                          "frac_of_8TBs": line["roofline"]["frac"], "roofline": line["roofline"],
                          "cpu_baseline": line["cpu_baseline"],
                          "request_sets_rotated": line["config"]["request_sets_rotated"]}),
              file=sys.stderr, flush=True)


def all_lines(a) -> None:
    """One JSON line per workload and sweep point on stderr: timing, the
    roofline with counter traffic when recorded for this kernel source, and
    the oracle on this host; then the plain streaming read per weight size,
    attn2 and LayerFront."""
    others = list(wl.WORKLOADS.values()) + [wl.sweep(m, k) for k in wl.SWEEP_NKV
                                            for m in wl.SWEEP_M]
    for o in others:
        oms, _ = time_front(o, rotated_sets(o, 0), a.steps, a.warmup, a.repeats)
        ogbs = o.algorithmic_bytes() / (oms * 1e-3) / 1e9
        traffic = measured_traffic(o)
        print(json.dumps({"workload": o.name, "M": o.M, "num_kv_heads": o.nkv, "N": o.N,
                          "us_per_call": round(oms * 1e3, 3), "GB_per_s": round(ogbs, 1),
                          "frac_of_8TBs": round(ogbs / HBM_PEAK_GBS, 4),
                          "weight_sets_rotated": rotated_sets(o, 0),
                          "roofline": {"bound": "hbm", "kernel": f"front_fused<{o.nkv}>",
                                       "achieved": round(ogbs, 2), "peak": HBM_PEAK_GBS,
                                       "unit": "GB/s", "frac": round(ogbs / HBM_PEAK_GBS, 4),
                                       "traffic": None if traffic is None else int(traffic)},
                          "cpu_baseline": cpu_baseline(o, a.all_cpu_seconds, single_core=False)}),
              file=sys.stderr, flush=True)
    # Context per weight size: the plain streaming read of one weight set,
    # rotated over as many sets as the front's sweep points use.
    for k in wl.SWEEP_NKV:
        sw = wl.sweep(1, k)
        ctx = stream_context(sw, rotated_sets(sw, 0), a.steps, a.repeats)
        print(json.dumps({"workload": f"stream_read_n{sw.N}", "bytes_per_call": ctx["bytes_per_call"],
                          "us_per_call": ctx["us_per_call"], "GB_per_s": ctx["GB_per_s"],
                          "frac_of_8TBs": ctx["frac_of_8TBs"],
                          "buffers_rotated": ctx["buffers_rotated"]}),
              file=sys.stderr, flush=True)
    attn2_all_lines(a)
    for lw in wl.LAYER_FRONT_WORKLOADS.values():
        line = layer_front_line(lw, a)
        line["cpu_baseline"] = layer_front_cpu_baseline(lw, a.all_cpu_seconds)
        print(json.dumps({"workload": lw.name, "us_per_call": line["us_per_call"],
                          "GB_per_s": line["value"], "frac_of_8TBs": line["roofline"]["frac"],
                          "roofline": line["roofline"], "cpu_baseline": line["cpu_baseline"],
                          "sets_rotated": line["config"]["sets_rotated"]}),
              file=sys.stderr, flush=True)


def main():
    a = parse()
    if a.summarize_profiles:
        summarize_profiles(a.summarize_profiles)
        return
    if a.summarize_attn2_profiles:
        summarize_attn2_profiles(a.summarize_attn2_profiles)
        return
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on exactly one GPU (asked for {a.gpus}); the front is a "
              "single-GPU kernel: several GPUs would each run it on their own KV heads' share "
              "of the weights and cache, with no traffic between them",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    if a.copy_calibration > 0:
        copy_calibration(a.copy_calibration, a.steps)
        return
    if a.profile_workloads:
        profile_workloads(a.profile_workloads.split(","), a.steps, a.warmup)
        return
    if a.route:
        if a.route not in wl.ROUTE_WORKLOADS:
            raise SystemExit(f"unknown routing workload {a.route}")
        print(json.dumps(route_line(wl.ROUTE_WORKLOADS[a.route], a)), flush=True)
        return
    if a.layer_front:
        if a.layer_front not in wl.LAYER_FRONT_WORKLOADS:
            raise SystemExit(f"unknown LayerFront workload {a.layer_front}")
        lw = wl.LAYER_FRONT_WORKLOADS[a.layer_front]
        line = layer_front_line(lw, a)
        line["cpu_baseline"] = layer_front_cpu_baseline(lw, a.cpu_baseline_seconds)
        print(json.dumps(line), flush=True)
        return
    if a.attn2_lines:
        attn2_all_lines(a)
        return
    if a.attn2:
        if a.attn2 not in wl.ATTN2_WORKLOADS:
            raise SystemExit(f"unknown attn2 workload {a.attn2}")
        aw = wl.ATTN2_WORKLOADS[a.attn2]
        line = attn2_line(aw, a)
        line["cpu_baseline"] = attn2_cpu_baseline(aw, a.cpu_baseline_seconds)
        print(json.dumps(line), flush=True)
        return
    w = workload_by_name(a.workload)
    sets = rotated_sets(w, a.wsets)
    ms, times = time_front(w, sets, a.steps, a.warmup, a.repeats)
    nbytes = w.algorithmic_bytes()
    gbs = nbytes / (ms * 1e-3) / 1e9
    if a.all:
        all_lines(a)
    base = cpu_baseline(w, a.cpu_baseline_seconds)
    traffic = measured_traffic(w)
    context = stream_context(w, sets, a.steps, a.repeats)
    out = {
        "metric": "QKV-front achieved HBM GB/s (algorithmic bytes per call / time per call); "
                  "us_per_call alongside, fraction of peak in roofline.frac",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 6),
        "us_per_call": round(ms * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": dict(wl.describe(w), weight_sets_rotated=sets,
                       algorithmic_bytes_per_call=nbytes),
        "roofline": {"bound": "hbm", "kernel": f"front_fused<{w.nkv}> (the whole call)",
                     "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else int(traffic)},
        "cpu_baseline": base,
        "stream_context": context,
        "repeats_ms": [round(t, 6) for t in times],
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
