"""Throughput of MoE dispatch (layout + scatter) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole dispatch hot path over one batch: the layout
(count, prefix sums, stable slots, inverse maps) and the row scatter into the
rank-contiguous and expert-major buffers, on inputs already resident in HBM.
The default workload is 4096 tokens x 7168 bf16, top-8 of 256 experts in 8
logical ranks with 5% of the routing entries masked.

Each timed step is one dispatch_layout_and_scatter call, started with a cold
Infinity Cache: before it, outside its HIP events, 512 MiB are written and
read back. Prints one JSON line with the throughput in algorithmic GB/s (bytes
the method must move per step / median event time per step), the scatter
kernel's roofline (achieved bandwidth against the 8 TB/s HBM peak, timed with
HIP events on the stream the kernel runs on, under the same flush), the same
step back to back without flushes as a side figure, and the CPU oracle's
throughput on the same input as a baseline.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "dispatch GB/s & % HBM peak, 4096 tok×7168 bf16, top-8 of 256 experts"
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
SCATTER_SOURCES = [os.path.join(ROOT, "moe_token_dispatch_amd", "csrc", f)
                   for f in ("dispatch_scatter.hip", "dispatch_device.hpp", "dispatch_common.hpp")]
COMBINE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "combine_traffic.json")
READ_AHEAD_MAX_BYTES = 160 << 20  # token rows + scale factors the layout reads ahead, at most
EXPAND_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "expand_scatter_traffic.json")
COMBINE_SOURCES = [os.path.join(ROOT, "moe_token_dispatch_amd", "csrc", f)
                   for f in ("dispatch_combine.hip", "dispatch_device.hpp")]


def traffic_file(workload):
    """Committed counter summary of the dispatch scatter on one workload."""
    return os.path.join(ROOT, "profiles", f"scatter_traffic_{workload}.json")


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100, help="timed steps, each after a cache flush")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--warm-steps", type=int, default=2000,
                    help="steps of the side figure timed back to back without flushes")
    ap.add_argument("--workload", default=None, help="workload name (default: the metric workload)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU oracle time budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph-steps", type=int, default=1000,
                    help="steps replayed from a captured HIP graph, reported beside the eager steps (0 = skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (for counter calibration)")
    ap.add_argument("--expand", action="store_true",
                    help="measure the receiver-side expand instead: S sources of the workload send to rank 0")
    ap.add_argument("--sources", type=int, default=8, help="sources for --expand")
    ap.add_argument("--combine", action="store_true",
                    help="measure the combine instead: weighted gather of the expert-major rows back to tokens")
    ap.add_argument("--latency", action="store_true",
                    help="per-step latency of small (decode-sized) batches of the workload's shape: "
                         "the one call against the layout and scatter calls (with --expand: small "
                         "receive buffers of --sources sources)")
    return ap.parse_args()


def algorithmic_bytes(t, k, e, r, idx_bytes, row_bytes, s, t_live, p_rows, n_rank):
    """Bytes the method must move per step (workspace traffic excluded).

    Routing read + each live token row read once + every rank row and every
    expert-major row (pads included) written + counts, psums, slot maps and
    inverse maps written.
    """
    row = row_bytes + 4 * s
    layout = t * k * idx_bytes + 4 * (2 * e + 2 * r + 2 + 2 * t * k + p_rows + n_rank)
    scatter_rows = t_live * row + (n_rank + p_rows) * row
    return layout + scatter_rows, layout, scatter_rows


def scatter_launch_bytes(t, k, e, row_bytes, s, t_live, p_rows, n_rank):
    """Algorithmic bytes of one scatter launch: live rows read once, slot maps
    read, every destination row written (pads as zeros)."""
    row = row_bytes + 4 * s
    return t_live * row + (n_rank + p_rows) * row + 2 * 4 * t * k + 4 * (2 * e + 1)


def source_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(path, sources=SCATTER_SOURCES, workload=None):
    """Bytes per launch of a kernel from committed rocprofv3 counters
    (L2-to-fabric bytes: FETCH_SIZE + WRITE_SIZE scaled by a plain copy), or
    None when they are missing, were taken on another workload or on another
    version of the kernel's source."""
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != source_digest(sources):
        return None
    if workload is not None and rec.get("workload") != workload:
        return None
    return rec.get("hbm_bytes_per_launch")


def copy_calibration():
    import torch

    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    reps = 20
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copy_GBps": 2 * n / dt / 1e9}), flush=True)


def measure_device_ceiling(torch):
    """Practical HBM ceilings on this machine: torch's device copy and fill."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(3)
    b = torch.empty_like(a)
    out = {}
    for name, fn, nbytes in (("copy", lambda: b.copy_(a), 2 * n), ("fill", lambda: b.fill_(7), n)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        out[f"{name}_GBps"] = round(nbytes * 10 / (time.perf_counter() - t0) / 1e9, 1)
    del a, b
    torch.cuda.empty_cache()
    return out


def cpu_baseline(inp, w, budget_s):
    """The CPU oracle as it stands (single-threaded C), layout + scatter of the
    same input, repeated until the time budget is spent, on one pinned core.
    Returns the medians of the step, the layout and the scatter."""
    import oracle

    prep = oracle.Prepared(inp.topk_idx, w.num_experts, w.num_ranks, w.alignment, inp.x_bytes(), inp.x_sf)
    # Pin this thread to one core while the oracle runs (restored afterwards).
    allowed = os.sched_getaffinity(0)
    os.sched_setaffinity(0, {min(allowed)})
    try:
        return _time_oracle(prep, budget_s)
    finally:
        os.sched_setaffinity(0, allowed)


def host_cpu():
    """Model name and logical CPU count of the host the oracle ran on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "logical_cpus": os.cpu_count(), "allowed_cpus": len(os.sched_getaffinity(0))}


def _time_oracle(prep, budget_s):
    prep.run_layout()
    prep.run_scatter()  # warm-up
    times, lay_t, sc_t = [], [], []
    t_end = time.perf_counter() + budget_s
    while time.perf_counter() < t_end or len(times) < 3:
        t0 = time.perf_counter()
        rc = prep.run_layout()
        t1 = time.perf_counter()
        rc |= prep.run_scatter()
        t2 = time.perf_counter()
        times.append(t2 - t0)
        lay_t.append(t1 - t0)
        sc_t.append(t2 - t1)
        if rc:
            raise RuntimeError(f"oracle status {rc}")
    return statistics.median(times), len(times), statistics.median(lay_t), statistics.median(sc_t)


def receive_buffer(base, s_count, t, rank, dev):
    """S sources, each the workload's shape at t tokens with its own seed, run
    the sender path on the GPU; receiver `rank` gets every source's block in a
    fixed-stride receive buffer of t rows per source (the most a source can
    send). Returns (recv_topk, counts, recv_buf, recv_sf, rows per source)."""
    import dataclasses

    import torch

    import moe_token_dispatch_amd as M
    import workloads as W

    k, e, r = base.num_topk, base.num_experts, base.num_ranks
    s_f, rb = base.sf_per_token, base.row_bytes
    m = t
    recv_buf = torch.zeros((s_count * m, rb), dtype=torch.uint8, device=dev)
    recv_sf = torch.zeros((s_count * m, s_f), dtype=torch.float32, device=dev) if s_f else None
    recv_topk = torch.full((s_count * m, k), -1, dtype=torch.int64, device=dev)
    counts = torch.zeros(s_count, dtype=torch.int32, device=dev)
    for s in range(s_count):
        w = dataclasses.replace(base, num_tokens=t, seed=base.seed * 1000 + s)
        inp = W.make_inputs(w)
        prob = M.make_problem(t, k, e, r, w.alignment, 8, rb, s_f)
        lay, ws, rows = M.alloc_layout(prob, dev), M.alloc_workspace(prob, dev), M.alloc_rows(prob, dev)
        topk_d = torch.from_numpy(inp.topk_idx).to(dev)
        x_d = inp.x.view(torch.uint8).to(dev)
        sf_d = None if inp.x_sf is None else torch.from_numpy(inp.x_sf).to(dev)
        M.dispatch_layout(prob, topk_d, lay, ws)
        M.dispatch_scatter(prob, lay, x_d, sf_d, rows.rank_x, rows.rank_sf, rows.recv_x, rows.recv_sf)
        lo, hi = int(lay.rank_psum[rank].item()), int(lay.rank_psum[rank + 1].item())
        n = hi - lo
        # Stand-in for the transport: the block lands at the source's region.
        recv_buf[s * m:s * m + n] = rows.rank_x[lo:hi]
        if s_f:
            recv_sf[s * m:s * m + n] = rows.rank_sf[lo:hi]
        recv_topk[s * m:s * m + n] = topk_d.index_select(0, lay.rank_src_token_idx[lo:hi].long())
        counts[s] = n
        del lay, ws, rows, topk_d, x_d, sf_d
    return recv_topk, counts, recv_buf, recv_sf, m


def expand_bench(args):
    """Receiver-side expand: S sources, each the chosen workload with its own
    seed, run the sender path on the GPU; receiver rank 0 gets every source's
    rank-0 block in a fixed-stride receive buffer (T rows per source, the
    most a source can send) and expands it into its expert-major buffer."""
    import torch

    import moe_token_dispatch_amd as M
    import workloads as W

    dev = "cuda:0"
    base = W.get(args.workload or W.METRIC_WORKLOAD)
    s_count, rank = args.sources, 0
    t, k, e, r = base.num_tokens, base.num_topk, base.num_experts, base.num_ranks
    s_f, rb = base.sf_per_token, base.row_bytes
    recv_topk, counts, recv_buf, recv_sf, m = receive_buffer(base, s_count, t, rank, dev)
    q = M.make_expand_problem(s_count, m, k, e, r, rank, base.alignment, 8, rb, s_f)
    elay = M.alloc_expand_layout(q, dev)
    ews = M.alloc_expand_workspace(q, dev)
    recv_x = torch.empty((max(q.recv_capacity_rows, 1), rb), dtype=torch.uint8, device=dev)
    out_sf = torch.empty((max(q.recv_capacity_rows, 1), s_f), dtype=torch.float32, device=dev) if s_f else None
    stream = torch.cuda.current_stream(dev)
    # A prepared plan: one C call per step (the layout and scatter kernels, or
    # one kernel for a small receive buffer).
    plan = M.ExpandPlan(q, recv_topk, counts, elay, ews, recv_buf, recv_sf, recv_x, out_sf, stream)
    scratch = torch.empty(64 << 20, dtype=torch.int64, device=dev)
    sink = torch.empty((), dtype=torch.int64, device=dev)

    def evict(i):  # as in the dispatch bench: 512 MiB written, then read back
        scratch.fill_(i)
        torch.sum(scratch, dim=0, out=sink)

    for _ in range(args.warmup):
        plan()
    torch.cuda.synchronize()
    if int(elay.status.item()) != 0:
        raise RuntimeError(f"expand status {int(elay.status.item())}")
    marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i, (e0, e1) in enumerate(marks):
        evict(i)
        e0.record(stream)
        plan()
        e1.record(stream)
    torch.cuda.synchronize()
    dt = statistics.median(a.elapsed_time(b) for a, b in marks) / 1e3
    dt_mean = statistics.mean(a.elapsed_time(b) for a, b in marks) / 1e3
    warm_steps = max(args.steps, args.warm_steps)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for _ in range(warm_steps):
        plan()
    torch.cuda.synchronize()
    warm_s = (time.perf_counter() - w0) / warm_steps
    received = int(counts.sum().item())
    p_rows = int(elay.expert_psum[-1].item())
    local = e // r
    row = rb + 4 * s_f
    total_b = received * k * 8 + 4 * s_count + received * row + p_rows * row + \
        4 * (2 * local + 2 + s_count * m * k + p_rows)
    # The expand's row copy alone on its saved layout, HIP events on the launch
    # stream: every received row read once, every expert-major row written
    # (pads as zeros), the slot map read.
    scatter_b = received * row + p_rows * row + 4 * s_count * m * k + 4 * (2 * local + 1)
    # The row copy under the same flush: the layout call, then an event, then
    # the scatter call, on at least 16 steps.
    roof = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(max(16, args.steps))]
    torch.cuda.synchronize()
    for i, (e0, e1, e2) in enumerate(roof):
        evict(i)
        e0.record(stream)
        plan.layout()
        e1.record(stream)
        plan.scatter()
        e2.record(stream)
    torch.cuda.synchronize()
    sc_s = statistics.mean(b.elapsed_time(c) for _, b, c in roof) / 1e3
    lay_s = statistics.mean(a.elapsed_time(b) for a, b, _ in roof) / 1e3
    del scratch, sink
    out = {
        "metric": "receiver-side expand GB/s & % HBM peak",
        "value": round(total_b / dt / 1e9, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(dt * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "u8", "data": "synthetic",
        "config": {"workload": f"expand of {s_count} x {base.name} into rank {rank}", "sources": s_count,
                   "rows_per_source": m, "received_rows": received, "expert_major_rows": p_rows,
                   "local_experts": local, "expert_alignment": base.alignment},
        "timing": ("median of HIP-event step times (one prepared call each); before each step, outside its "
                   "events, 512 MiB are written and read back"),
        "step_mean_us": round(dt_mean * 1e6, 2),
        "hbm_frac": round(total_b / dt / 1e9 / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_step": total_b,
        "layout_events_us_mean": round(lay_s * 1e6, 2),
        "warm_back_to_back": {"steps": warm_steps, "us_per_step": round(warm_s * 1e6, 2),
                              "value": round(total_b / warm_s / 1e9, 1),
                              "hbm_frac": round(total_b / warm_s / 1e9 / HBM_PEAK_GBPS, 4)},
        "roofline": {
            "kernel": "scatter_kernel (expand)", "bound": "hbm",
            "achieved": round(scatter_b / sc_s / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(scatter_b / sc_s / 1e9 / HBM_PEAK_GBPS, 4),
            "traffic": load_traffic(EXPAND_TRAFFIC_FILE, SCATTER_SOURCES, base.name),
            "algorithmic_bytes_per_launch": scatter_b, "launch_us_mean": round(sc_s * 1e6, 2),
            "event_samples": len(roof),
        },
    }
    print(json.dumps(out), flush=True)


def combine_bench(args):
    """Combine: out[t] = sum_k w[t, k] * y[expert_slot[t, k]] over the workload's
    layout, with y a bf16 expert-output buffer of the expert-major rows."""
    import numpy as np
    import torch

    import moe_token_dispatch_amd as M
    import workloads as W

    dev = "cuda:0"
    w = W.get(args.workload or W.METRIC_WORKLOAD)
    if w.dtype != "bf16":
        raise SystemExit("--combine needs a bf16 workload (expert outputs are bf16)")
    t, k = w.num_tokens, w.num_topk
    inp = W.make_inputs(w, with_x=False)
    prob = M.make_problem(t, k, w.num_experts, w.num_ranks, w.alignment, 8, w.row_bytes, 0,
                          flags=M.EXPERT_MAJOR)
    lay, ws = M.alloc_layout(prob, dev), M.alloc_workspace(prob, dev)
    M.dispatch_layout(prob, torch.from_numpy(inp.topk_idx).to(dev), lay, ws)
    torch.cuda.synchronize()
    if int(lay.status.item()) != 0:
        raise RuntimeError(f"layout status {int(lay.status.item())}")
    p_rows = int(lay.expert_psum[-1].item())
    y = W.make_expert_out(w, max(p_rows, 1)).to(dev)
    wts = torch.from_numpy(W.make_topk_weights(w, inp.topk_idx)).to(dev)
    slots = lay.expert_slot.view(t, k)
    out = torch.empty((t, w.hidden), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    lib = M.load_library()
    import ctypes
    q = M.CombineProblem(t, k, 0, w.hidden, y.shape[0])
    argv = (ctypes.byref(q), ctypes.c_void_p(slots.data_ptr()), ctypes.c_void_p(wts.data_ptr()),
            ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
    for _ in range(args.warmup):
        lib.dispatch_combine(*argv)
    torch.cuda.synchronize()
    rc = 0
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        rc |= lib.dispatch_combine(*argv)
    ev1.record(stream)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    if rc:
        raise RuntimeError(f"dispatch_combine returned {rc}")
    launch_s = ev0.elapsed_time(ev1) / 1e3 / max(args.steps, 1)
    pairs = int((inp.topk_idx >= 0).sum())
    total_b = t * k * 8 + pairs * w.row_bytes + t * w.row_bytes
    res = {
        "metric": "combine GB/s & % HBM peak",
        "value": round(total_b / dt / 1e9, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(dt * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"combine of {w.name}", "num_tokens": t, "hidden": w.hidden, "num_topk": k,
                   "routed_pairs": pairs, "expert_major_rows": p_rows},
        "hbm_frac": round(total_b / dt / 1e9 / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_step": total_b,
        "roofline": {
            "kernel": "combine_kernel", "bound": "hbm",
            "achieved": round(total_b / launch_s / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(total_b / launch_s / 1e9 / HBM_PEAK_GBPS, 4),
            "traffic": load_traffic(COMBINE_TRAFFIC_FILE, COMBINE_SOURCES, w.name),
            "algorithmic_bytes_per_launch": total_b, "launch_us_mean": round(launch_s * 1e6, 2),
        },
    }
    print(json.dumps(res), flush=True)


def expand_latency_bench(args):
    """Microseconds per step of the receiver-side expand for small receive
    buffers: S sources of t tokens of the workload's shape into rank 0,
    through a prepared plan; the layout and scatter calls against the one
    call (one kernel up to 2048 routing entries). HIP events on the launch
    stream around many back-to-back steps."""
    import torch

    import moe_token_dispatch_amd as M
    import workloads as W

    dev = "cuda:0"
    stream = torch.cuda.current_stream(dev)
    base = W.get(args.workload or W.METRIC_WORKLOAD)
    s_count, rank, reps = args.sources, 0, max(100, args.steps)
    k, e, r = base.num_topk, base.num_experts, base.num_ranks

    def per_step_us(fn):
        for _ in range(max(20, args.warmup)):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    rows_out = []
    for t in (1, 4, 16, 32, 48, 64):
        recv_topk, counts, recv_buf, recv_sf, m = receive_buffer(base, s_count, t, rank, dev)
        q = M.make_expand_problem(s_count, m, k, e, r, rank, base.alignment, 8, base.row_bytes, base.sf_per_token)
        lay, ws = M.alloc_expand_layout(q, dev), M.alloc_expand_workspace(q, dev)
        cap = max(q.recv_capacity_rows, 1)
        recv_x = torch.empty((cap, base.row_bytes), dtype=torch.uint8, device=dev)
        out_sf = torch.empty((cap, base.sf_per_token), dtype=torch.float32, device=dev) if base.sf_per_token else None
        plan = M.ExpandPlan(q, recv_topk, counts, lay, ws, recv_buf, recv_sf, recv_x, out_sf, stream)
        two = per_step_us(lambda: (plan.layout(), plan.scatter()))
        one = per_step_us(plan)
        if int(lay.status.item()) != 0:
            raise RuntimeError(f"expand status {int(lay.status.item())}")
        rows_out.append({"tokens_per_source": t, "receive_rows": s_count * m,
                         "received_rows": int(counts.sum().item()),
                         "us_two_calls": round(two, 2), "us_one_call": round(one, 2)})
    print(json.dumps({"metric": "receiver-side expand latency of small receive buffers", "unit": "us per step",
                      "higher_is_better": False, "workload": base.name, "sources": s_count, "steps": reps,
                      "what": "HIP events around back-to-back steps of a prepared expand plan",
                      "batches": rows_out}), flush=True)


def latency_bench(args):
    """Microseconds per step for small batches of the workload's shape (its
    experts, ranks, top-k and row width), through a prepared plan: the one
    call (one kernel up to 3072 (token, k) pairs, 2048 with zeroed pad rows)
    and the layout and scatter calls. HIP events on the launch stream around
    many back-to-back steps."""
    import dataclasses

    import torch

    import moe_token_dispatch_amd as M
    import workloads as W

    dev = "cuda:0"
    stream = torch.cuda.current_stream(dev)
    base = W.get(args.workload or W.METRIC_WORKLOAD)
    reps = max(100, args.steps)

    def per_step_us(fn):
        for _ in range(max(20, args.warmup)):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    rows_out = []
    for t in (1, 16, 64, 128, 256, 384):
        w = dataclasses.replace(base, num_tokens=t)
        inp = W.make_inputs(w)
        prob = M.make_problem(t, w.num_topk, w.num_experts, w.num_ranks, w.alignment, 8, w.row_bytes,
                              w.sf_per_token)
        lay, ws, rows = M.alloc_layout(prob, dev), M.alloc_workspace(prob, dev), M.alloc_rows(prob, dev)
        sf = None if inp.x_sf is None else torch.from_numpy(inp.x_sf).to(dev)
        plan = M.Plan(prob, torch.from_numpy(inp.topk_idx).to(dev), lay, ws, inp.x.view(torch.uint8).to(dev), sf,
                      rows, stream)
        two = per_step_us(lambda: (plan.layout(), plan.scatter()))
        one = per_step_us(plan)
        rows_out.append({"tokens": t, "kernels_one_call": M.dispatch_kernel_count(prob)[1],
                         "us_two_calls": round(two, 2), "us_one_call": round(one, 2)})
    print(json.dumps({"metric": "dispatch step latency of small batches", "unit": "us per step",
                      "higher_is_better": False, "workload": base.name, "steps": reps,
                      "what": "HIP events around back-to-back steps of a prepared plan", "batches": rows_out}),
          flush=True)


def graph_step(args, dev, stream, prob, topk_d, lay, ws, x_d, sf_d, rows, total_b, evict):
    """The same step (the combined call) captured once into a HIP graph and
    replayed, back to back and after the same flush as the timed steps: the
    kernels and buffers are the eager step's; only the launch path differs."""
    import statistics

    import torch

    import moe_token_dispatch_amd as M

    def call():
        M.dispatch_layout_and_scatter(prob, topk_d, lay, ws, x_d, sf_d, rows.rank_x, rows.rank_sf, rows.recv_x,
                                      rows.recv_sf)

    side = torch.cuda.Stream(device=dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        call()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        call()
    for _ in range(max(1, args.graph_steps // 10)):
        graph.replay()
    torch.cuda.synchronize()
    g0 = time.perf_counter()
    for _ in range(args.graph_steps):
        graph.replay()
    torch.cuda.synchronize()
    g_s = (time.perf_counter() - g0) / args.graph_steps
    marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(max(16, args.steps))]
    for i, (e0, e1) in enumerate(marks):
        evict(i)
        e0.record(stream)
        graph.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    flushed_us = statistics.mean(a.elapsed_time(b) * 1e3 for a, b in marks)
    if int(lay.status.item()) != 0:
        raise RuntimeError("graph replay left a non-zero layout status")
    return {"value": round(total_b / g_s / 1e9, 1), "unit": "GB/s", "steps": args.graph_steps,
            "us_per_step": round(g_s * 1e6, 2),
            "flushed_us_per_step": round(flushed_us, 2),
            "flushed_value": round(total_b / (flushed_us * 1e-6) / 1e9, 1),
            "what": "the combined call captured into a HIP graph and replayed (back to back; and flushed as "
                    "the timed steps)"}


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the dispatch path here has no cross-GPU exchange).", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.latency:
        expand_latency_bench(args) if args.expand else latency_bench(args)
        return
    if args.expand:
        expand_bench(args)
        return
    if args.combine:
        combine_bench(args)
        return

    import numpy as np
    import torch

    import moe_token_dispatch_amd as M
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = "cuda:0"
    w = W.get(args.workload or W.METRIC_WORKLOAD)
    inp = W.make_inputs(w)
    t, k = inp.topk_idx.shape
    s = w.sf_per_token
    prob = M.make_problem(t, k, w.num_experts, w.num_ranks, w.alignment, 8, w.row_bytes, s)
    lay = M.alloc_layout(prob, dev)
    ws = M.alloc_workspace(prob, dev)
    rows = M.alloc_rows(prob, dev)
    topk_d = torch.from_numpy(inp.topk_idx).to(dev)
    x_d = inp.x.view(torch.uint8).to(dev)
    sf_d = None if inp.x_sf is None else torch.from_numpy(inp.x_sf).to(dev)
    stream = torch.cuda.current_stream(dev)
    plan = M.Plan(prob, topk_d, lay, ws, x_d, sf_d, rows, stream)
    # A batch that fits one layout tile is dispatched by one kernel (the
    # combined call); then the events bracket that kernel. Otherwise the step
    # is the layout call and the scatter call, the same kernels the combined
    # call would launch, with the events around the scatter.
    _, step_kernels = M.dispatch_kernel_count(prob)
    one_kernel = step_kernels == 1

    # 512 MiB written, then read back, before every flushed step (outside its
    # events): the write evicts the step's data from the 256 MB Infinity Cache
    # and the read turns the lines the write left dirty into clean ones, so
    # that the timed step is not charged the sweep's own write-back.
    scratch = torch.empty(64 << 20, dtype=torch.int64, device=dev)
    sink = torch.empty((), dtype=torch.int64, device=dev)

    def evict(i):
        scratch.fill_(i)
        torch.sum(scratch, dim=0, out=sink)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    for _ in range(args.warmup):
        plan()
    torch.cuda.synchronize()
    if int(lay.status.item()) != 0:
        raise RuntimeError(f"dispatch status {int(lay.status.item())}")

    # The timed steps: one dispatch_layout_and_scatter call each (the layout
    # kernels read the token rows ahead, then the scatter), after a flush,
    # HIP events on the launch stream around the call.
    marks = [(ev(), ev()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i, (e0, e1) in enumerate(marks):
        evict(i)
        e0.record(stream)
        plan()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_us = [a.elapsed_time(b) * 1e3 for a, b in marks]

    # The dominant kernel on its own, under the same flush: the same two
    # parts the combined call enqueues (the read-ahead layout, then the
    # scatter with the read-ahead hint, which the library ignores for rows it
    # does not read ahead), with an event between them, on at least 16 steps.
    n_roof = max(16, args.steps)
    roof = [(ev(), ev(), ev()) for _ in range(n_roof)]
    torch.cuda.synchronize()
    for i, (e0, e1, e2) in enumerate(roof):
        evict(i)
        e0.record(stream)
        if one_kernel:
            plan()
        else:
            plan.layout_read_ahead()
            e1.record(stream)
            plan.scatter(read_ahead=True)
        e2.record(stream)
    torch.cuda.synchronize()
    if one_kernel:
        kernel_us = [a.elapsed_time(c) * 1e3 for a, _, c in roof]
        layout_us = [0.0]
    else:
        kernel_us = [b.elapsed_time(c) * 1e3 for _, b, c in roof]
        layout_us = [a.elapsed_time(b) * 1e3 for a, b, _ in roof]

    p_rows = int(lay.expert_psum[-1].item())
    n_rank = int(lay.rank_psum[-1].item())
    t_live = int((inp.topk_idx >= 0).any(axis=1).sum())
    p_valid = int((inp.topk_idx >= 0).sum())
    total_b, layout_b, _ = algorithmic_bytes(t, k, w.num_experts, w.num_ranks, 8, w.row_bytes, s,
                                             t_live, p_rows, n_rank)
    sc_b = scatter_launch_bytes(t, k, w.num_experts, w.row_bytes, s, t_live, p_rows, n_rank)
    # Rows that the layout reads ahead (up to 160 MB with their scale
    # factors) are copied by the split kernel, others by scatter_kernel.
    read_ahead = t * (w.row_bytes + 4 * s) <= READ_AHEAD_MAX_BYTES
    roof_kernel, roof_b = ("split_scatter_kernel" if read_ahead else "scatter_kernel"), sc_b
    if one_kernel:  # the one kernel moves the whole step's bytes
        roof_kernel, roof_b = "assign_kernel (one-kernel layout + scatter)", total_b
    # The figure is the median flushed step (the protocol's median of the
    # timed iterations); the mean, p10 and p90 are in step_events.
    step_median_us = statistics.median(step_us)
    ms_per_step = step_median_us / 1e3
    value = total_b / (step_median_us * 1e-6) / 1e9
    kernel_mean_us = statistics.mean(kernel_us)
    achieved = roof_b / (kernel_mean_us * 1e-6) / 1e9
    traffic = None if one_kernel else load_traffic(traffic_file(w.name), workload=w.name)

    def quant(us):
        v = sorted(us)
        q = lambda f: v[min(len(v) - 1, int(f * (len(v) - 1) + 0.5))]  # noqa: E731
        return {"mean_us": round(statistics.mean(v), 2), "p10_us": round(q(0.1), 2),
                "median_us": round(q(0.5), 2), "p90_us": round(q(0.9), 2)}

    # Back to back, no flush between steps (the rows and the layout's inputs
    # stay in the Infinity Cache from one step to the next): wall clock over
    # warm_steps combined calls.
    warm_steps = max(args.steps, args.warm_steps)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for _ in range(warm_steps):
        plan()
    torch.cuda.synchronize()
    warm_s = (time.perf_counter() - w0) / warm_steps
    warm = {"steps": warm_steps, "us_per_step": round(warm_s * 1e6, 2),
            "value": round(total_b / warm_s / 1e9, 1), "unit": "GB/s",
            "hbm_frac": round(total_b / warm_s / 1e9 / HBM_PEAK_GBPS, 4),
            "what": "the same combined call back to back with no flush (wall clock)"}

    # Cached dispatch: the same layout replayed, scatter only (the routing is
    # unchanged, so the layout is not recomputed), back to back.
    replay_steps = max(1, warm_steps // 4)
    torch.cuda.synchronize()
    r0 = time.perf_counter()
    for _ in range(replay_steps):
        plan.scatter()
    torch.cuda.synchronize()
    replay_s = (time.perf_counter() - r0) / replay_steps
    replay = {"value": round(sc_b / replay_s / 1e9, 1), "unit": "GB/s", "steps": replay_steps,
              "us_per_step": round(replay_s * 1e6, 2),
              "what": "dispatch_scatter alone on a saved layout (cached dispatch), back to back"}

    graph_res = None
    if args.graph_steps > 0:
        try:
            graph_res = graph_step(args, dev, stream, prob, topk_d, lay, ws, x_d, sf_d, rows, total_b, evict)
        except Exception as exc:  # an optional figure: report it, keep the contract line
            torch.cuda.synchronize()
            graph_res = {"error": f"{type(exc).__name__}: {exc}"}

    # Layout alone, back to back (HIP events on the launch stream).
    lay_steps = max(1, warm_steps // 4)
    ev_a, ev_b = ev(), ev()
    torch.cuda.synchronize()
    ev_a.record(stream)
    for _ in range(lay_steps):
        plan.layout()
    ev_b.record(stream)
    torch.cuda.synchronize()
    layout_only_us = ev_a.elapsed_time(ev_b) * 1e3 / lay_steps
    del scratch, sink
    torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        med, reps, med_lay, med_sc = cpu_baseline(inp, w, args.cpu_seconds)
        cpu = {"value": round(total_b / med / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"full {w.name} step (layout + scatter of all {t} tokens), median of {reps} runs, "
                         "single-threaded C oracle on pre-faulted host buffers",
               "ms_per_step": round(med * 1e3, 2), "layout_ms": round(med_lay * 1e3, 3),
               "scatter_ms": round(med_sc * 1e3, 2), "pinned_to_one_core": True, "host": host_cpu()}

    ceiling = measure_device_ceiling(torch)
    # The step and the scatter against the practical ceilings measured on the
    # same box (torch's own device copy and fill), beside the published peak.
    ceiling["step_frac_of_copy"] = round(value / ceiling["copy_GBps"], 4)
    ceiling["step_frac_of_fill"] = round(value / ceiling["fill_GBps"], 4)
    ceiling["scatter_frac_of_fill"] = round(achieved / ceiling["fill_GBps"], 4)
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic",
        "config": {
            "workload": w.name, "tokens": t, "hidden": w.hidden, "x_dtype": w.dtype,
            "sf_per_token": s, "experts": w.num_experts, "ranks": w.num_ranks, "topk": k,
            "routing": w.routing, "mask_frac": w.mask_frac, "expert_alignment": w.alignment,
            "outputs": "rank-contiguous + expert-major (zero pads)", "parallelism": "single GPU",
            "kernels_per_step": step_kernels, "seed": w.seed,
        },
        "timing": ("median of HIP-event step times over the timed steps; before each step, outside its "
                   "events, 512 MiB are written and read back, so the step starts with none of its data "
                   "in the Infinity Cache and no dirty lines to write back"),
        "hbm_frac": round(value / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_step": total_b,
        "step_events": quant(step_us),
        "wall_s_timed_loop_incl_flushes": round(wall, 4),
        "tokens_per_s": round(t / (ms_per_step * 1e-3), 1),
        "pairs_per_s": round(p_valid / (ms_per_step * 1e-3), 1),
        "payload_GBps": round((n_rank + p_valid) * (w.row_bytes + 4 * s) / (ms_per_step * 1e-3) / 1e9, 1),
        ("step_kernel_events" if one_kernel else "scatter_events"): quant(kernel_us),
        "layout_read_ahead_events": None if one_kernel else quant(layout_us),
        "layout_only_us_back_to_back": round(layout_only_us, 2),
        "warm_back_to_back": warm,
        "rows": {"expert_major": p_rows, "rank_contig": n_rank, "live_tokens": t_live, "pairs": p_valid},
        "roofline": {
            "kernel": roof_kernel,
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "traffic_counts": ("L2-to-fabric bytes (TCC_EA FETCH_SIZE + WRITE_SIZE, scaled by a plain copy); "
                               "Infinity Cache hits count in them, gfx950 exposes no DRAM-side byte counter"),
            "algorithmic_bytes_per_launch": roof_b,
            "event_samples": len(kernel_us),
            "launch_us_mean": round(kernel_mean_us, 2),
        },
        "replay_scatter_only": replay,
        "graph_step": graph_res,
        "device_ceiling": ceiling,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
