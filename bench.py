#!/usr/bin/env python3
"""Throughput of MoE token layout + dispatch + combine on one MI355X.

One step = ep_layout -> ep_dispatch (bf16) -> ep_combine over the headline
workload: T=8192 tokens, hidden 7168 bf16, 256 experts, top-8 distinct
uniform routing, fp32 row-normalised weights, identity experts (combine
reduces the dispatched rows).  Inputs are seeded synthetic data resident in
HBM before timing starts.  Every timed step and launch is preceded by a
1 GiB scratch read (outside its timing events), so inputs come from HBM,
not from the 256 MB last-level cache.  ``value`` is the dispatch + combine
algorithmic bytes of one step divided by the step's time (HIP events from
the layout launch to the end of the combine, layout included).

Also reported: per-kernel mean / median / p10 / p90 from HIP events recorded
on the launch stream, the fp8 dispatch and its variants (same shape, 1%
x100 outlier rows), the backward passes, the layout variants, the
per-(token, rank) path at 8 ranks, a plain device-to-device copy for
context, the roofline of the dominant kernel, the headline dispatch and
combine with the write-back they leave charged to them (a read pass after
each launch, minus the pass alone), and the CPU oracle timed on the host on
the same workload.  ``--warm`` adds the same steps back to back without
flushes, for context.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--warm]
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
METRIC = "dispatch+combine GB/s & tokens/s, T=8192 H=7168 E=256 k=8; % of HBM peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_headline.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# the source file of each kernel bench.py reports (plus the shared internal,
# device and cast headers and the build flags)
KERNEL_SOURCES = {
    "dispatch_bf16": "ep_dispatch.hip", "dispatch_fp8": "ep_dispatch.hip",
    "dispatch_fp8_e5m2_fp32": "ep_dispatch.hip", "dispatch_fp8_e4m3_pow2": "ep_dispatch.hip",
    "dispatch_fp8_e4m3_ue8m0": "ep_dispatch.hip", "dispatch_fp8_e5m2_ue8m0": "ep_dispatch.hip",
    "dispatch_fp8_prequantized": "ep_dispatch.hip", "dispatch_fp8_e4m3_fp32_colmajor": "ep_dispatch.hip",
    "dispatch_fp8_e4m3_fp32_colmajor_two_pass": "ep_dispatch.hip",
    "dispatch_fp8_prequantized_colmajor": "ep_dispatch.hip",
    "dispatch_fp8_prequantized_colmajor_two_pass": "ep_dispatch.hip",
    "dispatch_ranked_backward": "ep_ranked.hip",
    "routing_map": "ep_ranked.hip", "rank_count": "ep_ranked.hip", "rank_scatter": "ep_ranked.hip",
    "dispatch_ranked": "ep_ranked.hip", "combine_ranked": "ep_ranked.hip",
    "dispatch_fused_permute": "ep_ranked.hip",
    "dispatch_fused_permute_prequantized": "ep_ranked.hip",
    "dispatch_ranked_prequantized": "ep_ranked.hip",
    "dispatch_ranked_fp8": "ep_ranked.hip",
    "combine": "ep_combine.hip", "combine_backward": "ep_backward.hip",
    "layout_count": "ep_layout.hip",
    "layout_scatter": "ep_layout.hip",
}


def _code_only(text: str) -> str:
    """C++ source without comments and with whitespace runs collapsed, so
    that editing a comment does not count as changing the kernel."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest(kernel_key: str) -> str:
    """Digest of what a kernel's counters depend on: the code of its source
    file and of the internal, device and cast headers, and the hipcc flags."""
    from combine_ep_layout_04_amd.build import HIPCC_FLAGS

    csrc = os.path.join(ROOT, "combine_ep_layout_04_amd", "csrc")
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES[kernel_key], "ep_internal.h", "ep_device.h", "ep_cast.h"):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode() + b"\0" + _code_only(fh.read()).encode())
    h.update(" ".join(HIPCC_FLAGS).encode())
    return h.hexdigest()[:16]


def bytes_model(T, H, k, n):
    """Algorithmic bytes: what each operation must move at least once."""
    return {
        # read x once, write every dispatched row once, read slot once
        "dispatch_bf16": T * H * 2 + n * H * 2 + T * k * 4,
        # read x once, write codes and per-128 scales per row, read slot
        "dispatch_fp8": T * H * 2 + n * H + n * (H // 128) * 4 + T * k * 4,
        "dispatch_fp8_ue8m0": T * H * 2 + n * H + n * (H // 128) + T * k * 4,
        # read the code and scale rows once, write them per row, read slot
        "dispatch_prequantized": T * H + T * (H // 128) * 4 + n * H + n * (H // 128) * 4
                                 + T * k * 4,
        # read every dispatched row once, write out once, read slot and weights
        "combine": n * H * 2 + T * H * 2 + T * k * 4 + T * k * 4,
        # read g and every expert row once, write every row gradient once,
        # read slot and weights, write the weight gradients
        "combine_backward": T * H * 2 + 2 * n * H * 2 + T * k * 12,
        # read every row gradient once, write grad_x, read slot, gather the
        # row weight gradients into [T, k]
        "dispatch_backward": n * H * 2 + T * H * 2 + T * k * 4 + n * 4 + T * k * 4,
        # read topk_idx, write slot and src
        "layout": T * k * 8 + T * k * 4 + n * 4,
    }


def ranked_bytes_model(T, H, k, G, pairs):
    """Algorithmic bytes of the per-(token, rank) path for one rank's T
    tokens sent to ``pairs`` (token, destination rank) rows."""
    return {
        # read x once, write each (token, rank) row once, read the
        # sparse-to-dense rows, topk_idx and weights, write the weight rows
        "dispatch_ranked": T * H * 2 + pairs * H * 2 + T * G * 4 + T * k * 12 + pairs * k * 4,
        # read each (token, rank) row once, write out, read sparse-to-dense
        "combine_ranked": pairs * H * 2 + T * H * 2 + T * G * 4,
        # the same, plus topk_idx read, one weight gradient read and one
        # written per slot
        "dispatch_ranked_backward": pairs * H * 2 + T * H * 2 + T * G * 4 + T * k * 16,
    }


def variant_bytes_key(name: str) -> str:
    """The bytes-model entry of an 8-bit variant line."""
    if name.startswith("prequantized"):
        return "dispatch_prequantized"
    return "dispatch_fp8_ue8m0" if "ue8m0" in name else "dispatch_fp8"


def read_traffic(kernel_key: str):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE,
    scaled by a plain copy's counters; None when the measurement is missing
    or was taken on a different version of that kernel."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    for line in open(TRAFFIC_FILE):
        line = line.strip()
        if line.startswith("#") or not line.startswith("kernel="):
            continue
        fields = dict(kv.split("=", 1) for kv in line.split() if "=" in kv)
        if fields.get("kernel") == kernel_key:
            if fields.get("source_digest") != source_digest(kernel_key):
                return None
            return float(fields["hbm_bytes_per_launch"])
    return None


CPU_RUNS = 7   # about 13 s of oracle work at the headline workload


def cpu_baseline(inp, inp_fp8, E, nbytes):
    """The oracle as it stands (single-threaded C) on the full workload, and
    each of its operations timed alone (median of CPU_RUNS)."""
    import oracle

    times, ops = [], {"layout": [], "dispatch_bf16": [], "combine": [], "dispatch_fp8": []}
    for _ in range(CPU_RUNS):
        t0 = time.perf_counter()
        L = oracle.layout(inp.topk_idx, E)
        t1 = time.perf_counter()
        recv, _ = oracle.dispatch_bf16(inp.x_bits, L.slot)
        t2 = time.perf_counter()
        oracle.combine(recv, L.slot, inp.topk_weights)
        t3 = time.perf_counter()
        times.append(t3 - t0)
        ops["layout"].append(t1 - t0)
        ops["dispatch_bf16"].append(t2 - t1)
        ops["combine"].append(t3 - t2)
        del recv
        Lf = oracle.layout(inp_fp8.topk_idx, E)
        t4 = time.perf_counter()
        oracle.dispatch_fp8(inp_fp8.x_bits, Lf.slot)
        ops["dispatch_fp8"].append(time.perf_counter() - t4)
    t = statistics.median(times)
    # the same loops built with -fopenmp, token loops on all host cores
    # (layout stays the single-thread stable pass)
    ptimes, pops = [], {"dispatch_bf16": [], "combine": []}
    for _ in range(CPU_RUNS):
        t0 = time.perf_counter()
        L = oracle.layout(inp.topk_idx, E)
        t1 = time.perf_counter()
        recv = oracle.dispatch_bf16_parallel(inp.x_bits, L.slot)
        t2 = time.perf_counter()
        oracle.combine_parallel(recv, L.slot, inp.topk_weights)
        t3 = time.perf_counter()
        ptimes.append(t3 - t0)
        pops["dispatch_bf16"].append(t2 - t1)
        pops["combine"].append(t3 - t2)
        del recv
    tp = statistics.median(ptimes)
    threads = oracle.parallel_threads()
    return {"value": round(nbytes / t / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "full headline workload (T=8192, H=7168, E=256, k=8): oracle layout + "
                      f"bf16 dispatch + fp64 combine, single thread, median of {CPU_RUNS} runs "
                      f"({t:.2f} s each; the fp8 dispatch timed alone in each run too)",
            "seconds_per_step": round(t, 3),
            "seconds_per_op": {k: round(statistics.median(v), 4) for k, v in ops.items()},
            "host_cores_available": len(os.sched_getaffinity(0)),
            "openmp": {"value": round(nbytes / tp / 1e9, 3), "unit": "GB/s", "cores": threads,
                       "kind": "oracle loops built with -fopenmp",
                       "sample": "the same workload and step: single-thread layout, then the "
                                 f"bf16 dispatch and fp64 combine token loops on {threads} "
                                 f"threads, median of {CPU_RUNS} runs ({tp:.3f} s each)",
                       "seconds_per_step": round(tp, 4),
                       "seconds_per_op": {k: round(statistics.median(v), 4) for k, v in pops.items()}}}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle timing")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip timing the step replayed from a HIP graph")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the tiny / mid / skewed timings (profiling runs: the skewed config "
                         "shares the headline kernels)")
    ap.add_argument("--warm", action="store_true",
                    help="also time the steps back to back without cache flushes (context)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB elementwise copy (scale for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of dispatch and combine; it does not run on "
              "more than one GPU.", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        ap.error("--steps must be >= 1 and --warmup >= 0")

    import numpy as np
    import torch

    from combine_ep_layout_04_amd import ep
    from combine_ep_layout_04_amd.inputs import WORKLOADS, make_inputs

    dev = torch.device("cuda:0")
    L = ep.lib()
    w = WORKLOADS["headline"]
    T, H, E, k = w.T, w.H, w.E, w.k
    P = T * k
    log(f"[bench] generating workload headline T={T} H={H} E={E} k={k}")
    inp = make_inputs(w)

    stream = torch.cuda.Stream(device=dev)
    i32 = dict(dtype=torch.int32, device=dev)
    with torch.cuda.stream(stream):
        idx = torch.from_numpy(inp.topk_idx).to(dev)
        x = torch.from_numpy(inp.x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        wt = torch.from_numpy(inp.topk_weights).to(dev)
        counts = torch.empty(E, **i32)
        offsets = torch.empty(E + 1, **i32)
        slot = torch.empty((T, k), **i32)
        src = torch.empty(P, **i32)
        inval = torch.empty(1, **i32)
        ws_bytes = ep.layout_workspace_size(T, k, E)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        recv = torch.empty((P, H), dtype=torch.bfloat16, device=dev)
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        scratch = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
    stream.synchronize()
    s = stream.cuda_stream

    def flush():
        """Read 1 GiB of scratch (4x the 256 MB last-level cache) so the next
        launch finds its inputs in HBM, not in a cache.  A read leaves the
        caches full of clean lines: the write-back of whatever was dirty is
        paid here, not by the next kernel (a scratch *write* would leave
        256 MB of dirty lines for the timed kernel to write back).  Issued
        before every timed launch, outside its timing events."""
        with torch.cuda.stream(stream):
            scratch.sum()   # one reduction kernel over the 1 GiB, fp32 in and out
    p = {n: t.data_ptr() for n, t in dict(idx=idx, x=x, wt=wt, counts=counts, offsets=offsets,
                                          slot=slot, src=src, inval=inval, ws=ws, recv=recv,
                                          out=out).items()}

    def check(st, what):
        if st != 0:
            raise RuntimeError(f"{what}: {ep.status_string(st)}: {ep.last_error()}")

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        check(L.ep_layout(p["idx"], T, k, E, p["counts"], p["offsets"], p["slot"], p["src"],
                          p["inval"], p["ws"], ws_bytes, s), "ep_layout")
        if ev is not None:
            ev[1].record(stream)
        check(L.ep_dispatch(p["x"], T, H, k, p["slot"], None, 0, p["recv"], None, None, s),
              "ep_dispatch")
        if ev is not None:
            ev[2].record(stream)
        check(L.ep_combine(p["recv"], p["slot"], p["wt"], T, H, k, p["out"], s), "ep_combine")
        if ev is not None:
            ev[3].record(stream)

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        flush()
        step()
    stream.synchronize()
    n = int(offsets[E].item())

    # K steps, each after a cache flush; a step's time runs from its layout
    # launch to the end of its combine (HIP events on the launch stream, one
    # before the layout and one after the combine: an event recorded between
    # two launches adds a gap between them)
    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        flush()
        sev[i][0].record(stream)
        step()
        sev[i][1].record(stream)
    stream.synchronize()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_ms_step = (t1 - t0) * 1e3 / args.steps
    ms_step = statistics.fmean([e[0].elapsed_time(e[1]) for e in sev])
    # the same K steps again with events between the three launches, for
    # the per-kernel times
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps with per-kernel events")
    for i in range(args.steps):
        flush()
        step(evs[i])
    stream.synchronize()
    ms_step_staged = statistics.fmean([e[0].elapsed_time(e[3]) for e in evs])
    # context: the same step captured once in a HIP graph and replayed after
    # each flush
    graph = None
    if not args.no_graph:
        try:
            g = torch.cuda.CUDAGraph()
            stream.synchronize()
            with torch.cuda.graph(g, stream=stream):
                step()
            stream.synchronize()
            gev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
                   for _ in range(args.steps)]
            with torch.cuda.stream(stream):
                for i in range(args.steps):
                    flush()
                    gev[i][0].record(stream)
                    g.replay()
                    gev[i][1].record(stream)
            stream.synchronize()
            graph = {"ms_per_step": round(statistics.fmean([e[0].elapsed_time(e[1]) for e in gev]), 4)}
            del g
        except RuntimeError as e:   # context only: the step itself is timed above
            torch.cuda.synchronize()
            graph = {"error": str(e)[:200]}

    warm = None
    if args.warm:
        # context only: the same steps back to back, caches as the previous
        # step left them (x, read with cached loads, stays in the last-level
        # cache while the non-temporal streams pass it by)
        wev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        for i in range(args.steps):
            step(wev[i])
        stream.synchronize()
        wms = statistics.fmean([e[0].elapsed_time(e[3]) for e in wev])
        warm = {"ms_per_step": round(wms, 4),
                "dispatch_bf16_us": round(statistics.fmean([e[1].elapsed_time(e[2]) for e in wev]) * 1e3, 2),
                "combine_us": round(statistics.fmean([e[2].elapsed_time(e[3]) for e in wev]) * 1e3, 2)}

    lay = [e[0].elapsed_time(e[1]) for e in evs]
    dis = [e[1].elapsed_time(e[2]) for e in evs]
    com = [e[2].elapsed_time(e[3]) for e in evs]
    us = lambda v: statistics.fmean(v) * 1e3  # noqa: E731

    # ---- the dispatch and the combine charged with the write-back they
    # leave behind: each launch followed by a 256 MiB read pass, minus that
    # pass alone (caches emptied before each).  Stores that stayed dirty in
    # the last-level cache when the kernel ended would be written back
    # during the pass and make it slower; the row outputs are streaming
    # stores, so the charged time should not exceed the kernel's own (the
    # pass may overlap the kernel's last waves).  The pass reads a buffer of
    # its own, which the 1 GiB flush evicts: a pass over the flush's last
    # 256 MiB would find them in the last-level cache alone but not after a
    # kernel whose reads evict them, and charge that difference instead.
    with torch.cuda.stream(stream):
        tail = torch.zeros(1 << 26, dtype=torch.float32, device=dev)
    stream.synchronize()

    def tail_pass():
        with torch.cuda.stream(stream):
            tail.sum()

    def charged(fn, reps):
        evl = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        for i in range(-1, reps):
            flush()
            if i >= 0:
                evl[i][0].record(stream)
            fn()
            tail_pass()
            if i >= 0:
                evl[i][1].record(stream)
        stream.synchronize()
        return statistics.median([e[0].elapsed_time(e[1]) for e in evl])

    log("[bench] write-back charged timings")
    pass_alone = charged(lambda: None, args.steps)
    dis_charged = charged(lambda: check(L.ep_dispatch(p["x"], T, H, k, p["slot"], None, 0, p["recv"],
                                                      None, None, s), "ep_dispatch"), args.steps)
    com_charged = charged(lambda: check(L.ep_combine(p["recv"], p["slot"], p["wt"], T, H, k, p["out"],
                                                     s), "ep_combine"), args.steps)

    # correctness spot check of what was timed: identity experts give x back
    # (compared as values: a -0.0 in x comes back as +0.0)
    ok = bool(torch.equal(out.float(), x.float()))

    # ---- fp8 dispatch on the fp8 workload (same shape, 1% outlier rows)
    wf = WORKLOADS["fp8"]
    log("[bench] fp8 dispatch workload")
    inpf = make_inputs(wf)
    with torch.cuda.stream(stream):
        idxf = torch.from_numpy(inpf.topk_idx).to(dev)
        xf = torch.from_numpy(inpf.x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        slotf = torch.empty((T, k), **i32)
        q = torch.empty((P, H), dtype=torch.uint8, device=dev)
        sc = torch.empty((P, H // 128), dtype=torch.float32, device=dev)
    stream.synchronize()
    check(L.ep_layout(idxf.data_ptr(), T, k, E, p["counts"], p["offsets"], slotf.data_ptr(), None,
                      None, p["ws"], ws_bytes, s), "ep_layout")
    stream.synchronize()
    nf = int(offsets[E].item())

    def fp8_step():
        check(L.ep_dispatch(xf.data_ptr(), T, H, k, slotf.data_ptr(), None, 1, q.data_ptr(),
                            sc.data_ptr(), None, s), "ep_dispatch fp8")

    for _ in range(args.warmup):
        flush()
        fp8_step()
    fev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        flush()
        fev[i][0].record(stream)
        fp8_step()
        fev[i][1].record(stream)
    stream.synchronize()
    f8 = [e[0].elapsed_time(e[1]) for e in fev]

    # ---- backward passes on the headline layout (identity experts: y is
    # the dispatched rows; g and the row weight gradients are seeded N(0,1))
    from combine_ep_layout_04_amd.inputs import make_gradient
    with torch.cuda.stream(stream):
        gout = torch.from_numpy(make_gradient(T, H, 7).view(np.int16)).view(torch.bfloat16).to(dev)
        grad_y = torch.empty((P, H), dtype=torch.bfloat16, device=dev)
        grad_w = torch.empty((T, k), dtype=torch.float32, device=dev)
        grw = torch.randn(P, generator=torch.Generator().manual_seed(8)).to(dev)
    stream.synchronize()
    check(L.ep_layout(p["idx"], T, k, E, p["counts"], p["offsets"], p["slot"], p["src"],
                      p["inval"], p["ws"], ws_bytes, s), "ep_layout")
    check(L.ep_dispatch(p["x"], T, H, k, p["slot"], None, 0, p["recv"], None, None, s),
          "ep_dispatch")

    def time_call(fn, reps):
        evl = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        for i in range(-args.warmup, reps):
            flush()
            if i >= 0:
                evl[i][0].record(stream)
            fn()
            if i >= 0:
                evl[i][1].record(stream)
        stream.synchronize()
        return [e[0].elapsed_time(e[1]) for e in evl]

    cb_us = time_call(lambda: check(L.ep_combine_backward(
        gout.data_ptr(), p["recv"], p["slot"], p["wt"], T, H, k, grad_y.data_ptr(),
        grad_w.data_ptr(), s), "ep_combine_backward"), args.steps)
    db_us = time_call(lambda: check(L.ep_dispatch_backward(
        p["recv"], grw.data_ptr(), p["slot"], T, H, k, p["out"], grad_w.data_ptr(), s),
        "ep_dispatch_backward"), args.steps)
    del grad_y

    # ---- layout variants on the headline routing: segment starts aligned
    # to 128 rows, and a fixed 320 rows per expert (1.25x the mean load)
    def time_layout(alignment, capacity, reps):
        rows = ep.layout_max_rows(T, k, E, alignment, capacity)
        src_x = torch.empty(rows, **i32)
        drop = torch.empty(1, **i32)
        evl = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        for i in range(-args.warmup, reps):
            flush()
            if i >= 0:
                evl[i][0].record(stream)
            check(L.ep_layout_ex(p["idx"], T, k, E, alignment, capacity, p["counts"],
                                 p["offsets"], p["slot"], src_x.data_ptr(), p["inval"],
                                 drop.data_ptr(), p["ws"], ws_bytes, s), "ep_layout_ex")
            if i >= 0:
                evl[i][1].record(stream)
        stream.synchronize()
        return [e[0].elapsed_time(e[1]) for e in evl], int(drop.item())

    lay_a128, _ = time_layout(128, 0, args.steps)
    lay_cap, dropped_cap = time_layout(1, 320, args.steps)

    # ---- 8-bit cast variants and the pre-quantized copy (fp8 workload)
    variants = {}
    with torch.cuda.stream(stream):
        sc_b = torch.empty((P, H // 128), dtype=torch.uint8, device=dev)
        xq_tok = torch.empty((T, H), dtype=torch.uint8, device=dev)
        xs_tok = torch.empty((T, H // 128), dtype=torch.float32, device=dev)
        ident = torch.arange(T, dtype=torch.int32, device=dev).view(T, 1)
    stream.synchronize()
    # the tokens' own E4M3 rows and scales, for the pre-quantized input
    check(L.ep_dispatch(xf.data_ptr(), T, H, 1, ident.data_ptr(), None, 1, xq_tok.data_ptr(),
                        xs_tok.data_ptr(), None, s), "ep_dispatch fp8 (tokens)")
    # (column-major scales: [H/128, P], each block's scales contiguous over rows)
    for name, fmt, mode, sbuf, ld in (("e5m2_fp32", 2, 0, sc, 0), ("e4m3_pow2", 1, 1, sc, 0),
                                      ("e4m3_ue8m0", 1, 2, sc_b, 0), ("e5m2_ue8m0", 2, 2, sc_b, 0),
                                      ("e4m3_fp32_colmajor", 1, 0, sc, P)):
        variants[name] = time_call(lambda: check(L.ep_dispatch_ex(
            xf.data_ptr(), T, H, k, slotf.data_ptr(), None, fmt, mode, q.data_ptr(),
            sbuf.data_ptr(), None, ld, s), "ep_dispatch_ex"), args.steps)
    # the same column-major scales in two passes (codes and per-token scales
    # through a workspace, then the columns one receive row per lane)
    with torch.cuda.stream(stream):
        srcf = torch.empty(P, dtype=torch.int32, device=dev)
        cm_ws_bytes = L.ep_dispatch_colmajor_workspace_size(T, H, 0)
        cm_ws = torch.empty(cm_ws_bytes, dtype=torch.uint8, device=dev)
    stream.synchronize()
    check(L.ep_layout(idxf.data_ptr(), T, k, E, p["counts"], p["offsets"], slotf.data_ptr(),
                      srcf.data_ptr(), None, p["ws"], ws_bytes, s), "ep_layout")
    variants["e4m3_fp32_colmajor_two_pass"] = time_call(lambda: check(L.ep_dispatch_colmajor_scales(
        xf.data_ptr(), T, H, k, slotf.data_ptr(), srcf.data_ptr(), None, 1, 0, q.data_ptr(),
        sc.data_ptr(), None, P, P, cm_ws.data_ptr(), cm_ws_bytes, s), "ep_dispatch_colmajor_scales"),
        args.steps)
    variants["prequantized"] = time_call(lambda: check(L.ep_dispatch_prequantized(
        xq_tok.data_ptr(), xs_tok.data_ptr(), T, H, k, slotf.data_ptr(), None, q.data_ptr(),
        sc.data_ptr(), None, 0, s), "ep_dispatch_prequantized"), args.steps)
    # pre-quantized rows with column-major scales: one pass, and two (the
    # code rows, then the columns straight from the token scales)
    variants["prequantized_colmajor"] = time_call(lambda: check(L.ep_dispatch_prequantized(
        xq_tok.data_ptr(), xs_tok.data_ptr(), T, H, k, slotf.data_ptr(), None, q.data_ptr(),
        sc.data_ptr(), None, P, s), "ep_dispatch_prequantized"), args.steps)
    variants["prequantized_colmajor_two_pass"] = time_call(lambda: check(
        L.ep_dispatch_prequantized_colmajor(
            xq_tok.data_ptr(), xs_tok.data_ptr(), T, H, k, slotf.data_ptr(), srcf.data_ptr(), None,
            q.data_ptr(), sc.data_ptr(), None, P, P, s), "ep_dispatch_prequantized_colmajor"),
        args.steps)

    # ---- per-(token, rank) path: G = 8 ranks of the headline shape on this
    # device (rank 0 holds the headline tokens, ranks 1..7 uniform routing);
    # rank 0's share is timed: its routing bitmap, its layout over the
    # all-gathered map, the dispatch of its tokens once per destination rank
    # and the combine over ranks
    from combine_ep_layout_04_amd.inputs import make_routing
    import ctypes
    G = 8
    El = E // G
    W8 = (E + 7) // 8
    log(f"[bench] per-rank path, {G} ranks")
    with torch.cuda.stream(stream):
        gmap = torch.empty((G * T, W8), dtype=torch.uint8, device=dev)
        others = [torch.from_numpy(make_routing(T, E, k, 100 + r)).to(dev) for r in range(1, G)]
        rl = dict(s2d=torch.empty((T, G), **i32), lm=torch.empty((G * T, El), dtype=torch.uint8, device=dev),
                  rsrc=torch.empty(G * T, **i32), rti=torch.empty((G * T, k), dtype=torch.int64, device=dev),
                  ecnt=torch.empty(El, **i32), nrecv=torch.empty(1, **i32), novf=torch.empty(1, **i32))
        rl_ws_bytes = ep.rank_layout_workspace_size(T, E, G)
        rl_ws = torch.empty(rl_ws_bytes, dtype=torch.uint8, device=dev)
    stream.synchronize()
    for r in range(1, G):
        check(L.ep_routing_map(others[r - 1].data_ptr(), T, k, E, gmap[r * T].data_ptr(), None, s),
              "ep_routing_map")
    rm_us = time_call(lambda: check(L.ep_routing_map(p["idx"], T, k, E, gmap.data_ptr(), None, s),
                                    "ep_routing_map"), args.steps)
    rq = {n: t.data_ptr() for n, t in rl.items()}
    rk_us = time_call(lambda: check(L.ep_rank_layout(
        gmap.data_ptr(), T, E, G, 0, k, rq["s2d"], rq["lm"], rq["rsrc"], rq["rti"], rq["ecnt"],
        rq["nrecv"], rq["novf"], rl_ws.data_ptr(), rl_ws_bytes, s), "ep_rank_layout"), args.steps)
    stream.synchronize()
    s2d_h = rl["s2d"].cpu()
    pairs = int((s2d_h >= 0).sum())
    # rank 0's tokens come first in every receive buffer, so T rows hold them
    assert int(s2d_h.max()) < T
    with torch.cuda.stream(stream):
        dest = [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in range(G)]
        dest_w = [torch.empty((T, k), dtype=torch.float32, device=dev) for _ in range(G)]
        out_r = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    stream.synchronize()
    xtab = (ctypes.c_void_p * G)(*[t.data_ptr() for t in dest])
    wtab = (ctypes.c_void_p * G)(*[t.data_ptr() for t in dest_w])
    dr_us = time_call(lambda: check(L.ep_dispatch_ranked(
        p["x"], p["idx"], p["wt"], T, H, k, E, G, rq["s2d"], ctypes.addressof(xtab),
        ctypes.addressof(wtab), T, s), "ep_dispatch_ranked"), args.steps)
    # the combine over ranks reads back the rows just dispatched (each rank's
    # "partial output" of a token is the token itself): out[t] = bf16(n_t x[t])
    cr_us = time_call(lambda: check(L.ep_combine_ranked(
        ctypes.addressof(xtab), T, rq["s2d"], T, H, G, out_r.data_ptr(), s),
        "ep_combine_ranked"), args.steps)
    stream.synchronize()
    n_t = (s2d_h >= 0).sum(dim=1).to(dev).view(T, 1).float()
    ranked_ok = bool(torch.equal(out_r, (x.float() * n_t).bfloat16()))
    # the backward of the once-per-rank dispatch, with the rows and weight
    # rows just dispatched standing in for their gradients: the token
    # gradients are the combine over ranks, the weight gradients come back
    # to [T, k]
    with torch.cuda.stream(stream):
        gtw_r = torch.empty((T, k), dtype=torch.float32, device=dev)
    stream.synchronize()
    rb_us = time_call(lambda: check(L.ep_dispatch_ranked_backward(
        ctypes.addressof(xtab), ctypes.addressof(wtab), T, p["idx"], rq["s2d"], T, H, k, E, G,
        out_r.data_ptr(), gtw_r.data_ptr(), s), "ep_dispatch_ranked_backward"), args.steps)
    rbm = ranked_bytes_model(T, H, k, G, pairs)
    del dest

    # the same sends for 8-bit tokens (the fp8 workload's tokens, cast once
    # per token above): code and scale rows once per destination rank
    with torch.cuda.stream(stream):
        dest_q = [torch.empty((T, H), dtype=torch.uint8, device=dev) for _ in range(G)]
        dest_s = [torch.empty((T, H // 128), dtype=torch.float32, device=dev) for _ in range(G)]
    stream.synchronize()
    qtab = (ctypes.c_void_p * G)(*[t.data_ptr() for t in dest_q])
    stab = (ctypes.c_void_p * G)(*[t.data_ptr() for t in dest_s])
    drq_us = time_call(lambda: check(L.ep_dispatch_ranked_prequantized(
        xq_tok.data_ptr(), xs_tok.data_ptr(), p["idx"], p["wt"], T, H, k, E, G, rq["s2d"],
        ctypes.addressof(qtab), ctypes.addressof(stab), ctypes.addressof(wtab), T, s),
        "ep_dispatch_ranked_prequantized"), args.steps)
    drq_bytes = (T * H + T * (H // 128) * 4 + pairs * (H + (H // 128) * 4) + T * G * 4 + T * k * 12
                 + pairs * k * 4)
    # the same sends with the cast on the way (the fp8 workload's bf16
    # tokens, E4M3 with fp32 scales): no per-token code and scale buffers
    drf_us = time_call(lambda: check(L.ep_dispatch_ranked_fp8(
        xf.data_ptr(), p["idx"], p["wt"], T, H, k, E, G, rq["s2d"], 1, 0, ctypes.addressof(qtab),
        ctypes.addressof(stab), ctypes.addressof(wtab), T, s), "ep_dispatch_ranked_fp8"),
        args.steps)
    drf_bytes = (T * H * 2 + pairs * (H + (H // 128) * 4) + T * G * 4 + T * k * 12
                 + pairs * k * 4)
    del dest_q, dest_s, dest_w

    # receive side of rank 0 with the permute fused in: every token it
    # receives (from 8 ranks; ranks 1..7 hold seeded N(0,1) rows and unit-sum
    # weights) read once and written to its local-expert rows
    with torch.cuda.stream(stream):
        gen = torch.Generator(device=dev).manual_seed(11)
        src_x = [x] + [torch.randn((T, H), generator=gen, device=dev).bfloat16() for _ in range(1, G)]
        src_i = [idx] + others
        src_w = [wt] + [torch.full((T, k), 1.0 / k, dtype=torch.float32, device=dev)
                        for _ in range(1, G)]
        pc = torch.empty(El, **i32)
        po = torch.empty(El + 1, **i32)
        pslot = torch.empty((G * T, k), **i32)
        pws_bytes = ep.layout_workspace_size(G * T, k, El)
        pws = torch.empty(pws_bytes, dtype=torch.uint8, device=dev)
    stream.synchronize()
    check(L.ep_layout(rq["rti"], G * T, k, El, pc.data_ptr(), po.data_ptr(), pslot.data_ptr(), None,
                      None, pws.data_ptr(), pws_bytes, s), "ep_layout (received rows)")
    stream.synchronize()
    n_exp = int(po[El].item())
    n_recv = int(rl["nrecv"].item())
    with torch.cuda.stream(stream):
        perm_x = torch.empty((n_exp, H), dtype=torch.bfloat16, device=dev)
        perm_w = torch.empty(n_exp, dtype=torch.float32, device=dev)
    stream.synchronize()
    sxt = (ctypes.c_void_p * G)(*[t.data_ptr() for t in src_x])
    sit = (ctypes.c_void_p * G)(*[t.data_ptr() for t in src_i])
    swt = (ctypes.c_void_p * G)(*[t.data_ptr() for t in src_w])
    fp_us = time_call(lambda: check(L.ep_dispatch_fused_permute(
        ctypes.addressof(sxt), ctypes.addressof(sit), ctypes.addressof(swt), T, H, k, E, G, 0,
        rq["rsrc"], rq["rti"], rq["nrecv"], pslot.data_ptr(), n_exp, perm_x.data_ptr(),
        perm_w.data_ptr(), s),
        "ep_dispatch_fused_permute"), args.steps)
    # read each received token once, write each expert row once, read the
    # received rows' metadata (source, local experts, slots) and the senders'
    # topk rows, write the row weights (rows past the received count, read
    # on the device, are not visited)
    fp_bytes = (n_recv * H * 2 + n_exp * H * 2 + n_recv * (4 + k * 8 + k * 4) + n_recv * k * 12
                + n_exp * 4)
    del src_x, perm_x

    # the same receive for 8-bit tokens: rank 0's code and scale rows are the
    # fp8 workload's cast above, ranks 1..7 hold seeded bytes and unit scales
    nb = H // 128
    with torch.cuda.stream(stream):
        src_q = [xq_tok] + [torch.randint(0, 256, (T, H), generator=gen, device=dev,
                                          dtype=torch.uint8) for _ in range(1, G)]
        src_s = [xs_tok] + [torch.ones((T, nb), dtype=torch.float32, device=dev)
                            for _ in range(1, G)]
        perm_q = torch.empty((n_exp, H), dtype=torch.uint8, device=dev)
        perm_s = torch.empty((n_exp, nb), dtype=torch.float32, device=dev)
    stream.synchronize()
    sqt = (ctypes.c_void_p * G)(*[t.data_ptr() for t in src_q])
    sst = (ctypes.c_void_p * G)(*[t.data_ptr() for t in src_s])
    fpq_us = time_call(lambda: check(L.ep_dispatch_fused_permute_prequantized(
        ctypes.addressof(sqt), ctypes.addressof(sst), ctypes.addressof(sit), ctypes.addressof(swt),
        T, H, k, E, G, 0, rq["rsrc"], rq["rti"], rq["nrecv"], pslot.data_ptr(), n_exp,
        perm_q.data_ptr(), perm_s.data_ptr(), perm_w.data_ptr(), s),
        "ep_dispatch_fused_permute_prequantized"), args.steps)
    # as the bf16 receive with code rows of H bytes plus scale rows of H/128 fp32
    fpq_bytes = ((n_recv + n_exp) * (H + nb * 4) + n_recv * (4 + k * 8 + k * 4) + n_recv * k * 12
                 + n_exp * 4)
    del src_q, src_s, perm_q, perm_s

    # ---- the other seeded configs (tiny, mid, skewed): layout, dispatch and
    # combine each timed alone, caches emptied before every launch
    configs = {}
    for cname in (() if args.no_configs else ("tiny", "mid", "skewed")):
        wc = WORKLOADS[cname]
        ic = make_inputs(wc)
        Tc, Hc, Ec, kc = wc.T, wc.H, wc.E, wc.k
        with torch.cuda.stream(stream):
            c_idx = torch.from_numpy(ic.topk_idx).to(dev)
            c_x = torch.from_numpy(ic.x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
            c_w = torch.from_numpy(ic.topk_weights).to(dev)
            c_cnt = torch.empty(Ec, **i32)
            c_off = torch.empty(Ec + 1, **i32)
            c_slot = torch.empty((Tc, kc), **i32)
            c_ws_bytes = ep.layout_workspace_size(Tc, kc, Ec)
            c_ws = torch.empty(max(c_ws_bytes, 256), dtype=torch.uint8, device=dev)
            c_recv = torch.empty((Tc * kc, Hc), dtype=torch.bfloat16, device=dev)
            c_out = torch.empty((Tc, Hc), dtype=torch.bfloat16, device=dev)
        stream.synchronize()
        c_lay = time_call(lambda: check(L.ep_layout(
            c_idx.data_ptr(), Tc, kc, Ec, c_cnt.data_ptr(), c_off.data_ptr(), c_slot.data_ptr(),
            None, None, c_ws.data_ptr(), c_ws_bytes, s), "ep_layout"), args.steps)
        c_dis = time_call(lambda: check(L.ep_dispatch(
            c_x.data_ptr(), Tc, Hc, kc, c_slot.data_ptr(), None, 0, c_recv.data_ptr(), None, None,
            s), "ep_dispatch"), args.steps)
        c_com = time_call(lambda: check(L.ep_combine(
            c_recv.data_ptr(), c_slot.data_ptr(), c_w.data_ptr(), Tc, Hc, kc, c_out.data_ptr(), s),
            "ep_combine"), args.steps)
        stream.synchronize()
        nc = int(c_off[Ec].item())
        bmc = bytes_model(Tc, Hc, kc, nc)
        d_us, c_us = us(c_dis), us(c_com)
        # context at this size: torch's device-to-device copy of half the
        # dispatch's bytes into the other half (the same bytes moved), timed
        # the same way
        with torch.cuda.stream(stream):
            cp_src = torch.empty(bmc["dispatch_bf16"] // 2, dtype=torch.uint8, device=dev)
            cp_dst = torch.empty_like(cp_src)

        def copy_same_bytes():
            with torch.cuda.stream(stream):
                cp_dst.copy_(cp_src)

        cp_us = us(time_call(copy_same_bytes, args.steps))
        del cp_src, cp_dst
        configs[cname] = {
            "T": Tc, "H": Hc, "E": Ec, "k": kc, "dispatched_rows": nc,
            "layout_us": round(us(c_lay), 2),
            "dispatch_us": round(d_us, 2), "dispatch_GB_per_s": round(bmc["dispatch_bf16"] / d_us / 1e3, 1),
            "combine_us": round(c_us, 2), "combine_GB_per_s": round(bmc["combine"] / c_us / 1e3, 1),
            "dispatch_frac_of_hbm_peak": round(bmc["dispatch_bf16"] / d_us / 1e3 / HBM_PEAK_GBS, 4),
            "combine_frac_of_hbm_peak": round(bmc["combine"] / c_us / 1e3 / HBM_PEAK_GBS, 4),
            "d2d_copy_us_same_bytes": round(cp_us, 2),
            "dispatch_frac_of_d2d_copy": round(cp_us / d_us, 4),
            "combine_frac_of_d2d_copy": round(cp_us * bmc["combine"] / bmc["dispatch_bf16"] / c_us, 4),
        }
        del c_recv, c_out, c_x

    # the floor of this timing method: two events recorded back to back on the
    # stream after the same flush, nothing between them (short launches'
    # times include it)
    event_floor_us = us(time_call(lambda: None, args.steps))

    # ---- context: a plain device-to-device copy of 1 GiB (read + write)
    with torch.cuda.stream(stream):
        c_src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        c_dst = torch.empty_like(c_src)

    def copy_on_stream():
        with torch.cuda.stream(stream):
            c_dst.copy_(c_src)

    copy_ms = time_call(copy_on_stream, max(5, args.steps // 5))
    copy_gbs = 2.0 * (1 << 30) / (statistics.median(copy_ms) * 1e-3) / 1e9
    del c_src, c_dst

    if args.copy_calibration:
        # a plain elementwise kernel that reads and writes exactly 1 GiB each
        a = torch.ones(1 << 28, dtype=torch.int32, device=dev)
        b = torch.empty_like(a)
        torch.neg(a, out=b)
        torch.cuda.synchronize()
        del a, b

    bm = bytes_model(T, H, k, n)
    bmf = bytes_model(T, H, k, nf)

    def entry(ms, **extra):
        """mean (us, the roofline's figure), median and p10 / p90 of the
        per-launch HIP-event times."""
        q = statistics.quantiles(ms, n=10) if len(ms) > 1 else [ms[0]] * 9
        return {"us": round(us(ms), 2), "median_us": round(statistics.median(ms) * 1e3, 2),
                "p10_us": round(q[0] * 1e3, 2), "p90_us": round(q[-1] * 1e3, 2), **extra}

    per_kernel = {
        "layout": entry(lay),
        "dispatch_bf16": entry(dis, bytes=bm["dispatch_bf16"],
                               write_back_charged_median_us=round((dis_charged - pass_alone) * 1e3, 2)),
        "combine": entry(com, bytes=bm["combine"],
                         write_back_charged_median_us=round((com_charged - pass_alone) * 1e3, 2)),
        "dispatch_fp8": entry(f8, bytes=bmf["dispatch_fp8"],
                              workload="fp8: headline shape, 1% of rows x100"),
        "combine_backward": entry(cb_us, bytes=bm["combine_backward"]),
        "dispatch_backward": entry(db_us, bytes=bm["dispatch_backward"]),
        **{f"dispatch_fp8_{name}": entry(v, bytes=bmf[variant_bytes_key(name)])
           for name, v in variants.items()},
        "routing_map": entry(rm_us),
        "rank_layout": entry(rk_us, ranks=G),
        "dispatch_ranked": entry(dr_us, bytes=rbm["dispatch_ranked"], ranks=G,
                                 rows_written=pairs, expanded_rows=n),
        "combine_ranked": entry(cr_us, bytes=rbm["combine_ranked"], ranks=G, rows_read=pairs),
        "dispatch_ranked_backward": entry(rb_us, bytes=rbm["dispatch_ranked_backward"], ranks=G,
                                          rows_read=pairs),
        "dispatch_ranked_prequantized": entry(drq_us, bytes=drq_bytes, ranks=G, rows_written=pairs),
        "dispatch_ranked_fp8": entry(drf_us, bytes=drf_bytes, ranks=G, rows_written=pairs,
                                     workload="fp8 tokens, headline routing"),
        "dispatch_fused_permute": entry(fp_us, bytes=fp_bytes, ranks=G, tokens_received=n_recv,
                                        expert_rows_written=n_exp),
        "dispatch_fused_permute_prequantized": entry(fpq_us, bytes=fpq_bytes, ranks=G,
                                                     tokens_received=n_recv,
                                                     expert_rows_written=n_exp),
        "layout_aligned128": entry(lay_a128),
        "layout_capacity320": entry(lay_cap, dropped_pairs=dropped_cap),
    }
    for key, v in per_kernel.items():
        if "bytes" in v:
            gbs = v["bytes"] / (v["us"] * 1e-6) / 1e9
            v["GB_per_s"] = round(gbs, 1)
            v["GB_per_s_at_median"] = round(v["bytes"] / (v["median_us"] * 1e-6) / 1e9, 1)
            v["frac_of_hbm_peak"] = round(gbs / HBM_PEAK_GBS, 4)
            v["frac_of_d2d_copy"] = round(gbs / copy_gbs, 4)
            v["tokens_per_s"] = round(T / (v["us"] * 1e-6), 1)
        if key in KERNEL_SOURCES:
            v["traffic"] = read_traffic(key)

    dom = "combine" if per_kernel["combine"]["us"] >= per_kernel["dispatch_bf16"]["us"] else "dispatch_bf16"
    dk = per_kernel[dom]
    step_bytes = bm["dispatch_bf16"] + bm["combine"]
    value = step_bytes / (ms_step * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        cpu = cpu_baseline(inp, inpf, E, step_bytes)

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_with_kernel_events": round(ms_step_staged, 4),
        "graph_replay": graph,
        "wall_ms_per_step_incl_cache_flush": round(wall_ms_step, 4),
        "caches": "a 1 GiB scratch read before every timed launch and step (outside its events)",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 tokens, uniform distinct top-8 routing, "
                "row-normalised fp32 weights, identity experts)",
        "config": {"workload": "headline: T=8192 H=7168 E=256 k=8, step = layout + bf16 dispatch "
                               "+ weighted combine", "T": T, "H": H, "E": E, "k": k,
                   "dispatched_rows": n},
        "tokens_per_s": round(T / (ms_step * 1e-3), 1),
        "tokens_per_s_dispatch_plus_combine": round(
            T / ((per_kernel["dispatch_bf16"]["us"] + per_kernel["combine"]["us"]) * 1e-6), 1),
        "d2d_copy_GB_per_s": round(copy_gbs, 1),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": dk["GB_per_s"],
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dk["frac_of_hbm_peak"],
                     "traffic": read_traffic(dom)},
        "kernels": per_kernel,
        "combine_returns_x": ok,
        "ranked_combine_returns_n_x": ranked_ok,
        "cpu_baseline": cpu,
        "back_to_back": warm,
        "configs": configs,
        "event_timing_floor_us": round(event_floor_us, 2),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
