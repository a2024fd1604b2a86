"""Condense rocprofv3 CSV output into the short text kept under profiles/.

    python -m combine_ep_layout_04_amd.rocprof_summary stats DIR --cmd "..." > profiles/X.md
    python -m combine_ep_layout_04_amd.rocprof_summary pmc DIR --cmd "..." > profiles/X.md
    python -m combine_ep_layout_04_amd.rocprof_summary counters DIR --cmd "..." > profiles/X.md
    python -m combine_ep_layout_04_amd.rocprof_summary trace DIR --cmd "..." > profiles/X.md
    python -m combine_ep_layout_04_amd.rocprof_summary traffic FETCH_DIR WRITE_DIR \
        --cmd "..." --out profiles/hbm_traffic_headline.txt
    python -m combine_ep_layout_04_amd.rocprof_summary sequence DIR --kernel NAME \
        --labels a,b,c --per 3 --cmd "..."

``stats`` reads ``*_kernel_stats.csv`` (from ``--kernel-trace --stats``,
without ``-T`` so that template instances stay apart) and prints each
kernel's name without its namespace and argument list;
``sequence`` splits one kernel's dispatches, in dispatch order, into
consecutive groups of ``--per`` launches named by ``--labels`` (a driver
that runs the same kernel under several inputs) and reports each group's
median of every counter, with write latency and writes in flight derived
when the EA write counters are present;
``pmc`` reads ``*_counter_collection.csv`` (from ``--pmc``) and reports the
mean counter value per dispatch for each kernel; ``counters`` makes one row
per kernel with the median per dispatch of each counter; ``traffic`` takes one
FETCH_SIZE run and one WRITE_SIZE run of ``bench.py --copy-calibration``,
scales each counter by what it reads for the plain 1 GiB elementwise copy
(torch.neg on int32: 1 GiB read, 1 GiB written) and writes HBM bytes per
launch for each library kernel, tagged with the digest of the kernel
sources the counters were taken on.
"""

from __future__ import annotations

import argparse
import csv
import glob
import os
import re
import statistics
import sys
from collections import defaultdict


def _find(d: str, suffix: str):
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not hits:
        sys.exit(f"no *{suffix} under {d}")
    return hits


def short_name(name: str) -> str:
    """``void ep::(anonymous namespace)::k<1, 2>(int, ...)`` or ``void ep::k(...)`` -> ``k<1, 2>``
    or ``k``."""
    name = name.strip()
    if name.startswith("void "):
        name = name[5:]
    name = name.replace("ep::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
    if name.startswith("ep::"):
        name = name[4:]
    cut = name.find("(")
    if cut > 0 and not name.startswith("("):
        name = name[:cut]
    return name if len(name) < 90 else name[:87] + "..."


def stats(d: str):
    rows = []
    for f in _find(d, "kernel_stats.csv"):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    out = ["| kernel | calls | average (us) | min (us) | max (us) | share |",
           "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| {short_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                   f"{float(r['Percentage']):.1f}% |")
    return out


def pmc(d: str):
    vals = defaultdict(list)
    for f in _find(d, "counter_collection.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = r.get("Kernel_Name") or r.get("Kernel-Name") or r.get("KernelName")
                counter = r.get("Counter_Name") or r.get("Counter-Name")
                value = r.get("Counter_Value") or r.get("Counter-Value")
                vals[(name, counter)].append(float(value))
    out = ["| kernel | counter | dispatches | mean per dispatch |", "|---|---|---|---|"]
    for (name, counter), v in sorted(vals.items()):
        short = name if len(name) < 90 else name[:87] + "..."
        out.append(f"| {short} | {counter} | {len(v)} | {statistics.fmean(v):.1f} |")
    return out


def trace(d: str):
    """One row per (library kernel, grid size) from ``*_kernel_trace.csv``:
    the median duration of its dispatches.  The grid size tells apart the
    same kernel run on different workloads (e.g. the tiny, mid and headline
    configs)."""
    vals = defaultdict(list)
    for f in _find(d, "kernel_trace.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = short_name(r["Kernel_Name"])
                if not _library_kernel(name) or not name:
                    continue
                grid = int(r["Grid_Size_X"]) * int(r.get("Grid_Size_Y") or 1) * int(r.get("Grid_Size_Z") or 1)
                wg = int(r["Workgroup_Size_X"])
                dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                vals[(name, grid // max(wg, 1), wg)].append(dur)
    out = ["| kernel | workgroups | lanes per workgroup | dispatches | median (us) | min (us) |",
           "|---|---|---|---|---|---|"]
    for (name, wgs, wg), v in sorted(vals.items(), key=lambda kv: (kv[0][0], kv[0][1])):
        out.append(f"| {name} | {wgs} | {wg} | {len(v)} | {statistics.median(v):.2f} | {min(v):.2f} |")
    return out


def _library_kernel(short: str) -> bool:
    """The library's own kernels (not torch's or the HIP runtime's)."""
    return (not short.startswith(("at::", "__amd_rocclr", "(anonymous namespace)::elementwise",
                                  "elementwise_kernel"))
            and "at::native" not in short)


def counters(d: str):
    """One row per library kernel, one column per counter: the median per
    dispatch."""
    vals = defaultdict(list)
    names = set()
    for f in _find(d, "counter_collection.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = short_name(r.get("Kernel_Name") or r.get("Kernel-Name") or r.get("KernelName"))
                counter = r.get("Counter_Name") or r.get("Counter-Name")
                vals[(name, counter)].append(float(r.get("Counter_Value") or r.get("Counter-Value")))
                names.add(counter)
    cols = sorted(names)
    kernels = sorted({k for k, _ in vals if _library_kernel(k)})
    out = ["| kernel | dispatches | " + " | ".join(cols) + " |", "|---" * (len(cols) + 2) + "|"]
    for k in kernels:
        n = max(len(vals.get((k, c), [])) for c in cols)
        cells = [f"{statistics.median(vals[(k, c)]):.0f}" if (k, c) in vals else "" for c in cols]
        out.append(f"| {k} | {n} | " + " | ".join(cells) + " |")
    return out


def _counter_medians(d: str):
    vals = defaultdict(list)
    for f in _find(d, "counter_collection.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = r.get("Kernel_Name") or r.get("Kernel-Name") or r.get("KernelName")
                vals[name].append(float(r.get("Counter_Value") or r.get("Counter-Value")))
    return {k: statistics.median(v) for k, v in vals.items()}


# library kernels by the key bench.py reports them under, as a pattern on
# the full kernel name (the headline workload's instance: rows of 896
# vectors take the tiled bf16 dispatch, combine and per-rank kernels, and
# the row-major 8-bit casts the tiled cast in 64-lane tiles: 448 units end in
# a half tile at 128 lanes); the 8-bit cast is told apart by
# its template arguments <format (0 E4M3, 1 E5M2), scale (0 fp32, 1 power of
# two, 2 UE8M0), tile lanes, slots per workgroup>.  The median over a kernel's dispatches is used: the
# E4M3 / fp32 instance also runs once over the tokens themselves (T rows,
# one slot each) to make the pre-quantized input.  The combine line also
# counts the dispatch-backward launches, which run the same kernel over the
# same bytes plus a [T, k] gather.  A tuple names the launches of one
# operation (the combine backward's grad_y tiles and its grad_w pass), whose
# bytes are summed.
KERNEL_KEYS = {
    "dispatch_bf16": r"dispatch_bf16_tile_kernel<128>",
    "dispatch_fp8": r"dispatch_fp8_tile_kernel<0, 0, 64, 4, false>",
    "dispatch_fp8_e5m2_fp32": r"dispatch_fp8_tile_kernel<1, 0, 64, 4, false>",
    "dispatch_fp8_e4m3_pow2": r"dispatch_fp8_tile_kernel<0, 1, 64, 4, false>",
    "dispatch_fp8_e4m3_ue8m0": r"dispatch_fp8_tile_kernel<0, 2, 64, 4, false>",
    "dispatch_fp8_e5m2_ue8m0": r"dispatch_fp8_tile_kernel<1, 2, 64, 4, false>",
    # column-major scales: one pass per token, or the tiled cast into the
    # workspace followed by the column pass
    "dispatch_fp8_e4m3_fp32_colmajor": r"dispatch_fp8_kernel<7, 0, 0>",
    "dispatch_fp8_e4m3_fp32_colmajor_two_pass": (r"dispatch_fp8_tile_kernel<0, 0, 64, 4, true>",
                                                 r"scales_colmajor_kernel<0, true>"),
    "dispatch_fp8_prequantized": r"dispatch_prequant_kernel<7, 4, true>",
    # the pre-quantized copy with column-major scales: one wavefront per
    # token with the column stride (one pass), or the code rows through the
    # grouped copy with its scale stores off and then the column pass (the
    # same kernel as the cast's column pass, whose dispatches it shares)
    "dispatch_fp8_prequantized_colmajor": r"dispatch_prequant_kernel<7, 0, true>",
    "dispatch_fp8_prequantized_colmajor_two_pass": (r"dispatch_prequant_kernel<7, 4, false>",
                                                    r"scales_colmajor_kernel<0, true>"),
    "combine": r"[^_]combine_tile_kernel<",
    "combine_backward": (r"combine_backward_grad_y_tile_kernel",
                         r"combine_backward_kernel<128, 7, false>"),
    "layout_count": r"layout_count_kernel\(",
    "layout_scatter": r"layout_scatter(_wide)?_kernel\(",
    "routing_map": r"routing_map_kernel\(",
    "rank_count": r"rank_count_kernel<",
    "rank_scatter": r"rank_scatter_kernel<",
    # bf16 rows go through the tiled kernel, 8-bit code rows with their
    # scales (448 vectors: 64 lanes) through the per-token one
    "dispatch_ranked": r"dispatch_ranked_tile_kernel",
    "dispatch_ranked_prequantized": r"dispatch_ranked_kernel<64, 7, 4>",
    "dispatch_ranked_fp8": r"dispatch_ranked_fp8_tile_kernel<0, 0, 64>",
    "combine_ranked": r"combine_ranked_tile_kernel<128>",
    # the combine over ranks of the row gradients (the same kernel and bytes
    # as combine_ranked) and the weight-gradient gather
    "dispatch_ranked_backward": (r"combine_ranked_tile_kernel<128>", r"ranked_weight_grad_kernel"),
    "dispatch_fused_permute": r"dispatch_fused_permute_kernel<\d+, \d+, false>",
    "dispatch_fused_permute_prequantized": r"dispatch_fused_permute_kernel<\d+, \d+, true>",
}
COPY_KIB = float(1 << 20)  # the calibration kernel reads and writes 1 GiB


def traffic(fetch_dir: str, write_dir: str, digest, cmd: str):
    fetch, write = _counter_medians(fetch_dir), _counter_medians(write_dir)

    def pick(table, needle):
        hits = [v for k, v in table.items() if re.search(needle, k)]
        if len(hits) != 1:
            sys.exit(f"expected one kernel matching {needle!r}, found {len(hits)}")
        return hits[0]

    f_scale = COPY_KIB / pick(fetch, "neg_kernel")
    w_scale = COPY_KIB / pick(write, "neg_kernel")
    lines = ["# HBM traffic per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per dispatch,",
             "# median over the kernel's dispatches),",
             "# each scaled by the same counter on a plain 1 GiB elementwise copy (torch.neg,",
             "# int32): scale = 1048576 KiB / counter.  Commands:",
             *[f"#   {c}" for c in cmd.split(" ;; ")],
             "# source_digest: the code (comments and spacing left out) of the kernel's source",
             "# file and of the internal and device headers, and the hipcc flags",
             f"copy_scale fetch={f_scale:.4f} write={w_scale:.4f}"]
    for key, needle in KERNEL_KEYS.items():
        needles = needle if isinstance(needle, tuple) else (needle,)
        fk = sum(pick(fetch, n) for n in needles)
        wk = sum(pick(write, n) for n in needles)
        b = (fk * f_scale + wk * w_scale) * 1024.0
        lines.append(f"kernel={key} fetch_kib={fk:.1f} write_kib={wk:.1f} "
                     f"hbm_bytes_per_launch={b:.0f} source_digest={digest(key)}")
    return lines


def sequence(d: str, kernel: str, labels, per: int):
    """Median counters per group of ``per`` consecutive dispatches of
    ``kernel`` (dispatch order), one row per label."""
    by = defaultdict(dict)
    for f in _find(d, "counter_collection.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if kernel not in short_name(r["Kernel_Name"]):
                    continue
                c = by[int(r["Dispatch_Id"])]
                c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    runs = [by[k] for k in sorted(by)]
    if len(runs) != per * len(labels):
        sys.exit(f"{len(runs)} dispatches of {kernel}, expected {per} x {len(labels)}")
    cols = sorted({c for r in runs for c in r})
    derived = {"TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_LEVEL_sum", "GRBM_GUI_ACTIVE"} <= set(cols)
    head = ["input"] + cols + (["write latency (cycles)", "writes in flight"] if derived else [])
    out = ["| " + " | ".join(head) + " |", "|---" * len(head) + "|"]
    for i, lab in enumerate(labels):
        grp = runs[per * i: per * (i + 1)]
        med = {c: statistics.median(g.get(c, 0.0) for g in grp) for c in cols}
        cells = [f"{med[c]:.0f}" for c in cols]
        if derived:
            cells += [f"{med['TCC_EA0_WRREQ_LEVEL_sum'] / max(med['TCC_EA0_WRREQ_sum'], 1):.0f}",
                      f"{med['TCC_EA0_WRREQ_LEVEL_sum'] / max(med['GRBM_GUI_ACTIVE'], 1):.0f}"]
        out.append(f"| {lab} | " + " | ".join(cells) + " |")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("kind", choices=["stats", "pmc", "counters", "traffic", "trace", "sequence"])
    ap.add_argument("dir")
    ap.add_argument("dir2", nargs="?")
    ap.add_argument("--cmd", required=True, help="the command(s) that produced the data")
    ap.add_argument("--title", default="")
    ap.add_argument("--note", default="", help="a paragraph printed under the command")
    ap.add_argument("--out")
    ap.add_argument("--kernel", help="sequence: the kernel whose dispatches are grouped")
    ap.add_argument("--labels", help="sequence: comma-separated group names, in dispatch order")
    ap.add_argument("--per", type=int, default=3, help="sequence: dispatches per group")
    a = ap.parse_args()
    if a.kind == "traffic":
        root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
        sys.path.insert(0, root)
        from bench import source_digest
        text = "\n".join(traffic(a.dir, a.dir2, source_digest, a.cmd)) + "\n"
        if a.out:
            with open(a.out, "w") as fh:
                fh.write(text)
        print(text, end="")
        return
    lines = [f"# {a.title or a.kind}", "", "Command:", "", "```", a.cmd, "```", ""]
    if a.note:
        lines += [a.note, ""]
    if a.kind == "sequence":
        lines += sequence(a.dir, a.kernel, a.labels.split(","), a.per)
    else:
        lines += {"stats": stats, "pmc": pmc, "counters": counters, "trace": trace}[a.kind](a.dir)
    print("\n".join(lines))


if __name__ == "__main__":
    main()
