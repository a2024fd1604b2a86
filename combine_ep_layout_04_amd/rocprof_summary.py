"""Condense rocprofv3 CSV output into the short text kept under profiles/.

    python -m combine_ep_layout_04_amd.rocprof_summary stats DIR --cmd "..." > profiles/X.md
    python -m combine_ep_layout_04_amd.rocprof_summary pmc DIR --cmd "..." > profiles/X.md

``stats`` reads ``*_kernel_stats.csv`` (from ``--kernel-trace --stats``);
``pmc`` reads ``*_counter_collection.csv`` (from ``--pmc``) and reports the
mean counter value per dispatch for each kernel.
"""

from __future__ import annotations

import argparse
import csv
import glob
import os
import statistics
import sys
from collections import defaultdict


def _find(d: str, suffix: str):
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not hits:
        sys.exit(f"no *{suffix} under {d}")
    return hits


def stats(d: str):
    rows = []
    for f in _find(d, "kernel_stats.csv"):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    out = ["| kernel | calls | average (us) | min (us) | max (us) | share |",
           "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| {r['Name']} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("kind", choices=["stats", "pmc"])
    ap.add_argument("dir")
    ap.add_argument("--cmd", required=True, help="the command that produced the data")
    ap.add_argument("--title", default="")
    a = ap.parse_args()
    lines = [f"# {a.title or a.kind}", "", "Command:", "", "```", a.cmd, "```", ""]
    lines += stats(a.dir) if a.kind == "stats" else pmc(a.dir)
    print("\n".join(lines))


if __name__ == "__main__":
    main()
