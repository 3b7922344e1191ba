"""Summaries of rocprofv3 CSV output for the benchmark's kernels.

    python -m long_context_kv_hs2_amd.rocprof_summary stats DIR
        per-kernel calls, mean and total duration (from *_kernel_stats.csv)
    python -m long_context_kv_hs2_amd.rocprof_summary pmc DIR COUNTER
        per-kernel mean of a counter per dispatch (from *_counter_collection.csv)

DIR is the rocprofv3 output directory of a run with --output-format csv.
"""

from __future__ import annotations

import csv
import glob
import os
import sys
from collections import defaultdict


def _find(d, suffix):
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise SystemExit(f"no *{suffix} under {d}")
    return hits[0]


def _short(name, width=78):
    name = name.replace("void ", "")
    return name if len(name) <= width else name[: width - 3] + "..."


def stats(d):
    path = _find(d, "kernel_stats.csv")
    rows = list(csv.DictReader(open(path, newline="")))
    print(f"| kernel | calls | mean us | total us | % |")
    print(f"|---|---:|---:|---:|---:|")
    for r in rows:
        calls = int(r["Calls"])
        total = float(r["TotalDurationNs"]) / 1e3
        mean = float(r["AverageNs"]) / 1e3
        print(f"| {_short(r['Name'])} | {calls} | {mean:.2f} | {total:.1f} | {float(r['Percentage']):.1f} |")


def pmc(d, counter):
    path = _find(d, "counter_collection.csv")
    acc = defaultdict(list)
    for r in csv.DictReader(open(path, newline="")):
        if r.get("Counter_Name") != counter:
            continue
        acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    print(f"| kernel | dispatches | mean {counter} per dispatch (KiB) |")
    print(f"|---|---:|---:|")
    for name, vals in sorted(acc.items(), key=lambda kv: -sum(kv[1]) / len(kv[1])):
        print(f"| {_short(name)} | {len(vals)} | {sum(vals) / len(vals):.1f} |")


if __name__ == "__main__":
    if len(sys.argv) >= 3 and sys.argv[1] == "stats":
        stats(sys.argv[2])
    elif len(sys.argv) >= 4 and sys.argv[1] == "pmc":
        pmc(sys.argv[2], sys.argv[3])
    else:
        raise SystemExit(__doc__)
