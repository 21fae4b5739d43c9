"""Summaries of rocprofv3 output for the profiles/ folder (text tables, run on the host).

trace_summary(out_dir): the kernel trace of ``bench.py`` (``rocprofv3 --kernel-trace
--stats ... -- python bench.py``, with bench.py's own JSON line saved as
``<out_dir>/bench.json``) as a table of per-launch durations grouped by kernel and grid.

counter_summary(out_dir, kernels): the mean per dispatch of every counter of one
``rocprofv3 --pmc`` run, for the kernels whose names contain one of ``kernels``.

Nothing here touches a GPU; both read CSV files only.
"""

from __future__ import annotations

import collections
import csv
import glob
import json
import os


def _csv(out_dir: str, suffix: str):
    files = glob.glob(os.path.join(out_dir, "**", f"*{suffix}"), recursive=True)
    if not files:
        raise SystemExit(f"no *{suffix} under {out_dir}")
    rows = []
    for path in files:
        with open(path) as f:
            rows += list(csv.DictReader(f))
    return rows


def short_name(name: str) -> str:
    return name.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]


def trace_summary(out_dir: str, last: int = 20) -> str:
    rows = [r for r in _csv(out_dir, "kernel_trace.csv") if r.get("Kind", "KERNEL_DISPATCH") == "KERNEL_DISPATCH"]
    groups = collections.OrderedDict()
    for r in sorted(rows, key=lambda r: int(r["Start_Timestamp"])):
        name = r["Kernel_Name"]
        if "at::native::" in name:
            continue   # torch's input set-up and Infinity-Cache flushes, not this library's work
        key = (short_name(name), r["Grid_Size_X"], r["Grid_Size_Y"], r["Grid_Size_Z"])
        g = groups.setdefault(key, {"wg": r["Workgroup_Size_X"], "lds": r["LDS_Block_Size"],
                                    "vgpr": r["VGPR_Count"], "agpr": r["Accum_VGPR_Count"], "us": []})
        g["us"].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    lines = ["| kernel | grid (x, y, z) | block | LDS B | VGPR | AGPR | launches | avg µs | last "
             f"{last} avg µs | min µs | max µs |", "|---|---|---|---|---|---|---|---|---|---|---|"]
    for (name, gx, gy, gz), g in groups.items():
        us = g["us"]
        tail = us[-last:]
        lines.append(f"| `{name}` | {gx}, {gy}, {gz} | {g['wg']} | {g['lds']} | {g['vgpr']} | {g['agpr']} | "
                     f"{len(us)} | {sum(us) / len(us):.2f} | {sum(tail) / len(tail):.2f} | {min(us):.2f} | "
                     f"{max(us):.2f} |")
    bench = os.path.join(out_dir, "bench.json")
    if os.path.exists(bench):
        with open(bench) as f:
            line = json.loads([ln for ln in f.read().splitlines() if ln.startswith("{")][-1])
        lines += ["", "The same run's own JSON line (HIP-event timing inside bench.py):", ""]
        lines.append(f"* prefill: kernel_ms = {line['ms_per_step']}, {line['value']} {line['unit']}, "
                     f"roofline frac {line['roofline']['frac']}")
        for key in ("decode", "rope", "backward"):
            part = line.get(key) or {}
            if part:
                lines.append(f"* {part.get('workload', key)}: ms_per_call = {part.get('ms_per_call')}, "
                             f"{part.get('value')} {part.get('unit')}, roofline frac {part['roofline']['frac']}")
        for part in line.get("decode_sweep", []):
            lines.append(f"* {part['workload']}: ms_per_call = {part['ms_per_call']}, {part['value']} "
                         f"{part['unit']}, roofline frac {part['roofline']['frac']}")
        floors = [p_ for p_ in [line.get("decode")] + line.get("decode_sweep", []) if p_ and p_.get("read_floor")]
        if floors:
            lines += ["", "Streaming-read floor of each decode row (the row's algorithmic bytes read once, timed "
                      "the same way):", ""]
            for part in floors:
                f_ = part["read_floor"]
                lines.append(f"* {part['workload']}: floor {f_['ms_per_call']} ms ({f_['GB/s']} GB/s), "
                             f"row / floor = {f_['row_over_floor']}")
    return "\n".join(lines) + "\n"


def counter_summary(out_dir: str, kernels) -> str:
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in _csv(out_dir, "counter_collection.csv"):
        if any(k in r["Kernel_Name"] for k in kernels):
            vals[short_name(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    lines = []
    for name, ctr in vals.items():
        n = max(len(v) for v in ctr.values())
        lines += [f"`{name}` (mean of {n} dispatches):", "", "| counter | value |", "|---|---|"]
        for c in sorted(ctr):
            v = ctr[c]
            lines.append(f"| {c} | {sum(v) / len(v):,.0f} |")
        lines.append("")
    return "\n".join(lines)


if __name__ == "__main__":
    import sys

    if len(sys.argv) >= 3 and sys.argv[1] == "trace":
        print(trace_summary(sys.argv[2]), end="")
    elif len(sys.argv) >= 4 and sys.argv[1] == "counters":
        print(counter_summary(sys.argv[2], sys.argv[3].split(",")), end="")
    else:
        raise SystemExit("usage: python -m grouped_query_attention_prefill_amd.profiling trace OUT | counters OUT "
                         "KERNEL[,KERNEL...]")
