"""Summarise rocprofv3 CSV output into a short markdown table.

    python -m fp32_gemm_major_amd.profsummary --trace DIR/x_kernel_trace.csv \
        [--stats DIR/x_kernel_stats.csv] [--counters DIR/y_counter_collection.csv ...] \
        [--command "..."] > profiles/<kernel>_<workload>.md

Dispatches of one kernel are grouped by grid size as well as by name, since
one kernel runs several problem shapes in a benchmark run.
"""
from __future__ import annotations

import argparse
import collections
import csv
import statistics


def short(name: str) -> str:
    name = name.replace("sgemm::", "")
    if "(" in name:
        name = name[: name.index("(")]
    return name.replace("void ", "")


def trace_table(path):
    groups = collections.defaultdict(list)
    for r in csv.DictReader(open(path, newline="")):
        dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        grid = r.get("Grid_Size") or r.get("Grid_Size_X") or "?"
        wg = r.get("Workgroup_Size") or r.get("Workgroup_Size_X") or "?"
        groups[(short(r["Kernel_Name"]), grid, wg)].append(dur)
    out = ["| kernel | grid (work-items) | wg | calls | mean us | median us | min us | max us |",
           "|---|---|---|---|---|---|---|---|"]
    for (k, g, wg), d in sorted(groups.items(), key=lambda x: -sum(x[1])):
        out.append(f"| {k} | {g} | {wg} | {len(d)} | {statistics.mean(d)/1e3:.2f} | "
                   f"{statistics.median(d)/1e3:.2f} | {min(d)/1e3:.2f} | {max(d)/1e3:.2f} |")
    return out


def stats_table(path):
    out = ["| kernel | calls | average us | min us | max us | % |", "|---|---|---|---|---|---|"]
    for r in csv.DictReader(open(path, newline="")):
        out.append(f"| {short(r['Name'])} | {r['Calls']} | {float(r['AverageNs'])/1e3:.2f} | "
                   f"{float(r['MinNs'])/1e3:.2f} | {float(r['MaxNs'])/1e3:.2f} | "
                   f"{float(r['Percentage']):.2f} |")
    return out


def counter_table(paths):
    groups = collections.defaultdict(list)
    for path in paths:
        for r in csv.DictReader(open(path, newline="")):
            key = (short(r["Kernel_Name"]), r.get("Grid_Size", "?"), r["Counter_Name"])
            groups[key].append(float(r["Counter_Value"]))
    out = ["| kernel | grid | counter | dispatches | mean value |", "|---|---|---|---|---|"]
    for (k, g, c), v in sorted(groups.items()):
        out.append(f"| {k} | {g} | {c} | {len(v)} | {statistics.mean(v):.1f} |")
    return out


def traffic_entry(fetch_csv, write_csv, kernel_substr, grid, copy_bytes, workload,
                  kernel_name, source_hash):
    """HBM bytes per launch of one kernel from a FETCH_SIZE run and a
    WRITE_SIZE run (KiB per dispatch), each scaled by what the same counter
    reads for the plain device copy of ``copy_bytes`` in the same run."""
    def read(path, counter):
        vals, copy = [], None
        for r in csv.DictReader(open(path, newline="")):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"])
            if "copyBuffer" in r["Kernel_Name"]:
                copy = v
            elif kernel_substr in r["Kernel_Name"] and r.get("Grid_Size") == str(grid):
                vals.append(v)
        if not vals or copy is None:
            raise SystemExit(f"{path}: no {counter} values for the kernel or the copy")
        return statistics.mean(vals), copy
    f, fc = read(fetch_csv, "FETCH_SIZE")
    w, wc = read(write_csv, "WRITE_SIZE")
    copy_kib = copy_bytes / 1024.0
    fs, ws = copy_kib / fc, copy_kib / wc
    return {"workload": workload, "kernel": kernel_name, "source_hash": source_hash,
            "fetch_kib_raw": round(f, 1), "write_kib_raw": round(w, 1),
            "copy_bytes": copy_bytes, "copy_fetch_kib_raw": round(fc, 1),
            "copy_write_kib_raw": round(wc, 1), "fetch_scale": round(fs, 4),
            "write_scale": round(ws, 4),
            "hbm_bytes_per_launch": int(round((f * fs + w * ws) * 1024))}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace")
    ap.add_argument("--stats")
    ap.add_argument("--counters", nargs="*", default=[])
    ap.add_argument("--command", default="")
    ap.add_argument("--title", default="rocprofv3 summary")
    a = ap.parse_args(argv)
    lines = [f"# {a.title}", ""]
    if a.command:
        lines += ["Command:", "", "```", a.command, "```", ""]
    if a.stats:
        lines += ["rocprofv3 --stats (grouped by kernel name):", ""] + stats_table(a.stats) + [""]
    if a.trace:
        lines += ["Kernel trace grouped by kernel and grid size:", ""] + trace_table(a.trace) + [""]
    if a.counters:
        lines += ["Counters (per dispatch):", ""] + counter_table(a.counters) + [""]
    print("\n".join(lines))


if __name__ == "__main__":
    main()
