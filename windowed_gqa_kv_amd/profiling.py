"""Summaries of rocprofv3 output for the roofline numbers that bench.py reports.

    python -m windowed_gqa_kv_amd.profiling stats DIR [--by-grid]
        Markdown table of the kernel durations in DIR/*kernel_stats.csv, or,
        with --by-grid, from DIR/*kernel_trace.csv with one row per (kernel,
        grid size), which tells apart the workloads that launch one kernel.

    python -m windowed_gqa_kv_amd.profiling traffic --fetch DIR --write DIR \\
            --cal-fetch DIR --cal-write DIR --cal-mib N --kernel PATTERN \\
            --cal-kernel PATTERN --workload NAME --key KEY --out FILE [--grid N]
        HBM bytes per launch of the kernels whose names contain PATTERN (and,
        with --grid, whose grid holds N work-items), from
        two counter runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch).  Each
        counter is scaled by what it reads for a plain copy of N MiB (kernels
        matching the calibration pattern) so that a counter which reports a
        fixed fraction of the true bytes is corrected.  The record, keyed by
        KEY and stamped with a hash of the kernel sources, is merged into the
        JSON file FILE, where bench.py looks it up.

    python -m windowed_gqa_kv_amd.profiling counters DIR [DIR ...] --kernel PATTERN [--grid N]
        Markdown table of the mean per-dispatch value of every counter found in
        the DIRs' counter runs, over the kernels whose names contain PATTERN
        (and whose grid holds N work-items), with the dispatch count.

The sources that the hash covers are the ones bench.py names; a record taken
on other sources is ignored there.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))


def src_hash(names) -> str:
    """Short hash of kernel sources under csrc/ and of their per-file compiler
    flags (bench.py compares it): a record taken on other code is ignored."""
    from .build import FILE_FLAGS
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(PKG, "csrc", n), "rb") as f:
            h.update(f.read())
        h.update(" ".join(FILE_FLAGS.get(n, [])).encode())
    return h.hexdigest()[:16]


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def kernel_stats(d: str):
    """Rows of *kernel_stats.csv: (name, calls, avg_us, min_us, max_us)."""
    rows = []
    with open(_one(os.path.join(d, "**", "*kernel_stats.csv"))) as f:
        for r in csv.DictReader(f):
            rows.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                         float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
    return rows


def kernel_stats_by_grid(d: str):
    """Rows of *kernel_trace.csv grouped by (name, grid work-items):
    (name, grid, calls, avg_us, min_us, max_us)."""
    groups = {}
    with open(_one(os.path.join(d, "**", "*kernel_trace.csv"))) as f:
        for r in csv.DictReader(f):
            grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            groups.setdefault((r["Kernel_Name"], grid), []).append(us)
    return [(name, grid, len(v), sum(v) / len(v), min(v), max(v)) for (name, grid), v in groups.items()]


def counter_mean(d: str, counter: str, pattern: str, grid: int = 0):
    """Mean per-dispatch value (KiB for *_SIZE counters) and dispatch count of
    `counter` over the kernels whose names contain `pattern` (and whose grid
    holds `grid` work-items, if nonzero)."""
    vals = {}
    with open(_one(os.path.join(d, "**", "*counter_collection.csv"))) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter or pattern not in r["Kernel_Name"]:
                continue
            if grid and int(r["Grid_Size"]) != grid:
                continue
            # one row per dispatch (and counter); sum in case a counter is split
            key = r["Dispatch_Id"]
            vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    if not vals:
        raise ValueError(f"no {counter} rows for kernels matching {pattern!r} in {d}")
    return sum(vals.values()) / len(vals), len(vals)


def counter_names(d: str):
    """Counter names present in a counter run."""
    with open(_one(os.path.join(d, "**", "*counter_collection.csv"))) as f:
        return sorted({r["Counter_Name"] for r in csv.DictReader(f)})


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--by-grid", action="store_true")
    t = sub.add_parser("traffic")
    for k in ("fetch", "write", "cal_fetch", "cal_write", "kernel", "cal_kernel", "workload", "key", "out"):
        t.add_argument("--" + k.replace("_", "-"), required=True)
    t.add_argument("--cal-mib", type=float, required=True)
    t.add_argument("--sources", default="decode_mfma.hip,common.h,kernels.h")
    t.add_argument("--command", default="")
    t.add_argument("--grid", type=int, default=0)
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--kernel", required=True)
    c.add_argument("--grid", type=int, default=0)
    a = ap.parse_args(argv)

    if a.cmd == "counters":
        print("| counter | mean per dispatch | dispatches |")
        print("|---|---|---|")
        for d in a.dirs:
            for name in counter_names(d):
                mean, n = counter_mean(d, name, a.kernel, a.grid)
                print(f"| {name} | {mean:,.0f} | {n} |")
        return 0

    if a.cmd == "stats" and a.by_grid:
        print("| kernel | grid work-items | calls | avg us | min us | max us |")
        print("|---|---|---|---|---|---|")
        for name, grid, calls, avg, mn, mx in sorted(kernel_stats_by_grid(a.dir), key=lambda r: -r[2] * r[3]):
            print(f"| `{name}` | {grid} | {calls} | {avg:.2f} | {mn:.2f} | {mx:.2f} |")
        return 0
    if a.cmd == "stats":
        print("| kernel | calls | avg us | min us | max us |")
        print("|---|---|---|---|---|")
        for name, calls, avg, mn, mx in sorted(kernel_stats(a.dir), key=lambda r: -r[1] * r[2]):
            print(f"| `{name}` | {calls} | {avg:.2f} | {mn:.2f} | {mx:.2f} |")
        return 0

    fetch_kib, n_f = counter_mean(a.fetch, "FETCH_SIZE", a.kernel, a.grid)
    write_kib, n_w = counter_mean(a.write, "WRITE_SIZE", a.kernel, a.grid)
    cal_f, _ = counter_mean(a.cal_fetch, "FETCH_SIZE", a.cal_kernel)
    cal_w, _ = counter_mean(a.cal_write, "WRITE_SIZE", a.cal_kernel)
    true_kib = a.cal_mib * 1024.0
    f_scale, w_scale = true_kib / cal_f, true_kib / cal_w
    rec = {
        "kernel": a.kernel, "workload": a.workload, "grid": a.grid or None,
        "fetch_kib_per_dispatch": round(fetch_kib, 1), "write_kib_per_dispatch": round(write_kib, 1),
        "dispatches": [n_f, n_w],
        "copy_calibration": {"mib": a.cal_mib, "fetch_kib": round(cal_f, 1), "write_kib": round(cal_w, 1),
                             "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)},
        "bytes_per_launch": int(round((fetch_kib * f_scale + write_kib * w_scale) * 1024)),
        "src_hash": src_hash(a.sources.split(",")),
        "command": a.command,
    }
    table = {}
    if os.path.exists(a.out):
        with open(a.out) as f:
            table = json.load(f)
    table[a.key] = rec
    with open(a.out, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
        f.write("\n")
    json.dump(rec, sys.stdout, indent=1)
    print()
    return 0


if __name__ == "__main__":
    sys.exit(main())
