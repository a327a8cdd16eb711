"""Post-processing of rocprofv3 output for bench.py's profiles.

    python rocprof_summary.py trace <run_results.db> [--kernel SUBSTR --by-grid]
        Per-kernel table (calls, total/avg/min/max/median us) from a
        ``rocprofv3 --kernel-trace --stats`` database.  With --kernel and
        --by-grid, the matching kernel's launches split by grid size (one
        workload each) with their median and mean.

    python rocprof_summary.py traffic --fetch F.csv --write W.csv \\
        --copy-fetch CF.csv --copy-write CW.csv --kernel 'attn_split_kernel<true>' \\
        --splits 1 [--grid 131072] [--json out.json]
        HBM bytes per launch: FETCH_SIZE and WRITE_SIZE (KiB per dispatch,
        each from a ``--pmc`` run of its own) averaged over the kernel's
        dispatches and scaled by what the same counters read for the 256 MiB
        device copies of ``bench.py --copy-calibration``.  With --json the
        result is written where bench.py reads it, tagged with the hash of
        the kernel source it was measured on.

    python rocprof_summary.py counters --kernel SUBSTR [--first N] [--grid G] F.csv [...]
        Mean of every counter per dispatch of one kernel (any counters).
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import sqlite3
import statistics
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 256 * 2 ** 20


# ---------------------------------------------------------------- trace --

def short(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "")
    base = name.split("(")[0]
    return base if len(base) <= 70 else base[:67] + "..."


def trace_table(db: str) -> str:
    c = sqlite3.connect(db)
    rows = c.execute("select name, duration from kernels").fetchall()
    per = defaultdict(list)
    for name, dur in rows:
        per[name].append(dur / 1e3)
    out = ["| kernel | calls | total us | avg us | median us | min us | max us |",
           "|---|---|---|---|---|---|---|"]
    for name, d in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"| {short(name)} | {len(d)} | {sum(d):.1f} | {sum(d) / len(d):.2f} | "
                   f"{statistics.median(d):.2f} | {min(d):.2f} | {max(d):.2f} |")
    return "\n".join(out)


def trace_by_grid(db: str, kernel: str) -> str:
    """Launches of one kernel split by grid size (work-items)."""
    c = sqlite3.connect(db)
    cols = [r[1] for r in c.execute("pragma table_info(kernels)").fetchall()]
    gcol = next((g for g in ("grid_size", "grid_size_x", "grid_x") if g in cols), None)
    if gcol is None:
        raise SystemExit(f"no grid-size column in the kernels table: {cols}")
    rows = c.execute(f"select name, {gcol}, duration from kernels order by start").fetchall()
    per = defaultdict(list)
    for name, grid, dur in rows:
        if kernel in name:
            per[(short(name), int(grid))].append(dur / 1e3)
    out = ["| kernel | grid (work-items) | launches | median us | mean us | min us | max us |",
           "|---|---|---|---|---|---|---|"]
    for (name, grid), d in sorted(per.items(), key=lambda kv: (kv[0][1], kv[0][0])):
        out.append(f"| {name} | {grid} | {len(d)} | {statistics.median(d):.2f} | "
                   f"{sum(d) / len(d):.2f} | {min(d):.2f} | {max(d):.2f} |")
    return "\n".join(out)


# -------------------------------------------------------------- counters --

def counter_values(path: str, kernel_substr: str, counter: str, grid: int = 0):
    """Values of one counter for the dispatches of a kernel (only those of
    grid size `grid` work-items when it is nonzero)."""
    vals = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and kernel_substr in r["Kernel_Name"] and \
                    (not grid or int(r["Grid_Size"]) == grid):
                vals.append(float(r["Counter_Value"]))
    return vals


def calibration(path: str, counter: str) -> float:
    """True bytes / counted bytes for the device copies of 256 MiB."""
    vals = counter_values(path, "copyBuffer", counter)
    if not vals:
        vals = counter_values(path, "elementwise_kernel", counter)
    kib = max(vals)
    return COPY_BYTES / (kib * 1024.0)


def traffic(a) -> dict:
    fetch = counter_values(a.fetch, a.kernel, "FETCH_SIZE", a.grid)
    write = counter_values(a.write, a.kernel, "WRITE_SIZE", a.grid)
    if not fetch or not write:
        sys.exit(f"no dispatches of {a.kernel!r} in the counter files")
    f_cal = calibration(a.copy_fetch, "FETCH_SIZE")
    w_cal = calibration(a.copy_write, "WRITE_SIZE")
    f_kib = sum(fetch) / len(fetch)
    w_kib = sum(write) / len(write)
    read_b = f_kib * 1024.0 * f_cal
    write_b = w_kib * 1024.0 * w_cal
    res = {
        "kernel": a.kernel,
        "grid": a.grid or None,
        "dispatches": [len(fetch), len(write)],
        "fetch_size_kib_per_dispatch": round(f_kib, 3),
        "write_size_kib_per_dispatch": round(w_kib, 3),
        "fetch_calibration": round(f_cal, 4),
        "write_calibration": round(w_cal, 4),
        "hbm_read_bytes_per_launch": int(round(read_b)),
        "hbm_write_bytes_per_launch": int(round(write_b)),
        "hbm_bytes_per_launch": int(round(read_b + write_b)),
        "splits": a.splits,
    }
    if a.json:
        if ROOT not in sys.path:
            sys.path.insert(0, ROOT)
        import bench
        res["kernel_source_sha"] = bench.kernel_source_sha()
        with open(a.json, "w") as f:
            json.dump(res, f, indent=1)
            f.write("\n")
    return res


def counter_means(paths, kernel: str, first: int | None, grid: int = 0):
    per = defaultdict(dict)   # counter -> {dispatch id: value}
    for path in paths:
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if kernel in r["Kernel_Name"] and (not grid or int(r["Grid_Size"]) == grid):
                    d = int(r["Dispatch_Id"])
                    per[r["Counter_Name"]][d] = per[r["Counter_Name"]].get(d, 0.0) + \
                        float(r["Counter_Value"])
    out = {}
    for name, vals in per.items():
        ids = sorted(vals)[:first] if first else sorted(vals)
        out[name] = (sum(vals[i] for i in ids) / len(ids), len(ids))
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("--kernel")
    t.add_argument("--by-grid", action="store_true")
    f = sub.add_parser("traffic")
    for k in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--kernel"):
        f.add_argument(k, required=True)
    f.add_argument("--splits", type=int, required=True)
    f.add_argument("--grid", type=int, default=0,
                   help="only dispatches of this grid size in work-items (one workload)")
    f.add_argument("--json")
    c = sub.add_parser("counters")
    c.add_argument("--kernel", required=True)
    c.add_argument("--first", type=int)
    c.add_argument("--grid", type=int, default=0,
                   help="only dispatches of this grid size in work-items (one workload)")
    c.add_argument("csv", nargs="+")
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        print(trace_table(a.db))
        if a.kernel and a.by_grid:
            print()
            print(trace_by_grid(a.db, a.kernel))
    elif a.cmd == "traffic":
        print(json.dumps(traffic(a), indent=1))
    else:
        res = counter_means(a.csv, a.kernel, a.first, a.grid)
        print("| counter | mean per dispatch | dispatches |")
        print("|---|---|---|")
        for name in sorted(res):
            mean, n = res[name]
            print(f"| {name} | {mean:,.0f} | {n} |")


if __name__ == "__main__":
    main()
