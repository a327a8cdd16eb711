"""Turn rocprofv3 --pmc CSV output into HBM bytes per kernel launch.

    python -m tests.pmc_summary --fetch F.csv --write W.csv \
        --copy-fetch CF.csv --copy-write CW.csv --kernel attn_split_kernel<true> \
        --splits 1 [--grid 131072] [--json out.json]

FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the kernel are averaged over
its dispatches and scaled by what the same counters read for the 256 MiB
device copies of ``bench.py --copy-calibration`` (true bytes / counted
bytes), giving the kernel's HBM traffic per launch.  With --json the result
is written where bench.py reads it, tagged with the hash of the kernel
source it was measured on.
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

COPY_BYTES = 256 * 2 ** 20


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-fetch", required=True)
    ap.add_argument("--copy-write", required=True)
    ap.add_argument("--kernel", required=True)
    ap.add_argument("--splits", type=int, required=True)
    ap.add_argument("--grid", type=int, default=0,
                    help="only dispatches of this grid size in work-items (one workload)")
    ap.add_argument("--json")
    a = ap.parse_args()
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
        import bench
        res["kernel_source_sha"] = bench.kernel_source_sha()
        with open(a.json, "w") as f:
            json.dump(res, f, indent=1)
            f.write("\n")
    print(json.dumps(res, indent=1))


if __name__ == "__main__":
    main()
