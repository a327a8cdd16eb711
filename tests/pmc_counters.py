"""Average rocprofv3 --pmc counters per dispatch of one kernel.

    python -m tests.pmc_counters --kernel 'attn_split_kernel<false>' [--first N] F.csv [F.csv ...]

Reads run_counter_collection.csv files (any counters), keeps the dispatches
whose kernel name contains --kernel (the first N of them, in dispatch order,
with --first), and prints each counter's mean over those dispatches as a
markdown table row set.  The counters are summed over the whole device per
dispatch, as rocprofv3 reports them.
"""
from __future__ import annotations

import argparse
import csv
from collections import defaultdict


def averages(paths, kernel: str, first: int | None):
    per = defaultdict(dict)   # counter -> {dispatch id: value}
    for path in paths:
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if kernel in r["Kernel_Name"]:
                    d = int(r["Dispatch_Id"])
                    per[r["Counter_Name"]][d] = per[r["Counter_Name"]].get(d, 0.0) + float(r["Counter_Value"])
    out = {}
    for name, vals in per.items():
        ids = sorted(vals)[:first] if first else sorted(vals)
        out[name] = (sum(vals[i] for i in ids) / len(ids), len(ids))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--kernel", required=True)
    ap.add_argument("--first", type=int)
    ap.add_argument("csv", nargs="+")
    a = ap.parse_args()
    res = averages(a.csv, a.kernel, a.first)
    print("| counter | mean per dispatch | dispatches |")
    print("|---|---|---|")
    for name in sorted(res):
        mean, n = res[name]
        print(f"| {name} | {mean:,.0f} | {n} |")


if __name__ == "__main__":
    main()
