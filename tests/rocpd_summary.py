"""Summarise a rocprofv3 rocpd database (kernel table) as a markdown table.

    python -m tests.rocpd_summary <run_results.db> [title]
"""
import sqlite3
import sys


def short(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "")
    base = name.split("(")[0]
    return base if len(base) <= 70 else base[:67] + "..."


def summarize(db: str):
    c = sqlite3.connect(db)
    rows = c.execute("select name, count(*), sum(duration), avg(duration), min(duration), "
                     "max(duration) from kernels group by name order by sum(duration) desc").fetchall()
    out = ["| kernel | calls | total us | avg us | min us | max us |", "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| {short(r[0])} | {r[1]} | {r[2] / 1e3:.1f} | {r[3] / 1e3:.2f} | "
                   f"{r[4] / 1e3:.2f} | {r[5] / 1e3:.2f} |")
    return "\n".join(out)


if __name__ == "__main__":
    print(summarize(sys.argv[1]))
