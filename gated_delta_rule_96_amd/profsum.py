"""Summarise a rocprofv3 kernel trace (rocpd SQLite database or the
kernel_stats CSV) as a short text table: kernel, calls, total and average
duration (us), share of GPU time.

    python -m gated_delta_rule_96_amd.profsum <results.db | kernel_stats.csv>
"""
from __future__ import annotations

import csv
import sqlite3
import sys


def rows_from_db(path):
    con = sqlite3.connect(path)
    cur = con.execute("select name, total_calls, total_duration, average, percentage from top_kernels")
    # the top_kernels view reports microseconds
    return [(r[0], int(r[1]), float(r[2]), float(r[3]), float(r[4])) for r in cur]


def rows_from_csv(path):
    out = []
    with open(path) as f:
        for r in csv.DictReader(f):
            out.append((r["Name"], int(r["Calls"]), float(r["TotalDurationNs"]) / 1e3,
                        float(r["AverageNs"]) / 1e3, float(r["Percentage"])))
    return out


def main(path):
    rows = rows_from_db(path) if path.endswith(".db") else rows_from_csv(path)
    print(f"{'kernel':<60} {'calls':>6} {'total_us':>12} {'avg_us':>10} {'pct':>6}")
    for name, calls, tot, avg, pct in rows:
        short = name if len(name) <= 60 else name[:57] + "..."
        print(f"{short:<60} {calls:>6} {tot:>12.1f} {avg:>10.2f} {pct:>6.2f}")


if __name__ == "__main__":
    main(sys.argv[1])
