"""Summaries of rocprofv3 runs as short text.

Kernel trace (rocpd SQLite database or the kernel_stats CSV): kernel, calls,
total and average duration (us), share of GPU time.

    python -m gated_delta_rule_96_amd.profsum <results.db | kernel_stats.csv>

Memory counters of one kernel, calibrated by a plain copy of known size:

    python -m gated_delta_rule_96_amd.profsum pmc KERNEL_SUBSTRING \
        FETCH_counter_collection.csv WRITE_counter_collection.csv \
        COPY_FETCH_counter_collection.csv COPY_WRITE_counter_collection.csv COPY_BYTES

FETCH_SIZE and WRITE_SIZE are read per dispatch (KiB); each is scaled by
COPY_BYTES / (what the same counter reads for the copy), giving HBM bytes
per launch.  The summary also records the sha256 of the kernel sources, so
that a reader can tell whether the figures still describe the current code.
"""
from __future__ import annotations

import csv
import hashlib
import os
import sqlite3
import sys

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
SOURCES = ("kda_chunk.hip", "kda_device.h")


def source_sha256() -> str:
    """sha256 over the fused prefill kernel's sources (the code the counters describe)."""
    h = hashlib.sha256()
    for name in SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counter_per_dispatch(path, counter, kernel_sub):
    """Mean value of `counter` over the dispatches whose kernel name contains
    kernel_sub (values of one dispatch summed over its rows)."""
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and kernel_sub in r["Kernel_Name"]:
                per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} rows for kernels matching {kernel_sub!r} in {path}")
    return sum(per.values()) / len(per), len(per)


def pmc(kernel_sub, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_bytes):
    copy_bytes = float(copy_bytes)
    cf, ncf = counter_per_dispatch(copy_fetch_csv, "FETCH_SIZE", "copyBuffer")
    cw, ncw = counter_per_dispatch(copy_write_csv, "WRITE_SIZE", "copyBuffer")
    kf, nkf = counter_per_dispatch(fetch_csv, "FETCH_SIZE", kernel_sub)
    kw, nkw = counter_per_dispatch(write_csv, "WRITE_SIZE", kernel_sub)
    sf, sw = copy_bytes / cf, copy_bytes / cw
    print(f"kernel: {kernel_sub}")
    print(f"copy calibration: {copy_bytes:.0f} bytes each way; FETCH_SIZE {cf:.1f} KiB/dispatch "
          f"({ncf} dispatches) -> scale {sf:.4f} bytes per unit; WRITE_SIZE {cw:.1f} KiB/dispatch "
          f"({ncw}) -> scale {sw:.4f}")
    print(f"kernel FETCH_SIZE {kf:.1f} KiB/dispatch ({nkf} dispatches) -> {kf * sf:.0f} bytes read")
    print(f"kernel WRITE_SIZE {kw:.1f} KiB/dispatch ({nkw} dispatches) -> {kw * sw:.0f} bytes written")
    print(f"traffic_bytes_per_launch: {kf * sf + kw * sw:.0f}")
    print(f"source_sha256: {source_sha256()}")


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
    if sys.argv[1] == "pmc":
        pmc(*sys.argv[2:8])
    else:
        main(sys.argv[1])
