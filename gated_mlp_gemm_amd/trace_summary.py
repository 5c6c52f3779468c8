"""Per-kernel summary of a rocprofv3 kernel trace.

    python -m gated_mlp_gemm_amd.trace_summary DIR [--segment SUBSTR --skip S --count C]

DIR is the output directory of ``rocprofv3 --kernel-trace ... -d DIR`` (the
SQLite ``*_results.db`` it writes, or a ``*kernel_trace.csv`` of ``-f csv``).
Prints a markdown table of every kernel: calls, average, median, minimum and
maximum duration in microseconds.  ``--segment`` also averages one run of
dispatches: of the kernels whose short name (as in the table) contains SUBSTR, in dispatch order,
skip the first S and average the next C (e.g. the timed steps that follow a
bench loop's warm-up steps).
"""
from __future__ import annotations

import argparse
import csv
import glob
import os
import re
import sqlite3
import statistics
from typing import List, Tuple


def short_name(name: str) -> str:
    """Kernel name without namespace, return type and argument list."""
    n = re.sub(r"\(.*$", "", name.strip())
    n = n.replace("swiglu::", "")
    if n.startswith("void "):
        n = n[5:]
    return n


def load(directory: str) -> List[Tuple[str, int, int]]:
    """(name, start ns, duration ns) of every kernel dispatch, by start time."""
    dbs = sorted(glob.glob(os.path.join(directory, "**", "*_results.db"), recursive=True))
    if dbs:
        out = []
        for path in dbs:
            con = sqlite3.connect(path)
            out += con.execute("select name, start, duration from kernels").fetchall()
            con.close()
        return sorted(out, key=lambda r: r[1])
    csvs = sorted(glob.glob(os.path.join(directory, "**", "*kernel_trace.csv"), recursive=True))
    if not csvs:
        raise FileNotFoundError(f"no *_results.db or *kernel_trace.csv under {directory}")
    out = []
    for path in csvs:
        with open(path) as f:
            for r in csv.DictReader(f):
                s, e = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
                out.append((r["Kernel_Name"], s, e - s))
    return sorted(out, key=lambda r: r[1])


def table(rows) -> str:
    by = {}
    for name, _, dur in rows:
        by.setdefault(short_name(name), []).append(dur / 1e3)
    lines = ["| kernel | calls | avg µs | median µs | min µs | max µs |",
             "|---|---|---|---|---|---|"]
    for k, v in by.items():
        lines.append(f"| {k} | {len(v)} | {statistics.mean(v):.2f} | "
                     f"{statistics.median(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
    return "\n".join(lines)


def segment(rows, substr: str, skip: int, count: int):
    d = [dur / 1e3 for name, _, dur in rows if substr in short_name(name)][skip:skip + count]
    if not d:
        raise ValueError(f"no dispatches of {substr!r} after skipping {skip}")
    return {"calls": len(d), "avg_us": round(statistics.mean(d), 2),
            "min_us": round(min(d), 2), "max_us": round(max(d), 2)}


def main(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("directory")
    p.add_argument("--segment", action="append", default=[],
                   help="substring of the kernel name (repeatable, with --skip/--count each)")
    p.add_argument("--skip", type=int, action="append", default=[])
    p.add_argument("--count", type=int, action="append", default=[])
    a = p.parse_args(argv)
    rows = load(a.directory)
    print(table(rows))
    for i, sub in enumerate(a.segment):
        skip = a.skip[i] if i < len(a.skip) else 0
        count = a.count[i] if i < len(a.count) else 1 << 30
        print(f"\nsegment {sub!r} (skip {skip}, count {count}): {segment(rows, sub, skip, count)}")


if __name__ == "__main__":
    main()
