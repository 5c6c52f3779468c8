"""HBM traffic per call from rocprofv3 counter passes.

    python -m gated_mlp_gemm_amd.counters FETCH_DIR WRITE_DIR \
        [--workload M=4096,K=8192,N=29568] [--out profiles/traffic.json]

FETCH_DIR and WRITE_DIR hold the CSV output of two rocprofv3 runs of the same
command, one counter each (rocprofv3 collects what one pass allows):

    rocprofv3 --pmc FETCH_SIZE -f csv -d FETCH_DIR -o bench -- \
        python3 bench.py --steps 3 --warmup 1 --warmup-seconds 0 --repeats 1 \
            --no-cpu-baseline --no-per-workload --no-fp8 --copy-calibration
    rocprofv3 --pmc WRITE_SIZE -f csv -d WRITE_DIR -o bench -- (the same)

(or of ``bench.py --fp8 --fp8-workloads 1 --copy-calibration`` with
``--paths fp8`` for the FP8 kernel).

Both counters report KiB per dispatch.  Each is scaled by what it reads for
the plain 256 MiB device copy that ``--copy-calibration`` runs last (the copy
moves exactly 262144 KiB each way), and each path's kernels are summed with
their launches per call.  The entries record the hash of the kernel sources
they were taken on; the bench reports a figure only while the sources still
hash the same.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
from typing import Dict, List

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
COPY_KIB = 256 * 1024
PEAK_HBM_GBS = 8000.0   # MI355X HBM3E, published

# the kernels each bench path launches per call: (substrings every matching
# kernel name contains, launches per call).  A partly idle last round may add
# a split_reduce_kernel of the same epilogue, one per GEMM launch.
PATHS = {
    "i": [(("gemm_tiles_kernel", "PairMulEpilogueT<false>"), 1),
          (("split_reduce_kernel", "PairMulEpilogueT<false>"), 1)],
    "fp8": [(("gemm_tiles_kernel", "PairMulEpilogueT<true>"), 1),
            (("split_reduce_kernel", "PairMulEpilogueT<true>"), 1)],
    "s": [(("fused_sequential",), 1)],
    "ablation": [(("gemm_tiles_kernel", "StoreEpilogue"), 2),
                 (("split_reduce_kernel", "StoreEpilogue"), 2),
                 (("silu_mul_kernel",), 1)],
}


def _code_only(text: str) -> str:
    """C++/HIP source with comments removed and whitespace runs collapsed, so
    that edits to comments alone leave the hash unchanged.  String literals
    are kept (a '//' inside one is not a comment)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c == '"':                                    # string literal
            j = i + 1
            while j < n and text[j] != '"':
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """Hash of the code (comments and whitespace aside) of every file under
    csrc/, with the file names; 16 hex digits."""
    h = hashlib.sha256()
    csrc = os.path.join(PKG, "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def read_counter(directory: str, counter: str) -> Dict[str, List[float]]:
    """Kernel name -> the counter's values, in dispatch order."""
    rows = []
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"),
                          recursive=True):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"],
                                 float(r["Counter_Value"])))
    if not rows:
        raise SystemExit(f"no {counter} rows under {directory}")
    out: Dict[str, List[float]] = {}
    for _, name, value in sorted(rows):
        out.setdefault(name, []).append(value)
    return out


def copy_scale(values: Dict[str, List[float]]) -> float:
    """262144 KiB over the reading of the last device-copy dispatch."""
    copies = [v for name, vs in values.items() if "copyBuffer" in name for v in vs]
    if not copies:
        raise SystemExit("no device-copy dispatch found (run the bench with --copy-calibration)")
    return COPY_KIB / copies[-1]


def path_records(fetch: Dict[str, List[float]], write: Dict[str, List[float]],
                 source_hash: str) -> Dict[str, dict]:
    fs, ws = copy_scale(fetch), copy_scale(write)
    recs = {}
    for path, kernels in PATHS.items():
        names, launches, f_raw, w_raw = [], [], [], []
        for parts, per_call in kernels:
            for name in fetch:
                if all(p in name for p in parts) and name in write and name not in names:
                    names.append(name)
                    launches.append(per_call)
                    f_raw.append(round(statistics.median(fetch[name]), 1))
                    w_raw.append(round(statistics.median(write[name]), 1))
        if not names:
            continue
        kib = sum(n * (f * fs + w * ws) for n, f, w in zip(launches, f_raw, w_raw))
        recs[path] = {
            "kernel_source_hash": source_hash,
            "kernels": names,
            "launches_per_call": launches,
            "fetch_kib_raw": f_raw,
            "write_kib_raw": w_raw,
            "fetch_scale": round(fs, 4),
            "write_scale": round(ws, 4),
            "hbm_bytes_per_launch": int(round(kib * 1024)),
        }
    return recs


def _short(name: str) -> str:
    return name.split("(")[0].replace("void swiglu::", "").replace("swiglu::", "")


def kernel_table(mfma_dir: str, fetch: Dict[str, List[float]],
                 write: Dict[str, List[float]]) -> List[dict]:
    """Per kernel of a run: median duration and mean clock / MFMA busy from a
    `--kernel-trace --pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES` pass
    (first dispatch of each kernel dropped), and median HBM bytes from the
    FETCH_SIZE / WRITE_SIZE passes of the same command (copy-scaled).
    Clock = GRBM_GUI_ACTIVE / 8 XCDs / duration; MFMA busy =
    SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / those cycles."""
    durs = {}
    for path in glob.glob(os.path.join(mfma_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                durs[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    per: Dict[str, Dict[str, float]] = {}
    names: Dict[str, str] = {}
    for path in glob.glob(os.path.join(mfma_dir, "**", "*counter_collection.csv"),
                          recursive=True):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                per.setdefault(r["Dispatch_Id"], {})[r["Counter_Name"]] = float(r["Counter_Value"])
                names[r["Dispatch_Id"]] = r["Kernel_Name"]
    groups: Dict[str, List[tuple]] = {}
    for d in sorted(per, key=int):
        c, name = per[d], names[d]
        if d not in durs or "GRBM_GUI_ACTIVE" not in c or durs[d] <= 0:
            continue
        cycles = c["GRBM_GUI_ACTIVE"] / 8.0
        groups.setdefault(name, []).append(
            (durs[d], cycles / durs[d], c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / 1024.0 / cycles))
    fs, ws = copy_scale(fetch), copy_scale(write)
    rows = []
    for name, vals in groups.items():
        if "swiglu::" not in name or name not in fetch or name not in write:
            continue   # only the library's kernels
        vals = vals[1:] if len(vals) > 1 else vals
        dur = statistics.median(v[0] for v in vals)
        hbm = (statistics.median(fetch[name]) * fs + statistics.median(write[name]) * ws) * 1024
        rows.append({"kernel": _short(name), "dispatches": len(vals), "us": dur * 1e6,
                     "clock_ghz": statistics.mean(v[1] for v in vals) / 1e9,
                     "mfma_busy": statistics.mean(v[2] for v in vals),
                     "hbm_mb": hbm / 1e6, "hbm_gbs": hbm / dur / 1e9})
    return rows


def main(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("fetch_dir")
    p.add_argument("write_dir")
    p.add_argument("--workload", default="M=4096,K=8192,N=29568")
    p.add_argument("--out", default=os.path.join(ROOT, "profiles", "traffic.json"))
    p.add_argument("--paths", default=",".join(PATHS),
                   help="which paths of the run to record (default: all found)")
    p.add_argument("--mfma", default=None, metavar="DIR",
                   help="also print a per-kernel table (duration, clock, MFMA busy, HBM GB/s) "
                        "from a --kernel-trace --pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES "
                        "pass of the same command; writes nothing")
    a = p.parse_args(argv)
    if a.mfma:
        fetch = read_counter(a.fetch_dir, "FETCH_SIZE")
        write = read_counter(a.write_dir, "WRITE_SIZE")
        print("| kernel | dispatches | median µs | clock GHz | MFMA busy | HBM MB | HBM GB/s "
              "| % of 8 TB/s |")
        print("|---|---|---|---|---|---|---|---|")
        for r in kernel_table(a.mfma, fetch, write):
            print(f"| {r['kernel']} | {r['dispatches']} | {r['us']:.2f} | {r['clock_ghz']:.2f} | "
                  f"{100 * r['mfma_busy']:.1f} % | {r['hbm_mb']:.1f} | {r['hbm_gbs']:.0f} | "
                  f"{100 * r['hbm_gbs'] / PEAK_HBM_GBS:.0f} % |")
        return
    recs = path_records(read_counter(a.fetch_dir, "FETCH_SIZE"),
                        read_counter(a.write_dir, "WRITE_SIZE"), kernel_source_hash())
    keep = set(a.paths.split(","))
    recs = {k: v for k, v in recs.items() if k in keep}
    table = {}
    if os.path.exists(a.out):
        with open(a.out) as f:
            table = json.load(f)
    for path, rec in recs.items():
        table[f"{path}|{a.workload}"] = rec
    with open(a.out, "w") as f:
        json.dump(table, f, indent=1)
        f.write("\n")
    for path, rec in recs.items():
        print(f"{path}: {rec['hbm_bytes_per_launch'] / 1e6:.1f} MB per call "
              f"({', '.join(rec['kernels'])})")


if __name__ == "__main__":
    main()
