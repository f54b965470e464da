"""Fold rocprofv3 output into the counter records under ``profiles/``.

The benchmark prices its dominant kernel against measured HBM traffic read
from ``profiles/<name>.json``.  That record comes from three runs of the same
bench command: a kernel trace (``--kernel-trace --stats``), then one
``--pmc FETCH_SIZE`` and one ``--pmc WRITE_SIZE`` pass, each with
``--copy-mb N`` so that the same counters also read a plain device copy of
known size.  The counters are divided by the copy's reading of its own true
size (the calibration factor), averaged over the kernel's dispatches, and
stored with a digest of the kernel's sources so that a stale record is never
used.  Usage (from the repository root)::

    python -m rank_compressed_kv_lrkv_amd.profile_summary --name decode_scan_counters \\
        --kernel decode_mfma_kernel --workload mid_bf16_T8k --split 0 \\
        --trace <dir>/kt_kernel_stats.csv --fetch <dir>/fetch_counter_collection.csv \\
        --write <dir>/write_counter_collection.csv --copy-mb 1024 --command "python3 -u bench.py ..."
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def short_name(name):
    """Kernel name without `void`, the library namespace and an anonymous one."""
    return name.replace("void ", "").replace("(anonymous namespace)::", "").replace("lrkv::", "")


def counter_means(path, counter):
    """Mean value of `counter` per dispatch, keyed by kernel name (without
    arguments).  For the copy kernel only the dispatches of the largest grid
    count: those are the reference copies; the program's own small copies
    (uploads, staging) would dilute the calibration."""
    rows = []
    with open(path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == counter:
                rows.append(row)
    copy_grid = max((int(r["Grid_Size"]) for r in rows if COPY_KERNEL in r["Kernel_Name"]), default=None)
    acc = {}
    for row in rows:
        if COPY_KERNEL in row["Kernel_Name"] and int(row["Grid_Size"]) != copy_grid:
            continue
        name = short_name(row["Kernel_Name"]).split("(")[0]
        tot, n = acc.get(name, (0.0, 0))
        acc[name] = (tot + float(row["Counter_Value"]), n + 1)
    return {k: t / n for k, (t, n) in acc.items()}


def pick(means, kernel):
    hits = [v for k, v in means.items() if k.startswith(kernel)]
    if len(hits) != 1:
        raise SystemExit(f"expected one kernel named {kernel}* in the counters, found {sorted(means)}")
    return hits[0]


def trace_stats(path, kernel):
    with open(path) as f:
        for row in csv.DictReader(f):
            if short_name(row["Name"]).startswith(kernel):
                return {"calls": int(row["Calls"]), "avg_us": float(row["AverageNs"]) / 1e3,
                        "min_us": float(row["MinNs"]) / 1e3, "max_us": float(row["MaxNs"]) / 1e3}
    raise SystemExit(f"{kernel} not in {path}")


def main(argv=None):
    sys.path.insert(0, ROOT)
    from bench import KERNEL_SOURCES, source_digest
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--name", required=True, help="record name: profiles/<name>.json")
    ap.add_argument("--kernel", required=True, choices=sorted(KERNEL_SOURCES))
    ap.add_argument("--workload", required=True)
    ap.add_argument("--split", type=int, default=None)
    ap.add_argument("--trace", help="rocprofv3 kernel_stats.csv (optional)")
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-mb", type=int, required=True)
    ap.add_argument("--command", required=True)
    a = ap.parse_args(argv)

    copy_kib = a.copy_mb * 1024.0
    fetch, write = counter_means(a.fetch, "FETCH_SIZE"), counter_means(a.write, "WRITE_SIZE")
    cal_f, cal_w = pick(fetch, COPY_KERNEL) / copy_kib, pick(write, COPY_KERNEL) / copy_kib
    kf, kw = pick(fetch, a.kernel), pick(write, a.kernel)
    rec = {
        "kernel": a.kernel,
        "workload": a.workload,
        "source_sha256_16": source_digest(KERNEL_SOURCES[a.kernel]),
        "fetch_kib_per_dispatch": kf,
        "write_kib_per_dispatch": kw,
        "copy_calibration": {"fetch": cal_f, "write": cal_w},
        "hbm_bytes_per_launch": int(round((kf / cal_f + kw / cal_w) * 1024)),
        "command": a.command,
    }
    if a.split is not None:
        rec["split_tokens"] = a.split
    if a.trace:
        rec["trace"] = trace_stats(a.trace, a.kernel)
    out = os.path.join(ROOT, "profiles", a.name + ".json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    main()
