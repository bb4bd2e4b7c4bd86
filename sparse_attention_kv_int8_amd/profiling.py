"""rocprofv3 output -> short text summaries and calibrated HBM traffic.

    python -m sparse_attention_kv_int8_amd.profiling stats STATS_CSV --workload W --command "..." --out FILE.md
    python -m sparse_attention_kv_int8_amd.profiling traffic --fetch FETCH_CSV --write WRITE_CSV \
        --kernel REGEX --copy REGEX --copy-bytes N --workload W --kind KIND --command-fetch "..." \
        --command-write "..." --out FILE.json

`stats` tabulates a `--kernel-trace --stats` kernel_stats.csv.  `traffic`
reads two `--pmc` counter_collection.csv files (FETCH_SIZE, then
WRITE_SIZE; KiB per dispatch), takes the mean per dispatch of the kernels
matching --kernel, and scales each counter by copy_bytes / (the same
counter's mean for a plain elementwise copy of copy_bytes bytes in the
same run).  The record carries a digest of the kernel sources, so a reader
can tell whether the counters still describe the kernels being run.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
PROFILES = os.path.join(ROOT, "profiles")


def sources_digest() -> str:
    """sha256 over the HIP sources and the C header, in name order."""
    h = hashlib.sha256()
    csrc = os.path.join(PKG, "csrc")
    files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith((".hip", ".h")))
    files.append(os.path.join(ROOT, "include", "sd.h"))
    for p in files:
        h.update(os.path.basename(p).encode())
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def kernel_stats_md(stats_csv: str, workload: str, command: str) -> str:
    rows = list(csv.DictReader(open(stats_csv)))
    out = [f"# rocprofv3 kernel statistics: {workload}", "", "Command (from the repository root):", "",
           "```", command, "```", "",
           "| kernel | calls | avg µs | min µs | max µs | share % |", "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        name = r["Name"]
        if len(name) > 90:
            name = name[:87] + "..."
        out.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | {float(r['MinNs']) / 1e3:.3f} | "
                   f"{float(r['MaxNs']) / 1e3:.3f} | {float(r['Percentage']):.2f} |")
    return "\n".join(out) + "\n"


def _mean_counter(path: str, counter: str, regex: str) -> tuple[float, int]:
    pat = re.compile(regex)
    vals = []
    for r in csv.DictReader(open(path)):
        if r.get("Counter_Name") != counter or not pat.search(r.get("Kernel_Name", "")):
            continue
        vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"{path}: no {counter} rows for kernels matching {regex!r}")
    return statistics.fmean(vals), len(vals)


def traffic_record(fetch_csv: str, write_csv: str, kernel: str, copy: str, copy_bytes: int) -> dict:
    f_k, nf = _mean_counter(fetch_csv, "FETCH_SIZE", kernel)
    w_k, nw = _mean_counter(write_csv, "WRITE_SIZE", kernel)
    f_c, _ = _mean_counter(fetch_csv, "FETCH_SIZE", copy)
    w_c, _ = _mean_counter(write_csv, "WRITE_SIZE", copy)
    ff = copy_bytes / (f_c * 1024.0)
    fw = copy_bytes / (w_c * 1024.0)
    fetch = f_k * 1024.0 * ff
    write = w_k * 1024.0 * fw
    return {"fetch_kib_per_dispatch": round(f_k, 2), "write_kib_per_dispatch": round(w_k, 2),
            "dispatches": [nf, nw], "copy_fetch_kib": round(f_c, 2), "copy_write_kib": round(w_c, 2),
            "copy_bytes": copy_bytes, "factor_fetch": round(ff, 5), "factor_write": round(fw, 5),
            "fetch_bytes": round(fetch), "write_bytes": round(write), "traffic_bytes": round(fetch + write)}


def load_traffic(workload: str, kind: str) -> dict | None:
    """The stored traffic record of (workload, kernel kind), or None when there
    is none or the kernel sources changed since it was taken."""
    path = os.path.join(PROFILES, f"traffic_{kind}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("sources_sha256") != sources_digest():
        return None
    return rec


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--workload", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--copy", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--kind", required=True)
    t.add_argument("--command-fetch", required=True)
    t.add_argument("--command-write", required=True)
    t.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        open(a.out, "w").write(kernel_stats_md(a.csv, a.workload, a.command))
    else:
        rec = traffic_record(a.fetch, a.write, a.kernel, a.copy, a.copy_bytes)
        rec.update({"workload": a.workload, "kind": a.kind, "kernel_regex": a.kernel, "copy_regex": a.copy,
                    "command_fetch": a.command_fetch, "command_write": a.command_write,
                    "sources_sha256": sources_digest()})
        json.dump(rec, open(a.out, "w"), indent=1)
        open(a.out, "a").write("\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
