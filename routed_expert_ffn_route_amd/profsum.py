"""Summarise rocprofv3 output for one kernel of the benchmark into a short markdown file.

Inputs (CSV from `rocprofv3 --output-format csv`):
  --stats    a kernel_stats.csv from `--kernel-trace --stats` (mean duration per kernel)
  --fetch    a counter_collection.csv from `--pmc FETCH_SIZE --kernel-trace`
  --write    a counter_collection.csv from `--pmc WRITE_SIZE --kernel-trace`
  --kernel   substring of the kernel name to report
  --label    name the benchmark uses for that kernel (default: --kernel)
  --copy-bytes  size of the plain device-to-device copy the benchmark ran in the counter
             runs (`bench.py --copy-calibration N`): its FETCH_SIZE / WRITE_SIZE per
             dispatch calibrate the counters (factor = N / counter bytes)

The markdown ends with one line `TRAFFIC_JSON: {...}` that bench.py reads to fill the
roofline's `traffic` field (HBM bytes per launch) while the kernel source is unchanged.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = {
    "dec_": ["csrc/decode_impl.h", "csrc/select.h", "csrc/common.h"],
    "pf_": ["csrc/prefill.hip", "csrc/select.h", "csrc/common.h"],
}


def source_hash(kernel: str) -> str:
    files = next((v for k, v in KERNEL_SOURCES.items() if kernel.startswith(k)), [])
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(HERE, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def per_dispatch(csv_path, counter, match):
    vals = []
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] == counter and match(r["Kernel_Name"]):
            vals.append(float(r["Counter_Value"]))
    return vals


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--stats", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--kernel", required=True)
    ap.add_argument("--label", default=None)
    ap.add_argument("--copy-bytes", type=int, required=True)
    ap.add_argument("--algorithmic-bytes", type=float, required=True)
    ap.add_argument("--workload", required=True)
    ap.add_argument("--commands", required=True, help="file holding the exact commands run")
    a = ap.parse_args()
    label = a.label or a.kernel

    stats = list(csv.DictReader(open(a.stats)))
    krow = next(r for r in stats if a.kernel in r["Name"])
    avg_ns = float(krow["AverageNs"])
    is_k = lambda n: a.kernel in n  # noqa: E731
    is_copy = lambda n: "copyBuffer" in n or "copy" in n.lower() and "moe" not in n  # noqa: E731
    kf = per_dispatch(a.fetch, "FETCH_SIZE", is_k)
    kw = per_dispatch(a.write, "WRITE_SIZE", is_k)
    cf = [v for v in per_dispatch(a.fetch, "FETCH_SIZE", is_copy) if v * 1024 > 0.5 * a.copy_bytes]
    cw = [v for v in per_dispatch(a.write, "WRITE_SIZE", is_copy) if v * 1024 > 0.5 * a.copy_bytes]
    fetch_kib, write_kib = statistics.median(kf), statistics.median(kw)
    f_fac = a.copy_bytes / (statistics.median(cf) * 1024)
    w_fac = a.copy_bytes / (statistics.median(cw) * 1024)
    traffic = fetch_kib * 1024 * f_fac + write_kib * 1024 * w_fac
    out = {
        "kernel": label, "kernel_symbol": krow["Name"][:120], "workload": a.workload, "avg_ns": avg_ns,
        "fetch_bytes": round(fetch_kib * 1024 * f_fac), "write_bytes": round(write_kib * 1024 * w_fac),
        "traffic_bytes": round(traffic), "algorithmic_bytes": a.algorithmic_bytes,
        "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4),
        "source_hash": source_hash(label),
    }
    cmds = open(a.commands).read().strip()
    print(f"# {label} -- {a.workload}\n")
    print("Commands (run from the repository root on one MI355X):\n\n```\n" + cmds + "\n```\n")
    print(f"* mean duration (`--kernel-trace --stats`, {krow['Calls']} calls): {avg_ns / 1e3:.3f} us")
    print(f"* FETCH_SIZE per dispatch: {fetch_kib:.1f} KiB (median of {len(kf)}); "
          f"WRITE_SIZE: {write_kib:.1f} KiB (median of {len(kw)})")
    print(f"* copy calibration: a {a.copy_bytes} B device copy reads {statistics.median(cf):.1f} KiB "
          f"and writes {statistics.median(cw):.1f} KiB per dispatch -> factors "
          f"{f_fac:.4f} (fetch), {w_fac:.4f} (write)")
    print(f"* HBM traffic per launch: {traffic / 1e6:.3f} MB vs algorithmic {a.algorithmic_bytes / 1e6:.3f} MB "
          f"({traffic / a.algorithmic_bytes:.3f}x)")
    print(f"* achieved on algorithmic bytes: {a.algorithmic_bytes / avg_ns:.1f} GB/s\n")
    print("Library kernels (and the calibration copy) by total time:\n")
    print("| kernel | calls | mean us | total % |\n|---|---|---|---|")
    mine = [r for r in stats if "moe::" in r["Name"] or "copyBuffer" in r["Name"]]
    for r in sorted(mine, key=lambda r: -float(r["TotalDurationNs"]))[:8]:
        print(f"| {r['Name'][:90]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    print()
    print("TRAFFIC_JSON: " + json.dumps(out))


if __name__ == "__main__":
    main()
