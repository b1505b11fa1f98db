"""Summarise rocprofv3 output for one kernel of the benchmark into a short markdown file.

Inputs:
  --stats       kernel_stats.csv from `rocprofv3 --kernel-trace --stats --output-format csv`
  --fetch       counter_collection.csv from `rocprofv3 --pmc FETCH_SIZE --output-format csv`
  --write       counter_collection.csv from `rocprofv3 --pmc WRITE_SIZE --output-format csv`
  --bench-json  the JSON line bench.py wrote (--json-out) in the --kernel-trace run: the
                workload, and the algorithmic bytes and flops of every kernel (workmodel.py),
                so nothing here is typed by hand
  --kernel      the bench's label of the kernel (dec_gateup, pf_gateup, ...)
  --copy-bytes  size of the plain device copy the counter runs made (bench.py
                --copy-calibration N): its FETCH_SIZE / WRITE_SIZE per dispatch calibrate the
                counters (factor = N / counter bytes)
  --commands    file holding the exact commands that produced the inputs

The markdown ends with one line `PROFILE_JSON: {...}` that bench.py reads (while the kernel's
sources hash to the recorded value) for the roofline's `traffic` and the rocprofv3 mean.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = {
    "dec_": ["csrc/decode_impl.h", "csrc/select.h", "csrc/common.h", "csrc/kernels.h"],
    "pf_": ["csrc/prefill.hip", "csrc/route.hip", "csrc/select.h", "csrc/common.h", "csrc/kernels.h"],
}
# bench label -> regular expression over the demangled kernel name rocprofv3 reports
# (pf_gemm<MODE, BM, NS, weight dtype, precise>: the bf16 layer; pf_gemm_mix<MODE, weight dtype, W4A8>:
# the 4-bit layers, shared and routed tiles in one launch)
KERNEL_SYMBOLS = {
    "dec_router": r"dec_router<", "dec_select": r"dec_select<", "dec_gateup": r"dec_gateup<",
    "dec_down": r"dec_down<",
    "pf_router_split": r"pf_split_router\(", "pf_router": r"pf_gemm<2, ",
    "pf_gateup": r"pf_gemm<0, \d+, \d+, 1, false>|pf_gemm_mix<0,",
    "pf_down": r"pf_gemm<1, \d+, \d+, 1, false>|pf_gemm_mix<1,", "pf_quant_x": r"pf_quant_x\(",
    "pf_select": r"pf_select\(", "pf_combine": r"pf_combine\(",
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
    ap.add_argument("--bench-json", required=True)
    ap.add_argument("--kernel", required=True)
    ap.add_argument("--copy-bytes", type=int, required=True)
    ap.add_argument("--commands", required=True)
    a = ap.parse_args()

    bench = json.loads(open(a.bench_json).read().strip().splitlines()[-1])
    cfg = bench["config"]
    wk = bench["work"][a.kernel]
    sym = re.compile(KERNEL_SYMBOLS[a.kernel])
    is_k = lambda n: bool(sym.search(n))  # noqa: E731
    is_copy = lambda n: "copyBuffer" in n  # noqa: E731

    rows = [r for r in csv.DictReader(open(a.stats)) if is_k(r["Name"])]
    calls = sum(int(r["Calls"]) for r in rows)
    avg_ns = sum(float(r["TotalDurationNs"]) for r in rows) / calls
    kf = per_dispatch(a.fetch, "FETCH_SIZE", is_k)
    kw = per_dispatch(a.write, "WRITE_SIZE", is_k)
    cf = [v for v in per_dispatch(a.fetch, "FETCH_SIZE", is_copy) if v * 1024 > 0.25 * a.copy_bytes]
    cw = [v for v in per_dispatch(a.write, "WRITE_SIZE", is_copy) if v * 1024 > 0.5 * a.copy_bytes]
    fetch_kib, write_kib = statistics.median(kf), statistics.median(kw)
    f_fac = a.copy_bytes / (statistics.median(cf) * 1024)
    w_fac = a.copy_bytes / (statistics.median(cw) * 1024)
    traffic = fetch_kib * 1024 * f_fac + write_kib * 1024 * w_fac
    alg_b, alg_f = wk["bytes"], wk["flops"]
    T = cfg["T"]
    out = {
        "kernel": a.kernel, "kernel_symbol": rows[0]["Name"][:140], "workload": cfg["workload"], "T": T,
        "distinct_experts": cfg["distinct_experts_mean"], "calls": calls, "avg_ns": round(avg_ns, 1),
        "bound": wk["bound"], "algorithmic_bytes": alg_b, "algorithmic_flops": alg_f,
        "fetch_bytes": round(fetch_kib * 1024 * f_fac), "write_bytes": round(write_kib * 1024 * w_fac),
        "traffic_bytes": round(traffic), "traffic_ratio": round(traffic / alg_b, 4),
        "gbs_algorithmic": round(alg_b / avg_ns, 1), "tflops": round(alg_f / avg_ns / 1e3, 1),
        "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4),
        "source_hash": source_hash(a.kernel),
    }
    peak = 8000.0 if wk["bound"] == "hbm" else wk.get("peak_tflops", 2500.0)
    frac = (out["gbs_algorithmic"] if wk["bound"] == "hbm" else out["tflops"]) / peak
    out["frac"] = round(frac, 4)
    cmds = open(a.commands).read().strip()
    print(f"# {a.kernel} -- {cfg['workload']} T={T} (H={cfg['H']}, E={cfg['E']}, k={cfg['k']}, I={cfg['I']}, "
          f"{cfg['weights']} experts, {cfg['distinct_experts_mean']:g} distinct experts per call)\n")
    print("Commands (run from the repository root on one MI355X; the profsum line makes this file):\n\n```\n"
          + cmds + "\n```\n")
    print(f"* mean duration (`--kernel-trace --stats`, {calls} calls): {avg_ns / 1e3:.3f} us")
    print(f"* algorithmic work per launch (workmodel.py via the bench's JSON): {alg_b / 1e6:.3f} MB, "
          f"{alg_f / 1e9:.3f} GFLOP")
    if wk["bound"] == "hbm":
        print(f"* achieved: {alg_b / avg_ns:.1f} GB/s on algorithmic bytes = {frac:.3f} of 8000 GB/s")
    else:
        print(f"* achieved: {alg_f / avg_ns / 1e3:.1f} TFLOP/s = {frac:.3f} of {peak:g} TFLOP/s")
    print(f"* FETCH_SIZE per dispatch: {fetch_kib:.1f} KiB (median of {len(kf)}); "
          f"WRITE_SIZE: {write_kib:.1f} KiB (median of {len(kw)})")
    print(f"* copy calibration: a {a.copy_bytes} B device copy reads {statistics.median(cf):.1f} KiB "
          f"and writes {statistics.median(cw):.1f} KiB per dispatch -> factors "
          f"{f_fac:.4f} (fetch), {w_fac:.4f} (write)")
    print(f"* HBM traffic per launch: {traffic / 1e6:.3f} MB = {traffic / alg_b:.3f}x the kernel's algorithmic "
          f"bytes\n")
    print("Library kernels by total time (the `--kernel-trace --stats` run):\n")
    print("| kernel | calls | mean us | total % |\n|---|---|---|---|")
    stats = list(csv.DictReader(open(a.stats)))
    mine = [r for r in stats if "moe::" in r["Name"]]
    for r in sorted(mine, key=lambda r: -float(r["TotalDurationNs"]))[:10]:
        print(f"| {r['Name'][:100]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
              f"{float(r['Percentage']):.1f} |")
    print()
    print("PROFILE_JSON: " + json.dumps(out))


if __name__ == "__main__":
    main()
