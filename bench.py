"""Benchmark of the routed-expert FFN layer (libmoe) on one MI355X.

One step = one moe_forward call (router -> selection -> expert SwiGLU -> combine with the
shared expert) on one batch of synthetic tokens.  The default workload is batch-1 decode
with Qwen-style shapes: T=1, hidden 2048, 256 routed experts top-8 + 1 shared, expert and
shared intermediate 512, bf16 weights and activations, fp32 router; 48 independently drawn
layers are rotated call by call so that no layer's weights stay in the 256 MiB Infinity
Cache.  Other workloads (--workload): ling_verify (T=4, H=2560, E=512, I=768, d distinct
experts), ling_mxfp4 (same with MXFP4 experts; T=1 or 4), qwen_prefill (T=4096),
ling_mxfp4_prefill (T=4096, Ling shapes, MXFP4 experts, Zipf expert load).

Prints ONE JSON line: value = tokens/s of the whole layer (inputs resident in HBM), the
layer's GB/s or TFLOP/s against the MI355X peaks and the measured read ceiling, the roofline
of the dominant kernel (its algorithmic work per launch over its mean duration, both live:
the library launches each kernel with hipExtLaunchKernel events tied to the kernel itself),
and the CPU oracle timed on one pinned host core over a bounded sample.  The algorithmic work
of the layer and of every kernel comes from routed_expert_ffn_route_amd/workmodel.py, the
table the rocprofv3 summaries under profiles/ are computed from as well.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from routed_expert_ffn_route_amd import workmodel as W  # noqa: E402


def profile_record(kernel, workload, T):
    """The committed rocprofv3 summary of `kernel` on this workload (profiles/), if its kernel
    sources still hash to the recorded value; else None."""
    from routed_expert_ffn_route_amd import profsum
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_T{T}.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("PROFILE_JSON:"):
            d = json.loads(line.split(":", 1)[1])
            if d.get("source_hash") == profsum.source_hash(kernel):
                return d
    return None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(spec, layer_dev, seconds):
    """The oracle (plain single-threaded C) on one pinned host core, on a bounded sample of the
    workload: calls of up to 4 tokens (tokens are independent) on layer 0 with fresh seeded x,
    until `seconds` have passed."""
    import numpy as np

    import oracle
    from routed_expert_ffn_route_amd import synth
    T = spec["T"]
    Lh = synth.to_host(layer_dev)
    Ts = min(T, 4)
    Lh = Lh.with_T(Ts)
    if Lh.router_bias is not None and Lh.bias_t_stride:
        Lh.router_bias = np.ascontiguousarray(Lh.router_bias[:Ts])
    aff = os.sched_getaffinity(0)
    core = min(aff)
    os.sched_setaffinity(0, {core})   # this thread only: the oracle runs here
    try:
        rng = np.random.default_rng(1234)
        n, t0 = 0, time.perf_counter()
        while True:
            xr = rng.standard_normal((Ts, spec["H"]), dtype=np.float32)
            xh = synth.f32_to_bf16_bits(xr) if spec["act"] == "bf16" else xr
            oracle.forward(Lh, xh)
            n += 1
            if time.perf_counter() - t0 >= seconds and n >= 2:
                break
        dt = time.perf_counter() - t0
    finally:
        os.sched_setaffinity(0, aff)
    ncpu = os.cpu_count() or 1
    return {"value": round(n * Ts / dt, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "label": f"1 core of {ncpu}", "cpu": cpu_model(), "pinned_core": core,
            "sample": f"{n} oracle calls of {Ts} token(s) each on layer 0 of the workload (fresh seeded x per "
                      f"call), {dt:.1f} s on host core {core} (1 core of {ncpu}, {cpu_model()})"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="qwen_decode")
    ap.add_argument("--T", type=int, default=None)
    ap.add_argument("--d", type=int, default=None, help="distinct experts of a verify window (default min(32, 8 T))")
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of a HIP graph")
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="also run a plain device copy of this many bytes (counter calibration)")
    ap.add_argument("--json-out", default=None, help="also write the JSON line to this file")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the layer is built for a single MI355X; "
              "run it with --gpus 1 (multi-GPU sharding is described, not built).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from routed_expert_ffn_route_amd import binding as B
    from routed_expert_ffn_route_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    B.lib()
    spec = W.workload_spec(args.workload, args.T, args.d)
    nl = args.layers or spec["layers"]
    T = spec["T"]
    print(f"# generating {nl} layers of {args.workload} on the device", file=sys.stderr, flush=True)
    layers = []
    for li in range(nl):
        Ld, xd = synth.device_layer(T, spec["H"], spec["E"], spec["k"], spec["I"], spec["I_shared"],
                                    spec["act"], spec["expert"], spec["shared"], spec["out"], seed=li,
                                    bias=spec["bias"], d=spec["d"])
        if spec.get("act_quant"):
            Ld = dataclasses.replace(Ld, act_quant=spec["act_quant"])
        layers.append((Ld, xd, B.weights_of(Ld)))
    torch.cuda.synchronize()
    shape = B.shape_of(layers[0][0])
    path = B.path_name(shape)
    ws = B.workspace(shape)
    y = torch.empty((T, spec["H"]), device="cuda",
                    dtype=torch.float32 if spec["out"] == "f32" else torch.int16)
    stream = torch.cuda.current_stream()

    # distinct experts per layer (selected at decode, touched at prefill), from the library's
    # own routing: the bytes model counts each distinct expert once
    distinct = []
    for Ld, xd, _ in layers:
        r = B.layer_route(Ld, xd)
        distinct.append(len(set(r["ids"].cpu().numpy().ravel().tolist())))
    mean_distinct = float(np.mean(distinct))

    def step(i, sp):
        Ld, xd, w = layers[i % nl]
        B.forward(shape, xd, w, y, ws, sp)

    print(f"# path {path}; warmup {args.warmup}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i, stream.cuda_stream)
    torch.cuda.synchronize()

    def timed(fn, n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(torch.cuda.current_stream())
        fn()
        e1.record(torch.cuda.current_stream())
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # ---- eager: K back-to-back calls on the stream ----
    ms_eager = timed(lambda: [step(i, stream.cuda_stream) for i in range(args.steps)], args.steps)

    # ---- graph: the same K calls captured once into a HIP graph and replayed ----
    ms_graph = None
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        with torch.cuda.graph(g, stream=cs):
            for i in range(args.steps):
                step(i, cs.cuda_stream)
        g.replay()  # untimed
        torch.cuda.synchronize()
        ms_graph = timed(g.replay, args.steps)
    ms_step = ms_graph if ms_graph is not None else ms_eager

    # ---- isolated latency: one call on an idle GPU (synchronised before and after) ----
    iso = []
    for i in range(min(args.steps, 30)):
        iso.append(timed(lambda: step(i, stream.cuda_stream), 1))
    us_isolated = statistics.median(iso) * 1e3

    # ---- per-kernel durations: the library launches each kernel with hipExtLaunchKernel and a
    # pair of events tied to that kernel's own start and end ----
    ksteps = min(args.steps, 20)
    torch.cuda.synchronize()
    B.timing_begin(16 * ksteps)
    for i in range(ksteps):
        step(i, stream.cuda_stream)
    ktimes = B.timing_end()
    torch.cuda.synchronize()
    kern = {n: (c, ms / c) for n, (c, ms) in ktimes.items()}
    dom = max(kern, key=lambda n: kern[n][0] * kern[n][1])

    work = W.kernel_work(spec, mean_distinct)
    lbytes = W.layer_bytes(spec, mean_distinct)
    lflops = W.layer_flops(spec)
    t_s = ms_step / 1e3
    tok_s = T / t_s
    layer = {"bytes": int(lbytes), "flops": lflops, "gbs": round(lbytes / t_s / 1e9, 1),
             "frac_hbm": round(lbytes / t_s / 1e9 / W.HBM_PEAK_GBS, 4),
             "tflops": round(lflops / t_s / 1e12, 2),
             "frac_mfma": round(lflops / t_s / 1e12 / W.BF16_MFMA_PEAK_TFLOPS, 4),
             # the best the layer could do: bound by whichever of its flops and its bytes takes longer
             "attainable_frac": round(max(lflops / (W.BF16_MFMA_PEAK_TFLOPS * 1e12),
                                          lbytes / (W.HBM_PEAK_GBS * 1e9)) / t_s, 4)}

    # ---- read ceiling: the same byte count per call streamed with the decode kernels' access
    # pattern (16-byte loads over the whole chip), rotating through as many buffers as layers ----
    ceil_gbs = None
    if spec["T"] <= 16:
        nbuf = min(nl, max(2, int(8e9 // max(lbytes, 1))))
        per = (int(lbytes) + 255) // 256 * 256
        big = torch.empty(nbuf * per, dtype=torch.uint8, device="cuda")
        big.fill_(1)
        sink = torch.zeros(64, dtype=torch.int32, device="cuda")
        for i in range(5):
            B.read_ceiling(big[(i % nbuf) * per:], per, sink, stream.cuda_stream)
        gc = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        with torch.cuda.graph(gc, stream=cs):
            for i in range(args.steps):
                B.read_ceiling(big[(i % nbuf) * per:], per, sink, cs.cuda_stream)
        gc.replay()
        torch.cuda.synchronize()
        ms_read = timed(gc.replay, args.steps)
        ceil_gbs = round(per / (ms_read / 1e3) / 1e9, 1)
        layer["read_ceiling_gbs"] = ceil_gbs
        layer["frac_of_read_ceiling"] = round(layer["gbs"] / ceil_gbs, 4)
        del big, gc
    else:
        # operand-staging rates of the grouped GEMMs' load into LDS, by contiguous bytes per row
        # (4-bit weight rows: 16 per step; bf16 operand rows: 64; whole cache lines: 128), from a
        # 2 MiB region that stays in the L2
        reg = torch.empty(2 << 20, dtype=torch.uint8, device="cuda")
        reg.fill_(1)
        sink = torch.zeros(64, dtype=torch.int32, device="cuda")
        rates = {}
        for seg in (16, 64, 128):
            for _ in range(2):
                nb = B.stage_rate(reg, 2 << 20, seg, 256, sink, stream.cuda_stream)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(5):
                B.stage_rate(reg, 2 << 20, seg, 256, sink, stream.cuda_stream)
            e1.record(stream)
            torch.cuda.synchronize()
            gbs = 5 * nb / (e0.elapsed_time(e1) / 1e3) / 1e9
            rates[str(seg)] = {"gbs": round(gbs, 1), "bytes_per_clk_per_cu": round(gbs * 1e9 / 256 / 2.4e9, 1)}
        layer["stage_rate"] = rates
        del reg

    # ---- roofline of the dominant kernel ----
    roof = None
    if dom in work:
        wk = work[dom]
        dom_s = kern[dom][1] / 1e3
        if wk["bound"] == "hbm":
            amount, ach, peak, unit = wk["bytes"], wk["bytes"] / dom_s / 1e9, W.HBM_PEAK_GBS, "GB/s"
        else:
            amount, ach, peak, unit = wk["flops"], wk["flops"] / dom_s / 1e12, wk["peak_tflops"], "TFLOP/s"
        prof = profile_record(dom, args.workload, T)
        roof = {"bound": wk["bound"], "achieved": round(ach, 1), "peak": peak, "unit": unit,
                "frac": round(ach / peak, 4), "traffic": prof["traffic_bytes"] if prof else None,
                "kernel": dom, "kernel_us": round(kern[dom][1] * 1e3, 3),
                ("bytes_per_launch" if wk["bound"] == "hbm" else "flops_per_launch"): int(amount),
                "kernel_bytes_per_launch": wk["bytes"]}
        if prof:  # the committed rocprofv3 mean of the same kernel source
            roof["kernel_us_rocprof"] = round(prof["avg_ns"] / 1e3, 3)
            roof["frac_rocprof"] = round(amount / (prof["avg_ns"] * 1e-9) / (1e9 if unit == "GB/s" else 1e12) / peak, 4)
        if ceil_gbs and wk["bound"] == "hbm":
            roof["frac_of_read_ceiling"] = round(ach / ceil_gbs, 4)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(spec, layers[0][0], args.cpu_seconds)

    if args.copy_calibration:
        a = torch.ones(args.copy_calibration, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    out = {
        "metric": "MoE layer tok/s + HBM GB/s (% of peak) at T=1/T=4 decode; TFLOP/s at prefill",
        "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": spec["act"], "data": "synthetic",
        "config": {"workload": args.workload, "T": T, "H": spec["H"], "E": spec["E"], "k": spec["k"],
                   "I": spec["I"], "I_shared": spec["I_shared"], "weights": spec["expert"],
                   "layers_rotated": min(nl, args.steps), "layers_drawn": nl, "path": path,
                   "distinct_experts_mean": mean_distinct},
        "launch": "hipgraph" if ms_graph is not None else "eager",
        "us_per_call": round(ms_step * 1e3, 3), "us_per_call_eager": round(ms_eager * 1e3, 3),
        "us_isolated": round(us_isolated, 3),
        "layer": layer,
        "kernels_us": {n: round(v[1] * 1e3, 3) for n, v in kern.items()},
        "work": work,
        "roofline": roof, "cpu_baseline": cpu,
    }
    line = json.dumps(out)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
