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
roofline of the dominant kernel (its algorithmic bytes per launch over its mean launch time
from HIP events on the launch stream), and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16


def workload_spec(name, T_override=None, d=32):
    if name == "qwen_decode":
        return dict(T=T_override or 1, H=2048, E=256, k=8, I=512, I_shared=512, act="bf16", expert="bf16",
                    shared="bf16", out="bf16", bias=None, d=None, layers=48)
    if name == "ling_verify":
        return dict(T=T_override or 4, H=2560, E=512, k=8, I=768, I_shared=768, act="bf16", expert="bf16",
                    shared="bf16", out="bf16", bias="verify", d=d, layers=8)
    if name == "ling_mxfp4":
        T = T_override or 1
        return dict(T=T, H=2560, E=512, k=8, I=768, I_shared=768, act="bf16", expert="mxfp4",
                    shared="bf16", out="f32", bias=("verify" if T > 1 else None), d=(d if T > 1 else None),
                    layers=48)
    if name == "ling_mxfp4_prefill":
        return dict(T=T_override or 4096, H=2560, E=512, k=8, I=768, I_shared=768, act="bf16", expert="mxfp4",
                    shared="bf16", out="f32", bias="zipf", d=None, layers=8)
    if name == "qwen_prefill":
        return dict(T=T_override or 4096, H=2048, E=256, k=8, I=512, I_shared=512, act="bf16", expert="bf16",
                    shared="bf16", out="bf16", bias="zipf", d=None, layers=8)
    raise SystemExit(f"unknown workload {name}")


def expert_bytes(spec):
    """Bytes of one routed expert's gate+up and down weights."""
    H, I = spec["H"], spec["I"]
    if spec["expert"] == "mxfp4":
        gu = 2 * (I * H // 2 + I * H // 32)
        dn = H * I // 2 + H * I // 32
    else:
        es = 4 if spec["expert"] == "f32" else 2
        gu, dn = 2 * I * H * es, H * I * es
    return gu, dn


def algorithmic_bytes(spec, distinct):
    """Bytes the layer must move once: the distinct selected experts, the shared expert,
    the fp32 router, x and y."""
    H, E, T, Is = spec["H"], spec["E"], spec["T"], spec["I_shared"]
    gu, dn = expert_bytes(spec)
    ss = 2 if spec["shared"] == "bf16" else 4
    shared = 3 * Is * H * ss
    router = E * H * 4
    xs = T * H * (2 if spec["act"] == "bf16" else 4)
    ys = T * H * (2 if spec["out"] == "bf16" else 4)
    return distinct * (gu + dn) + shared + router + xs + ys


def traffic_from_profiles(kernel, workload, T):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary, or None
    when there is none or the kernel's source changed since the counters were taken."""
    from routed_expert_ffn_route_amd import profsum
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_T{T}.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("TRAFFIC_JSON:"):
            d = json.loads(line.split(":", 1)[1])
            if d.get("source_hash") == profsum.source_hash(kernel):
                return d["traffic_bytes"]
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="qwen_decode")
    ap.add_argument("--T", type=int, default=None)
    ap.add_argument("--d", type=int, default=32)
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of a HIP graph")
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="also run a plain device copy of this many bytes (counter calibration)")
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
    spec = workload_spec(args.workload, args.T, args.d)
    nl = args.layers or spec["layers"]
    T = spec["T"]
    print(f"# generating {nl} layers of {args.workload} on the device", file=sys.stderr, flush=True)
    layers = []
    for li in range(nl):
        Ld, xd = synth.device_layer(T, spec["H"], spec["E"], spec["k"], spec["I"], spec["I_shared"],
                                    spec["act"], spec["expert"], spec["shared"], spec["out"], seed=li,
                                    bias=spec["bias"], d=spec["d"])
        layers.append((Ld, xd, B.weights_of(Ld)))
    torch.cuda.synchronize()
    shape = B.shape_of(layers[0][0])
    path = B.path_name(shape)
    ws = B.workspace(shape)
    y = torch.empty((T, spec["H"]), device="cuda",
                    dtype=torch.float32 if spec["out"] == "f32" else torch.int16)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    # distinct experts per layer (for the bytes model), from the library's own routing
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

    def timed(fn):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(torch.cuda.current_stream())
        fn()
        e1.record(torch.cuda.current_stream())
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    # ---- eager: K back-to-back calls on the stream ----
    ms_eager = timed(lambda: [step(i, stream.cuda_stream) for i in range(args.steps)])

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
        ms_graph = timed(g.replay)
    ms_step = ms_graph if ms_graph is not None else ms_eager

    # ---- per-kernel durations: steps with every launch bracketed by HIP events on the launch
    # stream.  A few fills of a 1 GiB buffer go first so that the host has queued every timed
    # launch before the GPU reaches them: the intervals then hold GPU time only, not host gaps.
    ksteps = min(args.steps, 20)
    blocker = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    B.timing_begin(10 * ksteps)
    with torch.cuda.stream(stream):
        for _ in range(8):
            blocker.fill_(1.0)
    for i in range(ksteps):
        step(i, stream.cuda_stream)
    ktimes = B.timing_end()
    torch.cuda.synchronize()
    del blocker
    kern = {n: (c, ms / c) for n, (c, ms) in ktimes.items()}
    # an empty kernel bracketed the same way: reported beside the kernels (what the brackets
    # cost with no work); the kernels' durations are the bracketed times as measured
    ovh_ms = kern.pop("launch_overhead", (0, 0.0))[1]
    dom = max(kern, key=lambda n: kern[n][0] * kern[n][1])
    dom_ms = kern[dom][1]

    gu, dn = expert_bytes(spec)
    H, I, Is, E, k = spec["H"], spec["I"], spec["I_shared"], spec["E"], spec["k"]
    ss = 2 if spec["shared"] == "bf16" else 4
    layer_bytes = algorithmic_bytes(spec, mean_distinct)
    tok_s = T / (ms_step / 1e3)
    layer_gbs = layer_bytes / (ms_step / 1e3) / 1e9
    # algorithmic work of one launch of each kernel: bytes for the HBM-bound decode kernels,
    # flops for the prefill GEMMs
    work = {
        "dec_router": ("hbm", E * H * 4),
        "dec_select": ("hbm", 2 * Is * H * ss),  # the shared expert's gate/up rows (T > 1)
        "dec_gateup": ("hbm", mean_distinct * gu + (2 * Is * H * ss if T == 1 else 0)),
        "dec_down": ("hbm", mean_distinct * dn + Is * H * ss),  # + the shared expert's down rows
        "pf_gateup": ("mfma", 2.0 * 2 * (T * k * I + T * Is) * H),
        "pf_down": ("mfma", 2.0 * (T * k * I + T * Is) * H),
        "pf_router": ("mfma", 2.0 * 3 * T * E * H),
    }
    roof = None
    if dom in work:
        bound, amount = work[dom]
        if bound == "hbm":
            ach, peak, unit = amount / (dom_ms / 1e3) / 1e9, HBM_PEAK_GBS, "GB/s"
        else:
            ach, peak, unit = amount / (dom_ms / 1e3) / 1e12, BF16_MFMA_PEAK_TFLOPS, "TFLOP/s"
        roof = {"bound": bound, "achieved": round(ach, 1), "peak": peak, "unit": unit,
                "frac": round(ach / peak, 4), "traffic": traffic_from_profiles(dom, args.workload, T),
                "kernel": dom, "kernel_us": round(dom_ms * 1e3, 3),
                "empty_launch_us": round(ovh_ms * 1e3, 3),
                ("bytes_per_launch" if bound == "hbm" else "flops_per_launch"): int(amount)}

    # ---- CPU baseline: the oracle, single-threaded, on a bounded sample of the workload ----
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        Lh = synth.to_host(layers[0][0])
        Ts = min(T, 4)  # tokens are independent: the oracle runs a few at a time
        Lh = Lh.with_T(Ts)
        if Lh.router_bias is not None and Lh.bias_t_stride:
            Lh.router_bias = np.ascontiguousarray(Lh.router_bias[:Ts])
        n, t0 = 0, time.perf_counter()
        rng = np.random.default_rng(1234)
        while True:
            xr = rng.standard_normal((Ts, spec["H"]), dtype=np.float32)
            xh = synth.f32_to_bf16_bits(xr) if spec["act"] == "bf16" else xr
            oracle.forward(Lh, xh)
            n += 1
            if time.perf_counter() - t0 >= args.cpu_seconds and n >= 2:
                break
        dt = time.perf_counter() - t0
        cpu = {"value": round(n * Ts / dt, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"{n} oracle calls of {Ts} token(s) each on layer 0 of the workload "
                         f"(fresh seeded x per call), {dt:.1f} s on one host thread"}
        del Lh

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
        "scaling": "weak", "vs_baseline": None, "dtype": spec["expert"], "data": "synthetic",
        "config": {"workload": args.workload, "T": T, "H": spec["H"], "E": spec["E"], "k": spec["k"],
                   "I": spec["I"], "I_shared": spec["I_shared"], "layers_rotated": nl,
                   "path": path, "distinct_experts_mean": mean_distinct},
        "launch": "hipgraph" if ms_graph is not None else "eager",
        "us_per_call_eager": round(ms_eager * 1e3, 3),
        "layer_gbs": round(layer_gbs, 1), "layer_hbm_frac": round(layer_gbs / HBM_PEAK_GBS, 4),
        "layer_bytes": int(layer_bytes), "us_per_call": round(ms_step * 1e3, 3),
        "kernels_us": {n: round(v[1] * 1e3, 3) for n, v in kern.items()},
        "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
