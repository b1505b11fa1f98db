"""Workloads and the algorithmic work of the layer and of each of its kernels.

One table serves the benchmark (bench.py) and the rocprofv3 summaries (profsum.py), so the
bytes and flops a roofline fraction divides by are never typed by hand.

Algorithmic bytes count what must move once: the weights of the experts a call selects (each
distinct expert once), the shared expert, the fp32 router, and each kernel's own inputs and
outputs once ("Optimizing on-device inference for Apple Silicon", sections "Decode: bytes moved
per token" and "Limits of further optimization": a weight-streaming kernel is judged by the
bytes it must read against the rate the access pattern sustains).  Flops count 2 per
multiply-add of the contractions.
"""
from __future__ import annotations

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix cores
FP8_MFMA_PEAK_TFLOPS = 5000.0    # MI355X dense fp8 matrix cores (the W4A8 GEMMs' fp8 x fp4 rate)


def workload_spec(name, T_override=None, d=None):
    """Shapes and dtypes of the benchmark workloads (seeded synthetic inputs, see synth.py).
    d: distinct experts of a verify window (default 32, at most T * k)."""
    def window(T):
        return d if d is not None else min(32, T * 8)
    if name == "qwen_decode":
        return dict(T=T_override or 1, H=2048, E=256, k=8, I=512, I_shared=512, act="bf16", expert="bf16",
                    shared="bf16", out="bf16", bias=None, d=None, layers=48)
    if name == "ling_verify":
        T = T_override or 4
        return dict(T=T, H=2560, E=512, k=8, I=768, I_shared=768, act="bf16", expert="bf16",
                    shared="bf16", out="bf16", bias="verify", d=window(T), layers=8)
    if name == "ling_mxfp4":
        T = T_override or 1
        return dict(T=T, H=2560, E=512, k=8, I=768, I_shared=768, act="bf16", expert="mxfp4",
                    shared="bf16", out="f32", bias=("verify" if T > 1 else None), d=(window(T) if T > 1 else None),
                    layers=48)
    if name == "ling_mxfp4_prefill":
        return dict(T=T_override or 4096, H=2560, E=512, k=8, I=768, I_shared=768, act="bf16", expert="mxfp4",
                    shared="bf16", out="f32", bias="zipf", d=None, layers=8)
    if name == "qwen_prefill":
        return dict(T=T_override or 4096, H=2048, E=256, k=8, I=512, I_shared=512, act="bf16", expert="bf16",
                    shared="bf16", out="bf16", bias="zipf", d=None, layers=8)
    if name == "qwen_int4":   # the Qwen checkpoint's group-wise affine 4-bit experts
        return dict(T=T_override or 1, H=2048, E=256, k=8, I=512, I_shared=512, act="bf16", expert="int4g64",
                    shared="bf16", out="bf16", bias=None, d=None, layers=48)
    if name == "qwen_int4_prefill":
        return dict(T=T_override or 4096, H=2048, E=256, k=8, I=512, I_shared=512, act="bf16", expert="int4g64",
                    shared="bf16", out="bf16", bias="zipf", d=None, layers=8)
    if name == "ling_w4a8_prefill":   # Ling MXFP4 experts with MXFP8 activations
        return dict(T=T_override or 4096, H=2560, E=512, k=8, I=768, I_shared=768, act="bf16", expert="mxfp4",
                    shared="bf16", out="f32", bias="zipf", d=None, layers=8, act_quant="mxfp8")
    if name == "tiny":
        return dict(T=T_override or 4, H=256, E=16, k=2, I=128, I_shared=128, act="f32", expert="f32",
                    shared="f32", out="f32", bias=None, d=None, layers=1)
    raise ValueError(f"unknown workload {name}")


def _es(dt):
    return 4 if dt == "f32" else 2


def expert_bytes(spec):
    """Bytes of one routed expert's gate+up and of its down weights."""
    H, I = spec["H"], spec["I"]
    if spec["expert"] == "mxfp4":     # codes + one e8m0 byte per 32
        return 2 * (I * H // 2 + I * H // 32), H * I // 2 + H * I // 32
    if spec["expert"] == "int4g64":   # codes + a bf16 scale and a bf16 bias per 64
        return 2 * (I * H // 2 + I * H // 16), H * I // 2 + H * I // 16
    es = _es(spec["expert"])
    return 2 * I * H * es, H * I * es


def layer_bytes(spec, distinct):
    """Bytes the whole layer must move once: the distinct selected experts, the shared expert,
    the fp32 router, x and y."""
    H, E, T, Is = spec["H"], spec["E"], spec["T"], spec["I_shared"]
    gu, dn = expert_bytes(spec)
    return (distinct * (gu + dn) + 3 * Is * H * _es(spec["shared"]) + E * H * 4
            + T * H * _es(spec["act"]) + T * H * _es(spec["out"]))


def layer_flops(spec):
    """Flops of the layer: router, routed gate/up + down for T*k rows, shared expert for T."""
    T, H, E, k, I, Is = (spec[n] for n in ("T", "H", "E", "k", "I", "I_shared"))
    return 2.0 * T * E * H + 6.0 * T * k * I * H + 6.0 * T * Is * H


def kernel_work(spec, distinct):
    """{kernel name: {"bound": "hbm" | "mfma", "bytes": B, "flops": F}} for one call.  `distinct`
    is the number of distinct experts the call selects (decode) or touches (prefill)."""
    T, H, E, k, I, Is = (spec[n] for n in ("T", "H", "E", "k", "I", "I_shared"))
    gu, dn = expert_bytes(spec)
    ss, xs, ys = _es(spec["shared"]), _es(spec["act"]), _es(spec["out"])
    sh_gu, sh_dn = 2 * Is * H * ss, Is * H * ss
    S = T * k                                  # routed rows (slots); the shared expert adds T rows
    # MXFP4 and int4 prefill run the precise kernels: activations as bf16 hi + lo (4 B per value), fp32
    # slot rows; the shared expert's tiles run in the same launches (bf16, precise)
    p = spec["expert"] in ("mxfp4", "int4g64")
    ab, rb = (4, 4) if p else (2, 2)           # bytes per activation value, per slot-row value
    w = {
        # decode (T <= 16)
        "dec_router": ("hbm", E * H * 4 + T * H * xs + T * E * 4, 2.0 * T * E * H),
        # the shared expert's gate/up rows beside the selection (T > 1)
        "dec_select": ("hbm", sh_gu + T * H * xs + T * E * 4, 4.0 * T * Is * H),
        "dec_gateup": ("hbm", distinct * gu + (sh_gu if T == 1 else 0) + T * H * xs,
                       4.0 * S * I * H + (4.0 * T * Is * H if T == 1 else 0)),
        "dec_down": ("hbm", distinct * dn + sh_dn + T * H * ys, 2.0 * S * I * H + 2.0 * T * Is * H),
        # prefill (T > 16)
        "pf_router_split": ("hbm", E * H * 4 + 3 * E * H * 2, 0.0),
        # (the fp32 router runs as three bf16 parts, three times the MFMA work of its 2 T E H)
        "pf_router": ("mfma", 3 * E * H * 2 + T * H * 2 + T * E * 4, 2.0 * T * E * H),
        "pf_gateup": ("mfma", distinct * gu + sh_gu + T * H * 2 + (S * I + T * Is) * ab, 4.0 * (S * I + T * Is) * H),
        "pf_down": ("mfma", distinct * dn + sh_dn + S * (I * ab + H * rb) + T * (Is * ab + H * rb),
                    2.0 * (S * I + T * Is) * H),
        "pf_combine": ("hbm", (S + T) * H * rb + T * H * ys, 0.0),
    }
    w8 = spec.get("act_quant") == "mxfp8"
    if w8:   # W4A8: 1-byte activations + a scale byte per 32 on the routed tiles; shared tiles as bf16 precise
        xq = T * H + T * H // 32
        w["pf_quant_x"] = ("hbm", T * H * 2 + xq, 0.0)
        w["pf_gateup"] = ("mfma", distinct * gu + xq + S * I + S * I // 32 + sh_gu + T * H * 2 + T * Is * ab,
                          4.0 * (S * I + T * Is) * H)
        w["pf_down"] = ("mfma", distinct * dn + S * I + S * I // 32 + S * H * rb + sh_dn + T * (Is * ab + H * rb),
                        2.0 * (S * I + T * Is) * H)
    out = {n: {"bound": b, "bytes": int(by), "flops": float(f)} for n, (b, by, f) in w.items()}
    for n, v in out.items():   # the matrix-core peak each GEMM is measured against
        if v["bound"] == "mfma":
            v["peak_tflops"] = BF16_MFMA_PEAK_TFLOPS
    if w8:   # routed flops at the fp8 x fp4 rate, shared at the bf16 rate: the peak of the mix
        for n, share in (("pf_gateup", 4.0 * T * Is * H), ("pf_down", 2.0 * T * Is * H)):
            f = out[n]["flops"]
            out[n]["peak_tflops"] = round(f / ((f - share) / FP8_MFMA_PEAK_TFLOPS + share / BF16_MFMA_PEAK_TFLOPS), 1)
    return out
