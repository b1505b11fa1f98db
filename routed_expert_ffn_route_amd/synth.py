"""Seeded synthetic inputs for the routed-expert FFN layer.

This module only draws random numbers and lays them out as the bytes the
layer consumes; it holds none of the layer's arithmetic.  Both the GPU
library's tests/benchmark and the CPU oracle receive exactly these bytes.

Workloads (shapes from the pages; values synthetic, no trained weights):

* ``tiny``      T=4, H=256, E=16, k=2, I=I_s=128, all fp32.
* ``qwen_decode``  T=1, H=2048, E=256, k=8, I=I_s=512, bf16, fp32 router
  ("Optimizing on-device inference for Apple Silicon", section "Qwen creates
  three distinct workload shapes": 256 experts, eight selected, one shared).
* ``ling_verify``  T=4, H=2560, E=512, k=8, I=I_s=768, bf16, per-token router
  bias that makes the four tokens touch exactly ``d`` distinct experts
  ("Three ways to boost mixture-of-experts inference on NVIDIA DGX Spark",
  section "Optimization 3": a four-token verification window can touch up to
  32 experts where one token touches eight).
* ``ling_mxfp4``   Ling shapes with MXFP4 expert weights (uniform e2m1 codes,
  e8m0 scales 2^U{-4..2}), bf16 activations and shared expert, fp32 output,
  T=1 (no bias) or T=4 (the verify bias recipe).
* ``qwen_prefill`` T=4096 Qwen shapes, bf16, per-expert bias
  b_e = -1.1 * ln(pi(e) + 1) for a seeded permutation pi (Zipf-like load).
* ``qwen_int4``   Qwen shapes with group-wise affine 4-bit experts ("Optimizing
  on-device inference for Apple Silicon", section "Decode weights during
  matrix multiplication": a 4-bit code per weight, a bf16 scale and bias per
  64 weights): codes uniform over 0..15; per group s = (sigma / 3) * U[0.75,
  1.25] and b = -7.5 * s * U[0.9, 1.1], sigma = 1/sqrt(fan_in), both rounded
  to bf16 -- a group quantised from N(0, sigma^2) values spans about
  +-2.5 sigma, so (max - min) / 15 and min land there.

Distributions: x ~ N(0, 1); every weight ~ N(0, 1/fan_in) with fan_in = H for
router, gate and up and I (or I_s) for down; fp32 -> bf16 by round to nearest
even.  Host draws use numpy's PCG64 ``default_rng(seed)`` in the order x,
router, bias, then per expert gate, up, down, then shared gate, up, down.
Large timing-only layers may instead be drawn on the device with torch's
seeded generator (``device_layer``); their bytes are copied back for any
check against the oracle.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

BF16, F32, MXFP4, INT4 = "bf16", "f32", "mxfp4", "int4g64"


@dataclasses.dataclass
class Layer:
    T: int
    H: int
    E: int
    k: int
    I: int
    I_shared: int
    act_dtype: str
    expert_dtype: str
    shared_dtype: str
    out_dtype: str
    router_w: object            # [E][H] fp32
    router_bias: object = None  # None, [E] or [T][E] fp32
    bias_t_stride: int = 0      # 0: [E]; E: [T][E]
    gate: object = None         # [E][I][H]   (bf16 as uint16 bits / fp32 / MXFP4 codes [E][I][H/2])
    up: object = None           # [E][I][H]
    down: object = None         # [E][H][I]
    gate_s: object = None       # MXFP4: e8m0 [E][I][H/32]; INT4: bf16 scales [E][I][H/64]
    up_s: object = None
    down_s: object = None       # [E][H][I/32] / [E][H][I/64]
    sh_gate: object = None      # [I_s][H]
    sh_up: object = None        # [I_s][H]
    sh_down: object = None      # [H][I_s]
    gate_b: object = None       # INT4 only: bf16 biases [E][I][H/64]
    up_b: object = None
    down_b: object = None       # [E][H][I/64]
    act_quant: str = "none"     # "mxfp8": the routed experts' GEMM inputs quantised to MXFP8 (W4A8)

    def with_T(self, T: int) -> "Layer":
        return dataclasses.replace(self, T=T)

    def arrays(self):
        for f in ("router_w", "router_bias", "gate", "up", "down", "gate_s", "up_s", "down_s",
                  "sh_gate", "sh_up", "sh_down", "gate_b", "up_b", "down_b"):
            yield f, getattr(self, f)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal(rng, shape, std, dtype):
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if dtype == F32:
        return a
    return f32_to_bf16_bits(a)


def _mxfp4(rng, E, N, K):
    codes = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    scales = rng.integers(127 - 4, 127 + 3, size=(E, N, K // 32), dtype=np.uint8)
    return codes, scales


def _int4(rng, E, N, K, std):
    """Group-wise affine 4-bit weights: codes [E][N][K/2], bf16 scales and biases [E][N][K/64]."""
    codes = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    s = (std / 3.0) * rng.uniform(0.75, 1.25, size=(E, N, K // 64))
    b = -7.5 * s * rng.uniform(0.9, 1.1, size=(E, N, K // 64))
    return codes, f32_to_bf16_bits(s.astype(np.float32)), f32_to_bf16_bits(b.astype(np.float32))


def verify_bias(rng, T: int, E: int, k: int, d: int, boost: float = 8.0) -> np.ndarray:
    """Per-token bias [T][E]: +boost on each token's k experts, the T sets drawn
    so that their union is a seeded pool of exactly d distinct experts.

    The pool is shuffled and split into T near-equal groups (each at most k
    long since d <= T*k); token t takes its group plus k - |group| further
    experts drawn without replacement from the rest of the pool."""
    if not (k <= d <= min(T * k, E)):
        raise ValueError(f"d={d} must lie in [k, min(T*k, E)]")
    pool = rng.choice(E, size=d, replace=False)
    groups = np.array_split(rng.permutation(pool), T)
    bias = np.zeros((T, E), np.float32)
    for t, grp in enumerate(groups):
        rest = np.setdiff1d(pool, grp)
        extra = rng.choice(rest, size=k - len(grp), replace=False) if k > len(grp) else []
        bias[t, np.concatenate([grp, extra]).astype(np.int64)] = np.float32(boost)
    return bias


def zipf_bias(rng, E: int, s: float = 1.1) -> np.ndarray:
    """Per-expert bias b_e = -s * ln(pi(e) + 1), pi a seeded permutation."""
    pi = rng.permutation(E)
    return (-s * np.log(pi.astype(np.float64) + 1.0)).astype(np.float32)


def make_layer(T, H, E, k, I, I_shared, act=BF16, expert=BF16, shared=BF16, out=BF16,
               seed=0, bias: Optional[str] = None, d: Optional[int] = None):
    """Draw one layer and its input x on the host.  Returns (Layer, x)."""
    rng = np.random.default_rng(seed)
    x = _normal(rng, (T, H), 1.0, act)
    router_w = rng.standard_normal((E, H), dtype=np.float32) * np.float32(1.0 / math.sqrt(H))
    router_bias, stride = None, 0
    if bias == "verify":
        router_bias, stride = verify_bias(rng, T, E, k, d if d is not None else min(T * k, E)), E
    elif bias == "zipf":
        router_bias, stride = zipf_bias(rng, E), 0
    elif bias is not None:
        raise ValueError(bias)
    L = Layer(T, H, E, k, I, I_shared, act, expert, shared, out, router_w, router_bias, stride)
    if expert == MXFP4:
        # one expert at a time keeps the draw order "per expert gate, up, down"
        gs, us, ds, gc, uc, dc = [], [], [], [], [], []
        for _ in range(E):
            c, s_ = _mxfp4(rng, 1, I, H); gc.append(c); gs.append(s_)
            c, s_ = _mxfp4(rng, 1, I, H); uc.append(c); us.append(s_)
            c, s_ = _mxfp4(rng, 1, H, I); dc.append(c); ds.append(s_)
        L.gate, L.up, L.down = np.concatenate(gc), np.concatenate(uc), np.concatenate(dc)
        L.gate_s, L.up_s, L.down_s = np.concatenate(gs), np.concatenate(us), np.concatenate(ds)
    elif expert == INT4:
        parts = {f: [] for f in ("gate", "gate_s", "gate_b", "up", "up_s", "up_b", "down", "down_s", "down_b")}
        for _ in range(E):
            for f, (n, kk, fan) in (("gate", (I, H, H)), ("up", (I, H, H)), ("down", (H, I, I))):
                c, s_, b_ = _int4(rng, 1, n, kk, 1.0 / math.sqrt(fan))
                parts[f].append(c); parts[f + "_s"].append(s_); parts[f + "_b"].append(b_)
        for f, v in parts.items():
            setattr(L, f, np.concatenate(v))
    else:
        shp_in, shp_out = (I, H), (H, I)
        gt = np.empty((E, I, H), np.float32 if expert == F32 else np.uint16)
        ut = np.empty_like(gt)
        dt = np.empty((E, H, I), gt.dtype)
        for e in range(E):
            gt[e] = _normal(rng, shp_in, 1.0 / math.sqrt(H), expert)
            ut[e] = _normal(rng, shp_in, 1.0 / math.sqrt(H), expert)
            dt[e] = _normal(rng, shp_out, 1.0 / math.sqrt(I), expert)
        L.gate, L.up, L.down = gt, ut, dt
    if I_shared > 0:
        L.sh_gate = _normal(rng, (I_shared, H), 1.0 / math.sqrt(H), shared)
        L.sh_up = _normal(rng, (I_shared, H), 1.0 / math.sqrt(H), shared)
        L.sh_down = _normal(rng, (H, I_shared), 1.0 / math.sqrt(I_shared), shared)
    return L, x


# Named workloads --------------------------------------------------------------------------

def tiny(seed=0):
    return make_layer(4, 256, 16, 2, 128, 128, F32, F32, F32, F32, seed=seed)


def qwen_decode(seed=0, T=1):
    return make_layer(T, 2048, 256, 8, 512, 512, BF16, BF16, BF16, BF16, seed=seed)


def ling_verify(seed=0, d=32, T=4):
    return make_layer(T, 2560, 512, 8, 768, 768, BF16, BF16, BF16, BF16, seed=seed,
                      bias="verify", d=d)


def ling_mxfp4(seed=0, T=1, d=32):
    return make_layer(T, 2560, 512, 8, 768, 768, BF16, MXFP4, BF16, F32, seed=seed,
                      bias=("verify" if T > 1 else None), d=(d if T > 1 else None))


def qwen_prefill(seed=0, T=4096):
    return make_layer(T, 2048, 256, 8, 512, 512, BF16, BF16, BF16, BF16, seed=seed, bias="zipf")


# Device-side draws for large timing layers -------------------------------------------------

def device_layer(T, H, E, k, I, I_shared, act=BF16, expert=BF16, shared=BF16, out=BF16,
                 seed=0, bias=None, d=None, device="cuda"):
    """Same recipe as ``make_layer`` but drawn with torch's seeded generator on
    ``device`` (fast for multi-GB layers).  Returns (Layer of torch tensors, x)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    rng = np.random.default_rng(seed)  # small host draws (bias recipes)

    def normal(shape, std, dt):
        a = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            a.mul_(std)
        if dt == F32:
            return a
        return a.to(torch.bfloat16).view(torch.int16)

    x = normal((T, H), 1.0, act)
    router_w = normal((E, H), 1.0 / math.sqrt(H), F32)
    router_bias, stride = None, 0
    if bias == "verify":
        router_bias, stride = torch.from_numpy(verify_bias(rng, T, E, k, d)).to(device), E
    elif bias == "zipf":
        router_bias, stride = torch.from_numpy(zipf_bias(rng, E)).to(device), 0
    L = Layer(T, H, E, k, I, I_shared, act, expert, shared, out, router_w, router_bias, stride)
    def codes(shape):
        return torch.randint(0, 256, shape, generator=g, device=device, dtype=torch.int32).to(torch.uint8)
    if expert == MXFP4:
        def scales(shape):
            return torch.randint(123, 130, shape, generator=g, device=device, dtype=torch.int32).to(torch.uint8)
        L.gate, L.gate_s = codes((E, I, H // 2)), scales((E, I, H // 32))
        L.up, L.up_s = codes((E, I, H // 2)), scales((E, I, H // 32))
        L.down, L.down_s = codes((E, H, I // 2)), scales((E, H, I // 32))
    elif expert == INT4:
        def group_params(shape, std):  # the host recipe of _int4, drawn on the device
            s = torch.empty(shape, device=device).uniform_(0.75, 1.25, generator=g).mul_(std / 3.0)
            b = torch.empty(shape, device=device).uniform_(0.9, 1.1, generator=g).mul_(s).mul_(-7.5)
            return s.to(torch.bfloat16).view(torch.int16), b.to(torch.bfloat16).view(torch.int16)
        L.gate = codes((E, I, H // 2)); L.gate_s, L.gate_b = group_params((E, I, H // 64), 1.0 / math.sqrt(H))
        L.up = codes((E, I, H // 2)); L.up_s, L.up_b = group_params((E, I, H // 64), 1.0 / math.sqrt(H))
        L.down = codes((E, H, I // 2)); L.down_s, L.down_b = group_params((E, H, I // 64), 1.0 / math.sqrt(I))
    else:
        L.gate = torch.empty((E, I, H), device=device, dtype=torch.float32 if expert == F32 else torch.int16)
        L.up = torch.empty_like(L.gate)
        L.down = torch.empty((E, H, I), device=device, dtype=L.gate.dtype)
        # experts in chunks of up to 16 (a few kernels per chunk, bounded fp32 temporaries)
        for e0 in range(0, E, 16):
            n = min(16, E - e0)
            L.gate[e0:e0 + n] = normal((n, I, H), 1.0 / math.sqrt(H), expert)
            L.up[e0:e0 + n] = normal((n, I, H), 1.0 / math.sqrt(H), expert)
            L.down[e0:e0 + n] = normal((n, H, I), 1.0 / math.sqrt(I), expert)
    if I_shared > 0:
        L.sh_gate = normal((I_shared, H), 1.0 / math.sqrt(H), shared)
        L.sh_up = normal((I_shared, H), 1.0 / math.sqrt(H), shared)
        L.sh_down = normal((H, I_shared), 1.0 / math.sqrt(I_shared), shared)
    return L, x


def to_device(L: Layer, x, device="cuda"):
    import torch

    def mv(a):
        if a is None:
            return None
        if isinstance(a, np.ndarray):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:   # bf16 bit patterns travel as int16 on the device
                a = a.view(np.int16)
            return torch.from_numpy(a).to(device)
        return a.to(device)
    D = dataclasses.replace(L, **{f: mv(a) for f, a in L.arrays()})
    return D, mv(x)


def to_host(L: Layer, x=None):
    def mv(a):
        if a is None or isinstance(a, np.ndarray):
            return a
        h = a.detach().cpu().numpy()
        return h.view(np.uint16) if h.dtype == np.int16 else h
    H = dataclasses.replace(L, **{f: mv(a) for f, a in L.arrays()})
    return (H, mv(x)) if x is not None else H
