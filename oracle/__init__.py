"""Python access to the C reference ("oracle") of the routed-expert FFN layer.

TEST INFRASTRUCTURE ONLY.  The oracle is a plain single-threaded double
precision restatement of the layer (see ``oracle.h`` for the definition, the
page sections it follows and the readings taken where the pages are silent).
Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
it.  It shares no code with the GPU library and never touches a GPU.

Arrays are numpy arrays holding the exact bytes the GPU library receives:
fp32 as float32, bf16 as uint16 bit patterns, MXFP4 as uint8 code bytes plus
uint8 e8m0 scale bytes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# MOE_ORACLE_LIB: load another build of oracle.c instead (the sanitizer test's ASan/UBSan build)
_LOAD = os.environ.get("MOE_ORACLE_LIB") or _LIB

F32, BF16, MXFP4, INT4G64 = 0, 1, 2, 3
_DTYPES = {"f32": F32, "bf16": BF16, "mxfp4": MXFP4, "int4g64": INT4G64}


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc: -O2, no contraction, no fast-math."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-o", _LIB, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
    return _LIB


CLANG = "/opt/rocm/llvm/bin/clang"


def build_sanitized(outdir: str) -> str:
    """Compile oracle.c with clang under AddressSanitizer + UndefinedBehaviorSanitizer (any
    report aborts) into outdir/liboracle_san.so; loading it needs the clang ASan runtime
    preloaded (asan_runtime())."""
    os.makedirs(outdir, exist_ok=True)
    out = os.path.join(outdir, "liboracle_san.so")
    cmd = [CLANG, "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-shared-libsan",
           "-fPIC", "-shared", "-o", out, _SRC, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True)
    return out


def asan_runtime() -> str:
    return subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], check=True,
                          capture_output=True, text=True).stdout.strip()


class _Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "H", "E", "k", "I", "I_shared", "act_dtype", "expert_dtype",
                 "shared_dtype", "act_quant")]


class _Weights(ctypes.Structure):
    _fields_ = [("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
                ("bias_t_stride", ctypes.c_int64),
                ("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("gate_s", ctypes.c_void_p), ("up_s", ctypes.c_void_p), ("down_s", ctypes.c_void_p),
                ("sh_gate", ctypes.c_void_p), ("sh_up", ctypes.c_void_p), ("sh_down", ctypes.c_void_p),
                ("gate_b", ctypes.c_void_p), ("up_b", ctypes.c_void_p), ("down_b", ctypes.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LOAD == _LIB and not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LOAD)
        P = ctypes.c_void_p
        L.orc_bf16_to_double.restype = ctypes.c_double
        L.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.orc_e2m1_to_double.restype = ctypes.c_double
        L.orc_e2m1_to_double.argtypes = [ctypes.c_uint8]
        L.orc_e8m0_to_double.restype = ctypes.c_double
        L.orc_e8m0_to_double.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_to_double.restype = ctypes.c_double
        L.orc_e4m3_to_double.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_from_double.restype = ctypes.c_uint8
        L.orc_e4m3_from_double.argtypes = [ctypes.c_double]
        L.orc_weight.restype = ctypes.c_double
        L.orc_weight.argtypes = [P, P, P, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                 ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
        for name, args in {
            "orc_logits": [P, P, P, P],
            "orc_select": [P, ctypes.c_int, ctypes.c_int, P, P],
            "orc_set_weights": [P, ctypes.c_int, ctypes.c_int, P, P],
            "orc_plan": [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P],
            "orc_mxfp8_quantize": [P, ctypes.c_int, P, P],
            "orc_mxfp8_dequantize": [P, P, ctypes.c_int, P],
            "orc_forward_with_routing": [P, P, P, P, P, P],
            "orc_forward": [P, P, P, P, P, P, P],
        }.items():
            fn = getattr(L, name)
            fn.restype = ctypes.c_int
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "oracle needs C-contiguous numpy arrays"
    return a.ctypes.data


def _shape(layer) -> _Shape:
    return _Shape(layer.T, layer.H, layer.E, layer.k, layer.I, layer.I_shared,
                  _DTYPES[layer.act_dtype], _DTYPES[layer.expert_dtype],
                  _DTYPES[layer.shared_dtype], 1 if getattr(layer, "act_quant", "none") == "mxfp8" else 0)


def _weights(layer) -> tuple[_Weights, list]:
    keep = []

    def p(a):
        if a is not None:
            keep.append(a)
        return _ptr(a)

    w = _Weights(p(layer.router_w), p(layer.router_bias), layer.bias_t_stride,
                 p(layer.gate), p(layer.up), p(layer.down),
                 p(layer.gate_s), p(layer.up_s), p(layer.down_s),
                 p(layer.sh_gate), p(layer.sh_up), p(layer.sh_down),
                 p(getattr(layer, "gate_b", None)), p(getattr(layer, "up_b", None)), p(getattr(layer, "down_b", None)))
    return w, keep


def bf16_to_double(bits: int) -> float:
    return lib().orc_bf16_to_double(bits)


def e2m1_to_double(nibble: int) -> float:
    return lib().orc_e2m1_to_double(nibble)


def e8m0_to_double(bits: int) -> float:
    return lib().orc_e8m0_to_double(bits)


def e4m3_to_double(bits: int) -> float:
    return lib().orc_e4m3_to_double(bits)


def e4m3_from_double(v: float) -> int:
    return lib().orc_e4m3_from_double(v)


def mxfp8_quantize(v: np.ndarray):
    """MXFP8 (E4M3 elements, one e8m0 scale per 32): (codes uint8 [n], scales uint8 [n/32])."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    codes = np.empty(v.size, np.uint8)
    scales = np.empty(max(v.size // 32, 1), np.uint8)
    if lib().orc_mxfp8_quantize(_ptr(v), v.size, _ptr(codes), _ptr(scales)):
        raise ValueError("orc_mxfp8_quantize: n must be a multiple of 32")
    return codes, scales[: v.size // 32]


def mxfp8_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    v = np.empty(codes.size, np.float64)
    if lib().orc_mxfp8_dequantize(_ptr(codes), _ptr(scales), codes.size, _ptr(v)):
        raise ValueError("orc_mxfp8_dequantize: n must be a multiple of 32")
    return v


def weight(base: np.ndarray, scales, dtype: str, mat, rows, cols, r, c, biases=None) -> float:
    return lib().orc_weight(_ptr(base), _ptr(scales), _ptr(biases), _DTYPES[dtype], mat, rows, cols, r, c)


def logits(layer, x: np.ndarray) -> np.ndarray:
    """Router logits [T][E] as fp32 (double sum, one rounding)."""
    s = _shape(layer)
    w, keep = _weights(layer)
    out = np.empty((layer.T, layer.E), np.float32)
    rc = lib().orc_logits(ctypes.byref(s), _ptr(x), ctypes.byref(w), _ptr(out))
    if rc:
        raise ValueError(f"orc_logits failed ({rc})")
    return out


def select(logit_row: np.ndarray, k: int):
    """Top-k ids (descending logit, ties to lower index) and renormalised softmax weights."""
    lr = np.ascontiguousarray(logit_row, dtype=np.float32)
    ids = np.empty(k, np.int32)
    w = np.empty(k, np.float64)
    rc = lib().orc_select(_ptr(lr), lr.size, k, _ptr(ids), _ptr(w))
    if rc:
        raise ValueError(f"orc_select failed ({rc})")
    return ids, w


def set_weights(logit_row: np.ndarray, ids) -> np.ndarray:
    """Combine weights of a given expert set: softmax over all E renormalised over the set."""
    lr = np.ascontiguousarray(logit_row, dtype=np.float32)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.empty(ids.size, np.float64)
    rc = lib().orc_set_weights(_ptr(lr), lr.size, ids.size, _ptr(ids), _ptr(w))
    if rc:
        raise ValueError(f"orc_set_weights failed ({rc})")
    return w


def near_tie_selections(logit_row: np.ndarray, k: int, gap: float = 1e-5):
    """Every selection a token admits when logits within `gap` of its k-th largest logit
    count as tied: the experts strictly above that band, plus any choice of the rest from the
    band.  Returns a list of (ids in descending logit order, weights).  One selection when no
    logit outside the oracle's own choice lies in the band."""
    import itertools
    lr = np.ascontiguousarray(logit_row, dtype=np.float32)
    ids, _ = select(lr, k)
    kth = float(lr[ids[-1]])
    band = [e for e in range(lr.size) if abs(float(lr[e]) - kth) < gap]
    above = [int(e) for e in ids if abs(float(lr[e]) - kth) >= gap]
    out = []
    for extra in itertools.combinations(band, k - len(above)):
        s = above + sorted(extra, key=lambda e: (-float(lr[e]), e))
        out.append((np.array(s, np.int32), set_weights(lr, s)))
    return out


def select_all(logits_te: np.ndarray, k: int):
    T = logits_te.shape[0]
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    for t in range(T):
        ids[t], w[t] = select(logits_te[t], k)
    return ids, w


def plan(ids: np.ndarray, E: int):
    """Histogram, exclusive offsets and stable scatter of slots by expert."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    sorted_slot = np.empty(max(T * k, 1), np.int32)
    rc = lib().orc_plan(_ptr(ids), T, k, E, _ptr(counts), _ptr(offsets), _ptr(sorted_slot))
    if rc:
        raise ValueError(f"orc_plan failed ({rc})")
    return counts, offsets, sorted_slot[: T * k]


def forward_with_routing(layer, x: np.ndarray, ids: np.ndarray, cw: np.ndarray) -> np.ndarray:
    s = _shape(layer)
    w, keep = _weights(layer)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    cw = np.ascontiguousarray(cw, dtype=np.float64)
    y = np.empty((layer.T, layer.H), np.float64)
    rc = lib().orc_forward_with_routing(ctypes.byref(s), _ptr(x), ctypes.byref(w), _ptr(ids),
                                        _ptr(cw), _ptr(y))
    if rc:
        raise ValueError(f"orc_forward_with_routing failed ({rc})")
    return y


def forward(layer, x: np.ndarray):
    """Whole layer.  Returns (y [T][H] double, ids [T][k], weights [T][k], logits [T][E] fp32)."""
    s = _shape(layer)
    w, keep = _weights(layer)
    y = np.empty((layer.T, layer.H), np.float64)
    ids = np.empty((layer.T, layer.k), np.int32)
    cw = np.empty((layer.T, layer.k), np.float64)
    lg = np.empty((layer.T, layer.E), np.float32)
    rc = lib().orc_forward(ctypes.byref(s), _ptr(x), ctypes.byref(w), _ptr(y), _ptr(ids),
                           _ptr(cw), _ptr(lg))
    if rc:
        raise ValueError(f"orc_forward failed ({rc})")
    return y, ids, cw, lg
