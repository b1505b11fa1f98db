"""ctypes binding of libmoe.so (include/moe.h).  Argument marshalling only: every step
of the layer runs in the library's HIP kernels; torch supplies device memory and the
current stream.  Raises if the library has not been built -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB: load another build of the library (the sanitizer test's host-instrumented build)
LIB_PATH = os.environ.get("MOE_LIB") or os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EALIGN, MOE_EWORKSPACE, MOE_EHIP, MOE_ESCRATCH = 0, -1, -2, -3, -4, -5, -6
STATIC_SCRATCH_BYTES = 32 << 20   # MOE_STATIC_SCRATCH_BYTES
DTYPES = {"f32": 0, "bf16": 1, "mxfp4": 2, "int4g64": 3}
EXPORTS = ("moe_workspace_size", "moe_route", "moe_forward", "moe_forward_static", "moe_workspace_routing",
           "moe_path_name", "moe_strerror", "moe_timing_begin", "moe_timing_end", "moe_read_ceiling",
           "moe_stage_rate")


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "H", "E", "k", "I", "I_shared", "act_dtype", "expert_dtype", "shared_dtype",
                 "out_dtype", "act_quant")]


class Weights(ctypes.Structure):
    _fields_ = [("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
                ("bias_t_stride", ctypes.c_int64),
                ("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("gate_s", ctypes.c_void_p), ("up_s", ctypes.c_void_p), ("down_s", ctypes.c_void_p),
                ("sh_gate", ctypes.c_void_p), ("sh_up", ctypes.c_void_p), ("sh_down", ctypes.c_void_p),
                ("gate_b", ctypes.c_void_p), ("up_b", ctypes.c_void_p), ("down_b", ctypes.c_void_p)]


class RouteOut(ctypes.Structure):
    _fields_ = [("topk_ids", ctypes.c_void_p), ("topk_w", ctypes.c_void_p), ("logits", ctypes.c_void_p),
                ("expert_count", ctypes.c_void_p), ("expert_offset", ctypes.c_void_p),
                ("sorted_slot", ctypes.c_void_p)]


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 64), ("launches", ctypes.c_int32), ("total_ms", ctypes.c_double)]


class MoeError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {strerror(code)} ({code})")
        self.code = code


_lib = None


def lib():
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m routed_expert_ffn_route_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        L.moe_workspace_size.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(ctypes.c_size_t)]
        L.moe_route.argtypes = [ctypes.POINTER(Shape), P, ctypes.POINTER(Weights), P,
                                ctypes.POINTER(RouteOut), P, ctypes.c_size_t, P]
        L.moe_forward.argtypes = [ctypes.POINTER(Shape), P, ctypes.POINTER(Weights), P, P,
                                  ctypes.c_size_t, P]
        L.moe_forward_static.argtypes = [ctypes.POINTER(Shape), P, ctypes.POINTER(Weights), P, P]
        L.moe_workspace_routing.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(ctypes.c_size_t),
                                            ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
        L.moe_path_name.argtypes = [ctypes.POINTER(Shape)]
        L.moe_path_name.restype = ctypes.c_char_p
        L.moe_strerror.argtypes = [ctypes.c_int]
        L.moe_strerror.restype = ctypes.c_char_p
        L.moe_timing_begin.argtypes = [ctypes.c_int32]
        L.moe_timing_end.argtypes = [ctypes.POINTER(KernelTime), ctypes.c_int32,
                                     ctypes.POINTER(ctypes.c_int32)]
        L.moe_read_ceiling.argtypes = [P, ctypes.c_size_t, P, P]
        L.moe_stage_rate.argtypes = [P, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32, P, P]
        for n in ("moe_workspace_size", "moe_route", "moe_forward", "moe_forward_static", "moe_workspace_routing",
                  "moe_timing_begin", "moe_timing_end", "moe_read_ceiling", "moe_stage_rate"):
            getattr(L, n).restype = ctypes.c_int
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().moe_strerror(code).decode()


def _ptr(t):
    if t is None:
        return None
    return t.data_ptr() if hasattr(t, "data_ptr") else int(t)


def shape_of(layer) -> Shape:
    return Shape(layer.T, layer.H, layer.E, layer.k, layer.I, layer.I_shared,
                 DTYPES[layer.act_dtype], DTYPES[layer.expert_dtype], DTYPES[layer.shared_dtype],
                 DTYPES[layer.out_dtype], 1 if getattr(layer, "act_quant", "none") == "mxfp8" else 0)


def weights_of(layer) -> Weights:
    return Weights(_ptr(layer.router_w), _ptr(layer.router_bias), layer.bias_t_stride,
                   _ptr(layer.gate), _ptr(layer.up), _ptr(layer.down),
                   _ptr(layer.gate_s), _ptr(layer.up_s), _ptr(layer.down_s),
                   _ptr(layer.sh_gate), _ptr(layer.sh_up), _ptr(layer.sh_down),
                   _ptr(layer.gate_b), _ptr(layer.up_b), _ptr(layer.down_b))


def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def workspace_size(shape: Shape) -> int:
    n = ctypes.c_size_t(0)
    rc = lib().moe_workspace_size(ctypes.byref(shape), ctypes.byref(n))
    if rc:
        raise MoeError(rc, "moe_workspace_size")
    return n.value


def workspace(shape: Shape, device="cuda"):
    """A zero-filled workspace tensor of the size the library asks for."""
    import torch
    return torch.zeros(max(workspace_size(shape), 256), dtype=torch.uint8, device=device)


def route(shape: Shape, x, weights: Weights, out: RouteOut, ws, logits_in=None, stream=None) -> None:
    rc = lib().moe_route(ctypes.byref(shape), _ptr(x), ctypes.byref(weights), _ptr(logits_in),
                         ctypes.byref(out), _ptr(ws), ws.numel() if ws is not None else 0,
                         _stream(stream))
    if rc:
        raise MoeError(rc, "moe_route")


def forward(shape: Shape, x, weights: Weights, y, ws, stream=None) -> None:
    rc = lib().moe_forward(ctypes.byref(shape), _ptr(x), ctypes.byref(weights), _ptr(y), _ptr(ws),
                           ws.numel() if ws is not None else 0, _stream(stream))
    if rc:
        raise MoeError(rc, "moe_forward")


def workspace_routing_offsets(shape: Shape) -> tuple[int, int, int]:
    """Byte offsets of the logits, the selected ids and their weights that moe_forward
    leaves in its workspace."""
    lo, io, wo = ctypes.c_size_t(0), ctypes.c_size_t(0), ctypes.c_size_t(0)
    rc = lib().moe_workspace_routing(ctypes.byref(shape), ctypes.byref(lo), ctypes.byref(io), ctypes.byref(wo))
    if rc:
        raise MoeError(rc, "moe_workspace_routing")
    return lo.value, io.value, wo.value


def forward_routing(layer, ws):
    """(logits [T][E], ids [T][k] ascending per token, weights [T][k]) that the last moe_forward
    on workspace `ws` used, as views into the workspace tensor."""
    import torch
    lo, io, wo = workspace_routing_offsets(shape_of(layer))
    T, E, k = layer.T, layer.E, layer.k
    lg = ws[lo:lo + 4 * T * E].view(torch.float32).view(T, E)
    ids = ws[io:io + 4 * T * k].view(torch.int32).view(T, k)
    w = ws[wo:wo + 4 * T * k].view(torch.float32).view(T, k)
    return lg, ids, w


def forward_static(shape: Shape, x, weights: Weights, y, stream=None) -> None:
    """moe_forward_static: the layer with the library's static scratch as workspace."""
    rc = lib().moe_forward_static(ctypes.byref(shape), _ptr(x), ctypes.byref(weights), _ptr(y), _stream(stream))
    if rc:
        raise MoeError(rc, "moe_forward_static")


def path_name(shape: Shape) -> str:
    return lib().moe_path_name(ctypes.byref(shape)).decode()


def timing_begin(max_launches: int) -> None:
    rc = lib().moe_timing_begin(max_launches)
    if rc:
        raise MoeError(rc, "moe_timing_begin")


def timing_end(max_out: int = 32) -> dict:
    arr = (KernelTime * max_out)()
    n = ctypes.c_int32(0)
    rc = lib().moe_timing_end(arr, max_out, ctypes.byref(n))
    if rc:
        raise MoeError(rc, "moe_timing_end")
    return {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms) for i in range(n.value)}


def read_ceiling(buf, nbytes: int, sink, stream=None) -> None:
    """moe_read_ceiling: stream nbytes of buf once (the read-rate probe)."""
    rc = lib().moe_read_ceiling(_ptr(buf), nbytes, _ptr(sink), _stream(stream))
    if rc:
        raise MoeError(rc, "moe_read_ceiling")


def stage_rate(buf, region_bytes: int, seg_bytes: int, iters: int, sink, stream=None) -> int:
    """moe_stage_rate: the operand-staging probe; returns the bytes one call moves."""
    rc = lib().moe_stage_rate(_ptr(buf), region_bytes, seg_bytes, iters, _ptr(sink), _stream(stream))
    if rc:
        raise MoeError(rc, "moe_stage_rate")
    return 512 * 4 * iters * 6144


# Convenience on a synth.Layer of device tensors --------------------------------------------

def layer_forward(layer, x, y=None, ws=None, stream=None):
    """Run moe_forward on a synth.Layer whose arrays are device tensors."""
    import torch
    shape = shape_of(layer)
    if ws is None:
        ws = workspace(shape, x.device)
    if y is None:
        y = torch.empty((layer.T, layer.H), device=x.device,
                        dtype=torch.float32 if layer.out_dtype == "f32" else torch.int16)
    forward(shape, x, weights_of(layer), y, ws, stream)
    return y


def layer_route(layer, x, ws=None, logits_in=None, stream=None):
    import torch
    shape = shape_of(layer)
    dev = x.device if x is not None else logits_in.device
    if ws is None:
        ws = workspace(shape, dev)
    T, k, E = layer.T, layer.k, layer.E
    o = dict(ids=torch.empty((T, k), dtype=torch.int32, device=dev),
             w=torch.empty((T, k), dtype=torch.float32, device=dev),
             logits=torch.empty((T, E), dtype=torch.float32, device=dev),
             count=torch.empty(E, dtype=torch.int32, device=dev),
             offset=torch.empty(E + 1, dtype=torch.int32, device=dev),
             sorted=torch.empty(T * k, dtype=torch.int32, device=dev))
    out = RouteOut(_ptr(o["ids"]), _ptr(o["w"]), _ptr(o["logits"]), _ptr(o["count"]),
                   _ptr(o["offset"]), _ptr(o["sorted"]))
    route(shape, x, weights_of(layer), out, ws, logits_in, stream)
    return o
