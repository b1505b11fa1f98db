"""C-ABI checks that need no GPU: the library loads, exports every entry point the header
declares, and rejects bad arguments before it launches anything (validation runs on the
host first, so none of these calls touches a device)."""
import ctypes
import os
import re

import pytest

from routed_expert_ffn_route_amd import binding as B
from routed_expert_ffn_route_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libmoe.so is not built (run __graft_entry__.build())")
    return B.lib()


def test_header_declares_the_entry_points():
    assert _declared() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def _shape(**kw):
    base = dict(T=1, H=2048, E=256, k=8, I=512, I_shared=512, act_dtype=1, expert_dtype=1,
                shared_dtype=1, out_dtype=1, act_quant=0)
    base.update(kw)
    return B.Shape(*[base[n] for n, _ in B.Shape._fields_])


def _ws(shape):
    n = ctypes.c_size_t(0)
    rc = B.lib().moe_workspace_size(ctypes.byref(shape), ctypes.byref(n))
    return rc, n.value


def test_strerror_covers_codes(lib):
    for c in (0, -1, -2, -3, -4, -5, -6):
        assert B.strerror(c) and B.strerror(c) != "unknown error code"
    assert B.strerror(-99) == "unknown error code"


@pytest.mark.parametrize("kw,code", [
    (dict(T=0), B.MOE_EINVAL), (dict(k=0), B.MOE_EINVAL), (dict(E=4, k=8), B.MOE_EINVAL),
    (dict(I=0), B.MOE_EINVAL), (dict(I_shared=-32), B.MOE_EINVAL),
    (dict(H=2040), B.MOE_EUNSUPPORTED), (dict(I=500), B.MOE_EUNSUPPORTED),
    (dict(E=2048), B.MOE_EUNSUPPORTED), (dict(k=17, E=64), B.MOE_EUNSUPPORTED),
    (dict(act_dtype=0), B.MOE_EUNSUPPORTED), (dict(out_dtype=2), B.MOE_EUNSUPPORTED),
    (dict(expert_dtype=7), B.MOE_EUNSUPPORTED), (dict(shared_dtype=2), B.MOE_EUNSUPPORTED),
    # MXFP4 on the grouped-GEMM path: a tile's scale rows must fit in LDS (H, I <= 8192)
    (dict(T=64, expert_dtype=2, H=8224), B.MOE_EUNSUPPORTED),
    (dict(T=64, expert_dtype=2, I=8192 + 32), B.MOE_EUNSUPPORTED),
    # group-wise affine 4-bit: groups of 64 along H and I
    (dict(expert_dtype=3, H=2048 + 32), B.MOE_EUNSUPPORTED), (dict(expert_dtype=3, I=512 + 32), B.MOE_EUNSUPPORTED),
    # ... and on the grouped-GEMM path a wave's scale and bias blocks must fit in LDS beside the
    # ring (H <= 7680 for gate/up, I <= 6144 for down)
    (dict(T=64, expert_dtype=3, H=7680 + 64), B.MOE_EUNSUPPORTED),
    (dict(T=64, expert_dtype=3, I=6144 + 64), B.MOE_EUNSUPPORTED),
    (dict(expert_dtype=3, act_dtype=0, shared_dtype=0), B.MOE_EUNSUPPORTED),
    # W4A8: MXFP4 experts on the grouped-GEMM path only
    (dict(T=64, act_quant=1), B.MOE_EUNSUPPORTED), (dict(T=4, expert_dtype=2, act_quant=1), B.MOE_EUNSUPPORTED),
    (dict(T=64, expert_dtype=3, act_quant=1), B.MOE_EUNSUPPORTED), (dict(T=64, expert_dtype=2, act_quant=2), B.MOE_EUNSUPPORTED),
])
def test_shape_validation(lib, kw, code):
    rc, _ = _ws(_shape(**kw))
    assert rc == code
    assert B.path_name(_shape(**kw)) == "invalid"


def test_workspace_sizes_and_paths(lib):
    for kw, path in [(dict(), "decode.bf16"), (dict(T=4, H=2560, E=512, I=768, I_shared=768), "decode.bf16"),
                     (dict(expert_dtype=2, out_dtype=0), "decode.mxfp4"), (dict(T=16), "decode.bf16"),
                     (dict(T=17), "prefill.bf16"), (dict(T=4096), "prefill.bf16"),
                     (dict(T=4096, H=2560, E=512, I=768, I_shared=768, expert_dtype=2, out_dtype=0),
                      "prefill.mxfp4"), (dict(T=64, expert_dtype=2, H=8192), "prefill.mxfp4"),
                     (dict(expert_dtype=3), "decode.int4g64"), (dict(T=4096, expert_dtype=3), "prefill.int4g64"),
                     (dict(T=64, expert_dtype=3, H=7680, I=6144), "prefill.int4g64"),
                     (dict(T=4, expert_dtype=3, H=16384, I=8192), "decode.int4g64"),
                     (dict(T=4096, expert_dtype=2, out_dtype=0, act_quant=1), "prefill.mxfp4.w4a8"),
                     (dict(T=4, H=256, E=16, k=2, I=128, I_shared=128, act_dtype=0, expert_dtype=0,
                           shared_dtype=0, out_dtype=0), "decode.f32")]:
        s = _shape(**kw)
        rc, n = _ws(s)
        assert rc == 0 and n >= 256 and n % 256 == 0
        assert B.path_name(s) == path
    # a null shape or size pointer is rejected
    assert B.lib().moe_workspace_size(None, None) == B.MOE_EINVAL


def _call_forward(shape, x=0x1000, w=None, y=0x2000, ws=0x3000, ws_bytes=1 << 40):
    if w is None:
        w = B.Weights(0x10000, None, 0, 0x20000, 0x30000, 0x40000, None, None, None,
                      0x50000, 0x60000, 0x70000)
    return B.lib().moe_forward(ctypes.byref(shape), x, ctypes.byref(w), y, ws, ws_bytes, None)


def test_forward_argument_errors_enqueue_nothing(lib):
    s = _shape()
    good = B.Weights(0x10000, None, 0, 0x20000, 0x30000, 0x40000, None, None, None, 0x50000, 0x60000, 0x70000)
    assert _call_forward(s, x=None) == B.MOE_EINVAL
    assert _call_forward(s, y=None) == B.MOE_EINVAL
    w = B.Weights.from_buffer_copy(good); w.router_w = None
    assert _call_forward(s, w=w) == B.MOE_EINVAL
    w = B.Weights.from_buffer_copy(good); w.down = None
    assert _call_forward(s, w=w) == B.MOE_EINVAL
    w = B.Weights.from_buffer_copy(good); w.sh_up = None
    assert _call_forward(s, w=w) == B.MOE_EINVAL
    w = B.Weights.from_buffer_copy(good); w.router_bias = 0x80000; w.bias_t_stride = 7
    assert _call_forward(s, w=w) == B.MOE_EINVAL
    # MXFP4 needs its scale arrays, 16-byte aligned
    assert _call_forward(_shape(expert_dtype=2), w=good) == B.MOE_EINVAL
    w = B.Weights.from_buffer_copy(good); w.gate_s, w.up_s, w.down_s = 0x90000, 0xA0000, 0xB0000
    # group-wise affine 4-bit needs scales and biases, 16-byte aligned
    assert _call_forward(_shape(expert_dtype=3), w=w) == B.MOE_EINVAL
    w4 = B.Weights.from_buffer_copy(w); w4.gate_b, w4.up_b, w4.down_b = 0xC0000, 0xD0000, 0xE0000
    assert _call_forward(_shape(expert_dtype=3), w=w4, ws=None) == B.MOE_EWORKSPACE
    for f in ("gate_b", "up_b", "down_b", "down_s"):
        wm = B.Weights.from_buffer_copy(w4); setattr(wm, f, getattr(w4, f) + 2)
        assert _call_forward(_shape(expert_dtype=3), w=wm) == B.MOE_EALIGN, f
    rc, need = _ws(_shape(expert_dtype=2, out_dtype=0))
    assert _call_forward(_shape(expert_dtype=2, out_dtype=0), w=w, ws=None) == B.MOE_EWORKSPACE
    for f in ("gate_s", "up_s", "down_s"):
        wm = B.Weights.from_buffer_copy(w); setattr(wm, f, getattr(w, f) + 4)
        assert _call_forward(_shape(expert_dtype=2, out_dtype=0), w=wm) == B.MOE_EALIGN, f
    # misaligned pointers
    assert _call_forward(s, x=0x1004) == B.MOE_EALIGN
    assert _call_forward(s, y=0x2002) == B.MOE_EALIGN
    w = B.Weights.from_buffer_copy(good); w.gate = 0x20008
    assert _call_forward(s, w=w) == B.MOE_EALIGN
    # workspace
    rc, need = _ws(s)
    assert _call_forward(s, ws=None) == B.MOE_EWORKSPACE
    assert _call_forward(s, ws_bytes=need - 1) == B.MOE_EWORKSPACE
    # a shared-expert-free layer needs no shared pointers: everything validates up to the
    # workspace check
    s0 = _shape(I_shared=0)
    w = B.Weights.from_buffer_copy(good); w.sh_gate = w.sh_up = w.sh_down = None
    assert _call_forward(s0, w=w, ws=None) == B.MOE_EWORKSPACE


def test_route_argument_errors(lib):
    s = _shape()
    w = B.Weights(0x10000, None, 0, None, None, None, None, None, None, None, None, None)
    out = B.RouteOut(0x1000, 0x2000, None, None, None, None)
    L = B.lib()
    assert L.moe_route(ctypes.byref(s), 0x4000, ctypes.byref(w), None, None, 0x5000, 1 << 40, None) == B.MOE_EINVAL
    bad = B.RouteOut(None, 0x2000, None, None, None, None)
    assert L.moe_route(ctypes.byref(s), 0x4000, ctypes.byref(w), None, ctypes.byref(bad), 0x5000, 1 << 40, None) == B.MOE_EINVAL
    assert L.moe_route(ctypes.byref(s), None, ctypes.byref(w), None, ctypes.byref(out), 0x5000, 1 << 40, None) == B.MOE_EINVAL
    assert L.moe_route(ctypes.byref(s), 0x4000, ctypes.byref(w), None, ctypes.byref(out), None, 0, None) == B.MOE_EWORKSPACE
    assert L.moe_route(ctypes.byref(s), None, None, 0x6004, ctypes.byref(out), 0x5000, 1 << 40, None) == B.MOE_EALIGN


def test_workspace_routing_offsets(lib):
    """The forward pass's routing sits at the front of the workspace: logits [T][E] fp32, then
    ids and weights [T][k], each section 256-byte aligned and inside the workspace."""
    for kw in (dict(), dict(T=4, H=2560, E=512, I=768, I_shared=768), dict(T=4096),
               dict(T=300, expert_dtype=2, out_dtype=0)):
        s = _shape(**kw)
        lo, io, wo = B.workspace_routing_offsets(s)
        rc, need = _ws(s)
        assert lo == 0 and io >= 4 * s.T * s.E and wo >= io + 4 * s.T * s.k
        assert io % 256 == 0 and wo % 256 == 0 and wo + 4 * s.T * s.k <= need
    n = ctypes.c_size_t(0)
    assert B.lib().moe_workspace_routing(ctypes.byref(_shape()), None, ctypes.byref(n), ctypes.byref(n)) == B.MOE_EINVAL
    assert B.lib().moe_workspace_routing(ctypes.byref(_shape(T=0)), ctypes.byref(n), ctypes.byref(n),
                                         ctypes.byref(n)) == B.MOE_EINVAL


def test_static_forward_rejects_oversized_shapes_before_the_device(lib):
    """moe_forward_static refuses a shape whose workspace exceeds the static scratch with
    MOE_ESCRATCH before any device call (so this runs without a GPU), and validates the
    rest like moe_forward."""
    w = B.Weights(0x10000, None, 0, 0x20000, 0x30000, 0x40000, None, None, None, 0x50000, 0x60000, 0x70000)
    big = _shape(T=4096)
    rc, need = _ws(big)
    assert rc == 0 and need > B.STATIC_SCRATCH_BYTES
    assert B.lib().moe_forward_static(ctypes.byref(big), 0x1000, ctypes.byref(w), 0x2000, None) == B.MOE_ESCRATCH
    for kw in (dict(), dict(T=16, H=2560, E=512, I=768, I_shared=768),
               dict(T=16, H=2560, E=512, I=768, I_shared=768, expert_dtype=2, out_dtype=0)):
        rc, need = _ws(_shape(**kw))
        assert rc == 0 and need <= B.STATIC_SCRATCH_BYTES, kw   # every decode shape of the workloads fits
    s = _shape()
    assert B.lib().moe_forward_static(ctypes.byref(s), None, ctypes.byref(w), 0x2000, None) == B.MOE_EINVAL
    assert B.lib().moe_forward_static(ctypes.byref(s), 0x1004, ctypes.byref(w), 0x2000, None) == B.MOE_EALIGN
    assert B.lib().moe_forward_static(ctypes.byref(_shape(T=0)), 0x1000, ctypes.byref(w), 0x2000, None) == B.MOE_EINVAL


def test_read_ceiling_validates_arguments(lib):
    L = B.lib()
    assert L.moe_read_ceiling(None, 1024, 0x2000, None) == B.MOE_EINVAL
    assert L.moe_read_ceiling(0x1000, 8, 0x2000, None) == B.MOE_EINVAL
    assert L.moe_read_ceiling(0x1000, 1024, None, None) == B.MOE_EINVAL
    assert L.moe_read_ceiling(0x1008, 1024, 0x2000, None) == B.MOE_EALIGN


def test_stage_rate_validates_arguments(lib):
    L = B.lib()
    ok = (0x1000, 1 << 21, 64, 4, 0x2000, None)
    for i, bad in [(0, None), (1, 4096), (1, 3 << 20), (2, 8), (2, 48), (2, 2048), (3, 0), (4, None)]:
        a = list(ok)
        a[i] = bad
        assert L.moe_stage_rate(*a) == B.MOE_EINVAL, (i, bad)
    assert L.moe_stage_rate(0x1008, 1 << 21, 64, 4, 0x2000, None) == B.MOE_EALIGN
    assert L.moe_stage_rate(0x1000, 1 << 21, 64, 4, 0x2002, None) == B.MOE_EALIGN


def test_timing_api_rejects_misuse(lib):
    assert B.lib().moe_timing_begin(0) == B.MOE_EINVAL
    n = ctypes.c_int32(0)
    assert B.lib().moe_timing_end(None, 0, ctypes.byref(n)) == B.MOE_EINVAL


def test_binding_shapes_match_synth_layers():
    L, x = synth.tiny()
    s = B.shape_of(L)
    assert (s.T, s.H, s.E, s.k, s.I, s.I_shared) == (4, 256, 16, 2, 128, 128)
    assert (s.act_dtype, s.expert_dtype, s.shared_dtype, s.out_dtype) == (0, 0, 0, 0)
