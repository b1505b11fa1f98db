"""moe_forward_static (the entry point that allocates nothing: its workspace is the library's
static device scratch) against moe_forward on the same inputs, called through the C ABI: two
calls in a row, the second with a smaller input, bit for bit equal to moe_forward's output."""
import sys

import numpy as np
import pytest

from routed_expert_ffn_route_amd import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def B():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from routed_expert_ffn_route_amd import binding
    binding.lib()
    return binding


def _pair(B, kw, seed):
    import torch
    Lh, xh = synth.make_layer(**kw, seed=seed)
    Ld, xd = synth.to_device(Lh, xh)
    shape = B.shape_of(Ld)
    y_ref = B.layer_forward(Ld, xd)
    y = torch.full_like(y_ref, -1)
    B.forward_static(shape, xd, B.weights_of(Ld), y)
    torch.cuda.synchronize()
    return y_ref, y


@pytest.mark.parametrize("first,second", [
    # decode: Ling-shaped verify window, then a single token
    (dict(T=4, H=2560, E=64, k=8, I=768, I_shared=768), dict(T=1, H=2560, E=64, k=8, I=768, I_shared=768)),
    # MXFP4 decode, then prefill-sized batches (the grouped-GEMM path), larger then smaller
    (dict(T=5, H=1024, E=32, k=4, I=256, I_shared=128, act="bf16", expert="mxfp4", shared="bf16", out="f32"),
     dict(T=2, H=1024, E=32, k=4, I=256, I_shared=128, act="bf16", expert="mxfp4", shared="bf16", out="f32")),
    (dict(T=96, H=512, E=32, k=4, I=192, I_shared=64, bias="zipf"), dict(T=20, H=512, E=32, k=4, I=192, I_shared=64)),
    (dict(T=64, H=1024, E=16, k=2, I=512, I_shared=512, act="bf16", expert="mxfp4", shared="bf16", out="f32"),
     dict(T=17, H=1024, E=16, k=2, I=512, I_shared=512, act="bf16", expert="mxfp4", shared="bf16", out="f32")),
])
def test_static_forward_matches_forward(B, first, second):
    import torch
    for i, kw in enumerate((first, second)):
        say(f"[static] call {i + 1}: {kw}")
        y_ref, y = _pair(B, kw, seed=31 + i)
        assert torch.equal(y_ref.view(torch.int16) if y_ref.dtype == torch.int16 else y_ref.view(torch.int32),
                           y.view(torch.int16) if y.dtype == torch.int16 else y.view(torch.int32)), kw
        assert torch.isfinite(y.float() if y.dtype == torch.float32 else y.view(torch.bfloat16).float()).all()


def test_static_forward_rejects_a_shape_beyond_the_scratch(B):
    import torch
    Ld, xd = synth.device_layer(4096, 2048, 64, 8, 512, 512, seed=5)
    y = torch.empty((4096, 2048), dtype=torch.int16, device="cuda")
    with pytest.raises(B.MoeError) as e:
        B.forward_static(B.shape_of(Ld), xd, B.weights_of(Ld), y)
    assert e.value.code == B.MOE_ESCRATCH
