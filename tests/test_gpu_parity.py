"""GPU parity: the HIP library, called through its C ABI, against the CPU oracle on the
same seeded bytes.

Bars (floating point compared with the oracle's double-precision result):
  * routing fed the oracle's fp32 logits: indices bit-exact, plan counts/offsets exact,
    per-expert slot sets exact (order inside a group unspecified);
  * routing end to end: indices equal except on tokens whose k-th/(k+1)-th oracle logit gap
    is below 1e-5, where either order is accepted;
  * bf16 output: max relative error <= 2e-2 (|y - y_ref| / max(|y_ref|, rms(y_ref))) and
    relative L2 <= 5e-3;
  * MXFP4 experts with fp32 output: relative L2 <= 1e-3 on the decode path (T <= 16); on the
    grouped-GEMM path (T > 16) the MFMAs take bf16 activations, so the bf16 bars apply;
  * all-fp32 layer: relative L2 <= 1e-5 (fp32 accumulation over <= 2^12 terms stays
    near 1e-6).
"""
import dataclasses
import sys

import numpy as np
import pytest

from routed_expert_ffn_route_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch


@pytest.fixture(scope="module")
def B(torch_cuda):
    from routed_expert_ffn_route_amd import binding
    binding.lib()  # raises if libmoe.so is missing: no fallback
    return binding


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def errs(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    max_rel = float(np.max(np.abs(y - ref) / np.maximum(np.abs(ref), rms)))
    l2 = float(np.linalg.norm(y - ref) / np.linalg.norm(ref))
    return max_rel, l2


def y_host(L, y):
    a = y.cpu().numpy()
    if L.out_dtype == "bf16":
        return synth.bf16_bits_to_f32(a.view(np.uint16)).astype(np.float64)
    return a.astype(np.float64)


def check_out(L, y, ref, tag):
    max_rel, l2 = errs(y, ref)
    say(f"[{tag}] max_rel={max_rel:.3e} rel_l2={l2:.3e}")
    assert np.all(np.isfinite(y)), tag
    if L.expert_dtype == "mxfp4" and L.T <= 16:
        assert l2 <= 1e-3, tag
    elif L.expert_dtype == "mxfp4":  # grouped-GEMM path: bf16 activations feed the MFMAs
        assert max_rel <= 2e-2 and l2 <= 5e-3, tag
    elif L.out_dtype == "bf16":
        assert max_rel <= 2e-2 and l2 <= 5e-3, tag
    elif L.act_dtype == "f32" and L.expert_dtype == "f32":
        assert l2 <= 1e-5, tag
    else:
        assert l2 <= 5e-3, tag


def host_view_for_oracle(Ld, xd, ids_needed=None):
    """Host copy of a device layer for the oracle.  With ids_needed, only those experts'
    weights are copied; the rest are zero pages the oracle never reads."""
    import torch

    def cp(t):
        return None if t is None else t.cpu().numpy()
    Lh = synth.to_host(dataclasses.replace(Ld, gate=None, up=None, down=None, gate_s=None, up_s=None,
                                           down_s=None))
    for f in ("gate", "up", "down", "gate_s", "up_s", "down_s"):
        t = getattr(Ld, f)
        if t is None:
            continue
        if ids_needed is None:
            h = cp(t)
            setattr(Lh, f, h.view(np.uint16) if h.dtype == np.int16 else h)
        else:
            dt = cp(t[:1]).dtype
            arr = np.zeros(tuple(t.shape), dtype=np.uint16 if dt == np.int16 else dt)
            for e in sorted(set(int(i) for i in ids_needed)):
                arr[e] = t[e].cpu().numpy().view(arr.dtype)
            setattr(Lh, f, arr)
    return Lh, xd.cpu().numpy()


def oracle_routing(orc, Lh, xh):
    lg = orc.logits(Lh, xh)
    ids, w = orc.select_all(lg, Lh.k)
    return lg, ids, w


def gap_ok(lg_row, k, tol=1e-5):
    s = np.sort(lg_row.astype(np.float64))[::-1]
    return k >= len(s) or (s[k - 1] - s[k]) < tol


def check_routing(orc, Lh, xh, got_ids, lg, ids, tag):
    """Indices equal except on near-tie tokens.  Returns the tokens that differ."""
    diff = [t for t in range(Lh.T) if not np.array_equal(got_ids[t], ids[t])]
    for t in diff:
        assert gap_ok(lg[t], Lh.k), f"[{tag}] token {t} routing differs without a near tie"
        assert set(got_ids[t].tolist()) ^ set(ids[t].tolist()) <= set(np.argsort(-lg[t])[: Lh.k + 1].tolist())
    return diff


def forward_dev(B, Ld, xd, ws=None):
    import torch
    y = B.layer_forward(Ld, xd, ws=ws)
    torch.cuda.synchronize()
    return y


def full_check(orc, B, Lh, xh, Ld, xd, tag, copy_selected=False):
    """moe_route + moe_forward on the device vs the oracle on the host."""
    import torch
    if Lh is None:
        Lh, xh = host_view_for_oracle(dataclasses.replace(Ld, gate=None, up=None, down=None, gate_s=None,
                                                          up_s=None, down_s=None), xd)
    lg, ids, w = oracle_routing(orc, Lh, xh)
    if copy_selected:
        Lh, xh = host_view_for_oracle(Ld, xd, ids_needed=ids.ravel())
    r = B.layer_route(Ld, xd)
    torch.cuda.synchronize()
    got_ids = r["ids"].cpu().numpy()
    diff = check_routing(orc, Lh, xh, got_ids, lg, ids, tag)
    assert np.allclose(r["logits"].cpu().numpy(), lg, rtol=1e-4, atol=1e-5), tag
    y = y_host(Ld, forward_dev(B, Ld, xd))
    ref = orc.forward_with_routing(Lh, xh, ids, w)
    keep = [t for t in range(Lh.T) if t not in diff]
    check_out(Lh, y[keep], ref[keep], tag)
    return y, ids


# ------------------------------------------------------------------------------------------

def test_tiny_fp32_layer(orc, B):
    say("[tiny] T=4 H=256 E=16 k=2 I=Is=128 fp32")
    Lh, xh = synth.tiny(seed=0)
    Ld, xd = synth.to_device(Lh, xh)
    full_check(orc, B, Lh, xh, Ld, xd, "tiny")


@pytest.mark.parametrize("T,H,E,k", [(1, 256, 256, 8), (4, 256, 512, 8), (3, 64, 100, 16),
                                     (1, 64, 1024, 16), (8, 128, 64, 4), (2, 32, 7, 7)])
def test_forward_exact_ties(orc, B, T, H, E, k):
    """Router weights and activations in {-1, 0, 1} make every logit an exact integer, so many
    tokens have equal logits at the k-th place; the forward pass must take the lower expert
    index among equal logits, like the oracle, on every token (none is excused as a near tie)."""
    say(f"[forward-ties] T={T} H={H} E={E} k={k}")
    Lh, xh = synth.make_layer(T, H, E, k, 64, 64, seed=17 + E)
    rng = np.random.default_rng(23 + T * E)
    Lh.router_w = rng.integers(-1, 2, size=(E, H)).astype(np.float32)
    xi = rng.integers(-1, 2, size=(T, H)).astype(np.float32)
    xh = synth.f32_to_bf16_bits(xi) if Lh.act_dtype == "bf16" else xi
    Ld, xd = synth.to_device(Lh, xh)
    lg, ids, w = oracle_routing(orc, Lh, xh)
    s = -np.sort(-lg, axis=1)
    if k < E:
        assert np.any(s[:, k - 1] == s[:, k]), "the draw has no tie at the k-th place"
    y = y_host(Ld, forward_dev(B, Ld, xd))
    ref = orc.forward_with_routing(Lh, xh, ids, w)
    check_out(Lh, y, ref, f"ties T={T} E={E} k={k}")


@pytest.mark.parametrize("T,H,E,k,tie", [
    (4, 256, 16, 2, False), (1, 2048, 256, 8, False), (4, 2560, 512, 8, False),
    (16, 256, 64, 8, True), (3, 64, 1024, 16, True), (5, 96, 7, 7, True), (1, 32, 1, 1, False),
    (300, 256, 256, 8, True), (4096, 128, 256, 8, False)])
def test_route_bitexact_on_oracle_logits(orc, B, T, H, E, k, tie):
    """Fed the oracle's fp32 logits, the selection kernels reproduce its indices exactly
    (ties included: integer-valued inputs give integer logits with many exact ties)."""
    import torch
    say(f"[route-logits_in] T={T} H={H} E={E} k={k} tie={tie}")
    if tie:
        rng = np.random.default_rng(T * 7 + E)
        xi = rng.integers(-1, 2, (T, H)).astype(np.float32)
        wi = rng.integers(-1, 2, (E, H)).astype(np.float32)
        Lh = synth.Layer(T, H, E, k, 32, 0, "bf16", "bf16", "bf16", "bf16", wi)
        xh = synth.f32_to_bf16_bits(xi)
    else:
        Lh, xh = synth.make_layer(T, H, E, k, 32, 0, seed=E + T)
    lg = orc.logits(Lh, xh)
    ids, w = orc.select_all(lg, k)
    counts, offsets, sorted_slot = orc.plan(ids, E)
    Ld, _ = synth.to_device(Lh, xh)
    r = B.layer_route(Ld, None, logits_in=torch.from_numpy(lg).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(r["ids"].cpu().numpy(), ids)
    assert np.allclose(r["w"].cpu().numpy(), w, rtol=2e-6, atol=1e-7)
    assert np.array_equal(r["logits"].cpu().numpy(), lg)
    assert np.array_equal(r["count"].cpu().numpy(), counts)
    assert np.array_equal(r["offset"].cpu().numpy(), offsets)
    gs = r["sorted"].cpu().numpy()
    for e in range(E):
        assert set(gs[offsets[e]:offsets[e + 1]].tolist()) == set(sorted_slot[offsets[e]:offsets[e + 1]].tolist())


@pytest.mark.parametrize("T,H,E,k,bias", [(1, 2048, 256, 8, None), (4, 2560, 512, 8, "verify"),
                                          (64, 2048, 256, 8, "zipf"), (4096, 2048, 256, 8, "zipf")])
def test_route_end_to_end(orc, B, T, H, E, k, bias):
    import torch
    say(f"[route] T={T} H={H} E={E} k={k} bias={bias}")
    Lh, xh = synth.make_layer(T, H, E, k, 32, 0, seed=11, bias=bias, d=(32 if bias == "verify" else None))
    Ld, xd = synth.to_device(Lh, xh)
    lg, ids, w = oracle_routing(orc, Lh, xh)
    r = B.layer_route(Ld, xd)
    torch.cuda.synchronize()
    diff = check_routing(orc, Lh, xh, r["ids"].cpu().numpy(), lg, ids, "route")
    say(f"  near-tie tokens: {len(diff)}")
    assert np.allclose(r["logits"].cpu().numpy(), lg, rtol=1e-4, atol=1e-5)


@pytest.mark.parametrize("kw", [
    dict(T=1, H=256, E=8, k=2, I=64, I_shared=64),
    dict(T=4, H=512, E=32, k=4, I=96, I_shared=64),
    dict(T=5, H=800, E=40, k=8, I=160, I_shared=0),           # ragged rows, no shared expert
    dict(T=16, H=256, E=64, k=8, I=128, I_shared=96),          # largest decode batch
    dict(T=2, H=1024, E=1, k=1, I=224, I_shared=32),           # one expert
    dict(T=3, H=256, E=1024, k=16, I=32, I_shared=32),         # max E and k
    dict(T=4, H=4608, E=16, k=2, I=64, I_shared=64),           # row longer than one slice
    dict(T=16, H=4096, E=32, k=4, I=128, I_shared=64),         # x (128 KiB) too large for LDS
    dict(T=7, H=5120, E=24, k=3, I=96, I_shared=32),           # token tile 8, x from global
])
def test_decode_edge_shapes_bf16(orc, B, kw):
    say(f"[decode-edge] {kw}")
    Lh, xh = synth.make_layer(**kw, seed=3)
    Ld, xd = synth.to_device(Lh, xh)
    full_check(orc, B, Lh, xh, Ld, xd, f"edge {kw}")


def test_decode_fp32_single_token(orc, B):
    say("[decode-f32-T1]")
    Lh, xh = synth.make_layer(1, 512, 32, 4, 128, 96, "f32", "f32", "f32", "f32", seed=6)
    Ld, xd = synth.to_device(Lh, xh)
    full_check(orc, B, Lh, xh, Ld, xd, "f32 T=1")


def test_decode_fp32_out_from_bf16(orc, B):
    say("[decode-f32out]")
    Lh, xh = synth.make_layer(4, 512, 32, 4, 128, 128, out="f32", seed=4)
    Ld, xd = synth.to_device(Lh, xh)
    full_check(orc, B, Lh, xh, Ld, xd, "f32out")


def test_qwen_decode_full_size_and_nan_poison(orc, B):
    """Qwen-shaped decode (T=1, H=2048, 256 experts, top-8, I=I_s=512, bf16) at full size,
    drawn on the device.  Then every expert the oracle did not select is NaN-poisoned: the
    output must not change by a bit."""
    import torch
    for seed in (0, 47):
        say(f"[qwen-decode] seed={seed}")
        Ld, xd = synth.device_layer(1, 2048, 256, 8, 512, 512, seed=seed)
        y, ids = full_check(orc, B, None, None, Ld, xd, f"qwen seed={seed}", copy_selected=True)
        y0 = B.layer_forward(Ld, xd).clone()
        poison = torch.ones(256, dtype=torch.bool, device="cuda")
        poison[torch.from_numpy(ids.ravel().astype(np.int64)).cuda()] = False
        for f in ("gate", "up", "down"):
            getattr(Ld, f).view(torch.int16)[poison] = 0x7FC0   # bf16 quiet NaN
        y1 = B.layer_forward(Ld, xd)
        torch.cuda.synchronize()
        assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))


@pytest.mark.parametrize("d", [20, 24, 28, 32])
def test_ling_verify_window(orc, B, d):
    """Ling-shaped 4-token verify window (H=2560, 512 experts, top-8, I=I_s=768, bf16) whose
    per-token bias makes the tokens touch exactly d distinct experts."""
    say(f"[ling-verify] d={d}")
    Ld, xd = synth.device_layer(4, 2560, 512, 8, 768, 768, seed=100 + d, bias="verify", d=d)
    y, ids = full_check(orc, B, None, None, Ld, xd, f"ling d={d}", copy_selected=True)
    assert len(set(ids.ravel().tolist())) == d


@pytest.mark.parametrize("T,d", [(2, 8), (2, 16), (3, 13), (3, 24), (5, 21), (5, 40)])
def test_ling_verify_sweep(orc, B, T, d):
    """Verify windows of 2, 3 and 5 tokens at the Ling shapes, each at the fewest and the most
    distinct experts such a window can touch plus one value between."""
    say(f"[ling-verify-sweep] T={T} d={d}")
    Ld, xd = synth.device_layer(T, 2560, 512, 8, 768, 768, seed=300 + 10 * T + d, bias="verify", d=d)
    y, ids = full_check(orc, B, None, None, Ld, xd, f"ling T={T} d={d}", copy_selected=True)
    assert len(set(ids.ravel().tolist())) == d


@pytest.mark.parametrize("T,d", [(1, None), (4, 32), (4, 20), (3, 17), (5, 33)])
def test_ling_mxfp4(orc, B, T, d):
    """Ling shapes with MXFP4 experts (e2m1 codes, e8m0 scales 2^-4..2^2), bf16 activations
    and shared expert, fp32 output."""
    say(f"[ling-mxfp4] T={T} d={d}")
    Ld, xd = synth.device_layer(T, 2560, 512, 8, 768, 768, "bf16", "mxfp4", "bf16", "f32", seed=200 + T,
                                bias=("verify" if T > 1 else None), d=d)
    full_check(orc, B, None, None, Ld, xd, f"mxfp4 T={T}", copy_selected=True)


def test_mxfp4_small_shapes(orc, B):
    for kw in (dict(T=1, H=256, E=8, k=2, I=64, I_shared=64), dict(T=6, H=2048, E=16, k=4, I=512, I_shared=96),
               dict(T=16, H=2560, E=32, k=4, I=256, I_shared=64)):  # the last: x from global
        say(f"[mxfp4-small] {kw}")
        Lh, xh = synth.make_layer(**kw, act="bf16", expert="mxfp4", shared="bf16", out="f32", seed=5)
        Ld, xd = synth.to_device(Lh, xh)
        full_check(orc, B, Lh, xh, Ld, xd, f"mxfp4 {kw}")


def test_deterministic_and_workspace_reuse(orc, B):
    """Same inputs twice give identical bits; one workspace serves calls of different
    inputs back to back, and needs no initialisation (here: filled with garbage)."""
    import torch
    say("[determinism]")
    La, xa = synth.make_layer(4, 512, 64, 8, 128, 128, seed=21)
    Lb, xb = synth.make_layer(4, 512, 64, 8, 128, 128, seed=22)
    Lda, xda = synth.to_device(La, xa)
    Ldb, xdb = synth.to_device(Lb, xb)
    ws = B.workspace(B.shape_of(Lda))
    ws.fill_(0xA5)
    ya1 = B.layer_forward(Lda, xda, ws=ws).clone()
    yb = B.layer_forward(Ldb, xdb, ws=ws).clone()
    ya2 = B.layer_forward(Lda, xda, ws=ws).clone()
    torch.cuda.synchronize()
    assert torch.equal(ya1.view(torch.int16), ya2.view(torch.int16))
    ref_b = orc.forward(Lb, xb)[0]
    check_out(Lb, y_host(Lb, yb), ref_b, "ws-reuse")


# ---- prefill path (T > 16): grouped MFMA GEMMs ------------------------------------------

@pytest.mark.parametrize("kw", [
    dict(T=17, H=256, E=16, k=2, I=128, I_shared=128),           # smallest prefill batch
    dict(T=64, H=512, E=32, k=4, I=192, I_shared=64, bias="zipf"),  # ragged tiles, skewed load
    dict(T=300, H=1024, E=64, k=8, I=512, I_shared=512, bias="zipf"),
    dict(T=200, H=96, E=8, k=2, I=96, I_shared=0),               # K not a multiple of 64, no shared
    dict(T=129, H=2048, E=256, k=8, I=512, I_shared=512),        # Qwen shapes, one row past a tile
])
def test_prefill_small_bf16(orc, B, kw):
    say(f"[prefill] {kw}")
    Lh, xh = synth.make_layer(**kw, seed=7)
    Ld, xd = synth.to_device(Lh, xh)
    assert B.path_name(B.shape_of(Ld)) == "prefill.bf16"
    full_check(orc, B, Lh, xh, Ld, xd, f"prefill {kw}")


def test_prefill_f32_out(orc, B):
    say("[prefill-f32out]")
    Lh, xh = synth.make_layer(40, 256, 16, 4, 64, 64, out="f32", seed=8)
    Ld, xd = synth.to_device(Lh, xh)
    full_check(orc, B, Lh, xh, Ld, xd, "prefill f32out")


@pytest.mark.parametrize("kw", [
    dict(T=17, H=256, E=16, k=2, I=128, I_shared=128),
    dict(T=64, H=512, E=32, k=4, I=192, I_shared=64, bias="zipf"),   # ragged tiles, 6 scales per row
    dict(T=160, H=1024, E=4, k=2, I=512, I_shared=512, bias="zipf"),    # hot experts span 2 tiles
    dict(T=200, H=96, E=8, k=2, I=96, I_shared=0),                    # no shared expert
    dict(T=20, H=2560, E=16, k=4, I=768, I_shared=768),               # Ling widths
])
def test_prefill_small_mxfp4(orc, B, kw):
    """MXFP4 experts on the grouped-GEMM path: codes and scales unpacked to bf16 on the way
    from LDS into the MFMA; the shared expert (bf16) takes the bf16 kernel."""
    say(f"[prefill-mxfp4] {kw}")
    Lh, xh = synth.make_layer(**kw, act="bf16", expert="mxfp4", shared="bf16", out="f32", seed=9)
    Ld, xd = synth.to_device(Lh, xh)
    assert B.path_name(B.shape_of(Ld)) == "prefill.mxfp4"
    full_check(orc, B, Lh, xh, Ld, xd, f"prefill-mxfp4 {kw}")


def test_ling_mxfp4_prefill_full_size_sampled(orc, B):
    """Ling-shaped MXFP4 prefill (T=4096, 512 experts top-8, Zipf(1.1) bias) at full size in
    the benchmark's launch configuration; the oracle checks a sample of tokens."""
    import torch
    say("[ling-mxfp4-prefill] T=4096")
    Ld, xd = synth.device_layer(4096, 2560, 512, 8, 768, 768, "bf16", "mxfp4", "bf16", "f32", seed=3,
                                bias="zipf")
    y = y_host(Ld, forward_dev(B, Ld, xd))
    r = B.layer_route(Ld, xd)
    torch.cuda.synchronize()
    gids = r["ids"].cpu().numpy()
    counts = r["count"].cpu().numpy()
    assert counts.sum() == 4096 * 8
    hot = int(np.argmax(counts))
    rng = np.random.default_rng(1)
    pick = sorted(set(rng.choice(4096, 24, replace=False).tolist()) |
                  set(np.nonzero((gids == hot).any(axis=1))[0][:8].tolist()) | {0, 4095})
    Lh, xh = host_view_for_oracle(Ld, xd, ids_needed=gids[pick].ravel())
    sub = Lh.with_T(len(pick))
    xs = np.ascontiguousarray(xh[pick])
    lg, ids, w = oracle_routing(orc, sub, xs)
    diff = check_routing(orc, sub, xs, gids[pick], lg, ids, "mxfp4-prefill-4096")
    ref = orc.forward_with_routing(sub, xs, ids, w)
    keep = [i for i in range(len(pick)) if i not in diff]
    check_out(sub, y[pick][keep], ref[keep], "mxfp4-prefill-4096 sampled")
    assert np.all(np.isfinite(y))


def test_qwen_prefill_full_size_sampled(orc, B):
    """Qwen-shaped prefill (T=4096, 256 experts top-8, Zipf(1.1) expert bias, bf16) at full
    size in the benchmark's launch configuration; the oracle checks a sample of tokens one by
    one (tokens are independent), including tokens of the most loaded expert."""
    import torch
    say("[qwen-prefill] T=4096")
    Ld, xd = synth.device_layer(4096, 2048, 256, 8, 512, 512, seed=0, bias="zipf")
    y = y_host(Ld, forward_dev(B, Ld, xd))
    r = B.layer_route(Ld, xd)
    torch.cuda.synchronize()
    gids = r["ids"].cpu().numpy()
    counts = r["count"].cpu().numpy()
    say(f"  max tokens/expert {counts.max()}, idle experts {(counts == 0).sum()}")
    assert counts.sum() == 4096 * 8
    hot = int(np.argmax(counts))
    rng = np.random.default_rng(0)
    pick = sorted(set(rng.choice(4096, 40, replace=False).tolist()) |
                  set(np.nonzero((gids == hot).any(axis=1))[0][:12].tolist()) | {0, 4095})
    Lh, xh = host_view_for_oracle(Ld, xd)
    sub = Lh.with_T(len(pick))
    xs = np.ascontiguousarray(xh[pick])
    lg, ids, w = oracle_routing(orc, sub, xs)
    diff = check_routing(orc, sub, xs, gids[pick], lg, ids, "prefill-4096")
    ref = orc.forward_with_routing(sub, xs, ids, w)
    keep = [i for i in range(len(pick)) if i not in diff]
    check_out(sub, y[pick][keep], ref[keep], "prefill-4096 sampled")
    assert np.all(np.isfinite(y))
