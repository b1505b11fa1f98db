"""Pins for the CPU oracle: each test checks the oracle against something other
than itself -- a published value, a closed form, a library routine on a
special case, brute force on a tiny input, or an invariant of the layer -- so
that a plausible slip in the oracle (a dropped term, a wrong sign or index, a
transposed operand, swapped gate/up) fails at least one test.  CPU only.
"""
import itertools
import math
import os

import numpy as np
import pytest
import scipy.special

from routed_expert_ffn_route_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                a, b = line.split()
                rows.append((int(a, 0), float(b)))
    return rows


def _same(a, b):
    return (math.isnan(a) and math.isnan(b)) or (a == b and math.copysign(1, a) == math.copysign(1, b))


# --- element decoders -----------------------------------------------------------------------

def test_bf16_decode_matches_binary32_definition(orc):
    for bits, val in _read_table("bf16_values.txt"):
        assert _same(orc.bf16_to_double(bits), val), hex(bits)


def test_e2m1_decode_matches_mx_spec_table(orc):
    table = _read_table("e2m1_values.txt")
    assert len(table) == 16
    for code, val in table:
        assert _same(orc.e2m1_to_double(code), val), code


def test_e8m0_decode_closed_form(orc):
    for b in range(255):
        assert orc.e8m0_to_double(b) == math.ldexp(1.0, b - 127)
    assert math.isnan(orc.e8m0_to_double(255))


def test_mxfp4_roundtrip_all_codes_and_scales(orc):
    """quantise(dequantise(c, s)) == (c, s) for the 16 codes x the 7 scales the
    workloads use, keeping the sign of -0; every value is exact in fp32 and bf16."""
    table = dict(_read_table("e2m1_values.txt"))
    for s in range(123, 130):
        for c in range(16):
            codes = np.array([[[c | (c << 4)] * 16]], np.uint8)   # 1 x 1 x 32 elements
            scales = np.array([[[s]]], np.uint8)
            v = orc.weight(codes, scales, "mxfp4", 0, 1, 32, 0, 0)
            # quantise back: exact division by the power-of-two scale, then table search
            q = v / math.ldexp(1.0, s - 127)
            back = [cc for cc, tv in table.items() if _same(tv, q)]
            assert back == [c], (c, s, v)
            assert float(np.float32(v)) == v
            assert float(synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(np.array([v], np.float32)))[0]) == v


def test_mxfp4_layout_nibble_order_and_scale_index(orc):
    """Element 2i is the low nibble of byte i; one scale per 32 consecutive
    elements of a row; rows and experts are stacked [E][N][K/2]."""
    E, N, K = 2, 3, 64
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    scales = rng.integers(120, 134, (E, N, K // 32), dtype=np.uint8)
    table = dict(_read_table("e2m1_values.txt"))
    for e in range(E):
        for n in range(N):
            for c in range(K):
                byte = int(codes[e, n, c // 2])
                nib = byte & 15 if c % 2 == 0 else byte >> 4
                want = table[nib] * math.ldexp(1.0, int(scales[e, n, c // 32]) - 127)
                got = orc.weight(codes, scales, "mxfp4", e, N, K, n, c)
                assert _same(got, want), (e, n, c)


def test_int4_group_affine_closed_form(orc):
    """Group-wise affine 4-bit: weight = s * q + b with q the unsigned nibble (element 2i in the
    low nibble of byte i) and (s, b) the bf16 pair of the 64-element group the element falls in;
    rows and experts stacked [E][N][K/2] and [E][N][K/64].  Hand-made bytes: one row of 128
    elements, group 0 with s = 0.25, b = -1, group 1 with s = 2^-7, b = 3.5."""
    codes = np.zeros((1, 1, 64), np.uint8)
    codes[0, 0, 0] = 0x3A          # element 0 -> 10, element 1 -> 3
    codes[0, 0, 31] = 0xF0         # element 62 -> 0, element 63 -> 15
    codes[0, 0, 32] = 0x71         # element 64 -> 1, element 65 -> 7
    codes[0, 0, 63] = 0x0C         # element 126 -> 12, element 127 -> 0
    sc = synth.f32_to_bf16_bits(np.array([[[0.25, 2.0 ** -7]]], np.float32))
    bi = synth.f32_to_bf16_bits(np.array([[[-1.0, 3.5]]], np.float32))
    want = {0: 0.25 * 10 - 1, 1: 0.25 * 3 - 1, 62: -1.0, 63: 0.25 * 15 - 1, 64: 2.0 ** -7 + 3.5,
            65: 7 * 2.0 ** -7 + 3.5, 126: 12 * 2.0 ** -7 + 3.5, 127: 3.5, 2: -1.0, 100: 3.5}
    for c, v in want.items():
        assert orc.weight(codes, sc, "int4g64", 0, 1, 128, 0, c, biases=bi) == v, c


def test_int4_layout_and_roundtrip(orc):
    """Every element of random stacked int4 weights equals s*q + b read off the bytes by index
    arithmetic; and (w - b) / s recovers each of the 16 codes exactly for scales and biases of
    the workloads' kind (quantise(dequantise(q)) == q)."""
    E, N, K = 2, 3, 128
    rng = np.random.default_rng(15)
    codes, sc, bi = synth._int4(rng, E, N, K, 0.1)
    for e in range(E):
        for n in range(N):
            for c in range(0, K, 3):
                byte = int(codes[e, n, c // 2])
                q = byte & 15 if c % 2 == 0 else byte >> 4
                s_ = float(synth.bf16_bits_to_f32(sc[e, n, c // 64:c // 64 + 1])[0])
                b_ = float(synth.bf16_bits_to_f32(bi[e, n, c // 64:c // 64 + 1])[0])
                got = orc.weight(codes, sc, "int4g64", e, N, K, n, c, biases=bi)
                assert got == s_ * q + b_, (e, n, c)
                assert (got - b_) / s_ == q
    for q in range(16):
        row = np.full((1, 1, 32), q | (q << 4), np.uint8)
        for s_, b_ in ((0.03125, -0.234375), (2.0 ** -9 * 3, -2.0 ** -5 * 11), (1.0, 0.0)):
            w = orc.weight(row, synth.f32_to_bf16_bits(np.array([[[s_]]], np.float32)), "int4g64", 0, 1, 64, 0, 5,
                           biases=synth.f32_to_bf16_bits(np.array([[[b_]]], np.float32)))
            assert (w - b_) / s_ == q


# --- router: logits, selection, weights -----------------------------------------------------

def test_logits_exact_on_integer_inputs(orc):
    """Integer-valued x, router and bias make every partial sum exact, so the
    logits equal an int64 matrix product exactly (fp32 and bf16 activations)."""
    rng = np.random.default_rng(1)
    T, H, E = 3, 256, 16
    xi = rng.integers(-2, 3, (T, H))
    wi = rng.integers(-2, 3, (E, H))
    bi = rng.integers(-5, 6, (T, E))
    want = xi @ wi.T + bi
    for act in ("f32", "bf16"):
        x = xi.astype(np.float32) if act == "f32" else synth.f32_to_bf16_bits(xi.astype(np.float32))
        L = synth.Layer(T, H, E, 2, 32, 0, act, "f32", "f32", "f32", wi.astype(np.float32),
                        bi.astype(np.float32), E)
        got = orc.logits(L, x)
        assert np.array_equal(got.astype(np.int64), want)


def test_logits_single_rounding_of_double_sum(orc):
    rng = np.random.default_rng(2)
    L, x = synth.make_layer(2, 512, 8, 2, 32, 0, "bf16", "bf16", "bf16", "bf16", seed=3, bias="zipf")
    got = orc.logits(L, x)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    want = (xf @ L.router_w.astype(np.float64).T + L.router_bias.astype(np.float64)[None, :])
    # fp64 product vs sequential fp64 sum differ by ~1e-16 relative; after one
    # rounding to fp32 they agree to 1 ulp of fp32
    assert np.allclose(got, want.astype(np.float32), rtol=2 ** -23, atol=0)


def _brute_topk(lrow, k):
    order = sorted(range(len(lrow)), key=lambda e: (-float(lrow[e]), e))
    return order[:k]


def test_topk_brute_force_with_ties(orc):
    rng = np.random.default_rng(3)
    for trial in range(300):
        E = int(rng.integers(1, 40))
        k = int(rng.integers(1, E + 1))
        lrow = rng.integers(-3, 4, E).astype(np.float32)  # many ties
        ids, _ = orc.select(lrow, k)
        assert ids.tolist() == _brute_topk(lrow, k), (lrow, k)


def test_topk_subset_enumeration_small(orc):
    """For E <= 8, the selected set is the one subset of size k whose every member
    ranks before every non-member (larger logit, or equal logit and lower index)."""
    rng = np.random.default_rng(4)
    for trial in range(100):
        E = int(rng.integers(2, 9))
        k = int(rng.integers(1, E + 1))
        lrow = rng.integers(-2, 3, E).astype(np.float32)

        def before(a, b):
            return lrow[a] > lrow[b] or (lrow[a] == lrow[b] and a < b)
        good = [set(S) for S in itertools.combinations(range(E), k)
                if all(before(a, b) for a in S for b in range(E) if b not in S)]
        assert len(good) == 1
        ids, _ = orc.select(lrow, k)
        assert set(ids.tolist()) == good[0]
        assert all(before(ids[j], ids[j + 1]) for j in range(k - 1))


def test_weights_closed_forms(orc):
    # equal logits -> uniform over the k chosen
    ids, w = orc.select(np.zeros(16, np.float32), 4)
    assert ids.tolist() == [0, 1, 2, 3] and np.all(w == 0.25)
    # two experts whose logits differ by ln 3 -> 3/4 and 1/4
    l = np.array([-50.0, math.log(3.0), 0.0, -50.0], np.float32)
    ids, w = orc.select(l, 2)
    assert ids.tolist() == [1, 2]
    r = math.exp(float(np.float32(math.log(3.0))))
    assert abs(w[0] - r / (r + 1)) < 1e-15 and abs(w[1] - 1 / (r + 1)) < 1e-15
    # k = E reduces to the plain softmax (library routine)
    rng = np.random.default_rng(6)
    l = rng.standard_normal(10).astype(np.float32) * 3
    ids, w = orc.select(l, 10)
    sm = scipy.special.softmax(l.astype(np.float64))
    assert np.allclose(w, sm[ids], rtol=1e-14, atol=0)


def test_weights_equal_selected_ratio_and_sum_to_one(orc):
    """Renormalised softmax equals exp(l_j) / sum over the selected exp(l_i)
    (the full-softmax denominator cancels); weights sum to 1 and follow the
    rank order."""
    rng = np.random.default_rng(7)
    for _ in range(200):
        E = int(rng.integers(2, 64))
        k = int(rng.integers(1, min(E, 9) + 1))
        l = (rng.standard_normal(E) * 4).astype(np.float32)
        ids, w = orc.select(l, k)
        sel = l[ids].astype(np.float64)
        want = np.exp(sel - sel.max()) / np.exp(sel - sel.max()).sum()
        assert np.allclose(w, want, rtol=1e-13, atol=0)
        assert abs(w.sum() - 1.0) < k * 2 ** -52 * 4
        assert np.all(np.diff(w) <= 0)


def test_set_weights_are_the_softmax_of_the_set(orc):
    """Renormalising the full softmax over a set equals the plain softmax of the set's own
    logits (a library routine), in the order the set is given; shifting every logit by a
    constant changes nothing; the 3/4 : 1/4 closed form; duplicate or out-of-range ids are
    rejected."""
    rng = np.random.default_rng(9)
    for _ in range(200):
        E = int(rng.integers(2, 80))
        k = int(rng.integers(1, min(E, 16) + 1))
        l = (rng.standard_normal(E) * 3).astype(np.float32)
        ids = rng.choice(E, k, replace=False).astype(np.int32)
        w = orc.set_weights(l, ids)
        assert np.allclose(w, scipy.special.softmax(l[ids].astype(np.float64)), rtol=1e-13, atol=0)
        w2 = orc.set_weights((l.astype(np.float64) + 0.5).astype(np.float32), ids)
        assert np.allclose(w, w2, rtol=1e-6, atol=0)
    l = np.array([-50.0, math.log(3.0), 0.0, -50.0], np.float32)
    r = math.exp(float(np.float32(math.log(3.0))))
    w = orc.set_weights(l, [2, 1])
    assert abs(w[0] - 1 / (r + 1)) < 1e-15 and abs(w[1] - r / (r + 1)) < 1e-15
    for bad in ([1, 1], [0, 4], [-1, 2]):
        with pytest.raises(ValueError):
            orc.set_weights(l, bad)


def test_near_tie_selections(orc):
    """A token with no logit near its k-th admits exactly the oracle's selection; two logits
    tied at the k-th place admit both choices, each with its own renormalised weights; a band
    of three logits competing for two places admits the three pairs."""
    l = np.array([4.0, 1.0, 3.0, 0.0, 2.0], np.float32)
    sels = orc.near_tie_selections(l, 2)
    assert len(sels) == 1 and sels[0][0].tolist() == [0, 2]
    l = np.array([5.0, 2.0, 3.0, 3.0, 0.0], np.float32)
    sels = orc.near_tie_selections(l, 2)
    assert [s.tolist() for s, _ in sels] == [[0, 2], [0, 3]]
    for s, w in sels:
        assert np.allclose(w, scipy.special.softmax(l[s].astype(np.float64)), rtol=1e-13, atol=0)
    l = np.array([1.0, 1.0 + 2e-6, 9.0, 1.0 + 4e-6], np.float32)
    sels = orc.near_tie_selections(l, 3)
    assert sorted(tuple(sorted(s.tolist())) for s, _ in sels) == [(0, 1, 2), (0, 2, 3), (1, 2, 3)]
    assert all(s[0] == 2 for s, _ in sels)


# --- permutation plan ---------------------------------------------------------------------

def test_plan_histogram_2k_tokens(orc):
    """2,048 tokens routed to 8 of 256 experts give 16,384 assignments, 64 rows
    per expert on average ("Optimizing on-device inference for Apple Silicon",
    section "Match tile size to expert load")."""
    rng = np.random.default_rng(8)
    T, k, E = 2048, 8, 256
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    counts, offsets, sorted_slot = orc.plan(ids, E)
    assert counts.sum() == 16384 and counts.mean() == 64.0
    assert np.array_equal(counts, np.bincount(ids.ravel(), minlength=E))
    assert offsets[0] == 0 and offsets[-1] == T * k and np.all(np.diff(offsets) == counts)
    assert np.array_equal(np.sort(sorted_slot), np.arange(T * k))
    flat = ids.ravel()
    for e in range(E):
        grp = sorted_slot[offsets[e]:offsets[e + 1]]
        assert np.all(flat[grp] == e)
        assert np.all(np.diff(grp) > 0)   # stable: ascending slot order


def test_distinct_experts_bounded_by_tokens_times_k(orc):
    """One token touches k experts; a 4-token window touches at most 4k = 32
    ("Three ways to boost mixture-of-experts inference on NVIDIA DGX Spark",
    section "Optimization 3").  The verify bias recipe hits exactly d."""
    for d in (8, 20, 24, 28, 32):
        L, x = synth.make_layer(4, 64, 512, 8, 32, 0, "bf16", "bf16", "bf16", "bf16",
                                seed=d, bias="verify", d=d)
        lg = orc.logits(L, x)
        ids, _ = orc.select_all(lg, 8)
        assert len(set(ids.ravel().tolist())) == d <= min(32, 512)


# --- expert FFN and combine -----------------------------------------------------------------

def _np_w(a, dtype):
    if dtype == "f32":
        return a.astype(np.float64)
    if dtype == "bf16":
        return synth.bf16_bits_to_f32(a).astype(np.float64)
    raise ValueError(dtype)


def _np_mx(codes, scales):
    table = np.array([v for _, v in _read_table("e2m1_values.txt")], np.float64)
    lo = table[codes & 15]
    hi = table[codes >> 4]
    vals = np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)
    sc = np.ldexp(1.0, scales.astype(np.int64) - 127)
    return vals * np.repeat(sc, 32, axis=-1)


def _np_int4(codes, sc, bi):
    q = np.stack([codes & 15, codes >> 4], axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)
    s_ = synth.bf16_bits_to_f32(sc).astype(np.float64)
    b_ = synth.bf16_bits_to_f32(bi).astype(np.float64)
    return q * np.repeat(s_, 64, axis=-1) + np.repeat(b_, 64, axis=-1)


def _np_ffn(xv, Wg, Wu, Wd):
    g = Wg @ xv
    u = Wu @ xv
    a = g * scipy.special.expit(g) * u
    return Wd @ a


@pytest.mark.parametrize("dtype", ["f32", "bf16", "mxfp4", "int4g64"])
def test_single_expert_is_dense_swiglu(orc, dtype):
    """E = 1, k = 1, no shared expert: the layer is a dense SwiGLU FFN."""
    act = "f32" if dtype == "f32" else "bf16"
    L, x = synth.make_layer(3, 128, 1, 1, 64, 0, act, dtype, "bf16", "f32", seed=9)
    y, ids, w, _ = orc.forward(L, x)
    assert np.all(ids == 0) and np.all(w == 1.0)
    xs = _np_w(x, act)
    if dtype == "mxfp4":
        Wg, Wu, Wd = _np_mx(L.gate, L.gate_s)[0], _np_mx(L.up, L.up_s)[0], _np_mx(L.down, L.down_s)[0]
    elif dtype == "int4g64":
        Wg, Wu, Wd = (_np_int4(L.gate, L.gate_s, L.gate_b)[0], _np_int4(L.up, L.up_s, L.up_b)[0],
                      _np_int4(L.down, L.down_s, L.down_b)[0])
    else:
        Wg, Wu, Wd = _np_w(L.gate[0], dtype), _np_w(L.up[0], dtype), _np_w(L.down[0], dtype)
    for t in range(3):
        want = _np_ffn(xs[t], Wg, Wu, Wd)
        assert np.allclose(y[t], want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def test_combine_is_weighted_sum_plus_shared(orc):
    """With routing given, y = sum_j w_j FFN_{e_j}(x) + FFN_shared(x)."""
    L, x = synth.make_layer(2, 64, 6, 3, 32, 48, "bf16", "bf16", "bf16", "bf16", seed=10)
    ids = np.array([[4, 0, 2], [1, 5, 3]], np.int32)
    cw = np.array([[0.5, 0.3, 0.2], [0.7, 0.2, 0.1]])
    y = orc.forward_with_routing(L, x, ids, cw)
    xs = _np_w(x, "bf16")
    for t in range(2):
        want = sum(cw[t, j] * _np_ffn(xs[t], _np_w(L.gate[ids[t, j]], "bf16"), _np_w(L.up[ids[t, j]], "bf16"),
                                      _np_w(L.down[ids[t, j]], "bf16")) for j in range(3))
        want = want + _np_ffn(xs[t], _np_w(L.sh_gate, "bf16"), _np_w(L.sh_up, "bf16"), _np_w(L.sh_down, "bf16"))
        assert np.allclose(y[t], want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def test_shared_expert_is_additive(orc):
    L, x = synth.make_layer(2, 64, 8, 2, 32, 32, "bf16", "bf16", "bf16", "bf16", seed=11)
    y, *_ = orc.forward(L, x)
    no_shared = L.with_T(2)
    no_shared.I_shared = 0
    y0, *_ = orc.forward(no_shared, x)
    xs = _np_w(x, "bf16")
    for t in range(2):
        s = _np_ffn(xs[t], _np_w(L.sh_gate, "bf16"), _np_w(L.sh_up, "bf16"), _np_w(L.sh_down, "bf16"))
        assert np.allclose(y[t] - y0[t], s, rtol=1e-11, atol=1e-12 * np.abs(s).max())
    # zero routed output projections leave only the shared expert
    zd = L.with_T(2)
    zd.down = np.zeros_like(L.down)
    yz, *_ = orc.forward(zd, x)
    for t in range(2):
        s = _np_ffn(xs[t], _np_w(L.sh_gate, "bf16"), _np_w(L.sh_up, "bf16"), _np_w(L.sh_down, "bf16"))
        assert np.allclose(yz[t], s, rtol=1e-12, atol=1e-12 * np.abs(s).max())


def test_expert_storage_permutation_invariance(orc):
    """Relabelling experts (router rows, bias columns and weight stacks permuted
    together) maps the chosen ids exactly and leaves y unchanged up to the
    rounding of the softmax denominator (its sum over all E runs in storage
    order)."""
    L, x = synth.make_layer(4, 64, 12, 3, 32, 32, "bf16", "bf16", "bf16", "bf16", seed=12,
                            bias="verify", d=8)
    y, ids, w, _ = orc.forward(L, x)
    rng = np.random.default_rng(13)
    perm = rng.permutation(12)          # new expert n is old expert perm[n]
    inv = np.argsort(perm)
    P = L.with_T(4)
    P.router_w = np.ascontiguousarray(L.router_w[perm])
    P.router_bias = np.ascontiguousarray(L.router_bias[:, perm])
    P.gate = np.ascontiguousarray(L.gate[perm])
    P.up = np.ascontiguousarray(L.up[perm])
    P.down = np.ascontiguousarray(L.down[perm])
    yp, idp, wp, _ = orc.forward(P, x)
    assert np.array_equal(inv[ids], idp)
    assert np.allclose(w, wp, rtol=1e-15, atol=0)
    assert np.allclose(y, yp, rtol=1e-14, atol=1e-14 * np.abs(y).max())


def test_token_independence(orc):
    L, x = synth.make_layer(4, 64, 16, 4, 32, 32, "bf16", "bf16", "bf16", "bf16", seed=14)
    y, *_ = orc.forward(L, x)
    for t in range(4):
        yt, *_ = orc.forward(L.with_T(1), np.ascontiguousarray(x[t:t + 1]))
        assert np.array_equal(y[t:t + 1], yt)


def test_unselected_experts_are_never_read(orc):
    """NaN-poisoning every expert the router did not pick leaves y finite."""
    L, x = synth.make_layer(2, 64, 16, 2, 32, 32, "bf16", "bf16", "bf16", "bf16", seed=15)
    y, ids, *_ = orc.forward(L, x)
    P = L.with_T(2)
    nan16 = np.uint16(0x7FC0)
    P.gate, P.up, P.down = L.gate.copy(), L.up.copy(), L.down.copy()
    for e in set(range(16)) - set(ids.ravel().tolist()):
        P.gate[e] = nan16
        P.up[e] = nan16
        P.down[e] = nan16
    yp, *_ = orc.forward(P, x)
    assert np.all(np.isfinite(yp)) and np.array_equal(y, yp)


def test_hand_worked_example(orc):
    """T=1, H=2, E=3, k=2, I=I_s=1, fp32, worked by hand.
    x = (1, 0); router rows (2,0), (1,0), (0,0) -> logits 2, 1, 0 -> picks 0, 1
    with weights e^2/(e^2+e) and e/(e^2+e).  Expert e has gate row (1, 0), up row
    (e+1, 0), down column (1, -1): g = 1, u = e+1, a = silu(1)(e+1),
    o = a * (1, -1).  Shared: gate (2,0), up (1,0), down (0.5, 0.5): a = silu(2)."""
    f = np.float32
    L = synth.Layer(1, 2, 3, 2, 1, 1, "f32", "f32", "f32", "f32",
                    np.array([[2, 0], [1, 0], [0, 0]], f))
    L.gate = np.array([[[1, 0]]] * 3, f)
    L.up = np.array([[[1, 0]], [[2, 0]], [[3, 0]]], f)
    L.down = np.array([[[1], [-1]]] * 3, f)
    L.sh_gate = np.array([[2, 0]], f)
    L.sh_up = np.array([[1, 0]], f)
    L.sh_down = np.array([[0.5], [0.5]], f)
    x = np.array([[1, 0]], f)
    y, ids, w, lg = orc.forward(L, x)
    s1 = 1 / (1 + math.exp(-1))
    s2 = 2 / (1 + math.exp(-2))
    w0 = math.e ** 2 / (math.e ** 2 + math.e)
    w1 = math.e / (math.e ** 2 + math.e)
    routed = w0 * s1 * 1 + w1 * s1 * 2
    want = [routed + 0.5 * s2, -routed + 0.5 * s2]
    assert ids.tolist() == [[0, 1]] and lg.tolist() == [[2.0, 1.0, 0.0]]
    assert np.allclose(w[0], [w0, w1], rtol=1e-15)
    assert np.allclose(y[0], want, rtol=1e-14)


# --- MXFP8 activations (W4A8) -----------------------------------------------------------------

def test_e4m3_decode_matches_torch_float8(orc):
    """All 256 E4M3 codes against torch's float8_e4m3fn (an independent library decoder)."""
    import torch
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for c in range(256):
        assert _same(orc.e4m3_to_double(c), float(ref[c])), hex(c)
    assert orc.e4m3_to_double(0x7E) == 448.0 and orc.e4m3_to_double(0x08) == 2.0 ** -6
    assert orc.e4m3_to_double(0x01) == 2.0 ** -9 and math.isnan(orc.e4m3_to_double(0xFF))


def test_e4m3_rounding_matches_torch_and_saturates(orc):
    """In range, the encoder rounds like torch's float -> float8_e4m3fn cast (nearest, ties to
    even), exact midpoints and subnormals included; beyond 448 it saturates (the cast would give
    NaN there)."""
    import torch
    rng = np.random.default_rng(21)
    grid = torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    mids = (grid[1:] + grid[:-1]) / 2                       # every tie between neighbours
    vals = np.concatenate([rng.uniform(-440, 440, 4000), rng.uniform(-2 ** -6, 2 ** -6, 2000),
                           mids, -mids, grid, [0.0, -0.0, 447.9, 448.0]])
    want = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for v, w in zip(vals, want):
        assert orc.e4m3_from_double(float(v)) == int(w), v
    for v in (448.0001, 463.9, 464.0, 500.0, 1e30):
        assert orc.e4m3_from_double(v) == 0x7E and orc.e4m3_from_double(-v) == 0xFE


def test_mxfp8_scale_rule_and_round_trip(orc):
    """The shared scale is 2^(floor(log2 amax) - 8): a block whose amax is 2^k gets e8m0 byte
    127 + k - 8 and its amax element becomes 256 (code 0x78); a block with amax in [1.75, 2) 2^k
    saturates its largest element to 448; a zero block gets byte 0 and zero codes; values on the
    grid (E4M3 codes times a power of two, the largest with exponent 8) round-trip exactly."""
    rng = np.random.default_rng(22)
    for k in (-20, -3, 0, 5, 30):
        v = rng.uniform(-1, 1, 32) * 2.0 ** k * 0.9
        v[7] = 2.0 ** k
        c, s = orc.mxfp8_quantize(v)
        assert s[0] == 127 + k - 8 and c[7] == 0x78
        v[7] = -1.9 * 2.0 ** k
        c, s = orc.mxfp8_quantize(v)
        assert s[0] == 127 + k - 8 and c[7] == 0xFE
    c, s = orc.mxfp8_quantize(np.zeros(64))
    assert np.all(s == 0) and np.all(c == 0)
    for trial in range(50):
        e = int(rng.integers(-30, 30))
        codes = rng.integers(0, 0x7F, 32).astype(np.uint8) | rng.choice([0, 0x80], 32).astype(np.uint8)
        codes[int(rng.integers(32))] = 0x78 + int(rng.integers(0, 7))   # largest element: exponent field 15 (2^8)
        v = np.array([orc.e4m3_to_double(int(b)) for b in codes]) * 2.0 ** e
        c, s = orc.mxfp8_quantize(v)
        back = orc.mxfp8_dequantize(c, s)
        assert s[0] == 127 + e and np.array_equal(back, v)


def test_w4a8_dense_expert_quantises_both_gemm_inputs(orc):
    """E = 1, k = 1, a shared expert: with MXFP8 activations the routed expert computes
    Wd Q(silu(Wg Q(x)) * (Wu Q(x))), Q the quantise-dequantise round trip (pinned above), with
    the MXFP4 weights decoded by the spec table; the shared expert is left unquantised.  Checked
    against numpy matmuls."""
    import dataclasses
    L, x = synth.make_layer(2, 128, 1, 1, 64, 32, "bf16", "mxfp4", "bf16", "f32", seed=23)
    Lq = dataclasses.replace(L, act_quant="mxfp8")
    y, ids, w, _ = orc.forward(Lq, x)
    xs = _np_w(x, "bf16")
    Wg, Wu, Wd = _np_mx(L.gate, L.gate_s)[0], _np_mx(L.up, L.up_s)[0], _np_mx(L.down, L.down_s)[0]
    Sg, Su, Sd = _np_w(L.sh_gate, "bf16"), _np_w(L.sh_up, "bf16"), _np_w(L.sh_down, "bf16")

    def q(v):
        return orc.mxfp8_dequantize(*orc.mxfp8_quantize(v))
    for t in range(2):
        xq = q(xs[t])
        g, u = Wg @ xq, Wu @ xq
        a = q(g * scipy.special.expit(g) * u)
        want = Wd @ a + _np_ffn(xs[t], Sg, Su, Sd)
        assert np.allclose(y[t], want, rtol=1e-12, atol=1e-12 * np.abs(want).max())
    y_plain = orc.forward(L, x)[0]
    rel = np.linalg.norm(y - y_plain) / np.linalg.norm(y_plain)
    assert 1e-3 < rel < 1e-1, rel    # the quantisation is there, and of the expected size
