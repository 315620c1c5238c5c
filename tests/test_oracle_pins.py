"""Pins of the fp64 oracle against facts it does not compute itself: a dense
brute force that never sorts, closed forms, special cases that reduce to
textbook routines, library implementations of the same functions and the
published E2M1 table.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st, HealthCheck

import moe_inputs as mi
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _inputs(T, H, E, k, I, seed=0, skew=False):
    return mi.make(mi.Shape(T=T, H=H, E=E, k=k, I=I, skew=skew), seed=seed)


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# ------------------------------------------------------------------ shape
def test_golden_layer_shape_matches_configs():
    g = json.load(open(os.path.join(GOLDEN, "gemma4_moe_layer.json")))
    for name in ("decode", "prefill", "skew", "mxfp4"):
        s = mi.CONFIGS[name]
        assert (s.H, s.E, s.k, s.I) == (g["hidden_size"], g["num_experts"],
                                        g["top_k"], g["moe_intermediate_size"])
    assert mi.CONFIGS["prefill"].T == g["prefill_batch"] * g["prefill_seq_len"]
    assert mi.CONFIGS["decode"].T == g["decode_batch"]
    assert g["activation"] == "gelu_pytorch_tanh"
    sh = mi.CONFIGS["decode_shared"]
    assert (sh.H, sh.E, sh.k, sh.I, sh.T) == (g["hidden_size"], g["num_experts"], g["top_k"],
                                              g["moe_intermediate_size"], g["decode_batch"])
    assert sh.I_sh == g["dense_mlp_intermediate_size"]


# ------------------------------------------------------------------ brute force
def test_dense_brute_force_tiny_config():
    inp = mi.make("tiny")
    r = oracle.forward(inp)
    d = oracle.dense_forward(inp)
    assert _rel(r["out"], d) <= 1e-12


def test_dense_brute_force_skewed_bias():
    inp = _inputs(24, 64, 12, 3, 32, seed=3, skew=True)
    r = oracle.forward(inp)
    assert _rel(r["out"], oracle.dense_forward(inp)) <= 1e-12


@settings(max_examples=12, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(T=st.integers(1, 40), E=st.integers(1, 16), kf=st.floats(0, 1),
       H=st.sampled_from([32, 64, 128]), I=st.sampled_from([32, 64, 128]),
       seed=st.integers(0, 1000))
def test_dense_brute_force_random_shapes(T, E, kf, H, I, seed):
    k = 1 + int(kf * (E - 1))
    inp = _inputs(T, H, E, k, I, seed=seed)
    r = oracle.forward(inp)
    assert _rel(r["out"], oracle.dense_forward(inp)) <= 1e-12


# ------------------------------------------------------------------ top-k
def _rank_count_topk(L, k):
    """Selection by counting, per expert, the experts that beat it."""
    T, E = L.shape
    sel = []
    for t in range(T):
        chosen = []
        for e in range(E):
            beats = sum(1 for e2 in range(E)
                        if L[t, e2] > L[t, e] or (L[t, e2] == L[t, e] and e2 < e))
            if beats < k:
                chosen.append((beats, e))
        sel.append([e for _, e in sorted(chosen)])
    return np.array(sel)


def test_topk_matches_rank_count_with_many_ties():
    rng = np.random.default_rng(5)
    L = rng.integers(-3, 4, size=(50, 16)).astype(np.float64)   # heavy ties
    for k in (1, 3, 8, 16):
        ids, w = oracle.topk_softmax(L, k)
        assert (ids == _rank_count_topk(L, k)).all()


def test_all_equal_logits_pick_lowest_indices_with_equal_weights():
    L = np.full((4, 128), 0.37)
    ids, w = oracle.topk_softmax(L, 8)
    assert (ids == np.arange(8)).all()
    assert (w == 1.0 / 8).all()


def test_negative_zero_ties_with_zero():
    L = np.array([[-0.0, 0.0, -1.0]])
    ids, _ = oracle.topk_softmax(L, 1)
    assert ids[0, 0] == 0


def test_k_equals_E_gives_full_softmax():
    rng = np.random.default_rng(1)
    L = rng.standard_normal((10, 12))
    ids, w = oracle.topk_softmax(L, 12)
    full = torch.softmax(torch.from_numpy(L), dim=1).numpy()
    for t in range(10):
        assert np.allclose(w[t], full[t, ids[t]], rtol=0, atol=1e-15)
        assert (np.diff(L[t, ids[t]]) <= 0).all()


def test_topk_weights_are_renormalised_full_softmax():
    rng = np.random.default_rng(2)
    L = rng.standard_normal((20, 128)) * 3
    ids, w = oracle.topk_softmax(L, 8)
    full = torch.softmax(torch.from_numpy(L), dim=1).numpy()
    for t in range(20):
        p = full[t, ids[t]]
        assert np.allclose(w[t], p / p.sum(), rtol=1e-13, atol=0)


def test_shift_invariance_and_weight_invariants():
    rng = np.random.default_rng(3)
    L = rng.standard_normal((64, 128))
    ids, w = oracle.topk_softmax(L, 8)
    ids2, w2 = oracle.topk_softmax(L + 11.5, 8)
    assert (ids == ids2).all()
    assert np.allclose(w, w2, rtol=1e-12, atol=0)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert (np.diff(w, axis=1) <= 0).all()
    assert all(len(set(r)) == 8 for r in ids)


def test_margin():
    L = np.array([[5.0, 1.0, 3.0, 2.0]])
    assert oracle.routing_margin(L, 2)[0] == 1.0
    assert np.isinf(oracle.routing_margin(L, 4)[0])


# ------------------------------------------------------------------ permutation
def test_permutation_invariants_and_round_trip():
    T, E, k, H = 300, 16, 4, 48
    ids = mi.random_ids(T, E, k, seed=4, p=np.arange(1, E + 1)[::-1] / np.arange(1, E + 1).sum())
    counts, offsets = oracle.counts_offsets(ids, E)
    sorted_ids, inv = oracle.permutation(ids)
    A = T * k
    assert counts.sum() == A and offsets[0] == 0 and offsets[E] == A
    assert (np.diff(offsets) == counts).all()
    assert (np.bincount(ids.reshape(-1), minlength=E) == counts).all()
    assert sorted(sorted_ids.tolist()) == list(range(A))
    assert (inv[sorted_ids] == np.arange(A)).all()
    flat = ids.reshape(-1)
    for e in range(E):
        seg = sorted_ids[offsets[e]:offsets[e + 1]]
        assert (flat[seg] == e).all()
        assert (np.diff(seg // k) > 0).all()          # stable in token order
    tok_count = np.bincount(sorted_ids // k, minlength=T)
    assert (tok_count == k).all()                      # each token exactly k times
    x = mi.random_bf16((T, H), seed=9)
    x_perm = x[sorted_ids // k]
    back = x_perm[inv].reshape(T, k, H)
    assert (back == x[:, None, :]).all()               # bitwise round trip


def test_empty_experts_and_single_hot_expert():
    ids = np.tile(np.array([[0, 5]], dtype=np.int32), (7, 1))
    counts, offsets = oracle.counts_offsets(ids, 8)
    assert counts.tolist() == [7, 0, 0, 0, 0, 7, 0, 0]
    assert offsets.tolist() == [0, 7, 7, 7, 7, 7, 14, 14, 14]


# ------------------------------------------------------------------ GELU
def test_gelu_tanh_matches_torch_and_limits():
    z = np.linspace(-12, 12, 4001)
    ref = torch.nn.functional.gelu(torch.from_numpy(z), approximate="tanh").numpy()
    assert np.abs(oracle.gelu_tanh(z) - ref).max() <= 1e-14
    assert oracle.gelu_tanh(0.0) == 0.0
    assert oracle.gelu_tanh(40.0) == 40.0             # tanh saturates to 1
    assert oracle.gelu_tanh(-40.0) == 0.0
    exact = 0.5 * z * (1 + np.vectorize(math.erf)(z / math.sqrt(2)))
    assert np.abs(oracle.gelu_tanh(z) - exact).max() < 1e-3   # tanh form approximates erf form


# ------------------------------------------------------------------ layer special cases
def test_zero_input_gives_zero_output():
    inp = _inputs(5, 64, 6, 2, 32)
    inp.x[:] = 0
    assert (oracle.forward(inp)["out"] == 0).all()


def test_single_expert_is_a_dense_geglu_ffn():
    inp = _inputs(9, 64, 1, 1, 32, seed=7)
    r = oracle.forward(inp)
    x = torch.from_numpy(mi.bf16_bits_to_f32(inp.x).astype(np.float64))
    wgu = torch.from_numpy(mi.bf16_bits_to_f32(inp.w_gate_up[0]).astype(np.float64))
    wd = torch.from_numpy(mi.bf16_bits_to_f32(inp.w_down[0]).astype(np.float64))
    gate = torch.nn.functional.linear(x, wgu[:32])
    up = torch.nn.functional.linear(x, wgu[32:])
    ref = torch.nn.functional.linear(torch.nn.functional.gelu(gate, approximate="tanh") * up, wd)
    assert (r["w"] == 1.0).all()
    assert _rel(r["out"], ref.numpy()) <= 1e-13


def _bits(v):
    return mi.f32_to_bf16_bits(np.asarray(v, dtype=np.float32))


def test_gate_is_first_half_closed_form():
    """One token, H=2, two experts, k=2, I=1, weights chosen so every step has
    an exact closed form.  x = (8, 1).  Router rows make the logits (1, 0).
    Expert e: gate row (4, 0) -> gate pre-activation 32, gelu_tanh(32) = 32
    exactly in fp64; up row (0, u_e) -> up = u_e; down column d_e.  So
    Y_e = 32 u_e d_e and out = w0 Y_0 + w1 Y_1 with w0 = 1/(1+e^-1).
    Swapping gate and up would give gelu_tanh(u_e) * 32 instead."""
    s = mi.Shape(T=1, H=2, E=2, k=2, I=1)
    u = [0.5, -2.0]
    d = [[1.0, 0.25], [-0.5, 2.0]]
    inp = mi.Inputs(
        shape=s, seed=0,
        x=_bits([[8.0, 1.0]]),
        w_router=_bits([[0.125, 0.0], [0.0, 0.0]]),
        router_bias=None,
        w_gate_up=_bits([[[4.0, 0.0], [0.0, u[0]]], [[4.0, 0.0], [0.0, u[1]]]]),
        w_down=_bits([[[d[0][0]], [d[0][1]]], [[d[1][0]], [d[1][1]]]]),
    )
    r = oracle.forward(inp)
    w0 = 1.0 / (1.0 + math.exp(-1.0))
    w1 = 1.0 - w0
    expect = np.array([w0 * 32 * u[0] * d[0][0] + w1 * 32 * u[1] * d[1][0],
                       w0 * 32 * u[0] * d[0][1] + w1 * 32 * u[1] * d[1][1]])
    assert r["ids"].tolist() == [[0, 1]]
    assert np.allclose(r["w"][0], [w0, w1], rtol=1e-15, atol=0)
    assert np.allclose(r["out"][0], expect, rtol=1e-14, atol=0)


def test_forward_tokens_matches_forward():
    inp = _inputs(40, 64, 10, 3, 32, seed=11)
    r = oracle.forward(inp)
    sample = [0, 7, 39, 21]
    f = oracle.forward_tokens(inp, sample)
    assert (f["ids"] == r["ids"][sample]).all()
    assert _rel(f["out"], r["out"][sample]) <= 1e-13


def test_fp32_routing_override():
    inp = _inputs(30, 64, 10, 3, 32, seed=12)
    r = oracle.forward(inp)
    L32 = r["logits"].astype(np.float32)
    r32 = oracle.forward(inp, logits_fp32=L32)
    assert (r32["route_logits"] == L32.astype(np.float64)).all()


# ------------------------------------------------------------------ MXFP4
def _golden_e2m1():
    vals = {}
    for line in open(os.path.join(GOLDEN, "ocp_mx_e2m1.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        c, v = line.split()
        vals[int(c, 16)] = float(v)
    return vals


def test_mxfp4_decodes_every_code_to_the_published_table():
    table = _golden_e2m1()
    assert len(table) == 16
    for s in (127, 100, 140, 120):
        codes = np.arange(16, dtype=np.uint8)
        packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
        packed = np.tile(packed, 4)                     # 32 elements, one block
        scales = np.array([s], dtype=np.uint8)
        v = oracle.mxfp4_to_f64(packed, scales)
        for c in range(16):
            expect = table[c] * 2.0 ** (s - 127)
            assert v[c] == expect and np.signbit(v[c]) == (c >= 8)
    with pytest.raises(ValueError):
        oracle.mxfp4_to_f64(np.zeros(16, np.uint8), np.array([255], np.uint8))


def test_mxfp4_quantiser_round_trip_and_bf16_exactness():
    w = mi.random_bf16((6, 128), sigma=0.02, seed=8)
    packed, scales = mi.mxfp4_quantize(w)
    deq = oracle.mxfp4_to_f64(packed, scales)
    wf = mi.bf16_bits_to_f32(w).astype(np.float64)
    step = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1)
    # every element within half a grid step of the largest spacing (2 * scale)
    # unless saturated at 6 * scale
    sat = np.abs(wf) > 6 * step
    assert (np.abs(deq - wf)[~sat] <= step[~sat] + 0).all()
    assert (np.abs(deq[sat]) == 6 * step[sat]).all()
    # every decoded weight is exactly a bf16 value
    assert (mi.bf16_bits_to_f32(mi.f32_to_bf16_bits(deq.astype(np.float32))) == deq).all()
    # re-quantising the decoded weights reproduces the codes
    p2, s2 = mi.mxfp4_quantize(mi.f32_to_bf16_bits(deq.astype(np.float32)))
    assert (oracle.mxfp4_to_f64(p2, s2) == deq).all()


def test_mxfp4_tie_rounding_is_nearest_even():
    table = _golden_e2m1()
    # block max 4.0 -> scale 2^0; the midpoints 0.25, .75, 1.25, 1.75, 2.5, 3.5, 5
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    expect = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    row = np.zeros(32, dtype=np.float32)
    row[0] = 4.0
    row[1:8] = mids
    row[8:15] = [-m for m in mids]
    p, s = mi.mxfp4_quantize(mi.f32_to_bf16_bits(row)[None, :])
    v = oracle.mxfp4_to_f64(p, s)[0]
    assert s[0, 0] == 127
    assert v[1:8].tolist() == expect
    assert v[8:15].tolist() == [-e for e in expect]
    assert set(table.values()) >= set(abs(x) for x in expect)


def test_router_logits_match_torch_linear_with_bias():
    inp = _inputs(12, 64, 10, 3, 32, seed=13, skew=True)
    x = torch.from_numpy(mi.bf16_bits_to_f32(inp.x).astype(np.float64))
    W = torch.from_numpy(mi.bf16_bits_to_f32(inp.w_router).astype(np.float64))
    b = torch.from_numpy(inp.router_bias.astype(np.float64))
    ref = torch.nn.functional.linear(x, W, b).numpy()
    got = oracle.router_logits(oracle.bf16_to_f64(inp.x), oracle.bf16_to_f64(inp.w_router), inp.router_bias)
    assert np.allclose(got, ref, rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------- O10 dense MLP
def _torch_geglu_mlp(x_bits, gu_bits, d_bits):
    """Textbook dense GEGLU MLP from torch.nn.functional in float64."""
    x = torch.from_numpy(mi.bf16_bits_to_f32(x_bits).astype(np.float64))
    wgu = torch.from_numpy(mi.bf16_bits_to_f32(gu_bits).astype(np.float64))
    wd = torch.from_numpy(mi.bf16_bits_to_f32(d_bits).astype(np.float64))
    I = wgu.shape[0] // 2
    gate = torch.nn.functional.linear(x, wgu[:I])
    up = torch.nn.functional.linear(x, wgu[I:])
    return torch.nn.functional.linear(torch.nn.functional.gelu(gate, approximate="tanh") * up, wd).numpy()


def _without_shared(inp):
    import dataclasses
    return dataclasses.replace(inp, shape=dataclasses.replace(inp.shape, I_sh=0), w_sh_gate_up=None,
                               w_sh_down=None, sh_gu_scales=None, sh_d_scales=None)


def test_shared_mlp_adds_a_textbook_geglu_mlp():
    """forward with a dense MLP = forward without it + the torch GEGLU MLP."""
    s = mi.Shape(T=11, H=64, E=6, k=2, I=32, I_sh=96)
    inp = mi.make(s, seed=5)
    with_sh = oracle.forward(inp)["out"]
    without = oracle.forward(_without_shared(inp))["out"]
    mlp = _torch_geglu_mlp(inp.x, inp.w_sh_gate_up, inp.w_sh_down)
    assert _rel(with_sh - without, mlp) <= 1e-13
    assert np.abs(mlp).max() > 0
    # the brute force and the token-by-token path include it the same way
    assert _rel(oracle.dense_forward(inp), with_sh) <= 1e-12
    assert _rel(oracle.forward_tokens(inp, [0, 4, 10])["out"], with_sh[[0, 4, 10]]) <= 1e-13


def test_zero_shared_weights_change_nothing():
    s = mi.Shape(T=7, H=64, E=5, k=2, I=32, I_sh=64)
    inp = mi.make(s, seed=6)
    inp.w_sh_gate_up = np.zeros_like(inp.w_sh_gate_up)
    assert (oracle.forward(inp)["out"] == oracle.forward(_without_shared(inp))["out"]).all()


def test_shared_mlp_mxfp4_matches_its_decoded_weights():
    """MXFP4 dense weights: the oracle's MLP equals the torch MLP on the
    decoded (bf16-exact) weights."""
    s = mi.Shape(T=6, H=64, E=4, k=2, I=32, I_sh=64, mxfp4=True)
    inp = mi.make(s, seed=8)
    gu = oracle.mxfp4_to_f64(inp.w_sh_gate_up, inp.sh_gu_scales)
    d = oracle.mxfp4_to_f64(inp.w_sh_down, inp.sh_d_scales)
    ref = _torch_geglu_mlp(inp.x, mi.f32_to_bf16_bits(gu.astype(np.float32)), mi.f32_to_bf16_bits(d.astype(np.float32)))
    assert (mi.bf16_bits_to_f32(mi.f32_to_bf16_bits(gu.astype(np.float32))) == gu).all()   # exact in bf16
    got = oracle.shared_mlp(oracle.bf16_to_f64(inp.x), oracle.shared_weights(inp))
    assert _rel(got, ref) <= 1e-13


# ---------------------------------------------------------------- O11 W4A4
def test_mx_quantizer_matches_scalar_rule_and_generator_encoder():
    """The vectorised quantiser against the one-value rule, and against the
    generator's independent encoder of the same OCP conversion."""
    from oracle import moe_oracle as om
    rng = np.random.default_rng(3)
    v = (rng.standard_normal((40, 96)) * np.exp(rng.uniform(-6, 6, (40, 1)))).astype(np.float32)
    v = mi.bf16_bits_to_f32(mi.f32_to_bf16_bits(v)).astype(np.float64)
    codes, scales = oracle.mx_quantize(v)
    for r in range(0, 40, 7):
        for b in range(3):
            e = int(scales[r, b]) - 127
            for i in range(32):
                assert codes[r, 32 * b + i] == om._e2m1_code(v[r, 32 * b + i] / 2.0 ** e)
    packed, gscales = mi.mxfp4_quantize(mi.f32_to_bf16_bits(v.astype(np.float32)))
    assert (gscales == scales).all()
    assert (packed == (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)).all()


def test_mx_quantizer_representable_values_ties_saturation_zero():
    # every E2M1 value times a block scale that the block's amax selects comes back exactly
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    rng = np.random.default_rng(4)
    for e in (-10, 0, 7):
        blk = rng.choice(np.concatenate([grid, -grid]), size=32)
        blk[5] = 6.0                                   # amax 6 * 2^e -> exponent e
        vals = blk * 2.0 ** e
        c, s = oracle.mx_quantize(vals[None])
        assert s[0, 0] == e + 127
        assert (oracle.mx_dequantize(c, s)[0] == vals).all()
    # amax 7.9: floor(log2 7.9) = 2 -> exponent 0, so the values keep their
    # size; every midpoint goes to its even code and 7.9 saturates at 6
    blk = np.zeros(32)
    blk[:9] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.9, 4.0]
    c, s = oracle.mx_quantize(blk[None])
    assert s[0, 0] == 127
    assert c[0, :9].tolist() == [0, 2, 2, 4, 4, 6, 6, 7, 6]
    # amax 8 -> exponent 1: 8 / 2 = 4 (code 6), 4 / 2 = 2 (code 4)
    blk[7] = 8.0
    c, s = oracle.mx_quantize(blk[None])
    assert s[0, 0] == 128 and c[0, 7] == 6 and c[0, 8] == 4
    # zero block: scale byte 127, codes 0; negative zero keeps its sign bit
    z = np.zeros((1, 32))
    z[0, 3] = -0.0
    cz, sz = oracle.mx_quantize(z)
    assert sz[0, 0] == 127 and cz[0, 3] == 8 and cz[0, 0] == 0


def test_w4a4_single_expert_is_a_quantised_textbook_ffn():
    """E = 1, k = 1, W4A4: the torch GEGLU FFN on the quantised x, with h
    rounded to bf16 and quantised before the down projection."""
    s = mi.Shape(T=6, H=64, E=1, k=1, I=64, mxfp4=True, a4=True)
    inp = mi.make(s, seed=12)
    r = oracle.forward(inp)
    xq = torch.from_numpy(oracle.mx_round(oracle.bf16_to_f64(inp.x)))
    wgu = torch.from_numpy(oracle.mxfp4_to_f64(inp.w_gate_up[0], inp.gu_scales[0]))
    wd = torch.from_numpy(oracle.mxfp4_to_f64(inp.w_down[0], inp.d_scales[0]))
    g = torch.nn.functional.linear(xq, wgu[:64])
    u = torch.nn.functional.linear(xq, wgu[64:])
    h = torch.nn.functional.gelu(g, approximate="tanh") * u
    hq = torch.from_numpy(oracle.mx_round(oracle.round_to_bf16(h.numpy())))
    ref = torch.nn.functional.linear(hq, wd).numpy()
    assert _rel(r["out"], ref) <= 1e-13
    # quantising the activations changes the result (the path is exercised)
    plain = oracle.forward(mi.make(mi.Shape(T=6, H=64, E=1, k=1, I=64, mxfp4=True), seed=12))["out"]
    assert _rel(plain, ref) > 1e-4


def test_round_to_bf16_matches_torch():
    rng = np.random.default_rng(5)
    v = rng.standard_normal(1000) * np.exp(rng.uniform(-20, 20, 1000))
    ref = torch.from_numpy(v).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert (oracle.round_to_bf16(v) == ref).all()


# ------------------------------------------------------------------ NVFP4 (O12)
def _golden_e4m3():
    vals = {}
    for line in open(os.path.join(GOLDEN, "ocp_fp8_e4m3.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            c, v = line.split()
            vals[int(c, 16)] = float(v)
    return vals


def test_e4m3_table_matches_published_landmarks_and_torch():
    t = oracle.e4m3_to_f64(np.arange(256))
    for c, v in _golden_e4m3().items():
        assert t[c] == v
    # torch's float8_e4m3fn decoding (an independent implementation of the
    # same OCP format) agrees on every finite code; 0x7F and 0xFF are NaN
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    fin = ~np.isnan(ref)
    assert fin.sum() == 254
    assert (t[fin] == ref[fin]).all()
    assert np.isnan(t[~fin]).all()
    assert np.signbit(t[0x80]) and t[0x80] == 0.0


def test_nvfp4_decode_hand_built_row():
    e2m1 = _golden_e2m1()
    # one row of K = 32: two 16-element blocks; codes 0..15 in each block
    codes = np.arange(32, dtype=np.uint8) % 16
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    scales = np.array([0x38, 0x3C], dtype=np.uint8)      # 1.0 and 1.5
    v = oracle.nvfp4_to_f64(packed, scales, np.float32(0.25))
    for i in range(32):
        s = 1.0 if i < 16 else 1.5
        assert v[i] == e2m1[i % 16] * s * 0.25
    # the per-matrix scale is taken as fp32
    v2 = oracle.nvfp4_to_f64(packed, scales, 0.1)
    assert v2[2] == e2m1[2] * 1.0 * float(np.float32(0.1))
    with pytest.raises(ValueError):
        oracle.nvfp4_to_f64(packed, np.array([0x7F, 0x38], np.uint8), 1.0)


def test_nvfp4_element_times_block_scale_is_exact_in_bf16():
    # every E2M1 value times every finite E4M3 value has at most 6
    # significant bits and lies inside bf16's normal range: exactly a bf16
    e2m1 = np.array(sorted(_golden_e2m1().values()))
    sc = oracle.e4m3_to_f64(np.arange(0x7F))
    prod = (e2m1[:, None] * sc[None, :]).ravel()
    assert (oracle.round_to_bf16(prod) == prod).all()


def test_nvfp4_quantiser_round_trip_on_grid_values():
    # weights that are exactly element x block scale x matrix scale, with one
    # element per block at 6 x block scale, come back unchanged
    rng = np.random.default_rng(5)
    rows, K = 6, 64
    g = 2.0 ** -12            # a power of two keeps every product a bf16 value
    sc_codes = rng.integers(0x20, 0x60, size=(rows, K // 16))
    sc = oracle.e4m3_to_f64(sc_codes)
    e2m1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    el = e2m1[rng.integers(0, 8, size=(rows, K))] * rng.choice([-1.0, 1.0], size=(rows, K))
    el.reshape(rows, K // 16, 16)[:, :, 0] = 6.0
    sc[0, 0] = oracle.e4m3_to_f64(np.array([0x7E]))[0]     # the matrix max: 6 * 448 * g
    w = (el.reshape(rows, K // 16, 16) * sc[..., None]).reshape(rows, K) * g
    bits = mi.f32_to_bf16_bits(w.astype(np.float32))
    assert (mi.bf16_bits_to_f32(bits).astype(np.float64) == w).all()
    packed, s_codes, glob = mi.nvfp4_quantize(bits)
    assert glob == np.float32(g)
    back = oracle.nvfp4_to_f64(packed, s_codes, glob)
    assert (back == w).all()


def test_nvfp4_quantiser_error_bound():
    w = mi.random_bf16((8, 256), sigma=0.02, seed=9)
    packed, s_codes, glob = mi.nvfp4_quantize(w)
    deq = oracle.nvfp4_to_f64(packed, s_codes, glob)
    wf = mi.bf16_bits_to_f32(w).astype(np.float64)
    step = np.repeat(oracle.e4m3_to_f64(s_codes), 16, axis=1) * float(glob)
    sat = np.abs(wf) > 6 * step
    # within half the largest element spacing (2 x block step) of each value
    assert (np.abs(deq - wf)[~sat] <= step[~sat]).all()
    # a block's scale is its amax / 6 rounded to E4M3: the saturated excess is
    # at most the E4M3 rounding (relative 2^-4)
    assert (np.abs(wf[sat]) <= 6 * step[sat] * (1 + 2.0 ** -4)).all()


def test_nvfp4_single_expert_is_a_dense_geglu_ffn_on_decoded_weights():
    s = mi.Shape(T=5, H=64, E=1, k=1, I=32, nvfp4=True)
    inp = mi.make(s, seed=4)
    wgu, wd = oracle.expert_weights(inp, 0)
    assert wgu.shape == (64, 64) and wd.shape == (64, 32)
    x = torch.tensor(oracle.bf16_to_f64(inp.x))
    g = torch.tensor(wgu)
    h = torch.nn.functional.gelu(x @ g[:32].T, approximate="tanh") * (x @ g[32:].T)
    ref = (h @ torch.tensor(wd).T).numpy()
    out = oracle.forward(inp)["out"]
    assert _rel(out, ref) < 1e-12


# ------------------------------------------------------------------ NVFP4 activations (O13)
def _e4m3_midpoints():
    """Every value the E4M3 rounding must decide: the finite non-negative
    grid, the midpoints between neighbours, and values just off them."""
    grid = oracle.e4m3_to_f64(np.arange(127))
    mids = (grid[:-1] + grid[1:]) / 2
    return grid, mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf)


def test_e4m3_nearest_matches_torch_rounding_below_saturation():
    """torch's float8_e4m3fn cast rounds to the nearest even code; it agrees
    on the grid, every midpoint (ties to even) and random values up to the
    saturation point (the cast overflows to NaN from 464 on, where E4M3
    saturates at 448 by the OCP conversion)."""
    grid, mids, up, down = _e4m3_midpoints()
    rng = np.random.default_rng(1)
    rand = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(460.0), 4000))
    v = np.concatenate([grid, mids, up, down, rand, [0.0, 2.0 ** -10, 3 * 2.0 ** -11]])
    v = v[v < 464.0].astype(np.float32).astype(np.float64)      # the fp32 values a kernel rounds
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (oracle.e4m3_nearest(v) == ref).all()


def test_e4m3_nearest_saturation_and_generator_encoder():
    assert oracle.e4m3_nearest(np.array([448.0, 460.0, 464.0, 1e6, np.inf])).tolist() == [0x7E] * 5
    assert oracle.e4m3_nearest(np.array([0.0, 2.0 ** -9, 2.0 ** -10])).tolist() == [0, 1, 0]   # tie -> even
    # the generator's independently written encoder (arithmetic on the
    # exponent and mantissa) agrees everywhere it is defined
    grid, mids, up, down = _e4m3_midpoints()
    v = np.concatenate([grid, mids, up, down, [500.0, 1e4]])
    assert (oracle.e4m3_nearest(v) == mi.e4m3_encode(v)).all()


def _nv_scalar(block, g):
    """One 16-value block by the rule written out per value: fp32 amax, scale
    through the generator's E4M3 encoder, E2M1 through the scalar rule."""
    from oracle import moe_oracle as om
    f32 = np.float32
    amax = max(abs(f32(v)) for v in block)
    s = f32(amax) / (f32(6.0) * f32(g))
    sc = int(mi.e4m3_encode(np.array([float(s)]))[0])
    step = f32(oracle.e4m3_to_f64(sc)) * f32(g)
    if step == 0:
        return [0] * len(block), sc
    return [om._e2m1_code(float(f32(v) / step)) for v in block], sc


def test_nv_quantizer_matches_scalar_rule():
    rng = np.random.default_rng(3)
    rows = rng.standard_normal((6, 64)) * np.exp(rng.uniform(-6, 3, (6, 1)))
    rows = mi.bf16_bits_to_f32(mi.f32_to_bf16_bits(rows.astype(np.float32))).astype(np.float64)
    for g in (2.0 ** -8, 0.0037, 1.0):
        codes, sc = oracle.nv_quantize(rows, g)
        for r in range(rows.shape[0]):
            for b in range(4):
                c, s = _nv_scalar(rows[r, 16 * b:16 * b + 16], g)
                assert sc[r, b] == s and codes[r, 16 * b:16 * b + 16].tolist() == c


def test_nv_quantizer_representable_values_ties_saturation_zero():
    g = 2.0 ** -8
    # a block of E2M1 grid values times one E4M3 scale times g, whose amax is
    # 6 x scale x g, comes back unchanged
    rng = np.random.default_rng(4)
    for sc in (1, 8, 0x38, 0x55, 0x7E):
        s = oracle.e4m3_to_f64(sc)
        e2m1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
        vals = rng.choice(np.concatenate([e2m1, -e2m1]), 16)
        vals[3] = 6.0
        block = vals * s * g
        codes, scale = oracle.nv_quantize(block[None], g)
        assert scale[0, 0] == sc
        assert (oracle.nv_dequantize(codes, scale, g)[0] == block).all()
    # E2M1 midpoints relative to the step go to the even code
    step = 2.0 * g                                   # scale code 0x38 = 1.0 ... times 2: amax 12 g
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, -0.25, -5.0, 0, 0, 0, 0, 0, 0]) * step
    codes, scale = oracle.nv_quantize(mids[None], g)
    assert oracle.e4m3_to_f64(scale[0, 0]) == 2.0
    assert codes[0, :10].tolist() == [0, 2, 2, 4, 4, 6, 6, 7, 8, 14]
    # saturation: amax / (6 g) above 448 takes scale 448 and codes saturate at 6
    big = np.full(16, 1e4 * g)
    big[0] = -3e4 * g
    codes, scale = oracle.nv_quantize(big[None], g)
    assert scale[0, 0] == 0x7E and codes[0, 0] == 15 and (codes[0, 1:] == 7).all()
    # an all-zero block, and negative zeros: scale code 0, all-zero codes
    z = np.zeros((1, 16))
    z[0, 1] = -0.0
    codes, scale = oracle.nv_quantize(z, g)
    assert scale.tolist() == [[0]] and (codes == 0).all()


def test_nvfp4_w4a4_single_expert_is_a_quantised_textbook_ffn():
    """E = 1, k = 1, NVFP4 W4A4: the torch GEGLU FFN on the decoded weights
    and the quantised x, with h rounded to bf16 and quantised before the
    down projection."""
    s = mi.Shape(T=6, H=64, E=1, k=1, I=32, nvfp4=True, nv_a4=True)
    inp = mi.make(s, seed=13)
    r = oracle.forward(inp)
    wgu, wd = oracle.expert_weights(inp, 0)
    xq = torch.from_numpy(oracle.nv_round(oracle.bf16_to_f64(inp.x), inp.gu_input_scale))
    g = torch.nn.functional.linear(xq, torch.from_numpy(wgu[:32]))
    u = torch.nn.functional.linear(xq, torch.from_numpy(wgu[32:]))
    h = torch.nn.functional.gelu(g, approximate="tanh") * u
    hq = torch.from_numpy(oracle.nv_round(oracle.round_to_bf16(h.numpy()), inp.d_input_scale))
    ref = torch.nn.functional.linear(hq, torch.from_numpy(wd)).numpy()
    assert _rel(r["out"], ref) <= 1e-13
    plain = oracle.forward(mi.make(mi.Shape(T=6, H=64, E=1, k=1, I=32, nvfp4=True), seed=13))["out"]
    assert _rel(plain, ref) > 1e-4
