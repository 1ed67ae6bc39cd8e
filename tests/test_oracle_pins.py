"""Pins for the CPU oracle, checked against things other than the oracle itself:
library conversions (numpy, torch), full sorts, dense numpy products, closed
forms and hand-worked examples.  Sources are the "DeepSeek-V3 Technical Report"
page: §2.1.2 (DeepSeekMoE, auxiliary-loss-free balancing, node-limited
routing), §3.3 (fine-grained FP8 quantisation), §4.2 (hyper-parameters)."""
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import moe_synth as syn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32_of_bits(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# storage formats
# ---------------------------------------------------------------------------

def test_round_format_binary32_matches_hardware_cast(orc):
    rng = np.random.default_rng(1)
    mags = np.concatenate([rng.uniform(-140, 100, 4000), rng.uniform(-149, -120, 1000)])
    xs = rng.choice([-1.0, 1.0], mags.size) * np.exp2(mags) * (1 + rng.random(mags.size))
    for x in xs:
        want = float(np.float32(x))
        got = orc.round_format(x, 24, -126, float(np.finfo(np.float32).max))
        assert got == want, (x, got, want)


def test_bf16_rounding_matches_torch(orc):
    rng = np.random.default_rng(2)
    xs = (rng.standard_normal(20000) * np.exp2(rng.integers(-60, 60, 20000))).astype(np.float32)
    # exact ties between two bf16 neighbours: low 16 bits == 0x8000
    ties = (rng.integers(0, 2**31, 2000, dtype=np.uint32) & 0xFFFF0000 | 0x8000).view(np.float32)
    xs = np.concatenate([xs, ties[np.isfinite(ties)]])
    want = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for x, w in zip(xs, want):
        assert orc.encode_bf16(float(x)) == int(w), x


def test_e4m3_decode_matches_torch_all_codes(orc):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    for c in range(256):
        got = orc.decode_e4m3(c)
        if math.isnan(ref[c]):
            assert math.isnan(got)
        else:
            assert got == float(ref[c]), c
    assert orc.decode_e4m3(0x7E) == 448.0          # largest finite E4M3FN
    assert orc.decode_e4m3(0x01) == 2.0 ** -9       # smallest subnormal


def test_e4m3_encode_midpoints_and_torch(orc):
    vals = sorted({orc.decode_e4m3(c) for c in range(0x7F)})          # 0 .. 448, finite, positive
    for a, b in zip(vals[:-1], vals[1:]):
        mid = (a + b) / 2
        ca, cb = orc.encode_e4m3(a), orc.encode_e4m3(b)
        assert orc.decode_e4m3(ca) == a and orc.decode_e4m3(cb) == b
        even = ca if ca % 2 == 0 else cb
        assert orc.encode_e4m3(mid) == even                        # ties to even code
        assert orc.encode_e4m3(np.nextafter(mid, -np.inf)) == ca
        assert orc.encode_e4m3(np.nextafter(mid, np.inf)) == cb
        assert orc.encode_e4m3(-mid) == even | 0x80
    rng = np.random.default_rng(3)
    xs = np.concatenate([rng.uniform(-448, 448, 20000), rng.uniform(-0.05, 0.05, 20000)]).astype(np.float32)
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for x, r in zip(xs, ref):
        assert orc.encode_e4m3(float(x)) == int(r), x
    assert orc.encode_e4m3(1e6) == 0x7E                            # saturates at 448


def test_quant_closed_forms(orc):
    # a tile whose max is 448 has scale exactly 1 and quantises elementwise
    x = np.zeros((1, 128), np.float32)
    x[0, :8] = [448, -448, 1.0, 0.5, 3.0, -2.75, 0.0, 2.0 ** -9]
    q, s = orc.quant_1x128(x)
    assert s[0, 0] == 1.0
    assert [orc.decode_e4m3(c) for c in q[0, :8]] == [448, -448, 1.0, 0.5, 3.0, -2.75, 0.0, 2.0 ** -9]
    # an all-zero tile has scale 1 and code 0
    q, s = orc.quant_1x128(np.zeros((2, 256), np.float32))
    assert (s == 1.0).all() and (q == 0).all()
    # scale = fp32 quotient amax / 448
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 384)).astype(np.float32)
    q, s = orc.quant_1x128(x)
    amax = np.abs(x.reshape(3, 3, 128)).max(-1)
    assert (s == (amax / np.float32(448)).astype(np.float32)).all()
    # power-of-two rescaling leaves codes unchanged and scales the scale exactly
    q2, s2 = orc.quant_1x128(x * np.float32(8))
    assert (q2 == q).all() and (s2 == s * 8).all()


def test_quant_roundtrip_bound(orc):
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((16, 512)) * np.exp2(rng.integers(-8, 8, (16, 1)))).astype(np.float32)
    x[0, :5] = [100.0, -1e-4, 3e-3, 0.0, 7.0]           # outliers and small values in one tile
    q, s = orc.quant_1x128(x)
    dec = np.vectorize(orc.decode_e4m3)(q) * np.repeat(s, 128, axis=1)
    ratio = np.abs(x) / np.repeat(s, 128, axis=1)
    normal = ratio >= 2.0 ** -6
    err = np.abs(x.astype(np.float64) - dec)
    assert (err[normal] <= 2.0 ** -4 * np.abs(x[normal]) * (1 + 1e-6)).all()
    assert (err[~normal] <= 2.0 ** -10 * np.repeat(s, 128, axis=1)[~normal] * (1 + 1e-6)).all()


def test_quant_128x128_blocks(orc):
    rng = np.random.default_rng(6)
    w = rng.standard_normal((2, 256, 384)).astype(np.float32)
    w[1, 130, 300] = 50.0
    q, s = orc.quant_128x128(w)
    assert s.shape == (2, 2, 3)
    blocks = np.abs(w.reshape(2, 2, 128, 3, 128)).max(axis=(2, 4))
    assert (s == (blocks / np.float32(448)).astype(np.float32)).all()
    assert orc.decode_e4m3(q[1, 130, 300]) * s[1, 1, 2] == 50.0
    # a 128x128 block equals 128 rows of 1x128 tiles that share the block amax
    q1, s1 = orc.quant_1x128(w[0, :128, :128])
    assert s1.max() == s[0, 0, 0]


# ---------------------------------------------------------------------------
# routing (§2.1.2; group rule and tie rule are readings)
# ---------------------------------------------------------------------------

def brute_route(s, b, G, Mg, K):
    """Selection by full sorts (numpy lexsort), not by repeated arg-max."""
    T, Nr = s.shape
    gs = Nr // G
    sb = (s + b[None, :]).astype(np.float32)
    idx = np.empty((T, K), np.int64)
    for t in range(T):
        gsc = []
        for g in range(G):
            v = np.sort(sb[t, g * gs:(g + 1) * gs])[::-1]
            gsc.append(np.float32(v[0] + v[1]) if gs > 1 else v[0])
        gsc = np.array(gsc, np.float32)
        order_g = np.lexsort((np.arange(G), -gsc.astype(np.float64)))
        keep = set(order_g[:Mg].tolist())
        cand = np.array([i for i in range(Nr) if i // gs in keep])
        order = np.lexsort((cand, -sb[t, cand].astype(np.float64)))
        idx[t] = cand[order[:K]]
    return idx


@pytest.mark.parametrize("Nr,G,Mg,K", [(16, 4, 2, 2), (16, 4, 2, 5), (32, 8, 3, 6), (12, 1, 1, 4),
                                       (12, 3, 3, 4), (8, 8, 2, 2), (64, 8, 4, 8)])
def test_route_matches_brute_force_sort(orc, Nr, G, Mg, K):
    for seed in range(6):
        rng = np.random.default_rng(100 + seed)
        T = 64
        s = rng.random((T, Nr), dtype=np.float32)
        if seed % 2:                                   # force many exact ties
            s = (np.floor(s * 4) / 4).astype(np.float32)
        b = rng.uniform(-0.1, 0.1, Nr).astype(np.float32) if seed % 3 else np.zeros(Nr, np.float32)
        _, idx, w = orc.route(None, None, b, G=G, Mg=Mg, K=K, scores_in=s)
        assert (idx == brute_route(s, b, G, Mg, K)).all()
        den = np.zeros(T, np.float32)
        for j in range(K):
            den = (den + s[np.arange(T), idx[:, j]]).astype(np.float32)
        assert (w == (s[np.arange(T)[:, None], idx] / den[:, None]).astype(np.float32)).all()


@settings(max_examples=150, deadline=None, derandomize=True)
@given(data=st.data())
def test_route_property_matches_brute_force_sort(orc, data):
    """Hypothesis over tiny shapes, value grids (many exact ties) and biases:
    the oracle's selection equals the full-sort selection, and the gates are
    the selected un-biased affinities over their sum taken in slot order."""
    G = data.draw(st.sampled_from([1, 2, 3, 4, 8]), "G")
    per = data.draw(st.integers(1, 6), "experts per group")
    Nr = G * per
    Mg = data.draw(st.integers(1, G), "Mg")
    K = data.draw(st.integers(1, Mg * per), "K")
    T = data.draw(st.integers(1, 12), "T")
    levels = data.draw(st.sampled_from([2, 4, 16, 0]), "levels")   # 0: continuous values
    seed = data.draw(st.integers(0, 2**31 - 1), "seed")
    rng = np.random.default_rng(seed)
    s = rng.random((T, Nr), dtype=np.float32)
    if levels:
        s = (np.floor(s * levels) / levels + 1.0 / (2 * levels)).astype(np.float32)
    b = (rng.uniform(-0.2, 0.2, Nr) if data.draw(st.booleans(), "bias") else np.zeros(Nr)).astype(np.float32)
    _, idx, w = orc.route(None, None, b, G=G, Mg=Mg, K=K, scores_in=s)
    assert (idx == brute_route(s, b, G, Mg, K)).all()
    den = np.zeros(T, np.float32)
    for j in range(K):
        den = (den + s[np.arange(T), idx[:, j]]).astype(np.float32)
    assert (w == (s[np.arange(T)[:, None], idx] / den[:, None]).astype(np.float32)).all()


def test_route_single_group_is_plain_topk(orc):
    rng = np.random.default_rng(7)
    s = rng.random((128, 24), dtype=np.float32)
    b = np.zeros(24, np.float32)
    _, idx1, _ = orc.route(None, None, b, G=1, Mg=1, K=5, scores_in=s)
    _, idx2, _ = orc.route(None, None, b, G=4, Mg=4, K=5, scores_in=s)
    ref = np.argsort(-s, axis=1, kind="stable")[:, :5]
    assert (idx1 == ref).all() and (idx2 == ref).all()


def test_gates_sum_to_one(orc):
    rng = np.random.default_rng(8)
    s = rng.random((512, 64), dtype=np.float32)
    b = rng.uniform(-0.2, 0.2, 64).astype(np.float32)
    for K in (1, 2, 8):
        _, _, w = orc.route(None, None, b, G=8, Mg=4, K=K, scores_in=s)
        assert np.abs(w.astype(np.float64).sum(1) - 1).max() <= K * 2.0 ** -23
    _, _, w = orc.route(None, None, b, G=8, Mg=4, K=1, scores_in=s)
    assert (w == 1.0).all()


def test_bias_changes_selection_not_gates(orc):
    cfg = syn.CONFIGS["tiny"]
    u = syn.hidden(cfg)
    g, b = syn.router_params(cfg)
    kw = dict(G=cfg.G, Mg=cfg.Mg, K=cfg.K)
    s0, i0, w0 = orc.route(u, g, np.zeros_like(b), **kw)
    s1, i1, w1 = orc.route(u, g, b, **kw)
    assert (s0 == s1).all()
    assert (i0 != i1).any(), "the bias must change some selections"
    same = (i0 == i1).all(1)
    assert same.any() and (w0[same] == w1[same]).all()
    # gate = un-biased affinity over the sum of selected un-biased affinities
    T = u.shape[0]
    sel = s1[np.arange(T)[:, None], i1]
    assert np.allclose(w1, sel / sel.sum(1, keepdims=True), rtol=2e-7, atol=0)


def test_forced_routing(orc):
    rng = np.random.default_rng(9)
    s = rng.random((200, 32), dtype=np.float32)
    b = np.zeros(32, np.float32)
    b[13] = 10.0
    _, idx, w = orc.route(None, None, b, G=4, Mg=2, K=3, scores_in=s)
    assert (idx[:, 0] == 13).all()
    counts, _, _, _ = orc.permute(idx, 32)
    assert counts[13] == 200
    den = s[np.arange(200)[:, None], idx].astype(np.float32)
    assert np.allclose(w[:, 0], den[:, 0] / den.sum(1), rtol=3e-7)


def test_route_hand_worked_example(orc):
    with open(os.path.join(GOLDEN, "route_hand_example.json")) as f:
        cases = json.load(f)["cases"]
    for ex in cases:
        s = np.array(ex["scores"], np.float32)
        b = np.array(ex["bias"], np.float32)
        _, idx, w = orc.route(None, None, b, G=ex["G"], Mg=ex["Mg"], K=ex["K"], scores_in=s)
        assert idx.tolist() == ex["topk_idx"]
        assert np.allclose(w, np.array(ex["topk_w"]), rtol=0, atol=1e-7)


def test_affinity_matches_dense_numpy(orc):
    cfg = syn.CONFIGS["tiny"]
    u = syn.hidden(cfg)
    g, b = syn.router_params(cfg)
    s, _, _ = orc.route(u, g, b, G=cfg.G, Mg=cfg.Mg, K=cfg.K)
    z = u.astype(np.float64) @ g.astype(np.float64).T
    ref = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    ulp = np.spacing(ref)
    assert (np.abs(s - ref) <= ulp).all()
    # bf16 storage decodes as the upper half of binary32
    gb, ub = syn.to_bf16_bits(g), syn.to_bf16_bits(u)
    sb, _, _ = orc.route(ub, gb, b, G=cfg.G, Mg=cfg.Mg, K=cfg.K)
    z = f32_of_bits(ub).astype(np.float64) @ f32_of_bits(gb).astype(np.float64).T
    ref = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    assert (np.abs(sb - ref) <= np.spacing(ref)).all()


def test_sigmoid_closed_form(orc):
    # u . e = 0 for every expert  =>  every affinity is exactly 1/2
    u = np.zeros((4, 128), np.float32)
    g = np.random.default_rng(10).standard_normal((8, 128)).astype(np.float32)
    s, idx, w = orc.route(u, g, np.zeros(8, np.float32), G=2, Mg=1, K=2)
    assert (s == 0.5).all()
    assert (idx == [0, 1]).all() and (w == 0.5).all()      # ties go to the lower index


# ---------------------------------------------------------------------------
# dispatch
# ---------------------------------------------------------------------------

def test_permute_matches_stable_sort(orc):
    rng = np.random.default_rng(11)
    Nr, T, K = 40, 300, 6
    idx = np.stack([rng.permutation(Nr)[:K] for _ in range(T)]).astype(np.int32)
    idx[:50] = idx[0]                                        # a hot expert set
    counts, offsets, perm, inv = orc.permute(idx, Nr)
    assert counts.sum() == T * K and offsets[-1] == T * K
    assert (np.diff(offsets) == counts).all() and (counts == np.bincount(idx.ravel(), minlength=Nr)).all()
    order = np.argsort(idx.ravel(), kind="stable")           # library sort on (expert, flat index)
    assert (perm == order // K).all()
    assert (inv[order] == np.arange(T * K)).all()            # inverse permutation
    assert (perm[inv] == np.repeat(np.arange(T), K)).all()   # bijection back to tokens
    for e in range(Nr):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert (np.diff(seg) > 0).all()                      # ascending tokens inside an expert


def test_permute_empty_experts(orc):
    idx = np.array([[3, 1], [3, 1], [1, 3]], np.int32)
    counts, offsets, perm, inv = orc.permute(idx, 6)
    assert counts.tolist() == [0, 3, 0, 3, 0, 0]
    assert offsets.tolist() == [0, 0, 3, 3, 6, 6, 6]
    assert perm.tolist() == [0, 1, 2, 0, 1, 2]
    assert inv.tolist() == [3, 0, 4, 1, 2, 5]


# ---------------------------------------------------------------------------
# expert FFN and the whole layer
# ---------------------------------------------------------------------------

def swiglu_dense(x, wg, wu, wd, round_h, round_y):
    """Dense numpy fp64 SwiGLU with the storage roundings applied by the caller."""
    a = x @ wg.T
    b = x @ wu.T
    h = round_h(a / (1 + np.exp(-a)) * b)
    return round_y(h @ wd.T)


def small_cfg(Nr, G, Mg, K, Ns, d=128, I=128, T=48):
    return syn.LayerConfig("t", T=T, d=d, Nr=Nr, G=G, Mg=Mg, K=K, Ns=Ns, I=I, dtype="fp32")


def test_single_expert_reduces_to_dense_swiglu(orc):
    cfg = small_cfg(Nr=1, G=1, Mg=1, K=1, Ns=1)
    inp = syn.layer_inputs(cfg, seed=3)
    out, idx, w, _ = orc.moe_forward(inp["u"], inp["gate_w"], inp["bias"], (inp["wg"], inp["wu"], inp["wd"]),
                                     (inp["swg"], inp["swu"], inp["swd"]), G=1, Mg=1, K=1, w_code=orc.F32,
                                     out_code=orc.F32)
    assert (idx == 0).all() and (w == 1.0).all()
    f32 = lambda v: v.astype(np.float32).astype(np.float64)
    x = inp["u"].astype(np.float64)
    yr = swiglu_dense(x, inp["wg"][0].astype(np.float64), inp["wu"][0].astype(np.float64),
                      inp["wd"][0].astype(np.float64), f32, f32)
    ys = swiglu_dense(x, inp["swg"][0].astype(np.float64), inp["swu"][0].astype(np.float64),
                      inp["swd"][0].astype(np.float64), f32, f32)
    ref = (yr + ys).astype(np.float32)
    assert np.abs(out - ref).max() <= 4 * np.spacing(np.abs(ref)).max()


def test_single_expert_bf16_reduces_to_dense_swiglu(orc):
    cfg = syn.LayerConfig("t", T=32, d=256, Nr=1, G=1, Mg=1, K=1, Ns=0, I=128, dtype="bf16")
    inp = syn.layer_inputs(cfg, seed=4)
    out, _, _, _ = orc.moe_forward(inp["u"], inp["gate_w"], inp["bias"], (inp["wg"], inp["wu"], inp["wd"]), None,
                                   G=1, Mg=1, K=1, w_code=orc.BF16, out_code=orc.BF16)
    dec = lambda a: f32_of_bits(a).astype(np.float64)
    rb = lambda v: f32_of_bits(torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)).astype(np.float64)
    ref = swiglu_dense(dec(inp["u"]), dec(inp["wg"][0]), dec(inp["wu"][0]), dec(inp["wd"][0]), rb, rb)
    got = dec(out)
    # both round h and y to bf16; a product that lands next to a rounding
    # boundary may round the other way, so allow a couple of bf16 ulps
    assert np.abs(got - ref).max() <= 2 * 2.0 ** -7 * np.abs(ref).max()


def test_identical_experts_make_output_routing_independent(orc):
    cfg = small_cfg(Nr=16, G=4, Mg=2, K=3, Ns=1)
    inp = syn.layer_inputs(cfg, seed=5)
    for k in ("wg", "wu", "wd"):
        inp[k] = np.repeat(inp[k][:1], 16, axis=0)
    args = (inp["u"], inp["gate_w"])
    shared = (inp["swg"], inp["swu"], inp["swd"])
    routed = (inp["wg"], inp["wu"], inp["wd"])
    kw = dict(G=4, Mg=2, K=3, w_code=orc.F32, out_code=orc.F32)
    o1, i1, _, _ = orc.moe_forward(*args, np.zeros(16, np.float32), routed, shared, **kw)
    b = np.linspace(-0.3, 0.3, 16).astype(np.float32)
    o2, i2, _, _ = orc.moe_forward(*args, b, routed, shared, **kw)
    assert (i1 != i2).any()
    assert np.abs(o1 - o2).max() <= 1e-6 * np.abs(o1).max()


def test_down_projection_power_of_two_scaling_is_exact(orc):
    cfg = small_cfg(Nr=8, G=2, Mg=1, K=2, Ns=0)
    inp = syn.layer_inputs(cfg, seed=6)
    kw = dict(G=2, Mg=1, K=2, w_code=orc.F32, out_code=orc.F32)
    o1, _, _, _ = orc.moe_forward(inp["u"], inp["gate_w"], inp["bias"], (inp["wg"], inp["wu"], inp["wd"]), None, **kw)
    o2, _, _, _ = orc.moe_forward(inp["u"], inp["gate_w"], inp["bias"], (inp["wg"], inp["wu"], inp["wd"] * 2), None, **kw)
    assert (o2 == 2 * o1).all()


def test_layer_equals_its_steps(orc):
    """moe_forward = route -> permute -> grouped FFN (routed and shared) -> combine."""
    cfg = syn.CONFIGS["tiny"]
    inp = syn.layer_inputs(cfg)
    kw = dict(G=cfg.G, Mg=cfg.Mg, K=cfg.K)
    out, idx, w, s = orc.moe_forward(inp["u"], inp["gate_w"], inp["bias"], (inp["wg"], inp["wu"], inp["wd"]),
                                     (inp["swg"], inp["swu"], inp["swd"]), w_code=orc.F32, out_code=orc.F32, **kw)
    s2, idx2, w2 = orc.route(inp["u"], inp["gate_w"], inp["bias"], **kw)
    assert (idx == idx2).all() and (w == w2).all() and (s == s2).all()
    counts, offsets, perm, inv = orc.permute(idx, cfg.Nr)
    x = inp["u"][perm]
    rows = np.arange(cfg.T * cfg.K)
    y = orc.grouped_ffn(offsets, x, inp["wg"], inp["wu"], inp["wd"], rows=rows)
    ysh = orc.grouped_ffn(np.array([0, cfg.T]), inp["u"], inp["swg"], inp["swu"], inp["swd"], rows=np.arange(cfg.T))
    out2 = orc.combine(y, inv, w, T=cfg.T, y_shared=ysh)
    assert (out == out2).all()
    res = orc.combine(y, inv, w, T=cfg.T, y_shared=ysh, residual=inp["u"])
    assert np.abs(res - (out2 + inp["u"])).max() <= 2 * np.spacing(np.abs(res)).max()


def test_combine_closed_form(orc):
    rng = np.random.default_rng(12)
    T, K, d = 5, 3, 16
    y = rng.standard_normal((T * K, d)).astype(np.float32)
    inv = rng.permutation(T * K).astype(np.int32)
    w = np.zeros((T, K), np.float32)
    w[:, 1] = 1.0
    out = orc.combine(y, inv, w, T=T)
    assert (out == y[inv.reshape(T, K)[:, 1]]).all()
    ysh = rng.standard_normal((2, T, d)).astype(np.float32)
    w[:] = 0
    out = orc.combine(y, inv, w, T=T, y_shared=ysh)
    assert (out == (ysh[0].astype(np.float64) + ysh[1]).astype(np.float32)).all()


def test_fp8_ffn_matches_dense_on_dequantised_values(orc):
    cfg = syn.LayerConfig("t", T=16, d=256, Nr=2, G=1, Mg=1, K=1, Ns=0, I=256, dtype="bf16")
    inp = syn.layer_inputs(cfg, seed=7)
    (qg, sg), (qu, su), (qd, sd) = (orc.quant_128x128(inp[k]) for k in ("wg", "wu", "wd"))
    xq, xs = orc.quant_1x128(inp["u"])
    offsets = np.array([0, 7, 16])
    y = orc.grouped_ffn(offsets, xq, qg, qu, qd, rows=np.arange(16), x_scales=xs, w_scales=(sg, su, sd))
    dq = lambda q, s: np.vectorize(orc.decode_e4m3)(q) * np.kron(s, np.ones((128, 128)))
    xd = np.vectorize(orc.decode_e4m3)(xq) * np.repeat(xs, 128, axis=1)
    for r in range(16):
        e = 0 if r < 7 else 1
        a = dq(qg[e], sg[e]) @ xd[r]
        b = dq(qu[e], su[e]) @ xd[r]
        h = (a / (1 + np.exp(-a)) * b).astype(np.float32)
        hq, hs = orc.quant_1x128(h.reshape(1, -1))
        hd = np.vectorize(orc.decode_e4m3)(hq[0]) * np.repeat(hs[0], 128)
        ref = dq(qd[e], sd[e]) @ hd
        got = f32_of_bits(y[r]).astype(np.float64)
        assert np.abs(got - ref).max() <= 2.0 ** -8 * np.abs(ref).max() + 1e-30


def _fp8_weights(orc, inp, Ns):
    """128 x 128 e4m3 blocks of the routed and shared weights (§3.3)."""
    routed = [orc.quant_128x128(inp[k]) for k in ("wg", "wu", "wd")]
    shared = [orc.quant_128x128(inp[k]) for k in ("swg", "swu", "swd")] if Ns else None
    return routed, shared


def test_layer_equals_its_steps_e4m3(orc):
    """The E4M3 layer = route -> 1 x 128 tiles of u, gathered by the permutation
    -> e4m3 grouped FFN of the routed experts and of each shared expert over all
    tokens -> combine with the residual; bit for bit (§2.1.2 layer, §3.3 tiles
    and blocks).  Two shared experts with different block scales, so a shared
    expert reading another's scale grid would fail."""
    cfg = syn.LayerConfig("t", T=40, d=256, Nr=8, G=2, Mg=1, K=3, Ns=2, I=256, dtype="bf16", bias="uniform")
    inp = syn.layer_inputs(cfg, seed=21)
    routed, shared = _fp8_weights(orc, inp, cfg.Ns)
    assert not (shared[0][1][0] == shared[0][1][1]).all()
    kw = dict(G=cfg.G, Mg=cfg.Mg, K=cfg.K)
    out, idx, w, s = orc.moe_forward(inp["u"], inp["gate_w"], inp["bias"], tuple(q for q, _ in routed),
                                     tuple(q for q, _ in shared), w_code=orc.E4M3, out_code=orc.BF16,
                                     routed_scales=tuple(sc for _, sc in routed),
                                     shared_scales=tuple(sc for _, sc in shared), flags=1, **kw)
    s2, idx2, w2 = orc.route(inp["u"], inp["gate_w"], inp["bias"], **kw)
    assert (idx == idx2).all() and (w == w2).all() and (s == s2).all()
    counts, offsets, perm, inv = orc.permute(idx, cfg.Nr)
    assert len(np.unique(idx)) > 3
    uq, us = orc.quant_1x128(inp["u"])
    y = orc.grouped_ffn(offsets, uq[perm], *(q for q, _ in routed), rows=np.arange(cfg.T * cfg.K),
                        x_scales=us[perm], w_scales=tuple(sc for _, sc in routed))
    ysh = np.stack([orc.grouped_ffn(np.array([0, cfg.T]), uq, *(q[j:j + 1] for q, _ in shared),
                                    rows=np.arange(cfg.T), x_scales=us,
                                    w_scales=tuple(sc[j:j + 1] for _, sc in shared)) for j in range(cfg.Ns)])
    ref = orc.combine(y, inv, w, T=cfg.T, y_shared=ysh, residual=inp["u"])
    assert (out == ref).all()
    # and the routed part alone is what it is without the residual and shared experts
    no_res, _, _, _ = orc.moe_forward(inp["u"], inp["gate_w"], inp["bias"], tuple(q for q, _ in routed), None,
                                      w_code=orc.E4M3, out_code=orc.BF16,
                                      routed_scales=tuple(sc for _, sc in routed), **kw)
    assert (no_res == orc.combine(y, inv, w, T=cfg.T)).all()


def test_single_expert_fp8_reduces_to_dense_swiglu(orc):
    """N_r = K = 1 in e4m3 with two shared experts: the layer is three dense
    SwiGLU FFNs (numpy matmuls) on the dequantised 1 x 128 tiles of u and the
    dequantised 128 x 128 weight blocks, with each H re-tiled 1 x 128 and each
    expert output stored in bf16, summed once (§3.3; the gate is s/s = 1)."""
    cfg = syn.LayerConfig("t", T=24, d=384, Nr=1, G=1, Mg=1, K=1, Ns=2, I=256, dtype="bf16")
    inp = syn.layer_inputs(cfg, seed=22)
    routed, shared = _fp8_weights(orc, inp, cfg.Ns)
    out, idx, w, _ = orc.moe_forward(inp["u"], inp["gate_w"], inp["bias"], tuple(q for q, _ in routed),
                                     tuple(q for q, _ in shared), G=1, Mg=1, K=1, w_code=orc.E4M3,
                                     out_code=orc.BF16, routed_scales=tuple(sc for _, sc in routed),
                                     shared_scales=tuple(sc for _, sc in shared))
    assert (idx == 0).all() and (w == 1.0).all()
    dec = np.vectorize(orc.decode_e4m3)
    dq = lambda q, s: dec(q) * np.kron(s, np.ones((128, 128)))
    uq, us = orc.quant_1x128(inp["u"])
    x = dec(uq) * np.repeat(us, 128, axis=1)
    rb = lambda v: f32_of_bits(torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16)
                               .numpy().view(np.uint16)).astype(np.float64)

    def tiled(h):
        hq, hs = orc.quant_1x128(h.astype(np.float32))
        return dec(hq) * np.repeat(hs, 128, axis=1)

    total = np.zeros((cfg.T, cfg.d))
    for (qg, sg), (qu, su), (qd, sd), e in [(*routed, 0)] + [(*shared, j) for j in range(cfg.Ns)]:
        total += swiglu_dense(x, dq(qg[e], sg[e]), dq(qu[e], su[e]), dq(qd[e], sd[e]), tiled, rb)
    ref = rb(total)
    got = f32_of_bits(out).astype(np.float64)
    assert np.abs(got - ref).max() <= 2.0 ** -8 * np.abs(ref).max()
    # a shared expert that took the other's block scales would be far off
    wrong = swiglu_dense(x, dq(shared[0][0][1], shared[0][1][0]), dq(shared[1][0][1], shared[1][1][0]),
                         dq(shared[2][0][1], shared[2][1][0]), tiled, rb)
    right = swiglu_dense(x, dq(shared[0][0][1], shared[0][1][1]), dq(shared[1][0][1], shared[1][1][1]),
                         dq(shared[2][0][1], shared[2][1][1]), tiled, rb)
    assert np.abs(wrong - right).max() > 2.0 ** -8 * np.abs(ref).max()


# ---------------------------------------------------------------------------
# bias update (§2.1.2, gamma = 0.001 from §4.2)
# ---------------------------------------------------------------------------

def test_bias_update_closed_form(orc):
    T, K, Nr = 8192, 8, 256                    # mean load exactly 256
    counts = np.full(Nr, 256, np.int32)
    counts[0], counts[1] = 300, 212
    b = orc.bias_update(counts, np.zeros(Nr, np.float32), T, K, 0.001)
    assert b[0] == np.float32(-0.001) and b[1] == np.float32(0.001) and (b[2:] == 0).all()
    # ten steps at fixed loads move a bias by exactly ten fp32 additions
    bb = np.zeros(Nr, np.float32)
    for _ in range(10):
        bb = orc.bias_update(counts, bb, T, K, 0.001)
    ref = np.float32(0)
    for _ in range(10):
        ref = np.float32(ref - np.float32(0.001))
    assert bb[0] == ref and bb[1] == -ref


def test_bias_update_replay_and_resume(orc):
    rng = np.random.default_rng(13)
    steps = [rng.integers(0, 600, 64).astype(np.int32) for _ in range(10)]
    b = np.zeros(64, np.float32)
    for c in steps:
        b = orc.bias_update(c, b, 4096, 4)
    half = np.zeros(64, np.float32)
    for c in steps[:5]:
        half = orc.bias_update(c, half, 4096, 4)
    saved = np.frombuffer(half.tobytes(), np.float32).copy()      # save / restore as raw fp32
    for c in steps[5:]:
        saved = orc.bias_update(c, saved, 4096, 4)
    assert (saved.view(np.uint32) == b.view(np.uint32)).all()


# ---------------------------------------------------------------------------
# the pages' own numbers
# ---------------------------------------------------------------------------

def test_v3_configs_match_the_pages_hyper_parameters():
    with open(os.path.join(GOLDEN, "v3_moe_hyperparams.json")) as f:
        hp = json.load(f)
    for name in ("v3_prefill", "v3_decode", "v3_fp8", "v3_skew"):
        c = syn.CONFIGS[name]
        assert c.d == hp["hidden_dim"] and c.Nr == hp["routed_experts"] and c.Ns == hp["shared_experts"]
        assert c.I == hp["expert_intermediate"] and c.K == hp["routed_per_token"]
        assert c.Mg == hp["max_nodes_per_token"]
    assert hp["quant_group"] == 128 and hp["bias_update_speed"] == 0.001
    # FLOPs per token: 9 experts x 6 d I + 2 d Nr
    assert syn.CONFIGS["v3_prefill"].flops_per_token == 796_393_472


# ---------------------------------------------------------------------------
# complementary sequence-wise balance statistic (§2.1.2; alpha = 1e-4 from §4.2)
# ---------------------------------------------------------------------------

def test_seq_balance_even_routing_gives_alpha(orc):
    """Every expert taken equally often and equal affinities: f_i = 1 and
    P_i = 1/N_r, so the loss is alpha * N_r * (1/N_r) = alpha."""
    Nr, K, Ts = 32, 4, 64
    scores = np.full((Ts, Nr), 0.3, np.float32)
    idx = np.array([[(t * K + j) % Nr for j in range(K)] for t in range(Ts)], np.int32)
    loss, counts, share = orc.seq_balance(scores, idx, Ts, alpha=1e-4)
    assert (counts == Ts * K // Nr).all()
    assert np.allclose(share, 1.0 / Nr, rtol=0, atol=1e-8)
    assert loss[0] == np.float32(1e-4)


def test_seq_balance_concentrated_closed_form(orc):
    """All tokens pick the same K experts A, with affinity 1 on A and eps
    elsewhere: f_A = N_r/K, P_A = 1/(K + (N_r-K) eps), f = 0 off A, so
    loss = alpha * N_r / (K + (N_r - K) eps)."""
    Nr, K, Ts, eps = 64, 8, 50, 1e-3
    A = np.arange(5, 5 + K)
    scores = np.full((Ts, Nr), eps, np.float32)
    scores[:, A] = 1.0
    idx = np.tile(A.astype(np.int32), (Ts, 1))
    loss, counts, _ = orc.seq_balance(scores, idx, Ts, alpha=1e-4)
    expect = 1e-4 * Nr / (K + (Nr - K) * float(np.float32(eps)))
    assert abs(float(loss[0]) - expect) <= 2 ** -23 * expect
    assert counts[0, A].tolist() == [Ts] * K and counts[0].sum() == Ts * K


def test_seq_balance_invariants_and_sequence_split(orc):
    """Per sequence the counts sum to K*Ts and the affinity shares sum to 1;
    a batch of sequences gives each sequence the loss it has alone; a shorter
    last sequence is normalised by its own length."""
    rng = np.random.default_rng(4)
    Nr, K, L = 48, 6, 37
    T = 3 * L + 11
    scores = rng.uniform(0.01, 1.0, (T, Nr)).astype(np.float32)
    idx = np.stack([rng.permutation(Nr)[:K] for _ in range(T)]).astype(np.int32)
    loss, counts, share = orc.seq_balance(scores, idx, L)
    assert loss.shape == (4,)
    lens = [L, L, L, 11]
    for q, n in enumerate(lens):
        assert counts[q].sum() == K * n
        assert abs(share[q].astype(np.float64).sum() - 1.0) <= Nr * 2 ** -23
        alone, c1, s1 = orc.seq_balance(scores[q * L:q * L + n], idx[q * L:q * L + n], n)
        assert alone[0] == loss[q] and (c1[0] == counts[q]).all() and (s1[0] == share[q]).all()
    # permuting tokens inside a sequence changes nothing but rounding order
    perm = np.concatenate([rng.permutation(L), np.arange(L, T)])
    lp, cp, _ = orc.seq_balance(scores[perm], idx[perm], L)
    assert (cp == counts).all() and abs(float(lp[0]) - float(loss[0])) <= 1e-6 * float(loss[0])


# ---------------------------------------------------------------------------
# backward of the layer (fixed selection): exact forward + chain-rule gradient
# ---------------------------------------------------------------------------

def _tiny_f64(seed, T=5, d=16, Nr=8, Ns=1, K=3, I=8):
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((T, d))
    e = rng.standard_normal((Nr, d)) / np.sqrt(d)
    rw = (rng.standard_normal((Nr, I, d)) / np.sqrt(d), rng.standard_normal((Nr, I, d)) / np.sqrt(d),
          rng.standard_normal((Nr, d, I)) / np.sqrt(I))
    sw = (rng.standard_normal((Ns, I, d)) / np.sqrt(d), rng.standard_normal((Ns, I, d)) / np.sqrt(d),
          rng.standard_normal((Ns, d, I)) / np.sqrt(I))
    idx = np.stack([rng.permutation(Nr)[:K] for _ in range(T)]).astype(np.int32)
    dout = rng.standard_normal((T, d))
    return u, e, idx, rw, sw, dout


def test_exact_layer_matches_the_rounding_forward(orc):
    """layer_f64 on fp32 inputs equals the fp32-storage forward oracle (same
    selection) to fp32 rounding: two independent codings of one layer."""
    cfg = syn.CONFIGS["tiny"]
    inp = syn.layer_inputs(cfg)
    out_r, idx, w, _ = orc.moe_forward(inp["u"], inp["gate_w"], inp["bias"], (inp["wg"], inp["wu"], inp["wd"]),
                                       (inp["swg"], inp["swu"], inp["swd"]), G=cfg.G, Mg=cfg.Mg, K=cfg.K,
                                       w_code=orc.F32, out_code=orc.F32)
    out_x, g = orc.layer_f64(inp["u"], inp["gate_w"], idx, (inp["wg"], inp["wu"], inp["wd"]),
                             (inp["swg"], inp["swu"], inp["swd"]))
    assert np.abs(g - w).max() <= 4e-7
    assert np.abs(out_x - out_r).max() <= 2e-5 * np.abs(out_x).max()


@pytest.mark.parametrize("rs", [1.0, 2.5])
def test_backward_matches_finite_differences(orc, rs):
    """Central differences of sum(dout * layer) agree with the chain-rule
    gradient for u, the centroids and all six weight tensors, with and
    without a routed scaling factor on the gates."""
    u, e, idx, rw, sw, dout = _tiny_f64(11)
    g = orc.moe_backward(u, e, idx, rw, sw, dout, routed_scale=rs)
    assert np.allclose(orc.layer_f64(u, e, idx, rw, sw, routed_scale=rs)[1].sum(1), rs, rtol=1e-14)

    def loss(u_, e_, rw_, sw_):
        return float((orc.layer_f64(u_, e_, idx, rw_, sw_, routed_scale=rs)[0] * dout).sum())

    rng = np.random.default_rng(3)
    h = 1e-6
    checks = 0
    for name in ("u", "e", "rwg", "rwu", "rwd", "swg", "swu", "swd"):
        for _ in range(6):
            arrs = dict(u=u.copy(), e=e.copy(), rwg=rw[0].copy(), rwu=rw[1].copy(), rwd=rw[2].copy(),
                        swg=sw[0].copy(), swu=sw[1].copy(), swd=sw[2].copy())
            a = arrs[name]
            pos = tuple(rng.integers(0, n) for n in a.shape)
            if name == "e":   # a centroid that some token selected (others have zero gradient)
                pos = (int(idx[rng.integers(0, idx.shape[0]), rng.integers(0, idx.shape[1])]),) + pos[1:]
            grads = dict(u=g["du"], e=g["dgate_w"], rwg=g["dwg"], rwu=g["dwu"], rwd=g["dwd"],
                         swg=g["dswg"], swu=g["dswu"], swd=g["dswd"])
            v0 = a[pos]
            a[pos] = v0 + h
            lp = loss(arrs["u"], arrs["e"], (arrs["rwg"], arrs["rwu"], arrs["rwd"]), (arrs["swg"], arrs["swu"], arrs["swd"]))
            a[pos] = v0 - h
            lm = loss(arrs["u"], arrs["e"], (arrs["rwg"], arrs["rwu"], arrs["rwd"]), (arrs["swg"], arrs["swu"], arrs["swd"]))
            fd = (lp - lm) / (2 * h)
            an = grads[name][pos]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, pos, fd, an)
            checks += 1
    assert checks == 48
    # unselected centroids get no gradient
    unused = sorted(set(range(e.shape[0])) - set(idx.ravel().tolist()))
    assert all((g["dgate_w"][i] == 0).all() for i in unused)


def test_backward_single_expert_is_dense_swiglu_autograd(orc):
    """N_r = K = 1: the gate is s/s = 1, so the centroid gets no gradient and
    the rest is the gradient of two dense SwiGLU FFNs, here taken from torch
    autograd in float64."""
    u, e, _, rw, sw, dout = _tiny_f64(5, T=7, Nr=1, K=1)
    idx = np.zeros((7, 1), np.int32)
    g = orc.moe_backward(u, e, idx, rw, sw, dout)
    assert np.abs(g["dgate_w"]).max() <= 1e-15
    tu = torch.tensor(u, requires_grad=True)
    ws = [torch.tensor(w[0], requires_grad=True) for w in rw + sw]

    def ffn(x, wg, wu, wd):
        return torch.nn.functional.silu(x @ wg.T) * (x @ wu.T) @ wd.T

    out = ffn(tu, *ws[:3]) + ffn(tu, *ws[3:])
    (out * torch.tensor(dout)).sum().backward()
    assert np.allclose(g["du"], tu.grad.numpy(), rtol=1e-12, atol=1e-12)
    for mine, ref in zip((g["dwg"][0], g["dwu"][0], g["dwd"][0], g["dswg"][0], g["dswu"][0], g["dswd"][0]), ws):
        assert np.allclose(mine, ref.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_backward_token_and_expert_subsets(orc):
    """Listing tokens or experts gives the same rows as the full computation."""
    u, e, idx, rw, sw, dout = _tiny_f64(8, T=9, Nr=6, K=2)
    full = orc.moe_backward(u, e, idx, rw, sw, dout)
    sub = orc.moe_backward(u, e, idx, rw, sw, dout, tokens=[2, 7], experts=[4, 1], dgate=False, dshared=False)
    assert (sub["du"][[2, 7]] == full["du"][[2, 7]]).all() and (sub["du"][[0, 1, 3]] == 0).all()
    assert (sub["dg"][[2, 7]] == full["dg"][[2, 7]]).all()
    for k in ("dwg", "dwu", "dwd"):
        assert (sub[k][0] == full[k][4]).all() and (sub[k][1] == full[k][1]).all()


# ---------------------------------------------------------------------------
# FP8 backward (§3.3: Dgrad and Wgrad GEMMs in FP8)
# ---------------------------------------------------------------------------

def test_quant_128x1_is_the_transpose_of_1x128(orc):
    """One segment whose length is a multiple of 128: 128 x 1 tiles along the
    rows are the 1 x 128 tiles of the transposed matrix, bit for bit."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((256, 384)) * np.exp2(rng.integers(-6, 6, (1, 384)))).astype(np.float32)
    x[:, 5] = 0.0
    q, s = orc.quant_128x1(x, np.array([0, 256], np.int32))
    qt, st = orc.quant_1x128(np.ascontiguousarray(x.T))
    assert (q == qt.T).all() and (s.view(np.uint32) == st.T.view(np.uint32)).all()
    assert (s[:, 5] == 1.0).all() and (q[:, 5] == 0).all()


def test_quant_128x1_segments_gather_and_e4m3_input(orc):
    rng = np.random.default_rng(4)
    x = syn.to_bf16_bits(rng.standard_normal((500, 256)).astype(np.float32))
    off = np.array([0, 130, 130, 300, 431], np.int32)        # ragged runs, one empty segment
    gather = rng.integers(0, 500, 431).astype(np.int32)
    q, s = orc.quant_128x1(x, off, gather=gather)
    assert s.shape[0] == 2 + 0 + 2 + 2
    xg = x[gather]
    b = 0
    for e in range(4):
        seg = xg[off[e]:off[e + 1]]
        if len(seg) == 0:
            continue
        qa, sa = orc.quant_128x1(seg, np.array([0, len(seg)], np.int32))   # the segment alone
        assert (q[off[e]:off[e + 1]] == qa).all()
        assert (s[b:b + len(sa)].view(np.uint32) == sa.view(np.uint32)).all()
        b += len(sa)
    # e4m3 input with 1 x 128 scales equals its dequantised fp32 values
    c, cs = orc.quant_1x128(x)
    tab = np.array([orc.decode_e4m3(k) for k in range(256)])
    xd = (tab[c] * np.repeat(cs, 128, 1)).astype(np.float32)
    q8, s8 = orc.quant_128x1(c, off, x_scales=cs, gather=gather)
    qd, sd = orc.quant_128x1(xd, off, gather=gather)
    assert (q8 == qd).all() and (s8 == sd).all()


def _fp8_layer(seed, T=64, d=256, Nr=8, Ns=1, G=2, Mg=1, K=2, I=256):
    import oracle
    cfg = syn.LayerConfig("t", T=T, d=d, Nr=Nr, G=G, Mg=Mg, K=K, Ns=Ns, I=I, dtype="bf16", bias="uniform")
    inp = syn.layer_inputs(cfg, seed=seed)
    _, idx, _ = oracle.route(inp["u"], inp["gate_w"], inp["bias"], G=G, Mg=Mg, K=K)
    rq = [oracle.quant_128x128(inp[k]) for k in ("wg", "wu", "wd")]
    sq = [oracle.quant_128x128(inp[k]) for k in ("swg", "swu", "swd")] if Ns else None
    dout = syn.grad_output(cfg, seed=seed)
    doutf = (dout.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return inp, idx, rq, sq, doutf


def test_backward_fp8_within_e4m3_precision_of_the_exact_gradient(orc):
    """The FP8 chain (every Dgrad / Wgrad operand quantised) against the exact
    fp64 chain rule of the same layer (dequantised weights, the 1 x 128 tiles
    of u): every gradient within 8% of max|ref|.  e4m3 keeps 3 mantissa bits
    (at most 2^-4 relative per element, about 2% r.m.s.) and each gradient
    passes two to four quantisations; a transposed or dropped operand is off by
    O(1)."""
    inp, idx, rq, sq, dout = _fp8_layer(5)
    r8 = orc.moe_backward_fp8(inp["u"], inp["gate_w"], idx, [a for a, _ in rq], [b for _, b in rq],
                              [a for a, _ in sq], [b for _, b in sq], dout)
    tab = np.array([orc.decode_e4m3(c) for c in range(256)])

    def deq(q, s):
        return tab[q] * np.repeat(np.repeat(s, 128, 1), 128, 2)

    uq, us = orc.quant_1x128(inp["u"])
    ud = tab[uq] * np.repeat(us, 128, 1)
    gw = (inp["gate_w"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    r64 = orc.moe_backward(ud, gw, idx, [deq(a, b) for a, b in rq], [deq(a, b) for a, b in sq], dout)
    for k in ("du", "dg", "dgate_w", "dwg", "dwu", "dwd", "dswg", "dswu", "dswd"):
        err = np.abs(r8[k] - r64[k]).max() / np.abs(r64[k]).max()
        assert err <= 0.08, (k, err)
        assert err >= 1e-4, (k, err)          # the quantisation is really there


def test_backward_fp8_subsets_and_empty_expert(orc):
    inp, idx, rq, sq, dout = _fp8_layer(6, T=40, Nr=8, K=2)
    args = (inp["u"], inp["gate_w"], idx, [a for a, _ in rq], [b for _, b in rq], [a for a, _ in sq],
            [b for _, b in sq], dout)
    full = orc.moe_backward_fp8(*args)
    unused = sorted(set(range(8)) - set(idx.ravel().tolist()))
    sub = orc.moe_backward_fp8(*args, tokens=[3, 17], experts=[int(idx[3, 0])] + unused[:1], dgate=False,
                               dshared=False)
    assert (sub["du"][[3, 17]] == full["du"][[3, 17]]).all() and (sub["dg"][[3, 17]] == full["dg"][[3, 17]]).all()
    assert (sub["dwd"][0] == full["dwd"][idx[3, 0]]).all()
    for i in unused:
        assert (full["dwg"][i] == 0).all() and (full["dwd"][i] == 0).all() and (full["dgate_w"][i] == 0).all()
