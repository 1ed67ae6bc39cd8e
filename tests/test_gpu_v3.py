"""GPU parity at the V3 layer shape (d = 7168, 256 routed + 1 shared experts,
I = 2048, top-8 of 8 groups with top-4 groups; "DeepSeek-V3 Technical Report"
§4.2) in the launch configuration the benchmark times.

The layer runs on every token of the batch; the oracle recomputes a seeded
sample of tokens one by one (routing, every selected expert, the shared expert,
combine).  Layer-wide invariants (counts, gate sums, permutation) are checked
on every token."""
import numpy as np
import pytest

import moe_synth as syn
from _util import dec, oracle_codes, rel_err, routing_disagreement_is_near_tie, shape_of

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def moe():
    import mixture_experts_layer_35_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()
    return m


@pytest.fixture(scope="module")
def orc():
    import oracle
    oracle._load()
    return oracle


@pytest.fixture(scope="module")
def v3(moe):
    """Host master weights (bf16) and the device-resident bf16 layer."""
    from mixture_experts_layer_35_amd.layer import MoeLayer
    cfg = syn.CONFIGS["v3_prefill"]
    print("generating V3 inputs", flush=True)
    inp = syn.layer_inputs(cfg)
    print("uploading V3 layer", flush=True)
    layer = MoeLayer.from_host(shape_of(cfg), inp["gate_w"], inp["bias"], inp["wg"], inp["wu"], inp["wd"],
                               inp["swg"], inp["swu"], inp["swd"])
    return cfg, inp, layer


@pytest.fixture(scope="module")
def v3_routing(orc, v3):
    """The oracle's own affinities, selection and gates for every token of the batch."""
    cfg, inp, _ = v3
    print("oracle routing of all %d tokens" % cfg.T, flush=True)
    return orc.route(inp["u"], inp["gate_w"], inp["bias"], G=cfg.G, Mg=cfg.Mg, K=cfg.K)


def run(layer, cfg, u_host):
    from mixture_experts_layer_35_amd.layer import to_device, to_host
    T = u_host.shape[0]
    u = to_device(u_host)
    idx = torch.empty((T, cfg.K), dtype=torch.int32, device="cuda")
    w = torch.empty((T, cfg.K), dtype=torch.float32, device="cuda")
    counts = torch.empty(cfg.Nr, dtype=torch.int32, device="cuda")
    scores = torch.empty((T, cfg.Nr), dtype=torch.float32, device="cuda")
    out = layer.forward(u, topk_idx=idx, topk_w=w, counts=counts, scores=scores)
    torch.cuda.synchronize()
    return dict(out=to_host(out), idx=to_host(idx), w=to_host(w), counts=to_host(counts), scores=to_host(scores))


def row_blocks(m, bm=256):
    """First row of each row block when an expert's m rows are split evenly over
    ceil(m / bm) blocks (the expert kernel's tiles), plus m."""
    mt = -(-m // bm)
    mq, mr = divmod(m, mt)
    return [b * mq + min(b, mr) for b in range(mt)] + [m]


def covering_sample(idx_all, n, rng, experts):
    """n random tokens, plus for every row block of every listed expert (rows in
    token order, as the dispatch lays them out) one of its tokens if the random
    draw missed the block.  Returns the sorted tokens and the number of blocks."""
    T, _ = idx_all.shape
    tokens = set(rng.choice(T, n, replace=False).tolist())
    nblocks = 0
    for e in experts:
        rows = np.nonzero((idx_all == e).any(1))[0]           # the expert's tokens, increasing
        b = row_blocks(len(rows))
        for lo, hi in zip(b[:-1], b[1:]):
            nblocks += 1
            if not tokens.intersection(rows[lo:hi].tolist()):
                tokens.add(int(rng.choice(rows[lo:hi])))
    return np.array(sorted(tokens)), nblocks


def assert_covers(idx_all, tokens, experts):
    """Every row block of every listed expert holds a sampled token."""
    sample = set(tokens.tolist())
    for e in experts:
        rows = np.nonzero((idx_all == e).any(1))[0]
        b = row_blocks(len(rows))
        for lo, hi in zip(b[:-1], b[1:]):
            assert sample.intersection(rows[lo:hi].tolist()), (e, lo, hi)


def check(cfg, T, got, ref, tokens, bias, tol):
    out_r, idx_r, _, s_r = ref
    same = np.array([(got["idx"][t] == idx_r[n]).all() for n, t in enumerate(tokens)])
    for n, t in enumerate(tokens):
        if not same[n]:
            assert routing_disagreement_is_near_tie(s_r[n], bias, idx_r[n], got["idx"][t], cfg.G, 4e-6), t
    assert same.mean() >= 0.9
    err = rel_err(got["out"][tokens][same], out_r[same])
    print("sampled tokens %d, same routing %d, max|err|/max|ref| = %.3g" % (len(tokens), same.sum(), err), flush=True)
    assert err <= tol
    assert np.abs(got["scores"][tokens].astype(np.float64) - s_r).max() <= 2e-6
    assert got["counts"].sum() == T * cfg.K
    assert (got["counts"] == np.bincount(got["idx"].ravel(), minlength=cfg.Nr)).all()
    assert np.abs(got["w"].astype(np.float64).sum(1) - 1).max() <= cfg.K * 2.0 ** -23
    # every token keeps K distinct experts from at most topk_groups groups
    gs = cfg.Nr // cfg.G
    for row in got["idx"][:: max(1, T // 512)]:
        assert len(set(row.tolist())) == cfg.K and len(set((row // gs).tolist())) <= cfg.Mg


def test_v3_prefill_bf16(moe, orc, v3, v3_routing):
    cfg, inp, layer = v3
    print("forward V3 bf16 T=%d" % cfg.T, flush=True)
    got = run(layer, cfg, inp["u"])
    s_all, i_all, _ = v3_routing
    # 512 random tokens, completed so that every expert's row block holds one of them
    used = np.unique(i_all)
    tokens, nb = covering_sample(i_all, 512, np.random.default_rng(1), used)
    assert_covers(i_all, tokens, used)
    print("sample: %d tokens covering %d row blocks of %d experts" % (len(tokens), nb, len(used)), flush=True)
    wcode, ocode = oracle_codes(cfg)
    ref = orc.moe_forward(inp["u"], inp["gate_w"], inp["bias"], (inp["wg"], inp["wu"], inp["wd"]),
                          (inp["swg"], inp["swu"], inp["swd"]), G=cfg.G, Mg=cfg.Mg, K=cfg.K, w_code=wcode,
                          out_code=ocode, tokens=tokens)
    check(cfg, cfg.T, got, ref, tokens, inp["bias"], 2e-2)
    # the whole batch routes as the oracle does, up to near ties of the fp32 affinities
    same = (got["idx"] == i_all).all(1)
    for t in np.nonzero(~same)[0]:
        assert routing_disagreement_is_near_tie(s_all[t], inp["bias"], i_all[t], got["idx"][t], cfg.G, 4e-6), t
    print("tokens routed as the oracle does: %d / %d" % (same.sum(), cfg.T), flush=True)
    assert same.mean() >= 0.97
    # sequence-wise balance statistic of this batch's routing (4K-token sequences, §4.2), both
    # sides given the oracle's affinities and selection
    for seq_len in (4096, 1024):
        n_seq = cfg.T // seq_len
        shape = shape_of(cfg)
        loss = torch.empty(n_seq, dtype=torch.float32, device="cuda")
        counts = torch.empty((n_seq, cfg.Nr), dtype=torch.int32, device="cuda")
        ws = torch.empty(moe.moe_seq_balance_workspace_bytes(shape, seq_len), dtype=torch.uint8, device="cuda")
        moe.moe_seq_balance(shape, torch.from_numpy(s_all).cuda(), torch.from_numpy(i_all).cuda(), seq_len,
                            1e-4, loss, counts, None, ws)
        lr, cr, _ = orc.seq_balance(s_all, i_all, seq_len, 1e-4)
        print("seq balance loss (seq_len %d):" % seq_len, loss.cpu().numpy(), flush=True)
        assert (counts.cpu().numpy() == cr).all()
        assert np.allclose(loss.cpu().numpy(), lr, rtol=1e-5, atol=0)
    # the permutation of the same batch is a bijection with increasing tokens per expert
    shape = shape_of(cfg)
    T, K = cfg.T, cfg.K
    idx = torch.from_numpy(got["idx"]).cuda()
    counts, offsets = (torch.empty(n, dtype=torch.int32, device="cuda") for n in (cfg.Nr, cfg.Nr + 1))
    perm, inv = (torch.empty(T * K, dtype=torch.int32, device="cuda") for _ in range(2))
    ws = torch.empty(moe.moe_workspace_bytes(shape, moe.MOE_WS_PERMUTE), dtype=torch.uint8, device="cuda")
    moe.moe_permute(shape, idx, None, counts, offsets, perm, inv, None, None, ws)
    torch.cuda.synchronize()
    p, iv, off = perm.cpu().numpy(), inv.cpu().numpy(), offsets.cpu().numpy()
    assert (p[iv] == np.repeat(np.arange(T), K)).all()
    assert (np.sort(iv) == np.arange(T * K)).all()
    for e in range(0, cfg.Nr, 17):
        seg = p[off[e]:off[e + 1]]
        hit = got["idx"][seg] == e                        # each listed token routes to e exactly once
        assert (np.diff(seg) > 0).all() and (hit.sum(1) == 1).all()
        rows = iv[seg * K + np.argmax(hit, axis=1)]
        assert (rows == np.arange(off[e], off[e + 1])).all()


def test_v3_decode_bf16(moe, orc, v3):
    cfg0, inp, layer = v3
    cfg = syn.CONFIGS["v3_decode"]
    u = syn.hidden(cfg)
    assert (u == inp["u"][: cfg.T]).all()
    print("forward V3 bf16 T=%d" % cfg.T, flush=True)
    got = run(layer, cfg, u)
    tokens = np.arange(cfg.T)                                 # every token of the decode batch
    wcode, ocode = oracle_codes(cfg)
    ref = orc.moe_forward(u, inp["gate_w"], inp["bias"], (inp["wg"], inp["wu"], inp["wd"]),
                          (inp["swg"], inp["swu"], inp["swd"]), G=cfg.G, Mg=cfg.Mg, K=cfg.K, w_code=wcode,
                          out_code=ocode, tokens=tokens)
    check(cfg, cfg.T, got, ref, tokens, inp["bias"], 2e-2)


@pytest.fixture(scope="module")
def v3_fp8(moe, v3):
    """The e4m3 layer: weights quantised on the device from the same bf16 master weights."""
    from mixture_experts_layer_35_amd.layer import MoeLayer, quantize_weights_128x128
    _, inp, layer16 = v3
    cfg = syn.CONFIGS["v3_fp8"]
    rq, rs, sq, ss = [], [], [], []
    for w in layer16.routed_w:
        q, s = quantize_weights_128x128(w)
        rq.append(q)
        rs.append(s)
    for w in layer16.shared_w:
        q, s = quantize_weights_128x128(w)
        sq.append(q)
        ss.append(s)
    torch.cuda.synchronize()
    return cfg, MoeLayer(shape_of(cfg), layer16.gate_w, layer16.bias, rq, sq, rs, ss)


def quantise_for_oracle(orc, inp, experts):
    """The oracle's own 128 x 128 blocks of the listed routed experts (the others
    zero, scale 1: never read) and of the shared expert."""
    routed_q, routed_s = [], []
    for name in ("wg", "wu", "wd"):
        w = inp[name]
        q = np.zeros(w.shape, np.uint8)
        s = np.ones((w.shape[0], w.shape[1] // 128, w.shape[2] // 128), np.float32)
        q[experts], s[experts] = orc.quant_128x128(w[experts])
        routed_q.append(q)
        routed_s.append(s)
    shared = [orc.quant_128x128(inp[n]) for n in ("swg", "swu", "swd")]
    return routed_q, routed_s, [p[0] for p in shared], [p[1] for p in shared]


def test_v3_fp8(moe, orc, v3, v3_fp8):
    from mixture_experts_layer_35_amd.layer import to_host
    _, inp, _ = v3
    cfg, layer = v3_fp8
    # device quantisation of two experts is bit-identical to the oracle's
    for k, name in enumerate(("wg", "wu", "wd")):
        for e in (0, 255):
            qo, so = orc.quant_128x128(inp[name][e:e + 1])
            assert (to_host(layer.routed_w[k][e]) == qo[0]).all()
            assert (to_host(layer.routed_s[k][e]).view(np.uint32) == so[0].view(np.uint32)).all()
    u = syn.hidden(cfg)
    print("forward V3 fp8 T=%d" % cfg.T, flush=True)
    got = run(layer, cfg, u)
    print("oracle routing of all %d tokens" % cfg.T, flush=True)
    _, i_all, _ = orc.route(u, inp["gate_w"], inp["bias"], G=cfg.G, Mg=cfg.Mg, K=cfg.K)
    # 512 random tokens, completed so that both row blocks of every expert (about 512
    # rows each at T = 16384) hold one of them
    used = np.unique(i_all)
    tokens, nb = covering_sample(i_all, 512, np.random.default_rng(2), used)
    assert_covers(i_all, tokens, used)
    assert nb > len(used)
    print("sample: %d tokens covering %d row blocks of %d experts" % (len(tokens), nb, len(used)), flush=True)
    print("oracle: 128 x 128 blocks of the touched experts", flush=True)
    routed_q, routed_s, shared_q, shared_s = quantise_for_oracle(orc, inp, np.unique(i_all[tokens]))
    ref = orc.moe_forward(u, inp["gate_w"], inp["bias"], tuple(routed_q), tuple(shared_q), G=cfg.G,
                          Mg=cfg.Mg, K=cfg.K, w_code=orc.E4M3, out_code=orc.BF16, tokens=tokens,
                          routed_scales=tuple(routed_s), shared_scales=tuple(shared_s))
    check(cfg, cfg.T, got, ref, tokens, inp["bias"], 5e-2)


def test_v3_skew_bias_steps(moe, orc, v3):
    """The skewed-load layer (T = 8192, centroids scaled for a flattened
    Zipf(1.2) popularity, hottest expert ~8x the mean) over ten steps of the
    auxiliary-loss-free bias update (§2.1.2, gamma = 0.001 from §4.2).  Each
    step runs the whole layer on a fresh batch, starting from the oracle's
    bias chain.  The oracle routes every token itself; selections agree up to
    near ties of the fp32 affinities, the counts differ by exactly what those
    tokens moved, and the GPU's bias update equals the oracle's wherever the
    counts agree (elsewhere it is at most one step 2 gamma away).  Step 0 also
    checks sampled outputs against the oracle's experts."""
    from mixture_experts_layer_35_amd.layer import MoeLayer, to_device, to_host
    cfg0, inp, layer16 = v3
    cfg = syn.CONFIGS["v3_skew"]
    gate_w, bias_h = syn.router_params(cfg)
    layer = MoeLayer(shape_of(cfg), to_device(gate_w), to_device(bias_h), layer16.routed_w, layer16.shared_w)
    shape = shape_of(cfg)
    T, K, Nr = cfg.T, cfg.K, cfg.Nr
    mean = T * K / Nr
    ratios = []
    for step in range(syn.SKEW_STEPS):
        u = syn.hidden(cfg, seed=syn.SKEW_STEP_SEED + step)
        print("skew step %d T=%d" % (step, T), flush=True)
        bias_before = bias_h.copy()
        layer.bias.copy_(torch.from_numpy(bias_before))
        got = run(layer, cfg, u)
        moe.moe_bias_update(shape, torch.from_numpy(got["counts"]).cuda(), layer.bias, syn.SKEW_GAMMA)
        torch.cuda.synchronize()
        s_r, ir, wr = orc.route(u, gate_w, bias_before, G=cfg.G, Mg=cfg.Mg, K=K)
        same = (got["idx"] == ir).all(1)
        for t in np.nonzero(~same)[0]:
            assert routing_disagreement_is_near_tie(s_r[t], bias_before, ir[t], got["idx"][t], cfg.G, 4e-6), t
        assert same.mean() >= 0.97
        gw = got["w"][same].astype(np.float64)
        assert np.abs(gw - wr[same]).max() <= 1e-5
        cr, _, _, _ = orc.permute(ir, Nr)
        moved = np.bincount(got["idx"][~same].ravel(), minlength=Nr) - np.bincount(ir[~same].ravel(), minlength=Nr)
        assert (got["counts"].astype(np.int64) - cr == moved).all()
        bias_h = orc.bias_update(cr, bias_before, T, K, syn.SKEW_GAMMA)
        bias_g = to_host(layer.bias)
        eq = got["counts"] == cr
        assert (bias_g[eq].view(np.uint32) == bias_h[eq].view(np.uint32)).all()
        assert np.abs(bias_g[~eq].astype(np.float64) - bias_h[~eq]).max(initial=0.0) <= 2 * syn.SKEW_GAMMA + 1e-6
        print("  same routing %d / %d tokens, counts equal on %d / %d experts" % (same.sum(), T, eq.sum(), Nr),
              flush=True)
        ratios.append(cr.max() / mean)
        if step == 0:
            # the recipe's skew: hottest expert near 8x the mean load
            assert 6.5 <= ratios[0] <= 9.5, ratios[0]
            # 256 random tokens, completed so that every row block of the five hottest
            # experts (up to 8 blocks each, split over the XCD queues) holds one of them
            hot = np.argsort(-cr, kind="stable")[:5]
            tokens, nb = covering_sample(ir, 256, np.random.default_rng(5), hot)
            assert_covers(ir, tokens, hot)
            print("  sample: %d tokens covering %d row blocks of the hottest experts %s (rows %s)"
                  % (len(tokens), nb, hot.tolist(), cr[hot].tolist()), flush=True)
            wcode, ocode = oracle_codes(cfg)
            ref = orc.moe_forward(u, gate_w, bias_before, (inp["wg"], inp["wu"], inp["wd"]),
                                  (inp["swg"], inp["swu"], inp["swd"]), G=cfg.G, Mg=cfg.Mg, K=K, w_code=wcode,
                                  out_code=ocode, tokens=tokens)
            check(cfg, T, got, ref, tokens, bias_before, 2e-2)
    print("max/mean load per step:", " ".join("%.2f" % r for r in ratios), flush=True)
    assert np.abs(bias_h).max() <= syn.SKEW_GAMMA * syn.SKEW_STEPS + 1e-6


def test_v3_backward_sampled(moe, orc, v3, v3_routing):
    """The layer's backward at the V3 prefill shape in the launch configuration
    the benchmark times: input and gate gradients of sampled tokens and the
    weight gradients of three sampled experts (hottest, coldest, one at
    random) against the oracle's chain rule at its own routing.  Tokens whose
    selection differs from the oracle's by a near tie, and the experts they
    touch, are left out of the sample."""
    from mixture_experts_layer_35_amd.layer import to_device, to_host
    cfg, inp, layer = v3
    T, K, Nr = cfg.T, cfg.K, cfg.Nr
    u = to_device(inp["u"])
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    print("V3 backward: forward T=%d" % T, flush=True)
    layer.forward(u, topk_idx=idx)
    dout = syn.grad_output(cfg)
    dg = torch.empty((T, K), dtype=torch.float32, device="cuda")
    dW = tuple(torch.empty_like(w) for w in layer.routed_w)
    print("V3 backward: weight transposes and backward", flush=True)
    du = layer.backward(u, to_device(dout), d_routed_w=dW, dtopk_w=dg)
    torch.cuda.synchronize()
    gidx = to_host(idx)
    s_r, ir, _ = v3_routing
    same = (gidx == ir).all(1)
    for t in np.nonzero(~same)[0]:
        assert routing_disagreement_is_near_tie(s_r[t], inp["bias"], ir[t], gidx[t], cfg.G, 4e-6), t
    assert same.mean() >= 0.97
    touched = set(gidx[~same].ravel().tolist()) | set(ir[~same].ravel().tolist())
    counts = np.bincount(ir.ravel(), minlength=Nr)
    clean = [e for e in range(Nr) if e not in touched and counts[e] > 0]
    rng = np.random.default_rng(7)
    exps = sorted({max(clean, key=lambda e: counts[e]), min(clean, key=lambda e: counts[e]),
                   int(rng.choice(clean))})
    tokens = np.sort(rng.choice(np.nonzero(same)[0], 16, replace=False))
    print("V3 backward: oracle on tokens %s, experts %s (rows %s)" % (tokens.tolist(), exps,
                                                                       counts[exps].tolist()), flush=True)
    ref = orc.moe_backward(inp["u"], inp["gate_w"], ir, (inp["wg"], inp["wu"], inp["wd"]),
                           (inp["swg"], inp["swu"], inp["swd"]), dec(dout), tokens=tokens,
                           experts=np.array(exps, np.int32), dgate=False, dshared=False)
    errs = dict(du=rel_err(to_host(du)[tokens], ref["du"][tokens]),
                dtopk_w=rel_err(to_host(dg)[tokens], ref["dg"][tokens]))
    for name, a, key in zip(("dW_gate", "dW_up", "dW_down"), dW, ("dwg", "dwu", "dwd")):
        for q, e in enumerate(exps):
            errs["%s[%d]" % (name, e)] = rel_err(to_host(a[e]), ref[key][q])
    print("V3 backward errors:", {k: "%.2e" % v for k, v in errs.items()}, flush=True)
    del dW
    layer.drop_transposed()
    torch.cuda.empty_cache()
    for k, v in errs.items():
        assert v <= 2e-2, (k, v)


def test_v3_backward_fp8_sampled(moe, orc, v3, v3_fp8):
    """The e4m3 layer's backward (FP8 Dgrad and Wgrad GEMMs) at the V3 FP8
    shape (T = 16384) in the launch configuration the benchmark times: input
    and gate gradients of sampled tokens and the weight gradients of three
    sampled experts against the oracle's FP8 backward at its own routing, given
    its own 128 x 128 weight blocks."""
    from mixture_experts_layer_35_amd.layer import to_device, to_host
    _, inp, _ = v3
    cfg, layer = v3_fp8
    T, K, Nr = cfg.T, cfg.K, cfg.Nr
    uh = syn.hidden(cfg)
    u = to_device(uh)
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    print("V3 fp8 backward: forward T=%d" % T, flush=True)
    layer.forward(u, topk_idx=idx)
    dout = syn.grad_output(cfg)
    dg = torch.empty((T, K), dtype=torch.float32, device="cuda")
    dW = tuple(torch.empty(w.shape, dtype=torch.bfloat16, device="cuda") for w in layer.routed_w)
    print("V3 fp8 backward: weight transposes and backward", flush=True)
    du = layer.backward(u, to_device(dout), d_routed_w=dW, dtopk_w=dg)
    torch.cuda.synchronize()
    gidx = to_host(idx)
    print("V3 fp8 backward: oracle routing of all %d tokens" % T, flush=True)
    s_r, ir, _ = orc.route(uh, inp["gate_w"], inp["bias"], G=cfg.G, Mg=cfg.Mg, K=K)
    same = (gidx == ir).all(1)
    for t in np.nonzero(~same)[0]:
        assert routing_disagreement_is_near_tie(s_r[t], inp["bias"], ir[t], gidx[t], cfg.G, 4e-6), t
    assert same.mean() >= 0.97
    touched = set(gidx[~same].ravel().tolist()) | set(ir[~same].ravel().tolist())
    counts = np.bincount(ir.ravel(), minlength=Nr)
    clean = [e for e in range(Nr) if e not in touched and counts[e] > 0]
    rng = np.random.default_rng(8)
    exps = sorted({max(clean, key=lambda e: counts[e]), min(clean, key=lambda e: counts[e]),
                   int(rng.choice(clean))})
    tokens = np.sort(rng.choice(np.nonzero(same)[0], 16, replace=False))
    need = np.unique(np.concatenate([ir[tokens].ravel(), exps]))
    rq, rs, sq, ss = quantise_for_oracle(orc, inp, need)
    print("V3 fp8 backward: oracle on tokens %s, experts %s (rows %s)" % (tokens.tolist(), exps,
                                                                          counts[exps].tolist()), flush=True)
    ref = orc.moe_backward_fp8(uh, inp["gate_w"], ir, rq, rs, sq, ss, dec(dout), tokens=tokens,
                               experts=np.array(exps, np.int32), dgate=False, dshared=False)
    errs = dict(du=rel_err(to_host(du)[tokens], ref["du"][tokens]),
                dtopk_w=rel_err(to_host(dg)[tokens], ref["dg"][tokens]))
    for name, a, key in zip(("dW_gate", "dW_up", "dW_down"), dW, ("dwg", "dwu", "dwd")):
        for q, e in enumerate(exps):
            errs["%s[%d]" % (name, e)] = rel_err(to_host(a[e]), ref[key][q])
    print("V3 fp8 backward errors:", {k: "%.2e" % v for k, v in errs.items()}, flush=True)
    del dW
    layer.drop_transposed()
    torch.cuda.empty_cache()
    for k, v in errs.items():
        assert v <= 5e-2, (k, v)
