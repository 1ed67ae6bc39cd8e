#!/usr/bin/env python3
"""Throughput of the DeepSeekMoE layer forward pass on one MI355X.

A step is one moe_forward call (router, dispatch, gate/up and down expert
kernels, combine) over one batch of synthetic tokens already resident in HBM.
Default workload: the V3-shape bf16 prefill batch (T = 4096, d = 7168, 256
routed + 1 shared experts, top-8 of 8 groups with top-4 groups, I = 2048).

Prints one JSON line: tokens/s as `value`, plus layer TFLOP/s, per-stage times
measured with HIP events on the launch stream, a `roofline` object for the
dominant kernel and a `cpu_baseline` object (the CPU oracle on a bounded
sample of the same workload, timed on this host).

With --backward a step is one forward and one backward (moe_backward: input,
centroid and expert-weight gradients for an upstream gradient of the layer
output) of the same batch; the roofline then names the dominant backward
kernel and the CPU baseline times the oracle's input-gradient chain rule.

  python bench.py [--steps K] [--warmup W] [--config v3_prefill|v3_decode|v3_fp8|v3_skew|tiny] [--backward]
"""
import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0                          # MI355X HBM3E
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "fp32": 157.3}
STAGES = ("router", "dispatch", "ffn_gate_up", "ffn_down", "combine")
ROTATE_SEED = 2000          # u of rotated batch k > 0 is drawn with seed 2000 + k
FLUSH_BYTES = 512 << 20     # written between cold-stage launches: twice the 256 MB Infinity Cache


def rotation_batches(cfg):
    """Resident input batches the timed steps cycle through, so that a step's
    router does not find its u in the 256 MB memory-side cache: at least four,
    and together at least 512 MiB (at most 16)."""
    act = 4 if cfg.dtype == "fp32" else 2
    return int(min(16, max(4, -(-FLUSH_BYTES // (cfg.T * cfg.d * act)))))


def esz(dtype):
    return {"fp32": 4, "bf16": 2, "fp8": 1}[dtype]


def algorithmic(cfg, n_touched, saved=False):
    """Algorithmic FLOPs and HBM bytes per launch of the two expert kernels:
    every weight of a touched expert read once, activations in and H / y out
    once (no padding rows, no re-reads); saved: gate/up also writes the fp32
    SwiGLU inputs a | b of every row for the backward."""
    T, d, I, K, Ns = cfg.T, cfg.d, cfg.I, cfg.K, cfg.Ns
    rows = T * K + T * Ns
    wsz = esz(cfg.dtype)
    act = 2 if cfg.dtype != "fp32" else 4
    hsz = 1 if cfg.dtype == "fp8" else act
    sc = 4.0 / (128 * 128) if cfg.dtype == "fp8" else 0.0           # block scales per weight
    asc = 4.0 / 128 if cfg.dtype == "fp8" else 0.0                   # tile scales per activation
    xin = T * d * (1 + asc) if cfg.dtype == "fp8" else T * d * act   # u (or its e4m3 copy) read once
    experts = n_touched + Ns
    gu_bytes = experts * 2 * I * d * (wsz + sc) + xin + rows * I * (hsz + asc)
    if saved:
        gu_bytes += rows * 2 * I * 4
    dn_bytes = experts * I * d * (wsz + sc) + rows * I * (hsz + asc) + rows * d * act
    return dict(ffn_gate_up=(rows * 4.0 * I * d, gu_bytes), ffn_down=(rows * 2.0 * I * d, dn_bytes))


def stage_bytes(cfg):
    """Algorithmic HBM bytes of the three memory-bound stages (each operand
    read or written once): the router reads u and the centroids and writes
    the top-k indices and weights; dispatch reads the indices twice (histogram
    and scatter) and writes the permutation (and, for e4m3, reads u once and
    writes its 1x128-quantised copy); combine reads every expert output row,
    the shared output, the inverse permutation and gate weights, and writes
    the layer output."""
    T, d, K, Nr, Ns = cfg.T, cfg.d, cfg.K, cfg.Nr, cfg.Ns
    act = 4 if cfg.dtype == "fp32" else 2
    router = T * d * act + Nr * d * act + T * K * 8
    dispatch = T * K * 4 * 2 + T * K * 8 + Nr * 8
    if cfg.dtype == "fp8":
        dispatch += T * d * act + T * d * (1 + 4.0 / 128)
    combine = T * K * d * act + Ns * T * d * act + T * K * 8 + T * d * act
    return dict(router=router, dispatch=dispatch, combine=combine)


BWD_STAGES = ("bwd_combine", "bwd_dh", "bwd_swiglu", "bwd_dx", "bwd_token", "bwd_dgate", "wgrad_tile",
              "wgrad_down", "wgrad_gate_up")


def algorithmic_bwd(cfg, n_touched, saved=False):
    """Algorithmic (FLOPs, HBM bytes) per launch of each backward stage: every
    operand read or written once (weights of touched experts once, u once,
    activations per expert row once), no padding rows.  saved: the SwiGLU
    gradient reads the forward's fp32 (a, b) instead of recomputing them."""
    T, d, I, K, Ns, Nr = cfg.T, cfg.d, cfg.I, cfg.K, cfg.Ns, cfg.Nr
    fp8 = cfg.dtype == "fp8"
    a = 2 if fp8 else esz(cfg.dtype)                  # activations, gradients (bf16 for e4m3 layers)
    o = 1 + 4.0 / 128 if fp8 else a                   # GEMM operand: e4m3 code + its tile scale
    wb = 1 + 4.0 / (128 * 128) if fp8 else a          # weight element (+ block scale)
    rr, rs = T * K, T * Ns
    rows = rr + rs
    ex = n_touched + Ns
    gemm = 2.0 * rows * I * d
    # e4m3: the stages that produce a Dgrad input also write its 1x128 tiles
    q = o if fp8 else 0
    return dict(
        bwd_combine=(2.0 * rr * d, T * d * a + 2 * rr * d * a + rr * 12 + (rr + T) * d * q),
        bwd_dh=(gemm, ex * I * d * wb + (rr + T) * d * o + rows * I * a),
        bwd_swiglu=((0.0, rows * I * a + rows * 2 * I * 4 + rows * 2 * I * a) if saved else
                    (2 * gemm, ex * 2 * I * d * wb + T * d * o + rows * I * a + rows * 2 * I * (a + q))),
        bwd_dx=(2 * gemm, ex * 2 * I * d * wb + rows * 2 * I * o + rows * d * a),
        bwd_token=(2.0 * rows * d, rows * d * a + Nr * d * a + T * d * a + rr * 16),
        bwd_dgate=(2.0 * rr * d, T * d * a + Nr * d * 4 + rr * 8),
        # e4m3: both weight-gradient passes' operands re-tiled 128 x 1 (read once, written once)
        wgrad_tile=(0.0, (rr + T) * d * a + rows * I * o + rows * 2 * I * a + (rr + T) * d * o
                    + ((rr + T) * d + rows * I + rows * 2 * I + (rr + T) * d) * o if fp8 else 0.0),
        wgrad_down=(gemm, (rr + T) * d * o + rows * I * o + ex * I * d * a),
        wgrad_gate_up=(2 * gemm, rows * 2 * I * o + T * d * o + ex * 2 * I * d * a))


BWD_KERNELS = {"bwd_combine": "bwd_combine_kernel", "bwd_dh": "bwd_dh", "bwd_swiglu": "bwd_swiglu",
               "bwd_dx": "bwd_dx", "bwd_token": "bwd_token_kernel", "bwd_dgate": "dgate_kernel",
               "wgrad_tile": None,      # eight quantiser launches: no single kernel's traffic
               "wgrad_down": "wgrad_down", "wgrad_gate_up": "wgrad_gate_up"}


def profile_path(cfg, backward=False):
    return os.path.join(ROOT, "profiles", "moe_%s_%s_pmc.md" % ("backward" if backward else "forward", cfg.name))


STAGE_KERNELS = {"router": ("router_gemm_kernel", "router_select_kernel"),
                 "dispatch": ("perm_hist_kernel", "perm_scan_kernel", "perm_scatter_kernel", "quant_rows_kernel"),
                 "combine": ("combine_kernel",)}


def traffic_from_profile(cfg, kernel, backward=False):
    """HBM bytes per launch of `kernel` (a name or a tuple of names, summed)
    from the committed rocprofv3 PMC summary, or None when there is none for
    this workload or the kernel sources changed since it was taken."""
    if kernel is None:
        return None
    if isinstance(kernel, tuple):
        parts = [traffic_from_profile(cfg, k, backward) for k in kernel]
        parts = [p for p in parts if p is not None]
        return sum(parts) if parts else None
    from mixture_experts_layer_35_amd.profsum import source_hash
    path = profile_path(cfg, backward)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source_sha256_16:\s*([0-9a-f]+)", text)
    t = re.search(r"hbm_bytes_per_launch\[%s\]:\s*([0-9.eE+]+)" % re.escape(kernel), text)
    if not m or not t or m.group(1) != source_hash():
        return None
    return float(t.group(1))


def mfma_util_from_profile(cfg, kernel, backward=False):
    """MfmaUtil (% of MFMA-busy cycles over GPU-active cycles x SIMDs) of
    `kernel` from the committed rocprofv3 MFMA-counter summary, or None when
    there is none for this workload or the kernel sources changed since."""
    if kernel is None:
        return None
    from mixture_experts_layer_35_amd.profsum import source_hash
    path = profile_path(cfg, backward).replace("_pmc.md", "_mfma.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source_sha256_16:\s*([0-9a-f]+)", text)
    t = re.search(r"mfma_util\[%s\]:\s*([0-9.eE+]+)" % re.escape(kernel), text)
    if not m or not t or m.group(1) != source_hash():
        return None
    return float(t.group(1))


def cpu_model():
    """The host CPU as /proc/cpuinfo names it (model name, family / model /
    stepping of the first processor entry) and how many logical CPUs this
    process may run on."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    break                                   # first processor entry only
                k, _, v = line.partition(":")
                fields[k.strip()] = v.strip()
    except OSError:
        return None
    ids = ", ".join("%s %s" % (k, fields[k]) for k in ("cpu family", "model", "stepping") if k in fields)
    return "%s (%s); %d logical CPUs in this process's affinity of %d online" % (
        fields.get("model name", "?"), ids, len(os.sched_getaffinity(0)), os.cpu_count() or 0)


def cpu_baseline(cfg, inp, n_tokens):
    """The oracle on the first n/2 and the first n tokens of the batch: tokens/s
    of the larger sample, and both per-token times (the oracle's work is per
    token, so they agree when the sample rate stands for the whole batch)."""
    half = _cpu_forward(cfg, inp, max(1, n_tokens // 2))
    full = _cpu_forward(cfg, inp, n_tokens)
    full["per_token_s"] = [half.pop("_per_token"), full.pop("_per_token")]
    full["per_token_ratio"] = round(full["per_token_s"][1] / full["per_token_s"][0], 4)
    full["sample"] += "; also timed on the first %d tokens: per-token time ratio %.3f" % (
        max(1, n_tokens // 2), full["per_token_ratio"])
    return full


def _cpu_forward(cfg, inp, n_tokens):
    import numpy as np
    import oracle
    wcode = {"fp32": oracle.F32, "bf16": oracle.BF16, "fp8": oracle.E4M3}[cfg.dtype]
    ocode = oracle.F32 if cfg.dtype == "fp32" else oracle.BF16
    tokens = np.arange(min(n_tokens, cfg.T))
    routed = (inp["wg"], inp["wu"], inp["wd"])
    shared = (inp["swg"], inp["swu"], inp["swd"]) if cfg.Ns else None
    rs = ss = None
    if cfg.dtype == "fp8":
        # weights are quantised once before timing, as on the GPU; only the
        # experts this sample touches
        _, idx, _ = oracle.route(inp["u"], inp["gate_w"], inp["bias"], G=cfg.G, Mg=cfg.Mg, K=cfg.K, tokens=tokens)
        need = np.unique(idx)
        qs, ssc = [], []
        for w in routed:
            q = np.zeros(w.shape, np.uint8)
            s = np.ones((w.shape[0], w.shape[1] // 128, w.shape[2] // 128), np.float32)
            q[need], s[need] = oracle.quant_128x128(w[need])
            qs.append(q)
            ssc.append(s)
        routed, rs = tuple(qs), tuple(ssc)
        if shared is not None:
            pairs = [oracle.quant_128x128(w) for w in shared]
            shared, ss = tuple(p[0] for p in pairs), tuple(p[1] for p in pairs)
    t0 = time.perf_counter()
    oracle.moe_forward(inp["u"], inp["gate_w"], inp["bias"], routed, shared, G=cfg.G, Mg=cfg.Mg, K=cfg.K,
                       w_code=wcode, out_code=ocode, tokens=tokens, routed_scales=rs, shared_scales=ss)
    dt = time.perf_counter() - t0
    return {"value": round(len(tokens) / dt, 3), "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "cpu_model": cpu_model(), "_per_token": dt / len(tokens),
            "sample": "first %d tokens of the same %d-token batch: routing, %d routed + %d shared SwiGLU experts "
                      "each, combine (fp64 sums)%s; %.1f s" % (len(tokens), cfg.T, cfg.K, cfg.Ns,
                                                               ", activation and H quantisation (weights "
                                                               "pre-quantised)" if cfg.dtype == "fp8" else "",
                                                               dt)}


def cpu_baseline_backward(cfg, inp, n_tokens):
    """The oracle's chain rule for the input gradient (du, dL/dg) of the first
    n_tokens tokens taken as a batch of their own, at the oracle's routing."""
    import oracle
    import moe_synth as syn
    import numpy as np
    n = min(n_tokens, cfg.T)
    u = inp["u"][:n]
    dout = syn.grad_output(cfg)[:n]
    dout = (dout.astype(np.uint32) << 16).view(np.float32) if dout.dtype == np.uint16 else dout
    _, idx, _ = oracle.route(u, inp["gate_w"], inp["bias"], G=cfg.G, Mg=cfg.Mg, K=cfg.K)
    routed = (inp["wg"], inp["wu"], inp["wd"])
    shared = (inp["swg"], inp["swu"], inp["swd"]) if cfg.Ns else None
    none = np.zeros(0, np.int32)
    if cfg.dtype == "fp8":
        # weights quantised once before timing (only the experts the sample touches), as on the GPU
        need = np.unique(idx)
        rq, rsc = [], []
        for w in routed:
            qw = np.zeros(w.shape, np.uint8)
            sw = np.ones((w.shape[0], w.shape[1] // 128, w.shape[2] // 128), np.float32)
            qw[need], sw[need] = oracle.quant_128x128(w[need])
            rq.append(qw)
            rsc.append(sw)
        sp = [oracle.quant_128x128(w) for w in shared] if shared else None
        t0 = time.perf_counter()
        oracle.moe_backward_fp8(u, inp["gate_w"], idx, rq, rsc, [p[0] for p in sp] if sp else None,
                                [p[1] for p in sp] if sp else None, dout, experts=none, dgate=False, dshared=False)
    else:
        t0 = time.perf_counter()
        oracle.moe_backward(u, inp["gate_w"], idx, routed, shared, dout, experts=none, dgate=False, dshared=False)
    dt = time.perf_counter() - t0
    return {"value": round(n / dt, 3), "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": "input-gradient chain rule (du and dL/dg: %d routed + %d shared SwiGLU experts recomputed "
                      "and differentiated per token, fp64%s) for the first %d tokens of the %d-token batch; weight "
                      "and centroid gradients not in the sample; %.1f s" % (
                          cfg.K, cfg.Ns, ", Dgrad operands in e4m3 tiles" if cfg.dtype == "fp8" else "", n, cfg.T,
                          dt)}


def cold_stage_ms(moe, shape, cfg, layer, us, stream, n):
    """Median time of the router (moe_route) and of the combine (moe_combine)
    launched alone, each after a 512 MiB write that evicts L2 and the 256 MB
    Infinity Cache, so that every operand comes from HBM.  The router cycles
    through the resident batches; the combine reads the real routing of batch 0
    (its inverse permutation and gates) and seeded expert-output rows."""
    import numpy as np
    import torch
    T, K, Nr, d = cfg.T, cfg.K, cfg.Nr, cfg.d
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    scores = torch.empty((T, Nr), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    w = torch.empty((T, K), dtype=torch.float32, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
    rws = torch.empty(max(moe.moe_workspace_bytes(shape, moe.MOE_WS_ROUTE), 256), dtype=torch.uint8, device="cuda")
    for k in range(n):
        flush.fill_(k & 255)
        ev[2 * k].record(stream)
        moe.moe_route(shape, us[k % len(us)], layer.gate_w, layer.bias, None, scores, idx, w, rws, stream)
        ev[2 * k + 1].record(stream)
    torch.cuda.synchronize()
    router = float(np.median([ev[2 * k].elapsed_time(ev[2 * k + 1]) for k in range(n)]))
    moe.moe_route(shape, us[0], layer.gate_w, layer.bias, None, scores, idx, w, rws, stream)
    counts, offsets = (torch.empty(m, dtype=torch.int32, device="cuda") for m in (Nr, Nr + 1))
    perm, inv = (torch.empty(T * K, dtype=torch.int32, device="cuda") for _ in range(2))
    pws = torch.empty(max(moe.moe_workspace_bytes(shape, moe.MOE_WS_PERMUTE), 256), dtype=torch.uint8, device="cuda")
    moe.moe_permute(shape, idx, None, counts, offsets, perm, inv, None, None, pws, stream)
    dt = us[0].dtype
    gen = torch.Generator(device="cuda").manual_seed(7)
    y = torch.randn((T * K, d), generator=gen, device="cuda").to(dt)
    ysh = torch.randn((cfg.Ns, T, d), generator=gen, device="cuda").to(dt) if cfg.Ns else None
    out = torch.empty((T, d), dtype=dt, device="cuda")
    for k in range(n):
        flush.fill_(k & 255)
        ev[2 * k].record(stream)
        moe.moe_combine(shape, y, inv, w, ysh, None, out, stream)
        ev[2 * k + 1].record(stream)
    torch.cuda.synchronize()
    combine = float(np.median([ev[2 * k].elapsed_time(ev[2 * k + 1]) for k in range(n)]))
    del flush, y, ysh
    torch.cuda.empty_cache()
    return {"router": router, "combine": combine}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 20; 10 for v3_skew, whose run is 10 bias-update steps)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="v3_prefill")
    ap.add_argument("--cpu-tokens", type=int, default=640, help="tokens in the CPU-oracle sample (0: skip)")
    ap.add_argument("--backward", action="store_true",
                    help="time forward + backward (input, centroid and expert-weight gradients) per step")
    ap.add_argument("--recompute-swiglu", action="store_true",
                    help="with --backward: recompute the SwiGLU inputs in the backward instead of keeping them "
                         "from the forward (MOE_SAVE_SWIGLU_INPUTS, the default for --backward)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (reference kernel for HBM counter scaling)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the layer runs on a single GPU only (expert-parallel sharding across GPUs is "
              "not built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import moe_synth as syn
    import mixture_experts_layer_35_amd as moe
    from mixture_experts_layer_35_amd.layer import MoeLayer, to_device

    cfg = syn.CONFIGS[args.config]
    if args.steps is None:
        args.steps = syn.SKEW_STEPS if cfg.skew else 20
    torch.cuda.set_device(0)
    moe.lib()
    t_gen = time.perf_counter()
    inp = syn.layer_inputs(cfg)
    t_gen = time.perf_counter() - t_gen
    print("# inputs generated in %.1f s" % t_gen, file=sys.stderr, flush=True)
    # a training step keeps the SwiGLU inputs for the backward (fp32 a | b per expert row)
    saved = args.backward and not args.recompute_swiglu
    bwd_kernels = dict(BWD_KERNELS, bwd_swiglu="swiglu_grad_kernel") if saved else BWD_KERNELS
    shape = moe.make_shape(cfg.T, cfg.d, cfg.Nr, cfg.Ns, cfg.G, cfg.Mg, cfg.K, cfg.I, cfg.dtype,
                           flags=moe.MOE_SAVE_SWIGLU_INPUTS if saved else 0)
    layer = MoeLayer.from_host(shape, inp["gate_w"], inp["bias"], inp["wg"], inp["wu"], inp["wd"], inp["swg"],
                               inp["swu"], inp["swd"])
    T = cfg.T
    if cfg.skew:
        # the skewed-load run: step s routes batch s (seed 1000 + s) and then
        # moves the selection bias against that step's expert loads
        batches = [syn.hidden(cfg, seed=syn.SKEW_STEP_SEED + s) for s in range(syn.SKEW_STEPS)]
        inp["u"] = batches[0]
        us = [to_device(b) for b in batches]
    else:
        # several resident batches (batch 0 is the recipe's u), cycled through by the steps
        us = [to_device(inp["u"])] + [to_device(syn.hidden(cfg, seed=ROTATE_SEED + k))
                                      for k in range(1, rotation_batches(cfg))]
    out = torch.empty((T, cfg.d), dtype=us[0].dtype, device="cuda")
    counts = torch.zeros((max(args.steps, 1), cfg.Nr), dtype=torch.int32, device="cuda")
    ws = layer.workspace(T)
    stream = torch.cuda.current_stream()
    bias0 = layer.bias.clone()

    bw = None
    if args.backward:
        # weight transposes are weight preparation (once per weight update), timed apart
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        (rt, rts), (st, sts) = layer.transposed_weights(stream)
        e1.record()
        torch.cuda.synchronize()
        # weight gradients in the activation format (bf16 for e4m3 weights)
        grad_like = lambda ws: tuple(torch.empty(w.shape, dtype=us[0].dtype, device="cuda") for w in ws)
        bw = dict(rt=rt, rts=rts, st=st, sts=sts, transpose_ms=e0.elapsed_time(e1),
                  dout=to_device(syn.grad_output(cfg)), du=torch.empty_like(us[0]),
                  dgate=torch.empty((cfg.Nr, cfg.d), dtype=torch.float32, device="cuda"),
                  dr=grad_like(layer.routed_w),
                  ds=grad_like(layer.shared_w) if cfg.Ns else None,
                  ws=torch.empty(max(moe.moe_backward_workspace_bytes(shape), 256), dtype=torch.uint8,
                                 device="cuda"))

    def step(k, events=None, bevents=None):
        moe.moe_forward_timed(shape, us[k % len(us)], layer.gate_w, layer.bias, layer.routed_w, layer.routed_s,
                              layer.shared_w, layer.shared_s, out, None, None, counts[k], None, ws, stream, events)
        if bw is not None:
            moe.moe_backward_timed(shape, us[k % len(us)], layer.gate_w, layer.routed_w, layer.routed_s, bw["rt"],
                                   bw["rts"], layer.shared_w, layer.shared_s, bw["st"], bw["sts"], ws, bw["dout"],
                                   bw["du"], bw["dgate"], bw["dr"], bw["ds"], None, bw["ws"], stream, bevents)
        if cfg.skew:
            moe.moe_bias_update(shape, counts[k], layer.bias, syn.SKEW_GAMMA, stream)

    for _ in range(args.warmup):
        step(0)
    layer.bias.copy_(bias0)
    # events: created and recorded once so that their handles exist

    def event_rows(n):
        rows = []
        for _ in range(args.steps):
            row = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
            for e in row:
                e.record()
            rows.append(row)
        return rows

    evs = event_rows(6)
    bevs = event_rows(10) if bw is not None else None
    torch.cuda.synchronize()
    handles = [[e.cuda_event for e in row] for row in evs]
    bhandles = [[e.cuda_event for e in row] for row in bevs] if bevs else [None] * args.steps

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k, handles[k], bhandles[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1000.0 / args.steps
    stage_ms = {name: float(np.mean([evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(args.steps)]))
                for i, name in enumerate(STAGES)}
    bstage_ms = None
    if bevs:
        bstage_ms = {name: float(np.mean([bevs[k][i].elapsed_time(bevs[k][i + 1]) for k in range(args.steps)]))
                     for i, name in enumerate(BWD_STAGES)}

    cold = cold_stage_ms(moe, shape, cfg, layer, us, stream, n=max(5, min(args.steps, 20))) if bw is None else None
    cnt = counts.cpu().numpy()
    n_touched = int(np.mean([(c > 0).sum() for c in cnt]))
    skew = None
    if cfg.skew:
        mean = T * cfg.K / cfg.Nr
        skew = {"gamma": syn.SKEW_GAMMA, "step_seeds": "u of step s drawn with seed %d + s" % syn.SKEW_STEP_SEED,
                "max_over_mean": [round(float(c.max() / mean), 3) for c in cnt],
                "min_over_mean": [round(float(c.min() / mean), 3) for c in cnt],
                "step_ms": [round(float(evs[k][0].elapsed_time(evs[k][5])), 4) for k in range(args.steps)],
                "bias_range_after": [round(float(layer.bias.min()), 4), round(float(layer.bias.max()), 4)]}
    if bw is None:
        alg = algorithmic(cfg, n_touched, saved)
        dom = max(("ffn_gate_up", "ffn_down"), key=lambda k: stage_ms[k])
        t_dom = stage_ms[dom] / 1000.0
    else:
        alg = algorithmic_bwd(cfg, n_touched, saved)
        dom = max(BWD_STAGES, key=lambda k: bstage_ms[k])
        t_dom = bstage_ms[dom] / 1000.0
    flops, nbytes = alg[dom]
    peak_f = PEAK_TFLOPS[cfg.dtype]
    ridge = peak_f * 1e12 / (PEAK_HBM_GBS * 1e9)
    if flops / nbytes < ridge:
        roof = {"bound": "hbm", "achieved": round(nbytes / t_dom / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(flops / t_dom / 1e12, 1), "peak": peak_f, "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    tr = traffic_from_profile(cfg, dom) if bw is None else traffic_from_profile(cfg, bwd_kernels[dom], True)
    roof["traffic"] = tr
    roof["mfma_util_pct"] = (mfma_util_from_profile(cfg, dom) if bw is None
                             else mfma_util_from_profile(cfg, bwd_kernels[dom], True))
    roof["kernel"] = dom
    roof["algorithmic_bytes"] = nbytes
    roof["algorithmic_flops"] = flops
    roof["kernel_ms"] = round(t_dom * 1000.0, 4)
    bwd_stages = None
    if bw is not None:
        bwd_stages = {}
        for name in BWD_STAGES:
            f, nb = alg[name]
            t = bstage_ms[name] / 1000.0
            bwd_stages[name] = {"ms": round(bstage_ms[name], 4), "algorithmic_bytes": int(nb),
                                "algorithmic_flops": f,
                                "GB/s": round(nb / t / 1e9, 1) if t > 0 else None,
                                "TFLOP/s": round(f / t / 1e12, 1) if t > 0 else None,
                                "traffic": traffic_from_profile(cfg, bwd_kernels[name], True)}

    hbm_stages = {}
    for name, nb in stage_bytes(cfg).items():
        gbs = nb / (stage_ms[name] / 1000.0) / 1e9
        hbm_stages[name] = {"algorithmic_bytes": int(nb), "ms": round(stage_ms[name], 4), "GB/s": round(gbs, 1),
                            "frac": round(gbs / PEAK_HBM_GBS, 4),
                            "traffic": traffic_from_profile(cfg, STAGE_KERNELS[name])}
        if cold and name in cold:
            # the same call launched alone after a 512 MiB write (no operand in any cache)
            cg = nb / (cold[name] / 1000.0) / 1e9
            hbm_stages[name]["cold"] = {"ms": round(cold[name], 4), "GB/s": round(cg, 1),
                                        "frac": round(cg / PEAK_HBM_GBS, 4)}
    # "% attainable": the layer's algorithmic flops against min(MFMA peak, AI x HBM peak),
    # with AI over the algorithmic bytes of every stage of the step
    fwd_alg = algorithmic(cfg, n_touched, saved)
    layer_bytes = sum(stage_bytes(cfg).values()) + sum(b for _, b in fwd_alg.values())
    layer_flops = T * cfg.flops_per_token
    if bw is not None:
        layer_bytes += sum(b for _, b in alg.values())
        layer_flops += sum(f for name, (f, _) in alg.items() if name in ("bwd_dh", "bwd_swiglu", "bwd_dx",
                                                                         "wgrad_down", "wgrad_gate_up"))
    tflops = layer_flops / (ms / 1000.0) / 1e12
    attainable = min(peak_f, layer_flops / layer_bytes * PEAK_HBM_GBS / 1000.0)
    # per-step GPU time from the stage events (first to last event of each step)
    step_gpu = [evs[k][0].elapsed_time(evs[k][5]) + (bevs[k][0].elapsed_time(bevs[k][9]) if bevs else 0.0)
                for k in range(args.steps)]
    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    cpu = None
    if args.cpu_tokens > 0:
        cpu = cpu_baseline(cfg, inp, args.cpu_tokens) if bw is None else \
            cpu_baseline_backward(cfg, inp, max(1, args.cpu_tokens // 2))

    wl = ("%s: DeepSeekMoE layer %s, T=%d tokens, d=%d, %d routed + %d shared SwiGLU experts (I=%d), "
          "%d groups / top-%d groups / top-%d experts, %s" % (cfg.name, "forward" if bw is None else
                                                           "forward + backward (input, centroid and "
                                                           "expert-weight gradients)", T, cfg.d, cfg.Nr, cfg.Ns, cfg.I, cfg.G, cfg.Mg,
                                                           cfg.K, {"bf16": "bf16 storage, fp32 accumulation",
                                                                   "fp8": "e4m3 expert GEMMs (1x128 / 128x128 fp32 "
                                                                          "scales), bf16 in/out",
                                                                   "fp32": "fp32"}[cfg.dtype]))
    line = {
        "metric": "MoE layer tokens/s + achieved TFLOP/s (% MFMA peak), V3 shape bf16/fp8" if bw is None else
                  "MoE layer forward+backward tokens/s + achieved TFLOP/s, V3 shape bf16/fp8",
        "value": round(T / (ms / 1000.0), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8e4m3", "fp32": "f32"}[cfg.dtype],
        "data": "synthetic (seeded N(0,1) tokens, N(0,1/fan_in) weights; no trained weights)",
        "config": {"workload": wl, "T": T, "d": cfg.d, "n_routed": cfg.Nr, "n_shared": cfg.Ns, "topk": cfg.K,
                   "n_groups": cfg.G, "topk_groups": cfg.Mg, "inter": cfg.I, "parallelism": "single GPU",
                   **({"swiglu_inputs": "saved by the forward" if saved else "recomputed"} if args.backward else {})},
        "tflops": round(tflops, 2),
        "mfma_peak_frac": round(tflops / peak_f, 4),
        "attainable_tflops": round(attainable, 1),
        "attainable_frac": round(tflops / attainable, 4),
        "step_gpu_ms": {"median": round(float(np.median(step_gpu)), 4), "min": round(float(np.min(step_gpu)), 4),
                        "max": round(float(np.max(step_gpu)), 4)},
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "backward_stages": bwd_stages,
        "backward_ms": round(sum(bstage_ms.values()), 4) if bstage_ms else None,
        "weight_transpose_ms": round(bw["transpose_ms"], 4) if bw is not None else None,
        "experts_touched": n_touched,
        "roofline": roof,
        "hbm_stages": hbm_stages,
        "skew": skew,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
