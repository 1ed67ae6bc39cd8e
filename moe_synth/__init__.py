"""Seeded synthetic inputs for the DeepSeekMoE layer (shared by tests and bench).

This module only draws random numbers and stores them in the layer's input
formats.  It holds none of the layer's arithmetic, and imports neither the
GPU library nor the oracle, so both sides can consume the same inputs.

Recipe (shapes from §4.2 of the "DeepSeek-V3 Technical Report" page; trained
weights and the training corpus are not available, so normal draws stand in):
  * u ~ N(0, 1)                        hidden states, [T, d]
  * gate_w (centroids e_i) ~ N(0, 1/d) [Nr, d]
  * W_gate, W_up ~ N(0, 1/d)           [n, I, d]   (fan_in = d)
  * W_down ~ N(0, 1/I)                 [n, d, I]   (fan_in = I)
  * bias: zeros, or U(-0.1, 0.1) for the tiny fp32 layer
  * skewed-load layer: centroid row i scaled by a calibrated sigma_i so that
    expert popularity follows a flattened Zipf(1.2) whose hottest expert gets
    8x the mean load (calibrate_skew.py); step s of its bias-update run
    draws u with seed 1000 + s
Every tensor (and every expert's matrix) has its own numpy PCG64 stream seeded
by the tuple (seed, tag, index); draws are float32 and are rounded to nearest
even into bf16 when the layer stores bf16.  bf16 arrays are returned as uint16
bit patterns.
"""
from __future__ import annotations

import dataclasses
import json
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))

TAG_U, TAG_GATE, TAG_BIAS, TAG_WG, TAG_WU, TAG_WD, TAG_SWG, TAG_SWU, TAG_SWD, TAG_SCORES, TAG_DOUT = range(1, 12)


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    d: int
    Nr: int
    G: int
    Mg: int
    K: int
    Ns: int
    I: int
    dtype: str            # "fp32" | "bf16" | "fp8"
    bias: str = "zero"    # "zero" | "uniform"
    seed: int = 0
    skew: bool = False

    @property
    def flops_per_token(self) -> int:
        """Algorithmic FLOPs per token: router 2*d*Nr plus 6*d*I for each of
        the K routed and Ns shared experts (three d x I products)."""
        return 2 * self.d * self.Nr + (self.K + self.Ns) * 6 * self.d * self.I


CONFIGS = {
    "tiny": LayerConfig("tiny", T=256, d=256, Nr=16, G=4, Mg=2, K=2, Ns=1, I=128, dtype="fp32", bias="uniform"),
    "v3_prefill": LayerConfig("v3_prefill", T=4096, d=7168, Nr=256, G=8, Mg=4, K=8, Ns=1, I=2048, dtype="bf16"),
    "v3_decode": LayerConfig("v3_decode", T=128, d=7168, Nr=256, G=8, Mg=4, K=8, Ns=1, I=2048, dtype="bf16"),
    "v3_fp8": LayerConfig("v3_fp8", T=16384, d=7168, Nr=256, G=8, Mg=4, K=8, Ns=1, I=2048, dtype="fp8"),
    "v3_skew": LayerConfig("v3_skew", T=8192, d=7168, Nr=256, G=8, Mg=4, K=8, Ns=1, I=2048, dtype="bf16",
                           skew=True),
}


def _rng(seed, tag, index=0):
    return np.random.default_rng([int(seed), int(tag), int(index)])


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs).
    torch's CPU conversion is used for speed; it rounds the same way."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    try:
        import torch
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    except ImportError:
        b = x.view(np.uint32)
        r = ((b >> 16) & 1) + np.uint32(0x7FFF)
        return ((b + r) >> 16).astype(np.uint16)


def normal(shape, std, seed, tag, index=0, store="fp32"):
    a = _rng(seed, tag, index).standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
    if std != 1.0:
        a *= np.float32(std)
    return to_bf16_bits(a) if store == "bf16" else a


def _stack(shape_one, n, std, seed, tag, store, threads):
    out = np.empty((n,) + tuple(shape_one), dtype=np.uint16 if store == "bf16" else np.float32)

    def fill(e):
        out[e] = normal(shape_one, std, seed, tag, e, store)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(fill, range(n)))
    return out


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


SKEW_STEP_SEED = 1000
SKEW_STEPS = 10
SKEW_GAMMA = 0.001


def skew_sigma(cfg: LayerConfig) -> np.ndarray:
    """Per-expert row scales of the centroids that make expert popularity
    follow the skewed target of the skewed-load workload (calibrated once by
    calibrate_skew.py and stored in skew_sigma.json)."""
    with open(os.path.join(_HERE, "skew_sigma.json")) as f:
        table = json.load(f)
    assert table["Nr"] == cfg.Nr and table["d"] == cfg.d
    return np.asarray(table["sigma"], dtype=np.float32)


def store_of(cfg: LayerConfig) -> str:
    """Storage of u, centroids and master expert weights."""
    return "fp32" if cfg.dtype == "fp32" else "bf16"


def hidden(cfg: LayerConfig, seed=None, T=None):
    seed = cfg.seed if seed is None else seed
    T = cfg.T if T is None else T
    return normal((T, cfg.d), 1.0, seed, TAG_U, 0, store_of(cfg))


def router_params(cfg: LayerConfig, seed=None, sigma=None):
    """(gate_w [Nr, d], bias [Nr] fp32).  For the skewed-load workload each
    centroid row i is scaled by sigma[i] (the calibrated table unless
    `sigma` is given) before rounding to the storage format."""
    seed = cfg.seed if seed is None else seed
    g = normal((cfg.Nr, cfg.d), 1.0 / np.sqrt(cfg.d), seed, TAG_GATE, 0, "fp32")
    if cfg.skew or sigma is not None:
        g *= (skew_sigma(cfg) if sigma is None else np.asarray(sigma, np.float32))[:, None]
    if store_of(cfg) == "bf16":
        g = to_bf16_bits(g)
    if cfg.bias == "uniform":
        b = _rng(seed, TAG_BIAS).uniform(-0.1, 0.1, cfg.Nr).astype(np.float32)
    else:
        b = np.zeros(cfg.Nr, np.float32)
    return g, b


def expert_weights(cfg: LayerConfig, n=None, shared=False, seed=None, threads=None):
    """(W_gate [n, I, d], W_up [n, I, d], W_down [n, d, I]) master weights in
    the config's storage (float32 or bf16 bits)."""
    seed = cfg.seed if seed is None else seed
    threads = threads or default_threads()
    n = (cfg.Ns if shared else cfg.Nr) if n is None else n
    tg, tu, td = (TAG_SWG, TAG_SWU, TAG_SWD) if shared else (TAG_WG, TAG_WU, TAG_WD)
    st = store_of(cfg)
    wg = _stack((cfg.I, cfg.d), n, 1.0 / np.sqrt(cfg.d), seed, tg, st, threads)
    wu = _stack((cfg.I, cfg.d), n, 1.0 / np.sqrt(cfg.d), seed, tu, st, threads)
    wd = _stack((cfg.d, cfg.I), n, 1.0 / np.sqrt(cfg.I), seed, td, st, threads)
    return wg, wu, wd


def grad_output(cfg: LayerConfig, seed=None, T=None):
    """Upstream gradient dL/d(layer output) [T, d]: unit normal, in the
    activation storage (the backward takes it in the layer's own format)."""
    seed = cfg.seed if seed is None else seed
    T = cfg.T if T is None else T
    return normal((T, cfg.d), 1.0, seed, TAG_DOUT, 0, store_of(cfg))


def random_scores(T, Nr, seed, tag_index=0):
    """fp32 affinities in (0, 1) for selection-only tests (the same array is
    handed to both implementations)."""
    return _rng(seed, TAG_SCORES, tag_index).uniform(0.0, 1.0, (T, Nr)).astype(np.float32)


def layer_inputs(cfg: LayerConfig, seed=None, threads=None):
    """All inputs of one layer call as a dict of numpy arrays."""
    gate_w, bias = router_params(cfg, seed)
    rg, ru, rd = expert_weights(cfg, seed=seed, threads=threads)
    sg, su, sd = expert_weights(cfg, shared=True, seed=seed, threads=threads) if cfg.Ns else (None, None, None)
    return dict(u=hidden(cfg, seed), gate_w=gate_w, bias=bias, wg=rg, wu=ru, wd=rd, swg=sg, swu=su, swd=sd)
