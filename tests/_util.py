"""Shared helpers for the test suite (no layer arithmetic here)."""
import numpy as np

import moe_synth as syn


def dec(a):
    """Storage -> float64: bf16 bit patterns (uint16) or float32."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def rel_err(got, ref):
    """max |got - ref| / max |ref| over the whole tensor."""
    g, r = dec(got), dec(ref)
    return float(np.abs(g - r).max() / max(np.abs(r).max(), 1e-30))


def shape_of(cfg: syn.LayerConfig, T=None, flags=0, routed_scale=1.0):
    import mixture_experts_layer_35_amd as moe
    return moe.make_shape(cfg.T if T is None else T, cfg.d, cfg.Nr, cfg.Ns, cfg.G, cfg.Mg, cfg.K, cfg.I, cfg.dtype,
                          routed_scale, flags)


def oracle_codes(cfg):
    import oracle
    w = {"fp32": oracle.F32, "bf16": oracle.BF16, "fp8": oracle.E4M3}[cfg.dtype]
    o = oracle.F32 if cfg.dtype == "fp32" else oracle.BF16
    return w, o


def routing_disagreement_is_near_tie(s_ref, bias, idx_ref, idx_gpu, G, tol):
    """True when every expert chosen by one side and not the other has a biased
    affinity (or group score) within tol of a rival on the other side."""
    sb = (s_ref.astype(np.float32) + bias.astype(np.float32)).astype(np.float64)
    a, b = set(idx_ref.tolist()), set(idx_gpu.tolist())
    only_ref, only_gpu = a - b, b - a
    if not only_ref and not only_gpu:
        return True          # same set (order may still differ on a tie)
    gs = sb.size // G
    gsc = []
    for g in range(G):
        v = np.sort(sb[g * gs:(g + 1) * gs])[::-1]
        gsc.append(v[0] + (v[1] if gs > 1 else 0.0))
    for x in only_ref:
        near = any(abs(sb[x] - sb[y]) <= tol or abs(gsc[x // gs] - gsc[y // gs]) <= 2 * tol for y in only_gpu)
        if not near:
            return False
    return True
