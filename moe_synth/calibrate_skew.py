"""Writes skew_sigma.json: per-expert scales of the router centroids for the
skewed-load V3 layer (T = 8192, bf16).

Target load shares.  Expert popularity should follow Zipf with exponent 1.2
while the hottest expert gets about 8x the mean load.  A pure Zipf(1.2) over
256 ranks would give the hottest expert ~65x the mean, which top-8 routing
cannot produce (an expert takes at most one of a token's 8 slots, so at most
32x the mean).  The target is therefore the flattened law
    p_r  proportional to  (r + q)^(-1.2),   r = 1..Nr,
with q solved so that Nr * p_1 = 8.  Ranks go to experts through a seeded
permutation.

Calibration.  A larger centroid norm widens an expert's logits and wins it
more top-k picks, so row i of the centroids is scaled by sigma_i and sigma is
refined by the damped fixed-point step
    log sigma_i <- log sigma_i + eta * log(p_i / phat_i),
where phat is the load share the oracle router selects on a calibration batch
(seed 999, 8192 tokens, zero bias).  The share is a steep function of sigma
(an expert wins through the upper tail of its logits), so eta adapts: a step
that makes the L1 distance to the target worse is undone and eta halved,
otherwise eta grows by 1.25.  The best sigma found is kept; the run stops
once the hottest expert is within 5% of 8x the mean and the L1 distance is
below 0.05.

Only the oracle router is called.  Run from the repository root:
    python3 -m moe_synth.calibrate_skew
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import moe_synth as syn  # noqa: E402
import oracle  # noqa: E402

ZIPF_S = 1.2
HOT_OVER_MEAN = 8.0
CAL_SEED = 999
RANK_SEED = 7


def target_shares(Nr):
    r = np.arange(1, Nr + 1, dtype=np.float64)

    def hot(q):
        p = (r + q) ** -ZIPF_S
        return Nr * p[0] / p.sum()

    lo, hi = 0.0, 1000.0          # hot() falls as q grows
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if hot(mid) > HOT_OVER_MEAN:
            lo = mid
        else:
            hi = mid
    q = 0.5 * (lo + hi)
    p = (r + q) ** -ZIPF_S
    return q, p / p.sum()


def main():
    cfg = syn.CONFIGS["v3_skew"]
    q, p_rank = target_shares(cfg.Nr)
    perm = np.random.default_rng([RANK_SEED]).permutation(cfg.Nr)     # expert perm[r] has rank r
    p = np.empty(cfg.Nr)
    p[perm] = p_rank
    u = syn.hidden(cfg, seed=CAL_SEED)
    def measure(sigma):
        g, _ = syn.router_params(cfg, sigma=sigma.astype(np.float32))
        _, idx, _ = oracle.route(u, g, np.zeros(cfg.Nr, np.float32), G=cfg.G, Mg=cfg.Mg, K=cfg.K)
        cnt = np.bincount(idx.ravel(), minlength=cfg.Nr).astype(np.float64)
        return cnt, np.abs(cnt / cnt.sum() - p).sum()

    sigma = np.ones(cfg.Nr, np.float64)
    cnt, l1 = measure(sigma)
    best = (l1, sigma.copy(), cnt.max() / cnt.mean())
    eta = 0.1
    for it in range(80):
        phat = np.maximum(cnt, 0.5) / cnt.sum()
        trial = sigma * np.exp(eta * np.log(p / phat))
        trial /= np.exp(np.log(trial).mean())          # keep the geometric mean at 1
        tcnt, tl1 = measure(trial)
        hot = tcnt.max() / tcnt.mean()
        print("iter %2d eta %.3f: hottest %.2fx mean, coldest %.2fx, L1 %.4f" % (it, eta, hot,
                                                                                tcnt.min() / tcnt.mean(), tl1),
              flush=True)
        if tl1 < l1:
            sigma, cnt, l1 = trial, tcnt, tl1
            eta = min(eta * 1.25, 1.0)
            if l1 < best[0]:
                best = (l1, sigma.copy(), hot)
            if abs(hot / HOT_OVER_MEAN - 1) < 0.05 and l1 < 0.05:
                break
        else:
            eta *= 0.5
            if eta < 1e-3:
                break
    l1, sigma, hot = best
    out = {"Nr": cfg.Nr, "d": cfg.d, "zipf_s": ZIPF_S, "q": q, "hot_over_mean_target": HOT_OVER_MEAN,
           "calibration": {"seed": CAL_SEED, "T": cfg.T, "rank_seed": RANK_SEED, "hot_over_mean": hot, "l1": l1},
           "sigma": [float(np.float32(x)) for x in sigma]}
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "skew_sigma.json"), "w") as f:
        json.dump(out, f, indent=1)
    print("q = %.3f, hottest %.2fx, L1 %.4f" % (q, hot, l1))


if __name__ == "__main__":
    main()
