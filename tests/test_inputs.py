"""The synthetic-input recipe: seeded determinism and the skewed-load
workload's calibrated popularity (no GPU)."""
import json
import os

import numpy as np

import moe_synth as syn
from moe_synth import calibrate_skew


def test_seeded_inputs_are_reproducible_and_independent():
    cfg = syn.CONFIGS["tiny"]
    a, b = syn.layer_inputs(cfg), syn.layer_inputs(cfg)
    for k in a:
        assert (a[k] == b[k]).all()
    assert not np.array_equal(syn.hidden(cfg, seed=1), syn.hidden(cfg, seed=2))
    u = a["u"].astype(np.float64)                       # N(0, 1)
    assert abs(u.mean()) < 0.02 and abs(u.std() - 1) < 0.02
    wd = a["wd"].astype(np.float64)                     # N(0, 1/I)
    assert abs(wd.std() * np.sqrt(cfg.I) - 1) < 0.02
    assert ((a["bias"] >= -0.1) & (a["bias"] <= 0.1)).all()


def test_flattened_zipf_target():
    """p_r ~ (r + q)^-1.2 with the hottest rank at 8x the mean share; the
    coldest rank keeps a non-zero share and shares fall with rank."""
    q, p = calibrate_skew.target_shares(256)
    assert abs(p.sum() - 1) < 1e-12
    assert abs(256 * p[0] - 8.0) < 1e-9
    assert (np.diff(p) < 0).all()
    r = np.arange(1, 257)
    ratio = np.log(p[:-1] / p[1:]) / np.log((r[1:] + q) / (r[:-1] + q))
    assert np.allclose(ratio, 1.2)
    assert 10 < q < 20 and 256 * p[-1] > 0.1


def test_calibrated_skew_realises_the_target():
    """The stored centroid scales make the oracle router pick the hottest
    expert within 5% of 8x the mean load on the calibration batch."""
    import oracle
    cfg = syn.CONFIGS["v3_skew"]
    with open(os.path.join(os.path.dirname(syn.__file__), "skew_sigma.json")) as f:
        table = json.load(f)
    assert table["Nr"] == cfg.Nr and len(table["sigma"]) == cfg.Nr
    u = syn.hidden(cfg, seed=table["calibration"]["seed"])
    g, b = syn.router_params(cfg)
    assert (b == 0).all()
    _, idx, _ = oracle.route(u, g, b, G=cfg.G, Mg=cfg.Mg, K=cfg.K)
    cnt = np.bincount(idx.ravel(), minlength=cfg.Nr)
    assert cnt.sum() == cfg.T * cfg.K
    hot = cnt.max() / cnt.mean()
    assert abs(hot / 8.0 - 1) < 0.05, hot
