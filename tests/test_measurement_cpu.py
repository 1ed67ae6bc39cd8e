"""Host-side measurement logic: rocprofv3 summaries (profsum) and the
algorithmic work and profile lookups that bench.py reports.  No GPU."""
import csv
import importlib.util
import os

import pytest

from mixture_experts_layer_35_amd import profsum
import moe_synth as syn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

FFN_UP = "void moe::(anonymous namespace)::ffn_kernel<1, 1, false>(moe::FfnArgs, int)"
FFN_DOWN = "void moe::(anonymous namespace)::ffn_kernel<2, 0, false>(moe::FfnArgs, int)"
FFN_DOWN_WS = "void moe::(anonymous namespace)::ffn_kernel<1, 0, true>(moe::FfnArgs, int)"
WG_BF16 = "void moe::(anonymous namespace)::wgrad_bf16_kernel<1, 2>(moe::WgradArgs, long, long)"
WG_F32 = "void moe::(anonymous namespace)::wgrad_kernel<0, 0>(moe::WgradArgs, long, long)"
COPY = "__amd_rocclr_copyBuffer"


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _write_counters(path, rows):
    """rows: (dispatch, kernel, counter, value, start_ns, end_ns)"""
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
                    "End_Timestamp"])
        for r in rows:
            w.writerow(r)


def test_short_names():
    assert profsum.short_name(FFN_UP) == "ffn_gate_up"
    assert profsum.short_name(FFN_DOWN) == "ffn_down"
    assert profsum.short_name(FFN_DOWN_WS) == "ffn_down"
    assert profsum.short_name("void moe::(anonymous namespace)::ffn_kernel<1, 3>(moe::FfnArgs, int)") == "bwd_dh"
    assert profsum.short_name(WG_BF16) == "wgrad_gate_up"
    assert profsum.short_name(WG_F32) == "wgrad_down"
    assert profsum.short_name(COPY) == "copy_buffer"
    assert profsum.short_name("moe::(anonymous namespace)::perm_scan_kernel(int*, long, int, int*, int*)") \
        == "perm_scan_kernel"


def test_pmc_scales_by_the_copy_kernel(tmp_path):
    # the copy reads 1 GiB: FETCH_SIZE reports half of it (factor 2), WRITE_SIZE all of it (factor 1)
    gib_kib = (1 << 30) / 1024.0
    _write_counters(tmp_path / "f", [(1, COPY, "FETCH_SIZE", gib_kib / 2, 0, 1000),
                                     (2, FFN_UP, "FETCH_SIZE", 1000.0, 0, 3000),
                                     (3, FFN_UP, "FETCH_SIZE", 3000.0, 0, 5000)])
    _write_counters(tmp_path / "w", [(1, COPY, "WRITE_SIZE", gib_kib, 0, 1000),
                                     (2, FFN_UP, "WRITE_SIZE", 10.0, 0, 3000),
                                     (3, FFN_UP, "WRITE_SIZE", 30.0, 0, 5000)])
    out = tmp_path / "pmc.md"
    profsum.pmc(str(tmp_path / "f"), str(tmp_path / "w"), str(out), "w", ["cmd"])
    text = out.read_text()
    # mean fetch 2000 KiB x 2 + mean write 20 KiB x 1
    expect = (2000.0 * 2 + 20.0) * 1024.0
    line = [l for l in text.splitlines() if l.startswith("hbm_bytes_per_launch[ffn_gate_up]")][0]
    assert float(line.split(":")[1]) == pytest.approx(expect, rel=1e-6)
    assert "source_sha256_16: %s" % profsum.source_hash() in text


def test_mfma_summary(tmp_path):
    rows = []
    for d, util, mops, us in ((1, 30.0, 1.0e9, 2000.0), (2, 40.0, 1.0e9, 2000.0)):
        rows += [(d, FFN_UP, "MfmaUtil", util, 0, int(us * 1e3)),
                 (d, FFN_UP, "SQ_INSTS_VALU_MFMA_MOPS_BF16", mops, 0, int(us * 1e3)),
                 (d, FFN_UP, "SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0, 0, int(us * 1e3)),
                 (d, FFN_UP, "SQ_LDS_BANK_CONFLICT", 25.0, 0, int(us * 1e3)),
                 (d, FFN_UP, "SQ_LDS_IDX_ACTIVE", 100.0, 0, int(us * 1e3))]
    _write_counters(tmp_path / "m", rows)
    out = tmp_path / "mfma.md"
    profsum.mfma(str(tmp_path / "m"), str(out), "w", ["cmd"])
    text = out.read_text()
    assert "mfma_util[ffn_gate_up]: 35.00" in text
    row = [l for l in text.splitlines() if l.startswith("| ffn_gate_up")][0].split("|")
    # 1e9 MOPS x 512 flops over 2 ms, and 25 / 100 conflict cycles
    assert float(row[5]) == pytest.approx(5.12e11, rel=1e-3)
    assert float(row[6]) == pytest.approx(5.12e11 / 2e-3 / 1e12, rel=1e-3)
    assert row[7].strip() == "0.250"


def test_profile_lookups_need_the_current_sources(tmp_path):
    bench = _bench()
    bench.ROOT = str(tmp_path)
    os.makedirs(tmp_path / "profiles")
    cfg = syn.CONFIGS["v3_prefill"]
    pmc = tmp_path / "profiles" / "moe_forward_v3_prefill_pmc.md"
    mf = tmp_path / "profiles" / "moe_forward_v3_prefill_mfma.md"
    for h in (profsum.source_hash(), "0" * 16):
        pmc.write_text("source_sha256_16: %s\nhbm_bytes_per_launch[ffn_gate_up]: 1.5e+10\n" % h)
        mf.write_text("source_sha256_16: %s\nmfma_util[ffn_gate_up]: 37.18\n" % h)
        current = h == profsum.source_hash()
        assert bench.traffic_from_profile(cfg, "ffn_gate_up") == (1.5e10 if current else None)
        assert bench.mfma_util_from_profile(cfg, "ffn_gate_up") == (37.18 if current else None)
    assert bench.traffic_from_profile(cfg, "no_such_kernel") is None


def test_algorithmic_work_of_the_expert_kernels():
    bench = _bench()
    cfg = syn.CONFIGS["v3_prefill"]
    rows = cfg.T * (cfg.K + cfg.Ns)
    alg = bench.algorithmic(cfg, 256)
    f_gu, b_gu = alg["ffn_gate_up"]
    f_dn, b_dn = alg["ffn_down"]
    assert f_gu == rows * 4.0 * cfg.I * cfg.d and f_dn == rows * 2.0 * cfg.I * cfg.d
    # 257 experts' gate and up weights, u once, H once (bf16)
    assert b_gu == 257 * 2 * cfg.I * cfg.d * 2 + cfg.T * cfg.d * 2 + rows * cfg.I * 2
    assert b_dn == 257 * cfg.I * cfg.d * 2 + rows * cfg.I * 2 + rows * cfg.d * 2
    # the layer's flops per token: (K + N_s) SwiGLU experts plus the gate GEMM
    assert cfg.flops_per_token == (cfg.K + cfg.Ns) * 6 * cfg.d * cfg.I + 2 * cfg.d * cfg.Nr


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "2"})])
def test_bench_runs_on_one_gpu_only(argv, env):
    """More than one GPU is refused with a message before any GPU work."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv, capture_output=True, text=True,
                       timeout=120, env=dict(os.environ, **env), cwd=ROOT)
    assert r.returncode == 2, r.stderr
    assert "single GPU" in r.stderr and r.stdout == ""
