"""Summaries of rocprofv3 output for the layer's kernels (plain text tables).

  python -m mixture_experts_layer_35_amd.profsum stats DIR OUT.md --cmd "..."
      per-kernel call count and duration from a `--kernel-trace --stats` run
  python -m mixture_experts_layer_35_amd.profsum pmc FETCH_DIR WRITE_DIR OUT.md --workload NAME --cmd "..." --cmd "..."
      per-kernel HBM bytes per launch from one FETCH_SIZE and one WRITE_SIZE
      pass, scaled by what the same counters read for a 1 GiB device copy
  python -m mixture_experts_layer_35_amd.profsum mfma DIR OUT.md --workload NAME --cmd "..."
      per-kernel MFMA busy fraction (MfmaUtil), MFMA flops executed (MOPS
      counters x 512) and LDS bank-conflict cycles from one counter pass
  python -m mixture_experts_layer_35_amd.profsum counters DIR OUT.md --workload NAME --cmd "..."
      per-kernel average of every counter of one pass (wave-cycle breakdowns)

Only reads CSV files that rocprofv3 wrote; runs nothing on the GPU.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re
from collections import defaultdict

_HERE = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 1 << 30


def short_name(full: str) -> str:
    """Readable kernel name: the expert kernels by their projection, others
    by their function name."""
    m = re.search(r"ffn_kernel<(\d+), (\d+)(?:, (?:true|false))?>", full)
    if m:
        return {0: "ffn_down", 1: "ffn_gate_up", 2: "bwd_swiglu", 3: "bwd_dh", 4: "bwd_dx",
                5: "ffn_gate_up"}[int(m.group(2))]
    # the pass (0: dW_down, 1: dW_gate / dW_up) is the first template argument of the bf16
    # and e4m3 kernels and the second of the fp32 one
    m = re.search(r"wgrad_(?:bf16|fp8)_kernel<(\d+)", full) or re.search(r"wgrad_kernel<\d+, (\d+)>", full)
    if m:
        return "wgrad_gate_up" if m.group(1) == "1" else "wgrad_down"
    if "copyBuffer" in full:
        return "copy_buffer"
    head = full.replace("(anonymous namespace)", "").split("(")[0]
    head = re.sub(r"<.*$", "", head)
    return head.split("::")[-1].replace("void ", "").strip()


def source_hash() -> str:
    """Hash of the kernel sources (PMC figures are void once it changes)."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(os.path.join(_HERE, "csrc"))):
        if f.endswith((".hip", ".h")):
            with open(os.path.join(_HERE, "csrc", f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise SystemExit("no file matches %s" % pattern)
    return hits[0]


def stats(rdir: str, out: str, cmd: list[str]) -> None:
    path = _one(os.path.join(rdir, "**", "*kernel_stats.csv"))
    rows = list(csv.DictReader(open(path)))
    lines = ["# rocprofv3 kernel statistics", "", "Command (from the repository root):", ""]
    lines += ["    " + c for c in cmd]
    lines += ["", "| kernel | calls | avg us | min us | max us | total ms | share |", "|---|---|---|---|---|---|---|"]
    for r in rows:
        lines.append("| %s | %s | %.1f | %.1f | %.1f | %.3f | %.2f%% |" % (
            short_name(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["TotalDurationNs"]) / 1e6, float(r["Percentage"])))
    lines += ["", "Full kernel names:", ""]
    lines += ["- %s: `%s`" % (short_name(r["Name"]), r["Name"]) for r in rows]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def _counter(rdir: str, name: str):
    """{kernel: [values per dispatch]} and the copy kernel's largest value."""
    path = _one(os.path.join(rdir, "**", "*counter_collection.csv"))
    per = defaultdict(list)
    dur = defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != name:
            continue
        k = short_name(r["Kernel_Name"])
        per[k].append(float(r["Counter_Value"]))
        dur[k].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    if "copy_buffer" not in per:
        raise SystemExit("%s: no copy kernel in %s (run bench.py with --copy-calibration)" % (name, path))
    return per, dur, max(per["copy_buffer"])


def pmc(fdir: str, wdir: str, out: str, workload: str, cmd: list[str]) -> None:
    fetch, dur, fcopy = _counter(fdir, "FETCH_SIZE")
    write, _, wcopy = _counter(wdir, "WRITE_SIZE")
    ff = COPY_BYTES / 1024.0 / fcopy
    wf = COPY_BYTES / 1024.0 / wcopy
    lines = ["# HBM traffic per launch (rocprofv3 PMC), workload %s" % workload, "",
             "Commands (from the repository root), one counter per run:", ""]
    lines += ["    " + c for c in cmd]
    lines += ["",
              "Scale factors from a 1 GiB device-to-device copy in the same runs: FETCH_SIZE read %.0f KiB "
              "(x%.3f), WRITE_SIZE read %.0f KiB (x%.3f)." % (fcopy, ff, wcopy, wf),
              "",
              "source_sha256_16: %s" % source_hash(), "",
              "| kernel | launches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes per launch (scaled) | avg us (counter run) |",
              "|---|---|---|---|---|---|"]
    keys = [k for k in fetch if k != "copy_buffer" and k in write]
    keys.sort(key=lambda k: -sum(fetch[k]) / len(fetch[k]))
    for k in keys:
        fa = sum(fetch[k]) / len(fetch[k])
        wa = sum(write[k]) / len(write[k])
        lines.append("| %s | %d | %.0f | %.0f | %.4g | %.1f |" % (k, len(fetch[k]), fa, wa,
                                                                 (fa * ff + wa * wf) * 1024.0,
                                                                 sum(dur[k]) / len(dur[k])))
    lines.append("")
    for k in keys:
        fa = sum(fetch[k]) / len(fetch[k])
        wa = sum(write[k]) / len(write[k])
        lines.append("hbm_bytes_per_launch[%s]: %.6e" % (k, (fa * ff + wa * wf) * 1024.0))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


MFMA_COUNTERS = ("MfmaUtil", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F8",
                 "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE")


def mfma(rdir: str, out: str, workload: str, cmd: list[str]) -> None:
    """MfmaUtil is rocprofv3's derived metric: MFMA-busy cycles over (GPU-active
    cycles x SIMDs), in percent.  MOPS counters count MFMA multiply-adds / 512,
    so x 512 they give the flops the MFMAs executed, padding included."""
    path = _one(os.path.join(rdir, "**", "*counter_collection.csv"))
    per = defaultdict(lambda: defaultdict(list))
    dur = defaultdict(dict)
    for r in csv.DictReader(open(path)):
        k = short_name(r["Kernel_Name"])
        per[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
        dur[k][r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    lines = ["# MFMA and LDS counters per launch (rocprofv3 PMC), workload %s" % workload, "",
             "Command (from the repository root):", ""]
    lines += ["    " + c for c in cmd]
    lines += ["",
              "MfmaUtil = MFMA-busy cycles / (GPU-active cycles x 1024 SIMDs); MFMA flops = (MOPS_BF16 + MOPS_F8) x 512, "
              "padding rows included; the executed rate is those flops over the launch's duration in the counter run. "
              "LDS conflict share = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE (cycles).",
              "",
              "source_sha256_16: %s" % source_hash(), "",
              "| kernel | launches | avg us (counter run) | MfmaUtil % | MFMA flops per launch | executed TFLOP/s "
              "| LDS conflict share |",
              "|---|---|---|---|---|---|---|"]
    def avg(v):
        return sum(v) / len(v) if v else 0.0
    keys = [k for k in per if avg(per[k].get("MfmaUtil", [])) > 0 or avg(per[k].get("SQ_LDS_IDX_ACTIVE", [])) > 0]
    keys.sort(key=lambda k: -avg(list(dur[k].values())))
    util = {}
    for k in keys:
        c = per[k]
        us = avg(list(dur[k].values()))
        fl = (avg(c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", [])) + avg(c.get("SQ_INSTS_VALU_MFMA_MOPS_F8", []))) * 512
        lds = avg(c.get("SQ_LDS_IDX_ACTIVE", []))
        util[k] = avg(c.get("MfmaUtil", []))
        lines.append("| %s | %d | %.1f | %.1f | %.4g | %.1f | %s |" % (
            k, len(dur[k]), us, util[k], fl, fl / (us * 1e-6) / 1e12 if us > 0 else 0.0,
            "%.3f" % (avg(c.get("SQ_LDS_BANK_CONFLICT", [])) / lds) if lds > 0 else "-"))
    lines.append("")
    for k in keys:
        lines.append("mfma_util[%s]: %.2f" % (k, util[k]))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def counters(rdir: str, out: str, workload: str, cmd: list[str], kernels: list[str]) -> None:
    """Average per launch of every counter in one pass, for the named kernels
    (all kernels with a nonzero counter when none are named)."""
    path = _one(os.path.join(rdir, "**", "*counter_collection.csv"))
    per = defaultdict(lambda: defaultdict(list))
    dur = defaultdict(dict)
    names = []
    for r in csv.DictReader(open(path)):
        k = short_name(r["Kernel_Name"])
        if r["Counter_Name"] not in names:
            names.append(r["Counter_Name"])
        per[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
        dur[k][r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    keys = kernels or [k for k in per if any(sum(v) > 0 for v in per[k].values())]
    keys = [k for k in keys if k in per]
    keys.sort(key=lambda k: -sum(dur[k].values()) / len(dur[k]))
    lines = ["# rocprofv3 counters per launch, workload %s" % workload, "", "Command (from the repository root):", ""]
    lines += ["    " + c for c in cmd]
    lines += ["", "source_sha256_16: %s" % source_hash(), "",
              "| kernel | launches | avg us | " + " | ".join(names) + " |",
              "|---|---|---|" + "---|" * len(names)]
    for k in keys:
        vals = [sum(per[k][n]) / len(per[k][n]) if per[k][n] else 0.0 for n in names]
        lines.append("| %s | %d | %.1f | %s |" % (k, len(dur[k]), sum(dur[k].values()) / len(dur[k]),
                                                  " | ".join("%.4g" % v for v in vals)))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("out")
    s.add_argument("--cmd", action="append", default=[])
    p = sub.add_parser("pmc")
    p.add_argument("fetch_dir")
    p.add_argument("write_dir")
    p.add_argument("out")
    p.add_argument("--workload", required=True)
    p.add_argument("--cmd", action="append", default=[])
    m = sub.add_parser("mfma")
    m.add_argument("dir")
    m.add_argument("out")
    m.add_argument("--workload", required=True)
    m.add_argument("--cmd", action="append", default=[])
    c = sub.add_parser("counters")
    c.add_argument("dir")
    c.add_argument("out")
    c.add_argument("--workload", required=True)
    c.add_argument("--cmd", action="append", default=[])
    c.add_argument("--kernel", action="append", default=[])
    a = ap.parse_args()
    if a.mode == "counters":
        counters(a.dir, a.out, a.workload, a.cmd, a.kernel)
    elif a.mode == "stats":
        stats(a.dir, a.out, a.cmd)
    elif a.mode == "mfma":
        mfma(a.dir, a.out, a.workload, a.cmd)
    else:
        pmc(a.fetch_dir, a.write_dir, a.out, a.workload, a.cmd)


if __name__ == "__main__":
    main()
