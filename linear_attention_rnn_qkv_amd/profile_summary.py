"""Summaries of rocprofv3 runs of bench.py, and the source fingerprints that
tie measured HBM traffic to the kernel code it was measured on.

Usage (after the rocprofv3 runs listed in the summaries it writes):

    python -m linear_attention_rnn_qkv_amd.profile_summary \\
        --workload long-bf16-T131072 --trace DIR_kt --fetch DIR_f --write DIR_w \\
        --copy-fetch DIR_cf --copy-write DIR_cw --out profiles/

DIR_* are rocprofv3 ``-d`` output directories (CSV format). The copy runs are
``bench.py --calibrate-copy``: a plain device copy of exactly 1 GiB read and
1 GiB written per dispatch, whose FETCH_SIZE / WRITE_SIZE readings give the
factor from counter KiB to bytes.

``--mfma DIR`` adds a run with the matrix-core and LDS counters (MFMA_COUNTERS
below): per kernel, the fraction of the chip's SIMD cycles during which the
matrix cores were busy (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE, which
counts each XCD's active cycles, times the SIMDs per XCD), the MFMA flops the
counters saw (SQ_INSTS_VALU_MFMA_MOPS_* count units of 512 flops) and the share
of LDS-active cycles lost to bank conflicts. They go to
``mfma_counters.<workload>.json`` with the same source fingerprints.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
COPY_BYTES = 1 << 30
# one rocprofv3 --pmc pass (8 SQ counters and one GRBM counter)
MFMA_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F16",
                 "SQ_INSTS_MFMA", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS", "SQ_BUSY_CU_CYCLES",
                 "GRBM_GUI_ACTIVE"]
SIMDS_PER_XCD = 32 * 4  # 32 CUs of 4 SIMDs

# kernel symbol fragment -> (short name, sources its machine code is built from)
KERNELS = {
    "chunk_prep_kernel": ("chunk_prep_kernel", ["chunk_prep.hip", "mfma_tiles.h", "device_common.h",
                                                "gdn_internal.h"]),
    "chunk_state_kernel": ("chunk_state_kernel", ["chunk_state.hip", "mfma_tiles.h", "device_common.h",
                                                  "gdn_internal.h"]),
    "chunk_state_wide_kernel": ("chunk_state_wide_kernel", ["chunk_state_wide.hip", "mfma_tiles.h",
                                                            "device_common.h", "gdn_internal.h"]),
    "chunk_rule_kernel": ("chunk_rule_kernel", ["chunk_rule.hip", "device_common.h", "gdn_internal.h"]),
    "prologue_kernel": ("prologue_kernel", ["prologue.hip", "device_common.h", "gdn_internal.h"]),
    "decode_kernel": ("decode_kernel", ["decode.hip", "device_common.h", "gdn_internal.h"]),
    "gated_norm_kernel": ("gated_norm_kernel", ["gated_norm.hip", "device_common.h", "gdn_internal.h"]),
    "gated_norm_bwd_kernel": ("gated_norm_bwd_kernel", ["backward.hip", "device_common.h", "gdn_internal.h"]),
    "conv_bwd_kernel": ("conv_bwd_kernel", ["backward.hip", "device_common.h", "gdn_internal.h"]),
    "beta_g_bwd_kernel": ("beta_g_bwd_kernel", ["backward.hip", "device_common.h", "gdn_internal.h"]),
    "sum_partials_a": ("sum_partials_a", ["backward.hip", "device_common.h", "gdn_internal.h"]),
    "sum_partials_b": ("sum_partials_b", ["backward.hip", "device_common.h", "gdn_internal.h"]),
    "bwd_prep_kernel": ("bwd_prep_kernel", ["chunk_bwd.hip", "chunk_bwd_common.h", "mfma_tiles.h",
                                            "device_common.h", "gdn_internal.h"]),
    "bwd_states_kernel": ("bwd_states_kernel", ["chunk_bwd.hip", "chunk_bwd_common.h", "mfma_tiles.h",
                                                "device_common.h", "gdn_internal.h"]),
    "bwd_dstate_kernel": ("bwd_dstate_kernel", ["chunk_bwd.hip", "chunk_bwd_common.h", "mfma_tiles.h",
                                                "device_common.h", "gdn_internal.h"]),
    "bwd_grad_kernel": ("bwd_grad_kernel", ["chunk_bwd.hip", "chunk_bwd_common.h", "mfma_tiles.h",
                                            "device_common.h", "gdn_internal.h"]),
    "bwd_grad_mma_kernel": ("bwd_grad_mma_kernel", ["chunk_bwd_mma.hip", "chunk_bwd_common.h", "mfma_tiles.h",
                                                    "device_common.h", "gdn_internal.h"]),
    "bwd_state_passes_kernel": ("bwd_state_passes_kernel", ["chunk_bwd_state_mma.hip", "chunk_bwd_common.h",
                                                            "mfma_tiles.h", "device_common.h", "gdn_internal.h"]),
    "chunk_state_quad_kernel": ("chunk_state_quad_kernel", ["chunk_state.hip", "mfma_tiles.h", "device_common.h",
                                                            "gdn_internal.h"]),
}


def short_name(symbol: str) -> str | None:
    for frag, (name, _) in KERNELS.items():
        # mangled (name + template arguments "I..."), plain, or demangled
        # ("::name(" or "::name<") symbols
        if frag + "I" in symbol or symbol.endswith(frag) or "::" + frag + "(" in symbol or "::" + frag + "<" in symbol:
            return name
    return None


def source_hash(kernel: str) -> str:
    """SHA-256 (first 16 hex digits) of the sources a kernel is built from."""
    h = hashlib.sha256()
    for f in KERNELS[kernel][1]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _csv(d: str, suffix: str) -> list[dict]:
    files = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def kernel_stats(d: str) -> dict:
    out = {}
    for r in _csv(d, "_kernel_stats.csv"):
        n = short_name(r["Name"])
        if n:
            out[n] = {"symbol": r["Name"], "calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3,
                      "min_us": float(r["MinNs"]) / 1e3, "max_us": float(r["MaxNs"]) / 1e3}
    return out


def counter_per_dispatch(d: str, counter: str) -> dict:
    """Mean counter value (KiB) per dispatch, per kernel (short name or symbol)."""
    acc: dict[str, list[float]] = {}
    for r in _csv(d, "_counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        n = short_name(r["Kernel_Name"]) or r["Kernel_Name"]
        acc.setdefault(n, []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-fetch", required=True)
    ap.add_argument("--copy-write", required=True)
    ap.add_argument("--algorithmic", default="{}",
                    help='JSON {kernel: algorithmic bytes per launch} for the comparison column')
    ap.add_argument("--commands", default="", help="text block with the exact commands that were run")
    ap.add_argument("--mfma", default="", help="rocprofv3 --pmc run with MFMA_COUNTERS")
    ap.add_argument("--out", default="profiles")
    a = ap.parse_args()

    stats = kernel_stats(a.trace)
    fetch = counter_per_dispatch(a.fetch, "FETCH_SIZE")
    write = counter_per_dispatch(a.write, "WRITE_SIZE")
    cf = counter_per_dispatch(a.copy_fetch, "FETCH_SIZE")
    cw = counter_per_dispatch(a.copy_write, "WRITE_SIZE")
    copy_key = [k for k in cf if "copyBuffer" in k or "copy" in k.lower()]
    if not copy_key:
        raise SystemExit("no copy kernel in the calibration runs")
    kf = COPY_BYTES / (cf[copy_key[0]] * 1024.0)  # bytes per counted byte, fetch
    kw = COPY_BYTES / (cw[copy_key[0]] * 1024.0)
    algo = json.loads(a.algorithmic)

    traffic = {"workload": a.workload, "fetch_factor": kf, "write_factor": kw,
               "copy_counters_kib": {"FETCH_SIZE": cf[copy_key[0]], "WRITE_SIZE": cw[copy_key[0]]},
               "kernels": {}}
    for k in sorted(set(fetch) & set(write)):
        if k not in KERNELS:
            continue
        rb, wb = fetch[k] * 1024.0 * kf, write[k] * 1024.0 * kw
        traffic["kernels"][k] = {"source_hash": source_hash(k), "read_bytes": rb, "write_bytes": wb,
                                 "bytes": rb + wb, "FETCH_SIZE_kib": fetch[k], "WRITE_SIZE_kib": write[k]}
    os.makedirs(a.out, exist_ok=True)
    with open(os.path.join(a.out, f"hbm_traffic.{a.workload}.json"), "w") as fh:
        json.dump(traffic, fh, indent=1)

    lines = [f"# Kernel durations and HBM traffic, workload {a.workload}", ""]
    if a.commands:
        lines += ["Commands (run from the repository root on one MI355X):", "", "```", a.commands.strip(), "```", ""]
    lines += ["## rocprofv3 --kernel-trace --stats", "",
              "| kernel | calls | avg µs | min µs | max µs |", "|---|---|---|---|---|"]
    for k, v in sorted(stats.items(), key=lambda kv: -kv[1]["avg_us"]):
        lines.append(f"| {k} | {v['calls']} | {v['avg_us']:.1f} | {v['min_us']:.1f} | {v['max_us']:.1f} |")
    # stages of several launches ('+'-joined names): the sum of their averages
    for key in algo:
        parts = key.split("+")
        if len(parts) > 1 and all(q in stats for q in parts):
            lines.append(f"| {key} (sum) | - | {sum(stats[q]['avg_us'] for q in parts):.1f} | - | - |")
    lines += ["", "## HBM bytes per launch (rocprofv3 --pmc, one counter per run)", "",
              f"Calibration: a 1 GiB device copy reads FETCH_SIZE = {cf[copy_key[0]]:.0f} KiB and "
              f"WRITE_SIZE = {cw[copy_key[0]]:.0f} KiB per dispatch, so bytes = FETCH_SIZE x 1024 x "
              f"{kf:.4f} and WRITE_SIZE x 1024 x {kw:.4f}.", "",
              "| kernel | source hash | read GB | write GB | total GB | algorithmic GB | ratio |",
              "|---|---|---|---|---|---|---|"]
    rows = dict(traffic["kernels"])
    for key in algo:
        parts = key.split("+")
        if len(parts) > 1 and all(q in rows for q in parts):
            rows[key] = {"source_hash": "+".join(rows[q]["source_hash"][:6] for q in parts),
                         **{f: sum(rows[q][f] for q in parts) for f in ("read_bytes", "write_bytes", "bytes")}}
    for k, v in rows.items():
        al = algo.get(k)
        ratio = f"{v['bytes'] / al:.3f}" if al else "-"
        alt = f"{al / 1e9:.3f}" if al else "-"
        lines.append(f"| {k} | {v['source_hash']} | {v['read_bytes'] / 1e9:.3f} | {v['write_bytes'] / 1e9:.3f} | "
                     f"{v['bytes'] / 1e9:.3f} | {alt} | {ratio} |")
    if a.mfma:
        mf = {n: counter_per_dispatch(a.mfma, n) for n in MFMA_COUNTERS}
        recs = {}
        for k in sorted(set(mf["SQ_VALU_MFMA_BUSY_CYCLES"]) & set(stats)):
            if k not in KERNELS:
                continue
            busy = mf["SQ_VALU_MFMA_BUSY_CYCLES"][k]
            gui = mf["GRBM_GUI_ACTIVE"][k]
            mops = mf["SQ_INSTS_VALU_MFMA_MOPS_BF16"].get(k, 0.0) + mf["SQ_INSTS_VALU_MFMA_MOPS_F16"].get(k, 0.0)
            lds = mf["SQ_LDS_IDX_ACTIVE"].get(k, 0.0)
            recs[k] = {"source_hash": source_hash(k), "avg_us": stats[k]["avg_us"],
                       "mfma_busy": busy / (gui * SIMDS_PER_XCD) if gui else 0.0,
                       "mfma_instructions": mf["SQ_INSTS_MFMA"].get(k, 0.0),
                       "mfma_16bit_flops": mops * 512.0,
                       "mfma_16bit_TFLOP/s": mops * 512.0 / (stats[k]["avg_us"] * 1e-6) / 1e12,
                       "lds_bank_conflict_share": mf["SQ_LDS_BANK_CONFLICT"].get(k, 0.0) / lds if lds else 0.0,
                       "lds_instructions": mf["SQ_INSTS_LDS"].get(k, 0.0),
                       "counters": {n: mf[n].get(k) for n in MFMA_COUNTERS}}
        with open(os.path.join(a.out, f"mfma_counters.{a.workload}.json"), "w") as fh:
            json.dump({"workload": a.workload, "simds_per_xcd": SIMDS_PER_XCD, "kernels": recs}, fh, indent=1)
        lines += ["", "## Matrix cores and LDS (rocprofv3 --pmc, one pass of the counters below)", "",
                  "Counters: " + ", ".join(MFMA_COUNTERS) + ". MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / "
                  f"(GRBM_GUI_ACTIVE x {SIMDS_PER_XCD}): GRBM_GUI_ACTIVE sums each XCD's active cycles, so this "
                  "is the share of all SIMD cycles of the launch with the matrix core busy (a 16x16x32 "
                  "BF16/FP16 MFMA keeps it busy 16 cycles). MFMA flops = MOPS x 512.", "",
                  "| kernel | source hash | MFMA busy | MFMA instructions | MFMA TFLOP/s (16-bit, counted) | "
                  "LDS cycles lost to bank conflicts |", "|---|---|---|---|---|---|"]
        for k, r in recs.items():
            lines.append(f"| {k} | {r['source_hash']} | {r['mfma_busy']:.3f} | {r['mfma_instructions']:.3g} | "
                         f"{r['mfma_16bit_TFLOP/s']:.1f} | {r['lds_bank_conflict_share']:.3f} |")
    with open(os.path.join(a.out, f"layer_core_kernels.{a.workload}.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
