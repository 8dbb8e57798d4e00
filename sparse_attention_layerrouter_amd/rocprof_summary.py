"""Condense rocprofv3 CSV output into the short summaries kept under profiles/.

    python -m sparse_attention_layerrouter_amd.rocprof_summary stats DIR
        per-kernel launch count and average / min / max duration from the
        *kernel_stats.csv (and *kernel_trace.csv) files rocprofv3 wrote in DIR.
    python -m sparse_attention_layerrouter_amd.rocprof_summary traffic FETCH_DIR WRITE_DIR \\
            COPY_FETCH_DIR COPY_WRITE_DIR OUT_JSON
        HBM bytes per launch of the hot kernels from FETCH_SIZE / WRITE_SIZE
        passes (KiB per dispatch), each scaled by what the same counter reads
        for a plain 1 GiB read + 1 GiB write elementwise kernel.
    python -m sparse_attention_layerrouter_amd.rocprof_summary mfma DIR PROFILE_JSON OUT_JSON
        matrix-core evidence of the hot kernels from one counter pass with
        SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE
        and SQ_BUSY_CU_CYCLES (plus --kernel-trace for durations): executed MFMA
        flops (MOPS x 512) against the algorithmic flops bench.py --profile
        printed (PROFILE_JSON), the share of SIMD cycles the matrix cores were
        busy, and the clock the kernel ran at.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))

# kernels whose traffic the benchmark reports, by a substring of the demangled name
HOT_KERNELS = {
    "prefill_bf16_fa_131k": ("prefill_bf16_kernel<128, 1>", ("prefill.hip", "fa_common.h")),
    "prefill_bf16_sa_131k": ("prefill_bf16_kernel<128, 2>", ("prefill.hip", "fa_common.h")),
    "decode_bf16_fa_131k": ("decode_bf16_kernel<128, 4, 1, false>", ("decode.hip", "fa_common.h")),
    "decode_bf16_sa_131k": ("decode_bf16_kernel<128, 4, 2, false>", ("decode.hip", "fa_common.h")),
}
COPY_BYTES = 1 << 30


def source_hash(*names) -> str:
    """Hash of kernel sources, so stale counter data can be recognised."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(PKG, "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _rows(directory, suffix):
    out = []
    for path in sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True)):
        with open(path, newline="") as f:
            out.extend(csv.DictReader(f))
    return out


def stats(directory):
    rows = _rows(directory, "kernel_stats.csv")
    if not rows:
        raise SystemExit(f"no kernel_stats.csv under {directory}")
    lines = [f"{'calls':>6} {'avg_us':>11} {'min_us':>11} {'max_us':>11} {'total_%':>8}  kernel"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"{int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>11.2f} "
                     f"{float(r['MinNs']) / 1e3:>11.2f} {float(r['MaxNs']) / 1e3:>11.2f} "
                     f"{float(r['Percentage']):>8.2f}  {r['Name'][:150]}")
    return "\n".join(lines)


def _counter_avg(directory, counter):
    """{kernel name: average counter value per dispatch}."""
    acc = {}
    for r in _rows(directory, "counter_collection.csv"):
        if r.get("Counter_Name") != counter:
            continue
        name = r["Kernel_Name"]
        acc.setdefault(name, []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def _largest(d):
    return max(d.items(), key=lambda kv: kv[1])


def traffic(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, out_json):
    fetch = _counter_avg(fetch_dir, "FETCH_SIZE")
    write = _counter_avg(write_dir, "WRITE_SIZE")
    copy_name, copy_fetch = _largest(_counter_avg(copy_fetch_dir, "FETCH_SIZE"))
    _, copy_write = _largest(_counter_avg(copy_write_dir, "WRITE_SIZE"))
    f_scale = COPY_BYTES / (copy_fetch * 1024.0)
    w_scale = COPY_BYTES / (copy_write * 1024.0)
    out = {"_calibration": {"copy_kernel": copy_name[:120], "copy_bytes_each_way": COPY_BYTES,
                            "fetch_kib": copy_fetch, "write_kib": copy_write,
                            "fetch_scale": f_scale, "write_scale": w_scale}}
    for key, (needle, srcs) in HOT_KERNELS.items():
        fk = [v for k, v in fetch.items() if needle in k]
        wk = [v for k, v in write.items() if needle in k]
        if not fk or not wk:
            continue
        fb = fk[0] * 1024.0 * f_scale
        wb = wk[0] * 1024.0 * w_scale
        out[key] = {"kernel": needle, "fetch_bytes": fb, "write_bytes": wb,
                    "bytes_per_launch": fb + wb, "source_hash": source_hash(*srcs)}
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
    return out


# SIMDs of an MI355X (256 CUs x 4) and XCDs; GRBM_GUI_ACTIVE is reported summed over
# the 8 XCDs, each of which counts the same active cycles
N_SIMD = 1024
N_XCD = 8
MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE",
                 "SQ_BUSY_CU_CYCLES")


def _durations(directory):
    """{dispatch id: duration ns} from the kernel trace written beside the counters."""
    out = {}
    for r in _rows(directory, "kernel_trace.csv"):
        did = r.get("Dispatch_Id")
        if did is None:
            continue
        out[did] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    return out


def mfma(directory, profile_json, out_json):
    with open(profile_json) as f:
        prof = json.load(f)
    alg = prof.get("algorithmic", {})
    dur = _durations(directory)
    per = {}  # kernel key -> dispatch -> {counter: value}
    for r in _rows(directory, "counter_collection.csv"):
        cname = r.get("Counter_Name")
        if cname not in MFMA_COUNTERS:
            continue
        for key, (needle, _) in HOT_KERNELS.items():
            if needle in r["Kernel_Name"]:
                d = per.setdefault(key, {}).setdefault(r["Dispatch_Id"], {})
                d[cname] = d.get(cname, 0.0) + float(r["Counter_Value"])
    out = {"_note": ("per kernel: mean over its dispatches. executed_flop = MOPS_BF16 x 512; "
                     "mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 "
                     "SIMDs), the MfmaUtil expression; clock = GRBM_GUI_ACTIVE / 8 / kernel "
                     "duration; cu_busy = SQ_BUSY_CU_CYCLES x 4 / (GRBM_GUI_ACTIVE / 8 x 256)"),
           "_workload": {k: v for k, v in prof.items() if k != "algorithmic"}}
    for key, dispatches in per.items():
        n = len(dispatches)
        mean = {c: sum(d.get(c, 0.0) for d in dispatches.values()) / n for c in MFMA_COUNTERS}
        durs = [dur[i] for i in dispatches if i in dur]
        dns = sum(durs) / len(durs) if durs else None
        gui = mean["GRBM_GUI_ACTIVE"] / N_XCD
        e = {"kernel": HOT_KERNELS[key][0], "dispatches": n, "counters_mean": mean,
             "duration_us": dns / 1e3 if dns else None,
             "executed_flop": mean["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0,
             "mfma_busy": mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * N_SIMD) if gui else None,
             "cu_busy": mean["SQ_BUSY_CU_CYCLES"] * 4.0 / (gui * 256) if gui else None,
             "clock_ghz": gui / dns if dns else None}
        a = alg.get(key, {}).get("flop")
        if a:
            e["algorithmic_flop"] = a
            e["executed_over_algorithmic"] = e["executed_flop"] / a
            if dns:
                e["algorithmic_tflops"] = a / dns / 1e3
                # the same rate against the peak at the clock the kernel ran at
                e["peak_at_clock_tflops"] = 256 * 4096 * e["clock_ghz"] * 1e9 / 1e12
        e["source_hash"] = source_hash(*HOT_KERNELS[key][1])
        out[key] = e
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
    return out


if __name__ == "__main__":
    if len(sys.argv) >= 3 and sys.argv[1] == "stats":
        print(stats(sys.argv[2]))
    elif len(sys.argv) == 7 and sys.argv[1] == "traffic":
        print(json.dumps(traffic(*sys.argv[2:7]), indent=1))
    elif len(sys.argv) == 5 and sys.argv[1] == "mfma":
        print(json.dumps(mfma(*sys.argv[2:5]), indent=1))
    else:
        print(__doc__)
        sys.exit(2)
