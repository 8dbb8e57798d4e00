"""Condense rocprofv3 CSV output into the short summaries kept under profiles/.

    python -m sparse_attention_layerrouter_amd.rocprof_summary stats DIR
        per-kernel launch count and average / min / max duration from the
        *kernel_stats.csv (and *kernel_trace.csv) files rocprofv3 wrote in DIR.
    python -m sparse_attention_layerrouter_amd.rocprof_summary grids DIR NAME_SUBSTRING
        for the kernels whose name contains NAME_SUBSTRING: launch count and
        average / min / max duration per grid size, from the *kernel_trace.csv
        files (a kernel launched at several problem sizes in one run, e.g. the
        131072-token FA prefill layer beside the context sweep's).
    python -m sparse_attention_layerrouter_amd.rocprof_summary traffic FETCH_DIR WRITE_DIR \\
            COPY_FETCH_DIR COPY_WRITE_DIR OUT_JSON
        HBM bytes per launch of the hot kernels from FETCH_SIZE / WRITE_SIZE
        passes (KiB per dispatch), each scaled by what the same counter reads
        for a plain 1 GiB read + 1 GiB write elementwise kernel.
    python -m sparse_attention_layerrouter_amd.rocprof_summary counters DIR [DIR ...] \\
            PROFILE_JSON OUT_JSON
        per hot kernel, the mean of every counter of one or more counter passes
        (each run with --kernel-trace for durations) over its dispatches, and what
        follows from them: executed MFMA flops (MOPS x 512) against the
        algorithmic flops bench.py --profile printed (PROFILE_JSON), the clock,
        the matrix-core, LDS and VALU busy shares, LDS read bytes per clock,
        bank conflicts and the share of wave cycles spent waiting.
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
# (the launch header holds the decode split policy, which sets a decode launch's grid)
HOT_KERNELS = {
    "prefill_bf16_fa_131k": ("prefill_bf16_kernel<128, 1>", ("prefill.hip", "fa_common.h")),
    "prefill_bf16_sa_131k": ("prefill_bf16_kernel<128, 2>", ("prefill.hip", "fa_common.h")),
    "decode_bf16_fa_131k": ("decode_bf16_kernel<128, 4, 1, false, false>",
                            ("decode.hip", "fa_common.h", "fa_launch.h")),
    "decode_bf16_sa_131k": ("decode_bf16_kernel<128, 4, 2, false, true>",
                            ("decode.hip", "fa_common.h", "fa_launch.h")),
    "xa_score_131k": ("xa_score_kernel<128, 8>", ("xattn.hip", "fa_common.h")),
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


def grids(directory, needle):
    """Per grid size of the kernels matching `needle`: launches and durations."""
    acc = {}
    for r in _rows(directory, "kernel_trace.csv"):
        if needle not in r["Kernel_Name"]:
            continue
        key = (int(r["Grid_Size_X"]), int(r["Grid_Size_Y"]), int(r["Grid_Size_Z"]),
               int(r["Workgroup_Size_X"]))
        dur = (float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) / 1e3
        acc.setdefault(key, []).append(dur)
    if not acc:
        raise SystemExit(f"no launch of a kernel matching {needle!r} under {directory}")
    lines = [f"{'calls':>6} {'avg_us':>11} {'min_us':>11} {'max_us':>11}  grid (x, y, z) threads, "
             f"workgroup size  [{needle}]"]
    for key, v in sorted(acc.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{len(v):>6} {sum(v) / len(v):>11.2f} {min(v):>11.2f} {max(v):>11.2f}  "
                     f"({key[0]}, {key[1]}, {key[2]}), {key[3]}")
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


# SIMDs and CUs of an MI355X (256 CUs x 4 SIMDs) and XCDs; GRBM_GUI_ACTIVE is
# reported summed over the 8 XCDs, each of which counts the same active cycles
N_SIMD = 1024
N_CU = 256
N_XCD = 8


def _durations(directory):
    """{dispatch id: duration ns} from the kernel trace written beside the counters."""
    out = {}
    for r in _rows(directory, "kernel_trace.csv"):
        did = r.get("Dispatch_Id")
        if did is None:
            continue
        out[did] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    return out


def counters(directories, profile_json, out_json):
    """Per hot kernel: the mean of every counter over its dispatches (the passes in
    `directories` may collect different counters of the same program), and the
    figures derived from those present."""
    with open(profile_json) as f:
        prof = json.load(f)
    alg = prof.get("algorithmic", {})
    out = {"_note": ("mean over each kernel's dispatches of every counter, per pass; derived: "
                     "executed_flop = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; cycles = "
                     "GRBM_GUI_ACTIVE / 8 (per-XCD active cycles); clock = cycles / "
                     "duration; mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs) "
                     "(the MfmaUtil expression); lds_util = SQ_LDS_IDX_ACTIVE / (cycles x 256 "
                     "CUs) (LdsUtil); lds_read_bytes_per_clk_per_cu = "
                     "SQ_INSTS_LDS_LOAD_BANDWIDTH x 64 / (cycles x 256); valu_busy = "
                     "SQ_ACTIVE_INST_VALU / (cycles x 256) (VALUBusy); wait_fraction = "
                     "SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES"),
           "_workload": {k: v for k, v in prof.items() if k != "algorithmic"}}
    for directory in directories:
        dur = _durations(directory)
        per = {}  # kernel key -> dispatch -> {counter: value}
        for r in _rows(directory, "counter_collection.csv"):
            for key, (needle, _) in HOT_KERNELS.items():
                if needle in r["Kernel_Name"]:
                    d = per.setdefault(key, {}).setdefault(r["Dispatch_Id"], {})
                    c = r["Counter_Name"]
                    d[c] = d.get(c, 0.0) + float(r["Counter_Value"])
        for key, dispatches in per.items():
            e = out.setdefault(key, {"kernel": HOT_KERNELS[key][0],
                                     "source_hash": source_hash(*HOT_KERNELS[key][1]),
                                     "passes": []})
            names = sorted({c for d in dispatches.values() for c in d})
            mean = {c: sum(d.get(c, 0.0) for d in dispatches.values()) / len(dispatches)
                    for c in names}
            durs = [dur[i] for i in dispatches if i in dur]
            dns = sum(durs) / len(durs) if durs else None
            p = {"dispatches": len(dispatches), "counters_mean": mean,
                 "duration_us": dns / 1e3 if dns else None}
            cyc = mean.get("GRBM_GUI_ACTIVE", 0.0) / N_XCD
            if cyc and dns:
                p["clock_ghz"] = cyc / dns
            if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in mean:
                p["executed_flop"] = mean["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0
                a = alg.get(key, {}).get("flop")
                if a:
                    p["algorithmic_flop"] = a
                    p["executed_over_algorithmic"] = p["executed_flop"] / a
                    if dns:
                        p["algorithmic_tflops"] = a / dns / 1e3
            if cyc:
                for name, num, den in (
                        ("mfma_busy", "SQ_VALU_MFMA_BUSY_CYCLES", cyc * N_SIMD),
                        ("lds_util", "SQ_LDS_IDX_ACTIVE", cyc * N_CU),
                        ("valu_busy", "SQ_ACTIVE_INST_VALU", cyc * N_CU)):
                    if num in mean:
                        p[name] = mean[num] / den
                if "SQ_INSTS_LDS_LOAD_BANDWIDTH" in mean:
                    p["lds_read_bytes_per_clk_per_cu"] = (
                        mean["SQ_INSTS_LDS_LOAD_BANDWIDTH"] * 64.0 / (cyc * N_CU))
            if "SQ_WAIT_INST_ANY" in mean and mean.get("SQ_WAVE_CYCLES"):
                p["wait_fraction"] = mean["SQ_WAIT_INST_ANY"] / mean["SQ_WAVE_CYCLES"]
            if "SQ_LDS_BANK_CONFLICT" in mean and mean.get("SQ_LDS_IDX_ACTIVE"):
                p["lds_bank_conflict_per_active"] = (mean["SQ_LDS_BANK_CONFLICT"] /
                                                     mean["SQ_LDS_IDX_ACTIVE"])
            e["passes"].append(p)
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
    return out


if __name__ == "__main__":
    if len(sys.argv) >= 3 and sys.argv[1] == "stats":
        print(stats(sys.argv[2]))
    elif len(sys.argv) == 4 and sys.argv[1] == "grids":
        print(grids(sys.argv[2], sys.argv[3]))
    elif len(sys.argv) == 7 and sys.argv[1] == "traffic":
        print(json.dumps(traffic(*sys.argv[2:7]), indent=1))
    elif len(sys.argv) >= 5 and sys.argv[1] == "counters":
        print(json.dumps(counters(sys.argv[2:-2], sys.argv[-2], sys.argv[-1]), indent=1))
    else:
        print(__doc__)
        sys.exit(2)
