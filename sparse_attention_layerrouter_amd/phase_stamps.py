"""Clock stamps inside the prefill kernel: where a workgroup's time goes.

    python -m sparse_attention_layerrouter_amd.phase_stamps build
    python -m sparse_attention_layerrouter_amd.phase_stamps run [--seq 131072]

`build` compiles (on the host, in a temporary directory) a copy of the
attention library whose prefill kernel writes clock stamps into device arrays,
and places it beside the package as libfluxattn_stamps.so; the product library
is not touched.  `run` times one FA and one SA layer with the product library
(Llama-3.1-8B shape: 32 query / 8 KV heads, d 128; SA sink 128, window 2048,
block 64; seeded N(0, 1) inputs), then loads the instrumented copy instead in
the same process and runs the same layers again, reading back:

  * rounds: shader-clock stamps (s_memtime) at the phase boundaries of waves 0
    and 4 (one of each ping-pong group) of workgroup 0 of the FA layer, rounds
    500..531 (tiles 1000..1063): the MFMA block, softmax block and barrier
    cycles of each group, and the cycles per round of two tiles;
  * workgroups: realtime stamps (s_memrealtime, 100 MHz) of every workgroup
    of the SA and the FA layer at entry, main-loop start, main-loop end and
    end, with the CU's hardware ids: prologue, loop and epilogue times, and the
    gap between one workgroup's end and the next one's start on the same CU;
  * sa_rounds: realtime stamps at every round start of 8 SA workgroups.

The stamps are stores from one lane at a few points per phase, so the
instrumented kernel runs within a percent or two of the product kernel; the
layer times of both are printed beside the stamps.  Prints one JSON object.
"""
from __future__ import annotations

import argparse
import collections
import ctypes
import json
import math
import os
import shutil
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
STAMPS_LIB = os.path.join(PKG, "libfluxattn_stamps.so")

R0 = 500          # first recorded round of workgroup 0
NROUND = 32       # recorded rounds
SA_WG0 = 4096     # first of the 8 SA workgroups whose every round is stamped
MAX_WG = 65536


def _instrument(src: str) -> str:
    """The prefill source with the stamps added (fails loudly if an anchor moved)."""
    s = src

    def rep(old, new):
        nonlocal s
        assert old in s, f"anchor not found: {old[:60]!r}"
        s = s.replace(old, new, 1)

    rep("namespace fa {\nnamespace {", f"""__device__ unsigned long long g_st[2 * {NROUND} * 8];
__device__ unsigned long long g_wg[{MAX_WG} * 8];
__device__ unsigned long long g_rd[8 * 64];
extern "C" int fa_stamps_read(int which, void *host, size_t bytes)
{{
    if (which == 0) return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_st), bytes);
    if (which == 1) return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_wg), bytes);
    return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_rd), bytes);
}}
namespace fa {{
namespace {{""")
    rep("    const int l32 = lane & 31;\n", f"""    const int l32 = lane & 31;
    const unsigned long long ts0 = __builtin_amdgcn_s_memrealtime();
    const int dbg_w = (int)blockIdx.x - {SA_WG0};
    const bool dbg = dbg_w >= 0 && dbg_w < 8 && tid == 0;
    if (dbg) g_rd[dbg_w * 64 + 0] = ts0;
""")
    # phase stamps of the main loop
    a = s.index("auto run = [&](auto grp_tag)")
    e = s.index("    };\n", a) + len("    };\n")
    s = s[:a] + f"""auto run = [&](auto grp_tag) __attribute__((always_inline)) {{
        constexpr int GRP = decltype(grp_tag)::value;
        const bool rec_w = blockIdx.x == 0 && (wave == 0 || wave == 4);
        for (int p = 0; p < n_phases; p += 4) {{
            const int t0 = p >> 1;  // even tile index of this round
            const int rnd = (p >> 2) - {R0};
            const bool rec = rec_w && rnd >= 0 && rnd < {NROUND};
            auto ST = [&](int kk) __attribute__((always_inline)) {{
                if (rec && lane == 0) g_st[((wave >> 2) * {NROUND} + rnd) * 8 + kk] = __builtin_amdgcn_s_memtime();
            }};
            sync_even();
            if (dbg && (p >> 2) < 58) g_rd[dbg_w * 64 + 4 + (p >> 2)] = __builtin_amdgcn_s_memrealtime();
            ST(0);
            if constexpr (XA) xa_window(t0);
            if (GRP == 0) block_mfma(ic<1>{{}}, k_lds0, v_lds1, t0, k_lds1, v_lds0);
            else if (p > 0) block_valu(t0 - 1);
            ST(1);
            if (p + 1 >= n_phases) break;
            if (GRP == 0) block_valu(t0);
            else block_mfma(ic<0>{{}}, k_lds0, v_lds1, t0, nullptr, nullptr);
            ST(2);
            if (p + 2 >= n_phases) break;
            sync_even();
            ST(3);
            if (GRP == 0) block_mfma(ic<1>{{}}, k_lds1, v_lds0, t0 + 1, k_lds0, v_lds1);
            else block_valu(t0);
            ST(4);
            if (p + 3 >= n_phases) break;
            if (GRP == 0) block_valu(t0 + 1);
            else block_mfma(ic<0>{{}}, k_lds1, v_lds0, t0 + 1, nullptr, nullptr);
            ST(5);
        }}
    }};
""" + s[e:]
    rep("    if (grp == 0) run(ic<0>{});",
        "    const unsigned long long ts2 = __builtin_amdgcn_s_memrealtime();\n"
        "    if (dbg) g_rd[dbg_w * 64 + 1] = ts2;\n"
        "    if (grp == 0) run(ic<0>{});")
    a = s.index("    if (grp == 0) run(ic<0>{});")
    anchor = '    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");\n'
    b = s.index(anchor, a) + len(anchor)
    s = s[:b] + ("    const unsigned long long ts3 = __builtin_amdgcn_s_memrealtime();\n"
                 "    if (dbg) { g_rd[dbg_w * 64 + 2] = ts3; g_rd[dbg_w * 64 + 63] = (unsigned)n_tiles; }\n") + s[b:]
    end = ("            if (lse && g4 == 0) lse[row * hq + h] = (m_run[rg] + fast_log2(l_tot)) * kLn2;\n"
           "        }\n    }\n")
    rep(end, end + f"""    if (wave == 0 && lane == 0 && blockIdx.x < {MAX_WG}) {{
        const unsigned long long ts5 = __builtin_amdgcn_s_memrealtime();
        unsigned long long *w = g_wg + (size_t)blockIdx.x * 8;
        w[0] = ts0; w[1] = ts2; w[2] = ts3; w[3] = ts5;
        w[4] = (unsigned)__builtin_amdgcn_s_getreg((4) | (0 << 6) | (31 << 11));   // HW_ID
        w[5] = (unsigned)__builtin_amdgcn_s_getreg((20) | (0 << 6) | (31 << 11));  // XCC_ID
        w[6] = (unsigned)n_tiles; w[7] = 1;
    }}
    if (dbg) g_rd[dbg_w * 64 + 3] = __builtin_amdgcn_s_memrealtime();
""")
    return s


def build_instrumented() -> str:
    from sparse_attention_layerrouter_amd import build as b

    tmp = tempfile.mkdtemp(prefix="fa_stamps_")
    try:
        csrc = os.path.join(tmp, "csrc")
        shutil.copytree(os.path.join(PKG, "csrc"), csrc)
        path = os.path.join(csrc, "prefill.hip")
        with open(path) as f:
            src = f.read()
        with open(path, "w") as f:
            f.write(_instrument(src))
        return b.build_copy(csrc, STAMPS_LIB, os.path.join(tmp, "obj"))
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def _median(x):
    x = sorted(x)
    return x[len(x) // 2] if x else None


def run(T: int) -> dict:
    """Product layer times, then the instrumented copy's stamps (see the module doc)."""
    lib_path = STAMPS_LIB
    import numpy as np
    import torch

    from sparse_attention_layerrouter_amd import _lib, synth

    # the product path, then the instrumented copy (one library per process load)
    HQ, HKV, D = 32, 8, 128
    q = synth.device_normal((T, HQ, D), seed=100)
    k = synth.device_normal((T, HKV, D), seed=101)
    v = synth.device_normal((T, HKV, D), seed=102)
    o = torch.empty_like(q)
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")

    def layer_ms(bit):
        r = np.array([[bit]], np.uint8)
        rd = torch.from_numpy(r).cuda()
        f = lambda: _lib.fa_attn_prefill(q, k, v, o, cu, T, rd, 0, 128, 2048, 64,
                                         1 / math.sqrt(D), route_host=r)
        for _ in range(2):
            f()
        torch.cuda.synchronize()
        ts = []
        for _ in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(); f(); b.record(); b.synchronize()
            ts.append(a.elapsed_time(b))
        return _median(ts)

    out = {"seq": T, "product": {"fa_ms": layer_ms(1), "sa_ms": layer_ms(0)}}
    _lib.LIB_PATH = lib_path
    _lib._lib = None
    L = _lib.lib()
    L.fa_stamps_read.restype = ctypes.c_int
    L.fa_stamps_read.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t]

    def read(which, n):
        buf = (ctypes.c_ulonglong * n)()
        assert L.fa_stamps_read(which, buf, n * 8) == 0
        return np.array(buf, dtype=np.int64)

    out["instrumented"] = {}
    n_wg = HKV * ((T + 63) // 64)
    for name, bit in (("sa", 0), ("fa", 1)):
        out["instrumented"][name + "_ms"] = layer_ms(bit)
        w = read(1, n_wg * 8).reshape(n_wg, 8)
        assert (w[:, 7] == 1).all(), "a workgroup left no stamps"
        t0, t2, t3, t5 = (w[:, i] / 100.0 for i in range(4))  # 100 MHz ticks -> us
        hw, xcc, nt = w[:, 4], w[:, 5], w[:, 6]
        cuid = (xcc & 0xF) * 1000 + ((hw >> 13) & 7) * 100 + ((hw >> 12) & 1) * 20 + ((hw >> 8) & 15)
        by = collections.defaultdict(list)
        for i in range(n_wg):
            by[int(cuid[i])].append((t0[i], t5[i]))
        gaps = []
        for lst in by.values():
            lst.sort()
            gaps += [b0 - a1 for (a0, a1), (b0, b1) in zip(lst, lst[1:])]
        out[f"{name}_workgroups"] = {
            "workgroups": n_wg, "cus": len(by),
            "prologue_us": round(float(np.median(t2 - t0)), 2),
            "loop_us": round(float(np.median(t3 - t2)), 2),
            "tiles": int(np.median(nt)),
            "loop_us_per_tile": round(float(np.median((t3 - t2) / nt)), 3),
            "epilogue_us": round(float(np.median(t5 - t3)), 2),
            "gap_to_next_on_cu_us": {"median": round(float(np.median(gaps)), 2),
                                     "p10": round(float(np.percentile(gaps, 10)), 2),
                                     "p90": round(float(np.percentile(gaps, 90)), 2)},
        }
        if name == "sa" and n_wg >= SA_WG0 + 8:
            rd = read(2, 8 * 64).reshape(8, 64)
            rows = []
            for i in range(8):
                x = rd[i]
                ntl = int(x[63])
                nr = min((2 * ntl + 2 + 3) // 4, 58)
                base = x[0]
                starts = [(x[4 + j] - base) / 100.0 for j in range(nr)]
                rows.append({"workgroup": SA_WG0 + i, "tiles": ntl,
                             "loop_start_us": round((x[1] - base) / 100.0, 2),
                             "first_round_us": round(starts[0], 2),
                             "round_us": [round(b - a, 2) for a, b in zip(starts, starts[1:])],
                             "loop_end_us": round((x[2] - base) / 100.0, 2),
                             "end_us": round((x[3] - base) / 100.0, 2)})
            out["sa_rounds"] = rows
        if name == "fa":
            st = read(0, 2 * NROUND * 8).reshape(2, NROUND, 8)
            groups = {}
            for g, label in ((0, "group0_M_V_M_V"), (1, "group1_V_M_V_M")):
                x = st[g]
                d = np.diff(x[:, :6], axis=1)
                gap = x[1:, 0] - x[:-1, 5]
                groups[label] = {
                    "block_cycles": [round(float(d[:, i].mean())) for i in (0, 1, 3, 4)],
                    "barrier_cycles": [round(float(d[:, 2].mean())), round(float(gap.mean()))],
                    "round_cycles": round(float(np.diff(x[:, 0]).mean())),
                }
            out["fa_rounds"] = {"workgroup": 0, "rounds": [R0, R0 + NROUND - 1], **groups}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("what", choices=("build", "run"))
    ap.add_argument("--seq", type=int, default=131072)
    args = ap.parse_args()
    if args.what == "build":
        print(build_instrumented())
        return 0
    if not os.path.exists(STAMPS_LIB):
        raise SystemExit(f"{STAMPS_LIB} is missing: run `python -m "
                         "sparse_attention_layerrouter_amd.phase_stamps build` first")
    print(json.dumps(run(args.seq)))
    return 0


if __name__ == "__main__":
    sys.exit(main())
