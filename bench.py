#!/usr/bin/env python3
"""Benchmark of the layer-routed hybrid attention hot path on one MI355X.

One step = the whole hot path on one batch of synthetic, HBM-resident input:
  1. Layer Router: x_Q [131072, 4096] bf16, mean of the last 64 rows, fp32 MLP
     4096 -> 256 -> 32 (random Xavier), threshold -> 32 FA/SA bits;
  2. prefill of a 131072-token sequence through 32 Llama-3.1-8B-shaped
     attention layers (32 query / 8 KV heads, head_dim 128, bf16), each layer FA
     or SA (sink 128, window 2048, block 64) by the router's bit;
  3. one decode step of batch 8 over 32 layers with 131072-token bf16 KV caches
     (even layers FA, odd layers SA, same sparse configuration).
The prefill throughput of step 1+2 is `value` (tok/s at 128k); decode tok/s is
reported beside it.  Inputs are N(0, 1) drawn on the device from fixed seeds.
Per-layer and per-step times are reported as median / p10 / p90 over the timed
steps (the pages' protocol: warm-up iterations, then timed ones, medians).

Other legs: a context sweep, chunked prefill, ring caches, a batched-serving
sweep, the XAttention and Triangle Attention branches, single FA/SA layers at
32K, and the Qwen3-4B-shaped varlen workload (prefill, then 256 decode steps
that append to its caches); `--only-qwen` runs that workload alone and
`--cpu-full` runs the unsampled oracle timings and full-row parity.

Prints ONE JSON line.  `--gpus` above 1 is refused: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

HQ, HKV, D = 32, 8, 128
HIDDEN, ROUTER_HIDDEN, N_LAYERS, POOL = 4096, 256, 32, 64
SINK, WINDOW, BLOCK = 128, 2048, 64


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=3)
    p.add_argument("--warmup", type=int, default=1)
    p.add_argument("--seq", type=int, default=131072, help="prefill context length")
    p.add_argument("--decode-len", type=int, default=131072, help="KV cache length in decode")
    p.add_argument("--decode-batch", type=int, default=8)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-sweep", action="store_true",
                   help="skip the 8k/32k/64k/256k prefill sweep")
    p.add_argument("--no-serving", action="store_true",
                   help="skip the batched decode sweep (batch 8/16/24/32 at a 32K context)")
    p.add_argument("--no-chunked", action="store_true",
                   help="skip the chunked prefill (16384-token chunks over a growing key prefix)")
    p.add_argument("--no-xattn", action="store_true",
                   help="skip the XAttention sparse-branch timing (scores, selection, masked prefill)")
    p.add_argument("--no-qwen", action="store_true",
                   help="skip the Qwen3-4B-shaped varlen mixed-route leg")
    p.add_argument("--no-triangle", action="store_true",
                   help="skip the Triangle Attention sparse-branch timing")
    p.add_argument("--no-config2", action="store_true",
                   help="skip the single FA / SA layer timing at 32768 tokens")
    p.add_argument("--only-qwen", action="store_true",
                   help="run only the Qwen3-4B-shaped varlen leg (prefill + decode loop)")
    p.add_argument("--qwen-steps", type=int, default=256,
                   help="decode steps per sequence in the Qwen3-4B leg (each appends a token)")
    p.add_argument("--no-clock", action="store_true",
                   help="skip the graphics-clock window (e.g. under a profiler, whose "
                        "environment the amd-smi child would inherit)")
    p.add_argument("--cpu-full", action="store_true",
                   help="only the unsampled oracle timings (tiny case, one SA layer at 32K, one "
                        "FA and one SA decode layer at batch 8 x 131072), with full-row parity")
    p.add_argument("--cpu-rows", type=int, default=192,
                   help="query rows of the FA layer the oracle times (SA gets 4x)")
    p.add_argument("--profile", action="store_true",
                   help="short kernel-only run for rocprofv3 counter passes: one FA and one "
                        "SA prefill layer and one FA and one SA decode layer, twice")
    p.add_argument("--no-ceilings", action="store_true",
                   help="skip the ceiling streams (plain read, MFMA + LDS + softmax-mix "
                        "streams) timed before the inputs are allocated")
    p.add_argument("--only-ceilings", action="store_true",
                   help="run only the ceiling streams and print them")
    p.add_argument("--copy-probe", action="store_true",
                   help="only a plain 1 GiB read + 1 GiB write elementwise kernel (counter "
                        "calibration)")
    return p.parse_args()


# ---------------------------------------------------------------------------
# algorithmic work (visible (q, k) pairs; bytes of visible K/V rows)
# ---------------------------------------------------------------------------

def pairs_fa(T: int) -> int:
    return T * (T + 1) // 2


def pairs_sa(T: int, sink=SINK, window=WINDOW, block=BLOCK) -> int:
    """Visible pairs of one SA sequence: sum over rows of the kept-range sizes."""
    ns, nw = sink // block, window // block
    n = 0
    nqb = -(-T // block)
    for i in range(nqb):
        rows = min(block, T - i * block)
        # full kept blocks strictly before the diagonal block
        if i < ns:
            full = i
        else:
            full = ns + (i - max(ns, i - nw + 1))
        # rows of block i see `full` whole blocks and 1..rows keys of their own block
        n += rows * full * block + rows * (rows + 1) // 2
    return n


def pairs_ta(T: int, last_q: int, sink=SINK, window=WINDOW, block=BLOCK) -> int:
    """Visible pairs of one Triangle Attention sequence: the SA rows, plus every
    causal pair of the rows in the last last_q // block query blocks."""
    nqb = -(-T // block)
    tail0 = max(0, nqb - last_q // block) * block
    if tail0 >= T:
        return pairs_sa(T, sink, window, block)
    return pairs_sa(tail0, sink, window, block) + pairs_fa(T) - pairs_fa(tail0)


def flops_of_pairs(p: int) -> float:
    return 4.0 * D * HQ * p  # QK^T and PV, 2 flop per MAC, all query heads


def kept_tokens_decode(n: int, is_fa: bool, sink=SINK, window=WINDOW, block=BLOCK) -> int:
    if is_fa:
        return n
    i = (n - 1) // block
    sink_len = min(sink, n)
    win_start = min(max(sink, (i - window // block + 1) * block), n)
    return sink_len + n - win_start


def load_oracle():
    """The CPU oracle (test infrastructure) for the CPU-baseline leg only: the oracle's
    timing with its sampled parity (cpu_baseline), the needle-row parity, the Qwen
    decode loop's last-step check and the unsampled runs of --cpu-full.  With
    --no-cpu-baseline none of them runs and the oracle is never loaded."""
    import oracle

    return oracle


def read_traffic(kernel_key: str, src_hash: str):
    """HBM traffic per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    e = data.get(kernel_key)
    if not e or e.get("source_hash") != src_hash:
        return None
    return e.get("bytes_per_launch")


def log(msg: str):
    """Progress on stderr (the JSON result is the only stdout line)."""
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def dist(values_ms):
    """median / p10 / p90 / mean of a list of times in ms."""
    import numpy as np

    a = np.asarray(values_ms, dtype=np.float64)
    if a.size == 0:
        return None
    return {"median": round(float(np.median(a)), 4), "p10": round(float(np.percentile(a, 10)), 4),
            "p90": round(float(np.percentile(a, 90)), 4), "mean": round(float(a.mean()), 4),
            "n": int(a.size)}


def cpu_info():
    """Host CPU model and the number of cores this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return model, cores


class ClockSampler:
    """Samples the graphics clocks with `amd-smi metric --clock --json` from a
    background thread while a timed region runs (best effort: no samples when the
    tool is missing or its output cannot be read).  The value per sample is the
    mean current clock over the device's graphics domains (one per XCD)."""

    def __init__(self):
        import shutil
        import threading

        self.exe = shutil.which("amd-smi") or (
            "/opt/rocm/bin/amd-smi" if os.path.exists("/opt/rocm/bin/amd-smi") else None)
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._poll, daemon=True)

    def _read(self):
        import subprocess

        r = subprocess.run([self.exe, "metric", "--clock", "--json"], capture_output=True,
                           text=True, timeout=20)
        d = json.loads(r.stdout)
        if isinstance(d, dict):
            d = d.get("gpu_data", [d])
        clk = d[0]["clock"]
        vals = [v["clk"]["value"] for k, v in clk.items()
                if k.startswith("gfx") and isinstance(v, dict) and isinstance(v.get("clk"), dict)
                and isinstance(v["clk"].get("value"), (int, float))]
        return sum(vals) / len(vals) if vals else None

    def _poll(self):
        while not self._stop.is_set():
            try:
                v = self._read()
                if v is not None:
                    self.samples.append(v)
            except Exception:  # best effort: a failed read is just no sample
                pass
            self._stop.wait(0.25)

    def start(self):
        if self.exe:
            self._thread.start()
        return self

    def stop(self, during: str):
        if self.exe:
            self._stop.set()
            self._thread.join(timeout=30)
        if not self.samples:
            return None
        out = dist(self.samples)
        return {"unit": "MHz", "during": during, "source": "amd-smi metric --clock",
                **{k: (round(v, 1) if isinstance(v, float) else v) for k, v in out.items()}}


# ---------------------------------------------------------------------------

def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the routed attention step has no multi-GPU "
              "path (heads and sequences would shard with no exchange). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from sparse_attention_layerrouter_amd import _lib, synth
    from sparse_attention_layerrouter_amd.rocprof_summary import HOT_KERNELS, source_hash

    _lib.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe:
        x = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        torch.mul(x, 1.0, out=y)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_each_way": x.numel() * 4}))
        return
    stream = torch.cuda.current_stream()
    ceil = None
    if args.only_ceilings or not (args.no_ceilings or args.profile or args.only_qwen
                                  or args.cpu_full):
        ceil = ceilings_leg(stream)
        if args.only_ceilings:
            print(json.dumps({"ceilings": ceil}))
            return
    if args.only_qwen:
        print(json.dumps({"qwen3_4b_varlen": qwen_leg(args, stream)}))
        return
    if args.cpu_full:
        print(json.dumps({"cpu_full": cpu_full(stream)}))
        return
    T = args.seq
    NB, NC = args.decode_batch, args.decode_len
    if args.profile:
        n_dec_layers, n_sets = 2, 2
    else:
        n_dec_layers, n_sets = N_LAYERS, 4
    scale = 1.0 / math.sqrt(D)

    # ---- inputs, resident in HBM before any timing -------------------------
    x_q = synth.device_normal((T, HIDDEN), seed=11)
    rng = np.random.default_rng(0)
    w1, b1, w2, b2 = (torch.from_numpy(a).to(dev) for a in
                      synth.router_weights(rng, HIDDEN, ROUTER_HIDDEN, N_LAYERS))
    cu = torch.tensor([0, T], dtype=torch.int32, device=dev)
    route = torch.zeros((1, N_LAYERS), dtype=torch.uint8, device=dev)
    logits = torch.zeros((1, N_LAYERS), dtype=torch.float32, device=dev)
    ws_router = torch.empty(_lib.fa_router_workspace_size(1, HIDDEN, ROUTER_HIDDEN),
                            dtype=torch.uint8, device=dev)
    sets = []
    for s in range(n_sets):  # rotating per-layer Q/K/V sets, each far larger than the caches
        sets.append((synth.device_normal((T, HQ, D), seed=100 + 3 * s),
                     synth.device_normal((T, HKV, D), seed=101 + 3 * s),
                     synth.device_normal((T, HKV, D), seed=102 + 3 * s)))
    o_pre = torch.empty((T, HQ, D), dtype=torch.bfloat16, device=dev)

    dec_route_np = np.array([[1 if l % 2 == 0 else 0 for l in range(N_LAYERS)]] * NB, np.uint8)
    dec_route = torch.from_numpy(dec_route_np).to(dev)
    caches = []
    for l in range(n_dec_layers):  # one distinct cache per layer
        kc = torch.empty((NB, HKV, NC, D), dtype=torch.bfloat16, device=dev)
        vc = torch.empty_like(kc)
        for b in range(NB):
            kc[b] = synth.device_normal((HKV, NC, D), seed=1000 + 64 * l + 2 * b)
            vc[b] = synth.device_normal((HKV, NC, D), seed=1001 + 64 * l + 2 * b)
        caches.append((kc, vc))
    # compact SA ring caches (sink + window rows) for the SA layers of the decode stack
    RING = SINK + WINDOW
    rings = {}
    for l in range(n_dec_layers):
        if not dec_route_np[0, l]:
            rings[l] = (synth.device_normal((NB, HKV, RING, D), seed=5000 + 2 * l),
                        synth.device_normal((NB, HKV, RING, D), seed=5001 + 2 * l))
    q_dec = synth.device_normal((NB, HQ, D), seed=7)
    o_dec = torch.empty_like(q_dec)
    cache_len = torch.full((NB,), NC, dtype=torch.int32, device=dev)
    ws_dec = torch.empty(_lib.fa_decode_workspace_size(NB, HQ, D, NC), dtype=torch.uint8,
                         device=dev)
    torch.cuda.synchronize()
    log(f"inputs resident: prefill T={T}, decode {n_dec_layers} layers x batch {NB} x {NC}")

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # ---- one step -----------------------------------------------------------
    def step(rec=None, prefill_route=None):
        e_r0, e_r1 = ev(), ev()
        e_r0.record(stream)
        _lib.fa_router_decide(x_q, cu, POOL, w1, b1, w2, b2, route, logits, ws_router)
        e_r1.record(stream)
        r = route if prefill_route is None else prefill_route
        # the host learns the route once per request (decode reuses it as well); the
        # copy lets each layer launch the kernel compiled for its kind
        r_host = r.cpu().numpy()
        pre = []
        for l in range(N_LAYERS if not args.profile else 2):
            q, k, v = sets[l % n_sets]
            a, b_ = ev(), ev()
            a.record(stream)
            _lib.fa_attn_prefill(q, k, v, o_pre, cu, T, r, l, SINK, WINDOW, BLOCK, scale,
                                 route_host=r_host)
            b_.record(stream)
            pre.append((a, b_))
        dec = []
        for l in range(n_dec_layers):
            kc, vc = caches[l]
            a, b_ = ev(), ev()
            a.record(stream)
            _lib.fa_attn_decode(q_dec, o_dec, kc, vc, cache_len, dec_route, l, SINK, WINDOW,
                                BLOCK, scale, workspace=ws_dec, route_host=dec_route_np)
            b_.record(stream)
            dec.append((a, b_))
        if rec is not None:
            rec.append(((e_r0, e_r1), pre, dec))

    if args.profile:
        # kernel-only run for counter passes: layer 0 FA, layer 1 SA (prefill and decode),
        # then the XAttention score kernel
        for _ in range(2):
            step(prefill_route=torch.tensor([[1, 0] + [0] * 30], dtype=torch.uint8, device=dev))
        torch.cuda.synchronize()
        # the XAttention score kernel at the same length (block 128, stride 8), twice
        XBp, XSp = 128, 8
        nqb_p = (T + XBp - 1) // XBp
        sc_p = torch.empty((1, HQ, nqb_p, nqb_p), dtype=torch.float32, device=dev)
        xw_p = torch.empty(_lib.fa_xattn_workspace_size(1, HQ, nqb_p), dtype=torch.uint8,
                           device=dev)
        for _ in range(2):
            _lib.fa_xattn_scores(sets[0][0], sets[0][1], cu, T, XBp, XSp, scale, sc_p, xw_p)
        torch.cuda.synchronize()
        del sc_p, xw_p
        kept_sa = kept_tokens_decode(NC, False)
        alg = {
            "prefill_bf16_fa_131k": {"flop": flops_of_pairs(pairs_fa(T))},
            "prefill_bf16_sa_131k": {"flop": flops_of_pairs(pairs_sa(T))},
            "decode_bf16_fa_131k": {"flop": 4.0 * NB * HQ * NC * D,
                                    "bytes": NB * HKV * NC * D * 4 + 2 * NB * HQ * D * 2},
            "decode_bf16_sa_131k": {"flop": 4.0 * NB * HQ * kept_sa * D,
                                    "bytes": NB * HKV * kept_sa * D * 4 + 2 * NB * HQ * D * 2},
            "xa_score_131k": {"flop": float(HQ * (nqb_p * (nqb_p + 1) // 2) * 16 * 16 * (XSp * D)
                                            * 2)},
        }
        print(json.dumps({"profile_run": True, "seq": T, "decode_cache": NC,
                          "decode_batch": NB, "algorithmic": alg}))
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")
    recs = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(recs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"timed {args.steps} steps in {wall:.2f} s")

    # graphics clock under the FA prefill layer, sampled in an untimed window of its
    # own so that the sampling process cannot disturb the timed steps
    fa_route = torch.ones((1, N_LAYERS), dtype=torch.uint8, device=dev)
    fa_route_np = fa_route.cpu().numpy()
    clocks = ClockSampler()
    if args.no_clock:
        clocks.exe = None
    clocks.start()
    for i in range(24 if clocks.exe else 0):
        qs, ks, vs = sets[i % n_sets]
        _lib.fa_attn_prefill(qs, ks, vs, o_pre, cu, T, fa_route, 0, SINK, WINDOW, BLOCK, scale,
                             route_host=fa_route_np)
    torch.cuda.synchronize()
    gpu_clock = clocks.stop(f"24 FA prefill layers at {T} tokens, untimed, after the timed steps")

    route_full = route.clone()  # the sweeps below re-run the router on shorter inputs
    route_np = route.cpu().numpy()[0]
    logits_np = logits.cpu().numpy()[0]
    n_fa = int(route_np.sum())

    router_ms = np.array([a.elapsed_time(b) for (a, b), _, _ in recs])
    pre_ms = np.array([[a.elapsed_time(b) for a, b in pre] for _, pre, _ in recs])
    dec_ms = np.array([[a.elapsed_time(b) for a, b in dec] for _, _, dec in recs])
    t_router = float(router_ms.mean()) * 1e-3
    pre_t, dec_t = pre_ms * 1e-3, dec_ms * 1e-3
    t_prefill = t_router + pre_t.sum(axis=1).mean()
    t_decode = dec_t.sum(axis=1).mean()
    fa_layers = [l for l in range(N_LAYERS) if route_np[l]]
    sa_layers = [l for l in range(N_LAYERS) if not route_np[l]]
    t_fa = float(pre_t[:, fa_layers].mean()) if fa_layers else float("nan")
    t_sa = float(pre_t[:, sa_layers].mean()) if sa_layers else float("nan")
    dec_fa = [l for l in range(N_LAYERS) if dec_route_np[0, l]]
    dec_sa = [l for l in range(N_LAYERS) if not dec_route_np[0, l]]
    td_fa = float(dec_t[:, dec_fa].mean())
    td_sa = float(dec_t[:, dec_sa].mean())
    timing = {
        "protocol": (f"{args.warmup} warm-up steps, then {args.steps} timed steps; HIP events "
                     f"around every call on the launch stream; ms"),
        "prefill_step_ms": dist(router_ms + pre_ms.sum(axis=1)),
        "router_ms": dist(router_ms),
        "prefill_fa_layer_ms": dist(pre_ms[:, fa_layers].ravel()) if fa_layers else None,
        "prefill_sa_layer_ms": dist(pre_ms[:, sa_layers].ravel()) if sa_layers else None,
        "decode_step_ms": dist(dec_ms.sum(axis=1)),
        "decode_fa_layer_us": dist(dec_ms[:, dec_fa].ravel() * 1e3),
        "decode_sa_layer_us": dist(dec_ms[:, dec_sa].ravel() * 1e3),
    }

    # measured all-FA references: prefill with every layer FA (the same per-kind FA
    # kernel as the routed step's FA layers), one warm-up pass and up to three timed;
    # decode with every layer FA through the FA kernel (host route copy), with the
    # routed step's warm-up and timed counts
    allfa = torch.ones((1, N_LAYERS), dtype=torch.uint8, device=dev)
    ref = []
    for rep in range(1 + min(3, args.steps)):
        step(ref if rep else None, prefill_route=allfa)
    torch.cuda.synchronize()
    allfa_pre_ms = [ra.elapsed_time(rb) + sum(a.elapsed_time(b) for a, b in pre_ref)
                    for (ra, rb), pre_ref, _ in ref]
    t_prefill_allfa = float(np.median(allfa_pre_ms)) * 1e-3
    dec_allfa_np = np.ones((NB, N_LAYERS), np.uint8)
    dec_allfa_route = torch.from_numpy(dec_allfa_np).to(dev)
    allfa_dec_ms = []
    for rep in range(args.warmup + args.steps):
        a, b = ev(), ev()
        a.record(stream)
        for l in range(n_dec_layers):
            kc, vc = caches[l]
            _lib.fa_attn_decode(q_dec, o_dec, kc, vc, cache_len, dec_allfa_route, l, SINK,
                                WINDOW, BLOCK, scale, workspace=ws_dec,
                                route_host=dec_allfa_np)
        b.record(stream)
        torch.cuda.synchronize()
        if rep >= args.warmup:
            allfa_dec_ms.append(a.elapsed_time(b))
    t_decode_allfa = float(np.median(allfa_dec_ms)) * 1e-3
    t_decode_med = float(np.median(dec_ms.sum(axis=1))) * 1e-3
    timing["all_fa_prefill_ms"] = dist(allfa_pre_ms)
    timing["all_fa_decode_step_ms"] = dist(allfa_dec_ms)

    log("all-FA references done")

    # ---- decode step with ring caches on the SA layers (persistent-KV saving)
    ring_ms = []
    for rep in range(args.warmup + args.steps):
        a, b_ = ev(), ev()
        a.record(stream)
        for l in range(n_dec_layers):
            if l in rings:
                kr, vr = rings[l]
                _lib.fa_attn_decode_ring(q_dec, o_dec, kr, vr, cache_len, SINK, WINDOW, BLOCK,
                                         scale, workspace=ws_dec)
            else:
                kc, vc = caches[l]
                _lib.fa_attn_decode(q_dec, o_dec, kc, vc, cache_len, dec_route, l, SINK, WINDOW,
                                    BLOCK, scale, workspace=ws_dec, route_host=dec_route_np)
        b_.record(stream)
        torch.cuda.synchronize()
        if rep >= args.warmup:
            ring_ms.append(a.elapsed_time(b_))
    t_decode_ring = float(np.mean(ring_ms)) * 1e-3
    kv_full = 2 * n_dec_layers * NB * HKV * NC * D * 2
    kv_ring = sum(2 * NB * HKV * (RING if l in rings else NC) * D * 2 for l in range(n_dec_layers))
    log("ring-cache decode done")

    # ---- batched-serving decode sweep at a 32K context (batch 8/16/24/32): the
    # caches of each batch are prefix views of the per-layer buffers above
    serving = []
    if not args.no_serving and not args.profile and NB * NC >= 32 * 32768:
        SC = 32768
        rings32 = {l: (torch.empty((32, HKV, RING, D), dtype=torch.bfloat16, device=dev),
                       torch.empty((32, HKV, RING, D), dtype=torch.bfloat16, device=dev))
                   for l in rings}
        for l, (kr, vr) in rings32.items():
            kr.copy_(synth.device_normal((32, HKV, RING, D), seed=7000 + l))
            vr.copy_(synth.device_normal((32, HKV, RING, D), seed=7100 + l))
        ws_s = torch.empty(_lib.fa_decode_workspace_size(32, HQ, D, SC), dtype=torch.uint8,
                           device=dev)
        for bs in (8, 16, 24, 32):
            q_s = synth.device_normal((bs, HQ, D), seed=8000 + bs)
            o_s = torch.empty_like(q_s)
            cl_s = torch.full((bs,), SC, dtype=torch.int32, device=dev)
            r_np = np.array([[1 if l % 2 == 0 else 0 for l in range(N_LAYERS)]] * bs, np.uint8)
            r_d = torch.from_numpy(r_np).to(dev)
            def dec_pass(kind):
                for l in range(n_dec_layers):
                    kc, vc = caches[l]
                    n_el = bs * HKV * SC * D
                    kcv = kc.view(-1)[:n_el].view(bs, HKV, SC, D)
                    vcv = vc.view(-1)[:n_el].view(bs, HKV, SC, D)
                    if kind == "ring" and l in rings32:
                        kr, vr = rings32[l]
                        _lib.fa_attn_decode_ring(q_s, o_s, kr[:bs], vr[:bs], cl_s, SINK, WINDOW,
                                                 BLOCK, scale, workspace=ws_s)
                    else:
                        _lib.fa_attn_decode(q_s, o_s, kcv, vcv, cl_s, r_d, l, SINK, WINDOW,
                                            BLOCK, scale, workspace=ws_s, route_host=r_np)

            def median_ms(run):
                times = []
                for rep in range(6):  # one warm-up pass, the median of five timed passes
                    a, b_ = ev(), ev()
                    a.record(stream)
                    run()
                    b_.record(stream)
                    torch.cuda.synchronize()
                    if rep:
                        times.append(a.elapsed_time(b_))
                return float(np.median(times))

            ms = {kind: median_ms(lambda k_=kind: dec_pass(k_)) for kind in ("full", "ring")}
            # the full-cache step captured once as a HIP graph and replayed: the same
            # kernels, without 64 host launches per step
            dec_pass("full")
            torch.cuda.synchronize()
            o_eager = o_s.clone()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                dec_pass("full")
            torch.cuda.synchronize()
            ms["graph"] = median_ms(g.replay)
            graph_ok = bool(torch.equal(o_s.view(torch.int16), o_eager.view(torch.int16)))
            del g
            # the all-FA reference on the same caches
            r_fa_np = np.ones((bs, N_LAYERS), np.uint8)
            r_fa = torch.from_numpy(r_fa_np).to(dev)
            times = []
            for rep in range(6):
                a, b_ = ev(), ev()
                a.record(stream)
                for l in range(n_dec_layers):
                    kc, vc = caches[l]
                    n_el = bs * HKV * SC * D
                    _lib.fa_attn_decode(q_s, o_s, kc.view(-1)[:n_el].view(bs, HKV, SC, D),
                                        vc.view(-1)[:n_el].view(bs, HKV, SC, D), cl_s, r_fa, l,
                                        SINK, WINDOW, BLOCK, scale, workspace=ws_s,
                                        route_host=r_fa_np)
                b_.record(stream)
                torch.cuda.synchronize()
                if rep:
                    times.append(a.elapsed_time(b_))
            ms_fa = float(np.median(times))
            kv_full_s = 2 * n_dec_layers * bs * HKV * SC * D * 2
            kv_ring_s = sum(2 * bs * HKV * (RING if l in rings32 else SC) * D * 2
                            for l in range(n_dec_layers))
            serving.append({"batch": bs, "tok_s": round(bs / ms["full"] * 1e3, 1),
                            "ring_cache_tok_s": round(bs / ms["ring"] * 1e3, 1),
                            "graph_tok_s": round(bs / ms["graph"] * 1e3, 1),
                            "graph_matches_eager": graph_ok,
                            "all_fa_tok_s": round(bs / ms_fa * 1e3, 1),
                            "speedup_vs_all_fa": round(ms_fa / ms["full"], 3),
                            "persistent_kv_gib_full": round(kv_full_s / 2**30, 3),
                            "persistent_kv_gib_ring": round(kv_ring_s / 2**30, 3)})
        del rings32
        log("serving sweep done")

    # ---- context sweep of the routed prefill (router + 32 layers), one pass each
    sweep = []
    if not args.no_sweep:
        for Ts in (8192, 32768, 65536):
            if Ts >= T:
                continue
            cu_s = torch.tensor([0, Ts], dtype=torch.int32, device=dev)
            res = {}
            for kind in ("routed", "all_fa"):
                ms_pass = None
                for rep in range(2):  # first pass warms up, second is timed
                    a, b_ = ev(), ev()
                    a.record(stream)
                    _lib.fa_router_decide(x_q[:Ts], cu_s, POOL, w1, b1, w2, b2, route, logits,
                                          ws_router)
                    r_host = (route.cpu().numpy() if kind == "routed"
                              else np.ones((1, N_LAYERS), np.uint8))
                    r_dev = route if kind == "routed" else allfa
                    for l in range(N_LAYERS):
                        q, k, v = sets[l % n_sets]
                        _lib.fa_attn_prefill(q[:Ts], k[:Ts], v[:Ts], o_pre[:Ts], cu_s, Ts, r_dev,
                                             l, SINK, WINDOW, BLOCK, scale, route_host=r_host)
                    b_.record(stream)
                    torch.cuda.synchronize()
                    ms_pass = a.elapsed_time(b_)
                res[kind] = ms_pass
                if kind == "routed":
                    n_fa_s = int(route.cpu().numpy().sum())
            sweep.append({"seq": Ts, "tok_s": round(Ts / res["routed"] * 1e3, 1),
                          "ms": round(res["routed"], 3), "n_fa_layers": n_fa_s,
                          "all_fa_ms": round(res["all_fa"], 3),
                          "speedup_vs_all_fa": round(res["all_fa"] / res["routed"], 3)})
        sweep.append({"seq": T, "tok_s": round(T / t_prefill, 1), "ms": round(t_prefill * 1e3, 3),
                      "n_fa_layers": n_fa, "all_fa_ms": round(t_prefill_allfa * 1e3, 3),
                      "speedup_vs_all_fa": round(t_prefill_allfa / t_prefill, 3)})
        # twice the context (262144 at the defaults, the longest the pages evaluate),
        # on inputs of its own: one set of Q/K/V for all layers, one pass of each kind
        T2 = 2 * T
        if T2 <= 262144:
            x2 = synth.device_normal((T2, HIDDEN), seed=12)
            q2 = synth.device_normal((T2, HQ, D), seed=120)
            k2 = synth.device_normal((T2, HKV, D), seed=121)
            v2 = synth.device_normal((T2, HKV, D), seed=122)
            o2 = torch.empty_like(q2)
            cu2 = torch.tensor([0, T2], dtype=torch.int32, device=dev)
            res = {}
            for kind in ("routed", "all_fa"):
                a, b_ = ev(), ev()
                a.record(stream)
                _lib.fa_router_decide(x2, cu2, POOL, w1, b1, w2, b2, route, logits, ws_router)
                r_host = (route.cpu().numpy() if kind == "routed"
                          else np.ones((1, N_LAYERS), np.uint8))
                r_dev = route if kind == "routed" else allfa
                for l in range(N_LAYERS):
                    _lib.fa_attn_prefill(q2, k2, v2, o2, cu2, T2, r_dev, l, SINK, WINDOW, BLOCK,
                                         scale, route_host=r_host)
                b_.record(stream)
                torch.cuda.synchronize()
                res[kind] = a.elapsed_time(b_)
                if kind == "routed":
                    n_fa_2 = int(route.cpu().numpy().sum())
            sweep.append({"seq": T2, "tok_s": round(T2 / res["routed"] * 1e3, 1),
                          "ms": round(res["routed"], 3), "n_fa_layers": n_fa_2,
                          "all_fa_ms": round(res["all_fa"], 3),
                          "speedup_vs_all_fa": round(res["all_fa"] / res["routed"], 3)})
            del x2, q2, k2, v2, o2
        log("context sweep done")

    # ---- chunked prefill: the same routed 32-layer prefill in 16384-token chunks,
    # each chunk's queries against the whole key prefix (fa_attn_prefill_kv)
    chunked = None
    CHUNK = 16384
    if not args.no_chunked and T % CHUNK == 0 and T > CHUNK:
        r_host = route_full.cpu().numpy()
        cu_q = torch.tensor([0, CHUNK], dtype=torch.int32, device=dev)
        cu_ks = [torch.tensor([0, c1], dtype=torch.int32, device=dev)
                 for c1 in range(CHUNK, T + 1, CHUNK)]
        ms_pass = None
        for rep in range(2):  # first pass warms up, second is timed
            a, b_ = ev(), ev()
            a.record(stream)
            for ci, cu_k in enumerate(cu_ks):
                c0, c1 = ci * CHUNK, (ci + 1) * CHUNK
                for l in range(N_LAYERS):
                    q, k, v = sets[l % n_sets]
                    _lib.fa_attn_prefill_kv(q[c0:c1], k[:c1], v[:c1], o_pre[c0:c1], cu_q, cu_k,
                                            CHUNK, route_full, l, SINK, WINDOW, BLOCK, scale,
                                            route_host=r_host)
            b_.record(stream)
            torch.cuda.synchronize()
            ms_pass = a.elapsed_time(b_)
        t_chunked = ms_pass * 1e-3 + t_router
        chunked = {"chunk": CHUNK, "tok_s": round(T / t_chunked, 1),
                   "ms": round(t_chunked * 1e3, 3),
                   "vs_one_call": round(t_prefill / t_chunked, 3)}
        log("chunked prefill done")

    # ---- XAttention as the sparse branch of one layer at T: antidiagonal scores,
    # threshold selection and the block-masked prefill, on the i.i.d. inputs and on
    # locality-structured inputs (a positional code on Q and K, two strengths)
    xattn = None
    if not args.no_xattn:
        XB, XS, XTAU = 128, 8, 0.9
        nqb = -(-T // XB)
        nwx = -(-nqb // 32)
        sc = torch.empty((1, HQ, nqb, nqb), dtype=torch.float32, device=dev)
        mk = torch.empty((1, HQ, nqb, nwx), dtype=torch.int32, device=dev)
        xw = torch.empty(_lib.fa_xattn_workspace_size(1, HQ, nqb), dtype=torch.uint8,
                         device=dev)
        xa_flop = HQ * (nqb * (nqb + 1) // 2) * 16 * 16 * (XS * D) * 2
        xattn = {"block": XB, "stride": XS, "threshold": XTAU, "seq": T,
                 "fa_layer_ms": round(t_fa * 1e3, 3),
                 "sa_layer_ms": round(t_sa * 1e3, 3) if sa_layers else None,
                 "inputs": {}}
        inputs = [("iid", lambda: sets[0])]
        for alpha in (2.0, 3.0):
            inputs.append((f"positional_a{alpha:g}",
                           lambda a_=alpha: synth.device_positional_qkv(T, HQ, HKV, D, 31, a_)))
        for name, make in inputs:
            q, k, v = make()
            for rep in range(2):  # first run warms up, second is timed
                e = [ev() for _ in range(4)]
                e[0].record(stream)
                _lib.fa_xattn_scores(q, k, cu, T, XB, XS, scale, sc, xw)
                e[1].record(stream)
                _lib.fa_xattn_select(sc, cu, XB, XTAU, mk)
                e[2].record(stream)
                _lib.fa_attn_prefill_xattn(q, k, v, o_pre, cu, T, XB, mk, scale)
                e[3].record(stream)
                torch.cuda.synchronize()
            t3 = [e[i].elapsed_time(e[i + 1]) for i in range(3)]
            bits = mk.cpu().numpy().view(np.uint32)
            kept = int(np.unpackbits(bits.view(np.uint8)).sum())
            layer = sum(t3)
            xattn["inputs"][name] = {
                "density": round(kept / (HQ * nqb * (nqb + 1) // 2), 4),
                "scores_ms": round(t3[0], 3), "select_ms": round(t3[1], 3),
                "prefill_ms": round(t3[2], 3), "layer_ms": round(layer, 3),
                "speedup_vs_fa_layer": round(t_fa * 1e3 / layer, 3),
                "scores_tflops": round(xa_flop / (t3[0] * 1e-3) / 1e12, 1)}
            del q, k, v
        del sc, mk, xw
        log("xattn branch done")

    # ---- Triangle Attention as the sparse branch of one layer at T: the streaming
    # sink + window blocks plus a dense tail of the last query blocks
    tri = None
    if not args.no_triangle:
        r1 = np.zeros((1, 1), np.uint8)
        r1_dev = torch.from_numpy(r1).to(dev)
        q, k, v = sets[0]
        tri = {"seq": T, "sink": SINK, "window": WINDOW, "block": BLOCK,
               "fa_layer_ms": round(t_fa * 1e3, 3),
               "sa_layer_ms": round(t_sa * 1e3, 3) if sa_layers else None, "tails": []}
        for last_q in (128, 1024):
            ms = None
            for rep in range(3):  # first call warms up; the best of two timed calls
                a, b_ = ev(), ev()
                a.record(stream)
                _lib.fa_attn_prefill_triangle(q, k, v, o_pre, cu, T, r1_dev, 0, SINK, WINDOW,
                                              BLOCK, last_q, scale, route_host=r1)
                b_.record(stream)
                torch.cuda.synchronize()
                if rep:
                    ms = min(ms or 1e30, a.elapsed_time(b_))
            fl = flops_of_pairs(pairs_ta(T, last_q))
            tri["tails"].append({"last_q": last_q, "ms": round(ms, 3),
                                 "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                                 "pairs_vs_fa": round(pairs_ta(T, last_q) / pairs_fa(T), 5),
                                 "speedup_vs_fa_layer": round(t_fa * 1e3 / ms, 2)})
        log("triangle branch done")

    # ---- single FA and SA layers at 32768 tokens (one Llama-shaped layer run as
    # each kind), 10 warm-up and 50 timed calls
    config2 = None
    if not args.no_config2 and T >= 32768:
        config2 = config2_leg(stream, sets[0])
        log("32K single-layer leg done")

    # ---- Qwen3-4B-shaped mixed workload (prefill, then a decode loop appending to
    # its own caches); the Llama decode caches are not needed past this point
    caches.clear()
    rings.clear()
    torch.cuda.empty_cache()
    qwen = None
    if not args.no_qwen and not args.profile and n_dec_layers == N_LAYERS:
        qwen = qwen_leg(args, stream)
        torch.cuda.empty_cache()
        log("qwen3-4b varlen leg done")

    # ---- roofline --------------------------------------------------------------
    fa_flop = flops_of_pairs(pairs_fa(T))
    sa_flop = flops_of_pairs(pairs_sa(T))
    achieved_tflops = fa_flop / t_fa / 1e12
    pre_hash = source_hash(*HOT_KERNELS["prefill_bf16_fa_131k"][1])
    dec_hash = source_hash(*HOT_KERNELS["decode_bf16_fa_131k"][1])
    traffic_pre = read_traffic("prefill_bf16_fa_131k", pre_hash)
    dec_bytes = NB * HKV * NC * D * 2 * 2 + 2 * NB * HQ * D * 2
    dec_sa_bytes = NB * HKV * kept_tokens_decode(NC, False) * D * 2 * 2 + 2 * NB * HQ * D * 2
    achieved_gbs = dec_bytes / td_fa / 1e9

    result = {
        "metric": "routed-attn prefill tok/s @128k + decode tok/s; % MFMA / HBM roofline",
        "value": round(T / t_prefill, 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic N(0,1) on device, random-init Xavier router (no trained weights)",
        "config": {
            "workload": (f"Llama-3.1-8B-shaped attention (32 q / 8 kv heads, d 128): router "
                         f"{HIDDEN}->{ROUTER_HIDDEN}->{N_LAYERS} + 32-layer routed prefill of "
                         f"{T} tokens (SA: sink {SINK}, window {WINDOW}, block {BLOCK}) + "
                         f"32-layer decode step, batch {NB}, {NC}-token cache, 16 SA layers"),
            "seq_len": T, "global_batch": 1, "decode_batch": NB, "decode_cache": NC,
            "parallelism": "single GPU",
        },
        "prefill": {
            "tok_s": round(T / t_prefill, 1),
            "ms": round(t_prefill * 1e3, 3),
            "router_ms": round(t_router * 1e3, 4),
            "n_fa_layers": n_fa, "omega_msr": round(1 - n_fa / N_LAYERS, 4),
            "min_abs_logit": float(np.abs(logits_np).min()),
            "fa_layer_ms": round(t_fa * 1e3, 3), "sa_layer_ms": round(t_sa * 1e3, 3),
            "fa_layer_tflops": round(achieved_tflops, 1),
            "sa_layer_tflops": round(sa_flop / t_sa / 1e12, 1) if sa_layers else None,
            "all_fa_ms": round(t_prefill_allfa * 1e3, 3),
            "speedup_vs_all_fa": round(t_prefill_allfa / t_prefill, 3),
            "context_sweep": sweep,
            "chunked_16k": chunked,
            "xattn_branch": xattn,
            "triangle_branch": tri,
            "qwen3_4b_varlen": qwen,
            "single_layer_32k": config2,
        },
        "decode": {
            "tok_s": round(NB / t_decode, 1),
            "ms_per_token_step": round(t_decode * 1e3, 4),
            "fa_layer_us": round(td_fa * 1e6, 2), "sa_layer_us": round(td_sa * 1e6, 2),
            "fa_layer_gbs": round(achieved_gbs, 1),
            "sa_layer_gbs": round(dec_sa_bytes / td_sa / 1e9, 1),
            "all_fa_ms": round(t_decode_allfa * 1e3, 4),
            "speedup_vs_all_fa": round(t_decode_allfa / t_decode_med, 3),
            "ring_cache_tok_s": round(NB / t_decode_ring, 1),
            "ring_cache_ms_per_token_step": round(t_decode_ring * 1e3, 4),
            "persistent_kv_gib_full": round(kv_full / 2**30, 3),
            "persistent_kv_gib_ring": round(kv_ring / 2**30, 3),
            "persistent_kv_saving": round(1 - kv_ring / kv_full, 4),
            "serving_sweep_32k": serving,
        },
        "timing": timing,
        "gpu_clock_mhz": gpu_clock,
        "roofline": {
            "kernel": "prefill_bf16_kernel<128> (FA layer, 131072 tokens)",
            "bound": "mfma", "achieved": round(achieved_tflops, 1),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic_pre,
        },
        "roofline_decode": {
            "kernel": "fa_attn_decode FA layer (split + merge kernels)",
            "bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(achieved_gbs / PEAK_HBM_GBS, 4),
            "traffic": read_traffic("decode_bf16_fa_131k", dec_hash),
        },
    }
    if ceil is not None:
        ceil["fa_prefill_over_its_mix_stream"] = round(
            achieved_tflops / ceil["mix"]["prefill_mix_tflops"], 4)
        ceil["fa_decode_over_read_stream"] = round(achieved_gbs / ceil["read"]["best_gbs"], 4)
        if xattn is not None:
            ceil["xa_scores_iid_over_small_product_stream"] = round(
                xattn["inputs"]["iid"]["scores_tflops"] / ceil["mix"]["small_1_read_tflops"], 4)
        result["ceilings"] = ceil

    # ---- CPU oracle baseline (rank 0, N=1 only) and sampled parity -------------
    if not args.no_cpu_baseline:
        result["cpu_baseline"], result["parity"] = cpu_baseline(
            args, sets[0], route_np, T, scale, t_prefill)
        result["parity"]["needle"] = needle_parity(T, scale)
        result["parity"]["pass"] = bool(result["parity"]["pass"]
                                        and result["parity"]["needle"]["pass"])
    print(json.dumps(result))


def _host_bits(t):
    import numpy as np
    import torch

    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _f64(bits):
    import numpy as np

    from sparse_attention_layerrouter_amd import synth

    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def _parity_entry(o_gpu, o_ref, lse_gpu=None, l_ref=None):
    """Max abs error, reference scale and relative error of one set of checked outputs."""
    import numpy as np

    err = float(np.abs(o_gpu - o_ref).max())
    ref = float(np.abs(o_ref).max())
    out = {"rows": int(o_ref.shape[0]), "max_abs_err": err, "max_abs_ref": ref,
           "rel_err": err / ref if ref > 0 else None}
    if lse_gpu is not None:
        out["lse_max_abs_err"] = float(np.abs(lse_gpu - l_ref).max())
    return out


def _sa_row_pairs(rows, sink=SINK, window=WINDOW, block=BLOCK) -> int:
    """Visible (row, key) pairs of the given SA rows (per head)."""
    ns, nw = sink // block, window // block
    n = 0
    for t in rows:
        i = int(t) // block
        full = i if i < ns else ns + (i - max(ns, i - nw + 1))
        n += full * block + (int(t) - i * block + 1)
    return n


def _time_calls(stream, fn, warmup, timed):
    """HIP events around each of `timed` calls of fn after `warmup` untimed calls (ms)."""
    import torch

    for _ in range(warmup):
        fn()
    evs = []
    for _ in range(timed):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        evs.append((a, b))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def ceilings_leg(stream):
    """Measured ceilings of this board for the two hot kernels' mixes: a plain
    non-temporal read of 4 GiB (the FA decode layer's K/V bytes at batch 8 x
    131072) at three workgroup chunk sizes, and dependence-free streams of
    32x32x16 bf16 products (8 waves per CU) with 0, 1/2, 3/4 or 1 LDS operand
    read of 1 KiB per product, without and with the online softmax's VALU mix
    (one exponential, one FMA, one add and half a bf16 pair pack per product;
    the FA prefill kernel issues one exponential and about 2.6 other VALU
    instructions and 1 KiB of LDS reads per 32x32x16-sized product), and
    16x16x32 products with 0, 1/2 or 1 read per product, without and with the
    same softmax work per flop (the FA prefill kernel's own mix is 16x16x32
    with one 1 KiB read per two products; the XAttention score kernel's is one
    read per 16x16x32 product with little VALU work)."""
    from sparse_attention_layerrouter_amd import ceilings

    ceilings.lib()
    log("ceiling streams: read")
    rd = ceilings.measure_read(stream)
    log("ceiling streams: matrix products")
    mx = ceilings.measure_mix(stream)

    def pick(shape, reads, sm):
        return [r for r in mx["streams"] if r["shape"] == shape and r["softmax_mix"] == sm
                and r["lds_reads_per_product"] == reads][0]["tflops"]

    # the FA prefill kernel's mix: 16x16x32 products, one 1 KiB LDS fragment per two
    # products, the softmax's VALU work per flop
    mx["prefill_mix_tflops"] = pick("16x16x32", 0.5, True)
    mx["softmax_mix_1_read_tflops"] = pick("32x32x16", 1.0, True)
    mx["products_only_tflops"] = pick("32x32x16", 0.0, False)
    mx["small_1_read_tflops"] = pick("16x16x32", 1.0, False)
    log("ceiling streams: VALU issue")
    return {"read": rd, "mix": mx, "valu": ceilings.measure_valu(stream)}


def config2_leg(stream, qkv):
    """One Llama-shaped layer at 32768 tokens run as FA and as SA through the per-kind
    kernels: 10 warm-up and 50 timed calls each (median / p10 / p90)."""
    import numpy as np
    import torch

    from sparse_attention_layerrouter_amd import _lib

    T2 = 32768
    q, k, v = (x[:T2] for x in qkv)
    dev = q.device
    o = torch.empty_like(q)
    cu = torch.tensor([0, T2], dtype=torch.int32, device=dev)
    scale = 1.0 / math.sqrt(D)
    out = {"seq": T2, "sink": SINK, "window": WINDOW, "block": BLOCK}
    for name, bit, pairs in (("fa", 1, pairs_fa(T2)), ("sa", 0, pairs_sa(T2))):
        r = np.array([[bit]], np.uint8)
        r_dev = torch.from_numpy(r).to(dev)

        def call():
            _lib.fa_attn_prefill(q, k, v, o, cu, T2, r_dev, 0, SINK, WINDOW, BLOCK, scale,
                                 route_host=r)

        ms = _time_calls(stream, call, 10, 50)
        med = float(np.median(ms))
        fl = flops_of_pairs(pairs)
        out[name] = {"ms": dist(ms), "tok_s": round(T2 / med * 1e3, 1),
                     "algorithmic_flop": fl, "tflops": round(fl / (med * 1e-3) / 1e12, 1),
                     "mfma_frac": round(fl / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    out["fa_over_sa"] = round(out["fa"]["ms"]["median"] / out["sa"]["ms"]["median"], 3)
    return out


def qwen_leg(args, stream):
    """Qwen3-4B-shaped mixed workload: 36 layers, a varlen batch of 4 sequences
    (16384 / 32768 / 49152 / 65536 tokens), a 2560 -> 256 -> 36 router giving
    per-sequence masks (FA and SA sequences share a launch where their bits differ),
    SA sink 128 / window 4096 / block 128.  The routed prefill and its all-FA
    reference; then each layer's KV cache is filled from that layer's prefill K/V,
    and a loop of decode steps appends one token per sequence and step (the cache
    grows from T_b + 1 to T_b + steps tokens; decode reuses the router's mask), run
    routed and all-FA over the same caches.  The last step's outputs are checked
    against the oracle on the grown caches."""
    import numpy as np
    import torch

    from sparse_attention_layerrouter_amd import _lib, synth

    dev = torch.device("cuda:0")
    scale = 1.0 / math.sqrt(D)
    QL, QHID, QSINK, QWIN, QBLK = 36, 2560, 128, 4096, 128
    qlens = [16384, 32768, 49152, 65536]
    NS = args.qwen_steps
    qcu_np = synth.cu_seqlens_of(qlens)
    qtot, qmax = int(qcu_np[-1]), max(qlens)
    qcu = torch.from_numpy(qcu_np).to(dev)
    xq = synth.device_normal((qtot, QHID), seed=51)
    qw = [torch.from_numpy(a).to(dev)
          for a in synth.router_weights(np.random.default_rng(52), QHID, ROUTER_HIDDEN, QL)]
    qroute = torch.empty((4, QL), dtype=torch.uint8, device=dev)
    qlogits = torch.empty((4, QL), dtype=torch.float32, device=dev)
    ws_q = torch.empty(_lib.fa_router_workspace_size(4, QHID, ROUTER_HIDDEN), dtype=torch.uint8,
                       device=dev)
    qsets = [(synth.device_normal((qtot, HQ, D), seed=60 + 3 * i),
              synth.device_normal((qtot, HKV, D), seed=61 + 3 * i),
              synth.device_normal((qtot, HKV, D), seed=62 + 3 * i)) for i in range(2)]
    qo = torch.empty_like(qsets[0][0])

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def qwen_prefill(all_fa):
        a, b_ = ev(), ev()
        a.record(stream)
        _lib.fa_router_decide(xq, qcu, POOL, *qw, qroute, qlogits, ws_q)
        r_np = np.ones((4, QL), np.uint8) if all_fa else qroute.cpu().numpy()
        r_dev = torch.from_numpy(r_np).to(dev) if all_fa else qroute
        for l in range(QL):
            q_, k_, v_ = qsets[l % 2]
            _lib.fa_attn_prefill(q_, k_, v_, qo, qcu, qmax, r_dev, l, QSINK, QWIN, QBLK,
                                 scale, route_host=r_np)
        b_.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b_), r_np

    qwen_prefill(False)  # warm-up
    pre_ms, fa_ms = [], []
    for _ in range(3):
        ms, qr_np = qwen_prefill(False)
        pre_ms.append(ms)
    for _ in range(2):
        fa_ms.append(qwen_prefill(True)[0])
    del xq, qo
    log("qwen prefill timed")

    # ---- per-layer KV caches [4][8][T_b + steps][128], holding each layer's prefill K/V
    QC = qmax + NS
    caches = []
    for l in range(QL):
        _, k_, v_ = qsets[l % 2]
        kc = torch.empty((4, HKV, QC, D), dtype=torch.bfloat16, device=dev)
        vc = torch.empty_like(kc)
        for b in range(4):
            s, e = int(qcu_np[b]), int(qcu_np[b + 1])
            kc[b, :, :e - s] = k_[s:e].transpose(0, 1)
            vc[b, :, :e - s] = v_[s:e].transpose(0, 1)
        caches.append((kc, vc))
    del qsets
    torch.cuda.empty_cache()
    # per step and layer: a query, and the new token's K and V (appended by the call)
    qd_all = synth.device_normal((NS, QL, 4, HQ, D), seed=64)
    kn_all = synth.device_normal((NS, QL, 4, HKV, D), seed=65)
    vn_all = synth.device_normal((NS, QL, 4, HKV, D), seed=66)
    # the last step's queries point at one prefill key each, so its outputs are O(1)
    for l in range(QL):
        qd_all[NS - 1, l] = synth.device_needle_decode_q(caches[l][0], HQ, qlens, seed=700 + l)[0]
    cl0 = torch.tensor([n + 1 for n in qlens], dtype=torch.int32, device=dev)
    cl = cl0.clone()
    o_last = torch.empty((QL, 4, HQ, D), dtype=torch.bfloat16, device=dev)
    lse_last = torch.empty((QL, 4, HQ), dtype=torch.float32, device=dev)
    ws_qd = torch.empty(_lib.fa_decode_workspace_size(4, HQ, D, QC), dtype=torch.uint8,
                        device=dev)
    torch.cuda.synchronize()
    log(f"qwen decode caches resident ({QL} layers x 4 x {QC} tokens)")

    def decode_loop(r_np, n_steps):
        """n_steps appending decode steps from cache length T_b + 1; per-step ms."""
        r_dev = torch.from_numpy(r_np).to(dev)
        cl.copy_(cl0)
        evs = []
        for j in range(n_steps):
            a, b_ = ev(), ev()
            a.record(stream)
            for l in range(QL):
                kc, vc = caches[l]
                _lib.fa_attn_decode(qd_all[j, l], o_last[l], kc, vc, cl, r_dev, l, QSINK, QWIN,
                                    QBLK, scale, workspace=ws_qd, k_new=kn_all[j, l],
                                    v_new=vn_all[j, l], lse=lse_last[l], route_host=r_np)
            b_.record(stream)
            cl.add_(1)  # the cache grows by the appended token
            evs.append((a, b_))
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in evs]

    decode_loop(qr_np, 2)  # warm-up: writes the same tokens as the first two steps below
    routed_ms = decode_loop(qr_np, NS)
    final = [n + NS for n in qlens]
    o_fin, lse_fin = o_last.clone(), lse_last.clone()
    allfa_np = np.ones((4, QL), np.uint8)
    allfa_ms = decode_loop(allfa_np, NS)
    log("qwen decode loops timed")

    # ---- (CPU-baseline leg) the last routed step against the oracle on the grown
    # caches: a layer with mixed routes, an all-FA and an all-SA layer (when the mask
    # has them), KV heads 0, 7
    oracle = None if args.no_cpu_baseline else load_oracle()
    G = HQ // HKV
    n_fa = qr_np.sum(axis=0)
    picks = {}
    for kind, sel in (("mixed", (n_fa > 0) & (n_fa < 4)), ("fa", n_fa == 4), ("sa", n_fa == 0)):
        idx = np.nonzero(sel)[0]
        if idx.size:
            picks[kind] = int(idx[0])
    checks = {} if oracle is not None else None
    ok = True
    for kind, l in (picks.items() if oracle is not None else ()):
        kc, vc = caches[l]
        errs, lerrs, refs = [], [], []
        for g in (0, HKV - 1):
            o_ref, l_ref = oracle.attn_decode(
                _host_bits(qd_all[NS - 1, l][:, g * G:(g + 1) * G]), _host_bits(kc[:, g:g + 1]),
                _host_bits(vc[:, g:g + 1]), final, qr_np, l, QSINK, QWIN, QBLK, scale)
            og = _f64(_host_bits(o_fin[l][:, g * G:(g + 1) * G]))
            errs.append(float(np.abs(og - o_ref).max()))
            lerrs.append(float(np.abs(lse_fin[l][:, g * G:(g + 1) * G].cpu().numpy()
                                      - l_ref).max()))
            refs.append(float(np.abs(o_ref).max()))
        checks[kind] = {"layer": l, "max_abs_err": max(errs), "lse_max_abs_err": max(lerrs),
                        "max_abs_ref": max(refs)}
        ok = ok and max(errs) <= 2e-2 and max(lerrs) <= 1e-3
    # appended tokens landed at their positions (the last one of each sequence)
    for b in range(4):
        kc, _ = caches[picks.get("mixed", 0)]
        ok = ok and torch.equal(kc[b, :, final[b] - 1], kn_all[NS - 1, picks.get("mixed", 0), b])

    # algorithmic bytes of the routed loop: the kept K/V rows of every step
    def kept(n, fa):
        return kept_tokens_decode(n, fa, QSINK, QWIN, QBLK)

    loop_bytes = 0
    for j in range(NS):
        for b in range(4):
            n = qlens[b] + 1 + j
            for l in range(QL):
                loop_bytes += kept(n, bool(qr_np[b, l])) * HKV * D * 4
    t_routed, t_allfa = sum(routed_ms) * 1e-3, sum(allfa_ms) * 1e-3
    out = {
        "layers": QL, "lengths": qlens, "sink": QSINK, "window": QWIN, "block": QBLK,
        "fa_layers_per_seq": [int(x) for x in qr_np.sum(axis=1)],
        "mixed_layers": int(((n_fa > 0) & (n_fa < 4)).sum()),
        "prefill_tok_s": round(qtot / float(np.median(pre_ms)) * 1e3, 1),
        "prefill_ms": dist(pre_ms), "all_fa_prefill_ms": dist(fa_ms),
        "prefill_speedup_vs_all_fa": round(float(np.median(fa_ms) / np.median(pre_ms)), 3),
        "decode": {
            "steps_per_seq": NS, "cache_len_first": [n + 1 for n in qlens], "cache_len_last": final,
            "tok_s": round(4 * NS / t_routed, 1),
            "step_ms": dist(routed_ms),
            "all_fa_tok_s": round(4 * NS / t_allfa, 1),
            "all_fa_step_ms": dist(allfa_ms),
            "speedup_vs_all_fa": round(t_allfa / t_routed, 3),
            "algorithmic_bytes": loop_bytes,
            "achieved_gbs": round(loop_bytes / t_routed / 1e9, 1),
            "parity_last_step": checks,
            "parity_pass": bool(ok) if checks is not None else None,
        },
    }
    del caches, qd_all, kn_all, vn_all
    return out


def needle_parity(T, scale):
    """FA and SA prefill at T on needle inputs (every query row a copy of one earlier
    key, so outputs are O(1)) through the per-kind kernels, sampled rows against the
    oracle: the check a dropped or mis-read tile cannot pass."""
    import numpy as np
    import torch

    oracle = load_oracle()
    from sparse_attention_layerrouter_amd import _lib, synth

    dev = torch.device("cuda:0")
    q, k, v, _ = synth.device_needle_qkv(T, HQ, HKV, D, seed=301)
    cu = torch.tensor([0, T], dtype=torch.int32, device=dev)
    qh, kh, vh = _host_bits(q), _host_bits(k), _host_bits(v)
    out, ok = {}, True
    for name, bit, n_rand in (("fa", 1, 10), ("sa", 0, 96)):
        o = torch.empty_like(q)
        lse = torch.empty((T, HQ), dtype=torch.float32, device=dev)
        r = np.array([[bit]], np.uint8)
        _lib.fa_attn_prefill(q, k, v, o, cu, T, torch.from_numpy(r).to(dev), 0, SINK, WINDOW,
                             BLOCK, scale, lse=lse, route_host=r)
        torch.cuda.synchronize()
        rng = np.random.default_rng(40 + bit)
        rows = np.array(sorted({0, T // 2, T - 2, T - 1}
                               | set(rng.integers(0, T, n_rand).tolist())), np.int32)
        o_ref, l_ref = oracle.attn_prefill(qh, kh, vh, [0, T], r, 0, SINK, WINDOW, BLOCK, scale,
                                           rows=rows)
        e = _parity_entry(_f64(_host_bits(o)[rows]), o_ref, lse.cpu().numpy()[rows], l_ref)
        heads = slice(None) if bit else slice(1, None, 2)
        e["min_row_max_abs_ref"] = float(np.abs(o_ref[:, heads]).max(axis=(1, 2)).min())
        ok = ok and e["max_abs_err"] <= 2e-2 and e["lse_max_abs_err"] <= 1e-3 \
            and e["min_row_max_abs_ref"] >= 0.1
        out[name] = e
    out["inputs"] = ("needle: query row t of head h = 2 K[g][h/4], g drawn in [0, t] (even "
                     "heads) or among the first 128 / last 64 positions (odd heads, kept by SA)")
    out["pass"] = bool(ok)
    return out


def cpu_baseline(args, qkv, route_np, T, scale, t_prefill_gpu):
    """Time the oracle on a bounded sample of the same prefill workload, on every core
    the process may use and on one core, and scale each to the metric's unit by
    visible-pair count.  The sampled GPU rows are compared per layer kind."""
    import numpy as np
    import torch

    oracle = load_oracle()
    from sparse_attention_layerrouter_amd import _lib

    q, k, v = qkv
    dev = q.device
    cu = torch.tensor([0, T], dtype=torch.int32, device=dev)
    model, cores = cpu_info()
    qh, kh, vh = _host_bits(q), _host_bits(k), _host_bits(v)
    samples, kinds = {}, {}
    for name, bit, n_rows in (("fa", 1, args.cpu_rows), ("sa", 0, 4 * args.cpu_rows)):
        o = torch.empty_like(q)
        lse = torch.empty((T, HQ), dtype=torch.float32, device=dev)
        r = np.array([[bit]], np.uint8)
        _lib.fa_attn_prefill(q, k, v, o, cu, T, torch.from_numpy(r).to(dev), 0, SINK, WINDOW,
                             BLOCK, scale, lse=lse, route_host=r)
        torch.cuda.synchronize()
        rng = np.random.default_rng(5 + bit)
        rows = np.sort(rng.choice(T, size=n_rows, replace=False)).astype(np.int32)
        t0 = time.perf_counter()
        o_ref, l_ref = oracle.attn_prefill(qh, kh, vh, [0, T], r, 0, SINK, WINDOW, BLOCK, scale,
                                           rows=rows, n_threads=cores)
        dt = time.perf_counter() - t0
        log(f"oracle {name}: {len(rows)} rows in {dt:.1f} s on {cores} threads")
        sp = int((rows + 1).sum()) if bit else _sa_row_pairs(rows)
        samples[name] = (dt, sp, pairs_fa(T) if bit else pairs_sa(T), len(rows))
        kinds[name] = _parity_entry(_f64(_host_bits(o)[rows]), o_ref, lse.cpu().numpy()[rows],
                                    l_ref)
    # one core, smaller samples
    one = {}
    for name, bit, n_rows in (("fa", 1, max(2, args.cpu_rows // 32)),
                              ("sa", 0, max(8, args.cpu_rows // 8))):
        rng = np.random.default_rng(8 + bit)
        rows = np.sort(rng.choice(T, size=n_rows, replace=False)).astype(np.int32)
        t0 = time.perf_counter()
        oracle.attn_prefill(qh, kh, vh, [0, T], np.array([[bit]], np.uint8), 0, SINK, WINDOW,
                            BLOCK, scale, rows=rows, n_threads=1)
        dt = time.perf_counter() - t0
        sp = int((rows + 1).sum()) if bit else _sa_row_pairs(rows)
        one[name] = (dt, sp, len(rows))
    log(f"oracle one core: {one['fa'][0]:.1f} s + {one['sa'][0]:.1f} s")
    n_fa = int(route_np.sum())
    n_sa = N_LAYERS - n_fa

    def scaled(fa, sa):  # seconds for the routed 32-layer prefill
        return (n_fa * fa[0] * pairs_fa(T) / fa[1] + n_sa * sa[0] * pairs_sa(T) / sa[1])

    t_cpu = scaled(samples["fa"][:2], samples["sa"][:2])
    t_cpu1 = scaled(one["fa"][:2], one["sa"][:2])
    out = {
        "value": round(T / t_cpu, 4), "unit": "tok/s", "cores": cores, "kind": "oracle",
        "cpu_model": model,
        "sample": (f"oracle (fp64 sums, {cores} threads) on {samples['fa'][3]} random query rows "
                   f"x 32 heads of one FA layer ({samples['fa'][0]:.1f} s) and "
                   f"{samples['sa'][3]} rows of one SA layer ({samples['sa'][0]:.1f} s) at {T} "
                   f"tokens, extrapolated by visible-pair count to the routed 32-layer prefill "
                   f"({n_fa} FA layers); router time ignored"),
        "value_1core": round(T / t_cpu1, 5),
        "sample_1core": (f"{one['fa'][2]} FA rows ({one['fa'][0]:.1f} s) and {one['sa'][2]} SA "
                         f"rows ({one['sa'][0]:.1f} s) on one thread, extrapolated the same way"),
        "gpu_over_cpu": round(t_cpu / t_prefill_gpu, 1),
    }
    ok = all(kinds[n]["max_abs_err"] <= 2e-2 and kinds[n]["lse_max_abs_err"] <= 1e-3
             for n in kinds)
    parity = {"workload_rows": kinds, "tolerance": 2e-2, "lse_tolerance": 1e-3, "pass": ok,
              "note": ("workload rows are i.i.d. N(0,1): late FA rows have |O| ~ sqrt(e/T), "
                       "so max_abs_ref shows how much the bar can see; the needle rows below "
                       "have O(1) outputs")}
    return out, parity


def cpu_full(stream):
    """Unsampled oracle runs, timed on every core the process may use, with full-row
    parity of the same GPU launches: the tiny two-layer case (router + FA + SA, fp32),
    one SA and one FA layer at 32768 tokens (Llama shape, bf16; the FA layer runs in
    eight row chunks, each logged, as it takes minutes), and one FA and one SA decode
    layer at batch 8 over 131072-token caches (every head)."""
    import numpy as np
    import torch

    oracle = load_oracle()
    from sparse_attention_layerrouter_amd import _lib, synth

    dev = torch.device("cuda:0")
    model, cores = cpu_info()
    out = {"cpu_model": model, "cores": cores}

    # ---- the tiny case, every output
    c = synth.tiny_case(0)
    cfg = c["cfg"]
    cu_np = c["cu_seqlens"]
    cu = torch.from_numpy(cu_np).to(dev)
    route = torch.zeros((1, 2), dtype=torch.uint8, device=dev)
    logits = torch.zeros((1, 2), dtype=torch.float32, device=dev)
    _lib.fa_router_decide(torch.from_numpy(c["x_q"]).to(dev), cu, cfg["pool"],
                          *(torch.from_numpy(c[n]).to(dev) for n in ("w1", "b1", "w2", "b2")),
                          route, logits)
    sc = 1 / math.sqrt(cfg["d"])
    og, lg = [], []
    for layer, (q, k, v) in enumerate(c["layers"]):
        o = torch.empty((cfg["seq"], cfg["hq"], cfg["d"]), dtype=torch.float32, device=dev)
        lse = torch.empty((cfg["seq"], cfg["hq"]), dtype=torch.float32, device=dev)
        _lib.fa_attn_prefill(*(torch.from_numpy(x).to(dev) for x in (q, k, v)), o, cu,
                             cfg["seq"], route, layer, cfg["sink"], cfg["window"], cfg["block"],
                             sc, lse=lse)
        og.append(o)
        lg.append(lse)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    r_ref, _, _ = oracle.router(c["x_q"], cu_np, cfg["pool"], c["w1"], c["b1"], c["w2"], c["b2"])
    refs = [oracle.attn_prefill(q, k, v, cu_np, r_ref, layer, cfg["sink"], cfg["window"],
                                cfg["block"], sc, n_threads=cores)
            for layer, (q, k, v) in enumerate(c["layers"])]
    dt = time.perf_counter() - t0
    out["tiny_case"] = {
        "kind": "full", "seconds": round(dt, 4),
        "route_bits_equal": bool(np.array_equal(route.cpu().numpy(), r_ref)),
        "layers": [_parity_entry(og[i].cpu().numpy().astype(np.float64), refs[i][0],
                                 lg[i].cpu().numpy(), refs[i][1]) for i in range(2)],
        "tolerance": 1e-4}
    log("cpu-full: tiny case done")

    # ---- one SA and one FA layer at 32768 tokens, every row
    T2 = 32768
    q = synth.device_normal((T2, HQ, D), seed=0)
    k = synth.device_normal((T2, HKV, D), seed=1)
    v = synth.device_normal((T2, HKV, D), seed=2)
    qh, kh, vh = _host_bits(q), _host_bits(k), _host_bits(v)
    cu2 = torch.tensor([0, T2], dtype=torch.int32, device=dev)
    sc = 1 / math.sqrt(D)
    for name, bit in (("sa_layer_32k", 0), ("fa_layer_32k", 1)):
        r = np.array([[bit]], np.uint8)
        o = torch.empty_like(q)
        lse = torch.empty((T2, HQ), dtype=torch.float32, device=dev)
        gpu_ms = _time_calls(stream, lambda: _lib.fa_attn_prefill(
            q, k, v, o, cu2, T2, torch.from_numpy(r).to(dev), 0, SINK, WINDOW, BLOCK, sc,
            lse=lse, route_host=r), 2, 5)
        parts, dt = [], 0.0
        for rows in np.array_split(np.arange(T2, dtype=np.int32), 8 if bit else 1):
            t0 = time.perf_counter()
            parts.append(oracle.attn_prefill(qh, kh, vh, [0, T2], r, 0, SINK, WINDOW, BLOCK,
                                             sc, rows=rows, n_threads=cores))
            dt += time.perf_counter() - t0
            log(f"cpu-full: {name} rows {rows[0]}..{rows[-1]} ({dt:.0f} s so far)")
        o_ref = np.concatenate([p_[0] for p_ in parts])
        l_ref = np.concatenate([p_[1] for p_ in parts])
        e = _parity_entry(_f64(_host_bits(o)), o_ref, lse.cpu().numpy(), l_ref)
        out[name] = {"kind": "full", "rows": T2, "seconds": round(dt, 3),
                     "gpu_ms": dist(gpu_ms),
                     "cpu_over_gpu": round(dt / (np.median(gpu_ms) * 1e-3), 1),
                     "parity": e}
        log(f"cpu-full: {name} {dt:.1f} s")
    del q, k, v, o

    # ---- one FA and one SA decode layer at batch 8 over 131072-token caches, every head
    B, n = 8, 131072
    kc = torch.empty((B, HKV, n, D), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    for b in range(B):
        kc[b] = synth.device_normal((HKV, n, D), seed=1000 + 2 * b)
        vc[b] = synth.device_normal((HKV, n, D), seed=1001 + 2 * b)
    qd = synth.device_normal((B, HQ, D), seed=7)
    cl = torch.full((B,), n, dtype=torch.int32, device=dev)
    r = np.array([[1, 0]] * B, np.uint8)
    rd = torch.from_numpy(r).to(dev)
    ws = torch.empty(_lib.fa_decode_workspace_size(B, HQ, D, n), dtype=torch.uint8, device=dev)
    kch, vch, qdh = _host_bits(kc), _host_bits(vc), _host_bits(qd)
    for name, layer in (("decode_fa_layer_b8_131k", 0), ("decode_sa_layer_b8_131k", 1)):
        o = torch.empty_like(qd)
        lse = torch.empty((B, HQ), dtype=torch.float32, device=dev)
        gpu_ms = _time_calls(stream, lambda: _lib.fa_attn_decode(
            qd, o, kc, vc, cl, rd, layer, SINK, WINDOW, BLOCK, sc, lse=lse, route_host=r,
            workspace=ws), 5, 20)
        t0 = time.perf_counter()
        o_ref, l_ref = oracle.attn_decode(qdh, kch, vch, [n] * B, r, layer, SINK, WINDOW, BLOCK,
                                          sc, n_threads=cores)
        dt = time.perf_counter() - t0
        out[name] = {"kind": "full", "seconds": round(dt, 3), "gpu_ms": dist(gpu_ms),
                     "cpu_over_gpu": round(dt / (np.median(gpu_ms) * 1e-3), 1),
                     "parity": _parity_entry(_f64(_host_bits(o)), o_ref, lse.cpu().numpy(),
                                             l_ref)}
        log(f"cpu-full: {name} {dt:.1f} s")
    return out


if __name__ == "__main__":
    main()
