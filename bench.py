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

Prints ONE JSON line.  `--gpus` above 1 is refused: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
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
    p.add_argument("--cpu-rows", type=int, default=192,
                   help="query rows of the FA layer the oracle times (SA gets 4x)")
    p.add_argument("--profile", action="store_true",
                   help="short kernel-only run for rocprofv3 counter passes: one FA and one "
                        "SA prefill layer and one FA and one SA decode layer, twice")
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
    from sparse_attention_layerrouter_amd.rocprof_summary import source_hash

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
        # kernel-only run for counter passes: layer 0 FA, layer 1 SA (prefill and decode)
        for _ in range(2):
            step(prefill_route=torch.tensor([[1, 0] + [0] * 30], dtype=torch.uint8, device=dev))
        torch.cuda.synchronize()
        print(json.dumps({"profile_run": True, "seq": T, "decode_cache": NC}))
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

    route_full = route.clone()  # the sweeps below re-run the router on shorter inputs
    route_np = route.cpu().numpy()[0]
    logits_np = logits.cpu().numpy()[0]
    n_fa = int(route_np.sum())

    t_router = np.mean([a.elapsed_time(b) for (a, b), _, _ in recs]) * 1e-3
    pre_t = np.array([[a.elapsed_time(b) * 1e-3 for a, b in pre] for _, pre, _ in recs])
    dec_t = np.array([[a.elapsed_time(b) * 1e-3 for a, b in dec] for _, _, dec in recs])
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

    # measured all-FA references (one pass each, same events)
    allfa = torch.ones((1, N_LAYERS), dtype=torch.uint8, device=dev)
    ref = []
    step(ref, prefill_route=allfa)
    torch.cuda.synchronize()
    (ra, rb), pre_ref, _ = ref[0]
    t_prefill_allfa = ra.elapsed_time(rb) * 1e-3 + sum(a.elapsed_time(b) for a, b in pre_ref) * 1e-3
    dec_allfa_route = torch.ones((NB, N_LAYERS), dtype=torch.uint8, device=dev)
    a, b = ev(), ev()
    a.record(stream)
    for l in range(N_LAYERS):
        kc, vc = caches[l]
        _lib.fa_attn_decode(q_dec, o_dec, kc, vc, cache_len, dec_allfa_route, l, SINK, WINDOW,
                            BLOCK, scale, workspace=ws_dec)
    b.record(stream)
    torch.cuda.synchronize()
    t_decode_allfa = a.elapsed_time(b) * 1e-3

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
            r_fa = torch.ones((bs, N_LAYERS), dtype=torch.uint8, device=dev)
            times = []
            for rep in range(6):
                a, b_ = ev(), ev()
                a.record(stream)
                for l in range(n_dec_layers):
                    kc, vc = caches[l]
                    n_el = bs * HKV * SC * D
                    _lib.fa_attn_decode(q_s, o_s, kc.view(-1)[:n_el].view(bs, HKV, SC, D),
                                        vc.view(-1)[:n_el].view(bs, HKV, SC, D), cl_s, r_fa, l,
                                        SINK, WINDOW, BLOCK, scale, workspace=ws_s)
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

    # ---- Qwen3-4B-shaped mixed workload: 36 layers, a varlen batch of 4 sequences
    # (16384 / 32768 / 49152 / 65536 tokens), a 2560 -> 256 -> 36 router giving
    # per-sequence masks (FA and SA sequences share a launch where their bits
    # differ), SA sink 128 / window 4096 / block 128; the routed prefill and its
    # all-FA reference, then decode steps with the first token after the prompt
    qwen = None
    if not args.no_qwen and not args.profile and n_dec_layers == N_LAYERS:
        QL, QHID, QSINK, QWIN, QBLK = 36, 2560, 128, 4096, 128
        qlens = [16384, 32768, 49152, 65536]
        qcu_np = synth.cu_seqlens_of(qlens)
        qtot, qmax = int(qcu_np[-1]), max(qlens)
        qcu = torch.from_numpy(qcu_np).to(dev)
        xq = synth.device_normal((qtot, QHID), seed=51)
        qw = [torch.from_numpy(a).to(dev)
              for a in synth.router_weights(np.random.default_rng(52), QHID, ROUTER_HIDDEN, QL)]
        qroute = torch.empty((4, QL), dtype=torch.uint8, device=dev)
        qlogits = torch.empty((4, QL), dtype=torch.float32, device=dev)
        ws_q = torch.empty(_lib.fa_router_workspace_size(4, QHID, ROUTER_HIDDEN),
                           dtype=torch.uint8, device=dev)
        qsets = [(synth.device_normal((qtot, HQ, D), seed=60 + 3 * i),
                  synth.device_normal((qtot, HKV, D), seed=61 + 3 * i),
                  synth.device_normal((qtot, HKV, D), seed=62 + 3 * i)) for i in range(2)]
        qo = torch.empty_like(qsets[0][0])

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
        ms_q, qr_np = qwen_prefill(False)
        ms_q_fa, _ = qwen_prefill(True)
        # decode: caches are prefix views of the per-layer decode buffers above
        QC = qmax + 8
        n_el = 4 * HKV * QC * D
        qcl = torch.tensor([n + 1 for n in qlens], dtype=torch.int32, device=dev)
        qd = synth.device_normal((4, HQ, D), seed=63)
        qod = torch.empty_like(qd)
        ws_qd = torch.empty(_lib.fa_decode_workspace_size(4, HQ, D, QC), dtype=torch.uint8,
                            device=dev)
        dec_ms = {}
        for kind in ("routed", "all_fa"):
            r_np = qr_np if kind == "routed" else np.ones((4, QL), np.uint8)
            r_dev = torch.from_numpy(r_np).to(dev)
            times = []
            for rep in range(4):  # one warm-up step, the median of three
                a, b_ = ev(), ev()
                a.record(stream)
                for l in range(QL):
                    kc, vc = caches[l % len(caches)]
                    _lib.fa_attn_decode(qd, qod, kc.view(-1)[:n_el].view(4, HKV, QC, D),
                                        vc.view(-1)[:n_el].view(4, HKV, QC, D), qcl, r_dev, l,
                                        QSINK, QWIN, QBLK, scale, workspace=ws_qd,
                                        route_host=r_np)
                b_.record(stream)
                torch.cuda.synchronize()
                if rep:
                    times.append(a.elapsed_time(b_))
            dec_ms[kind] = float(np.median(times))
        qwen = {"layers": QL, "lengths": qlens, "sink": QSINK, "window": QWIN, "block": QBLK,
                "fa_layers_per_seq": [int(x) for x in qr_np.sum(axis=1)],
                "mixed_layers": int(((qr_np.sum(axis=0) > 0) & (qr_np.sum(axis=0) < 4)).sum()),
                "prefill_tok_s": round(qtot / ms_q * 1e3, 1), "prefill_ms": round(ms_q, 3),
                "all_fa_prefill_ms": round(ms_q_fa, 3),
                "prefill_speedup_vs_all_fa": round(ms_q_fa / ms_q, 3),
                "decode_tok_s": round(4 / dec_ms["routed"] * 1e3, 1),
                "decode_ms_per_step": round(dec_ms["routed"], 3),
                "all_fa_decode_ms": round(dec_ms["all_fa"], 3),
                "decode_speedup_vs_all_fa": round(dec_ms["all_fa"] / dec_ms["routed"], 3)}
        del xq, qsets, qo
        log("qwen3-4b varlen leg done")

    # ---- roofline --------------------------------------------------------------
    fa_flop = flops_of_pairs(pairs_fa(T))
    sa_flop = flops_of_pairs(pairs_sa(T))
    achieved_tflops = fa_flop / t_fa / 1e12
    pre_hash = source_hash("prefill.hip", "fa_common.h")
    dec_hash = source_hash("decode.hip", "fa_common.h")
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
        },
        "decode": {
            "tok_s": round(NB / t_decode, 1),
            "ms_per_token_step": round(t_decode * 1e3, 4),
            "fa_layer_us": round(td_fa * 1e6, 2), "sa_layer_us": round(td_sa * 1e6, 2),
            "fa_layer_gbs": round(achieved_gbs, 1),
            "sa_layer_gbs": round(dec_sa_bytes / td_sa / 1e9, 1),
            "all_fa_ms": round(t_decode_allfa * 1e3, 4),
            "speedup_vs_all_fa": round(t_decode_allfa / t_decode, 3),
            "ring_cache_tok_s": round(NB / t_decode_ring, 1),
            "ring_cache_ms_per_token_step": round(t_decode_ring * 1e3, 4),
            "persistent_kv_gib_full": round(kv_full / 2**30, 3),
            "persistent_kv_gib_ring": round(kv_ring / 2**30, 3),
            "persistent_kv_saving": round(1 - kv_ring / kv_full, 4),
            "serving_sweep_32k": serving,
        },
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

    # ---- CPU oracle baseline (rank 0, N=1 only) and sampled parity -------------
    if not args.no_cpu_baseline:
        result["cpu_baseline"], result["parity"] = cpu_baseline(
            args, sets[0], route_np, T, scale, t_prefill)
    print(json.dumps(result))


def cpu_baseline(args, qkv, route_np, T, scale, t_prefill_gpu):
    """Time the oracle on a bounded sample of the same prefill workload and scale it to
    the metric's unit by visible-pair count.  Also compares the sampled GPU rows."""
    import numpy as np
    import torch

    import oracle
    from sparse_attention_layerrouter_amd import _lib

    q, k, v = qkv
    dev = q.device
    cu = torch.tensor([0, T], dtype=torch.int32, device=dev)
    out = {}
    errs = []
    cores = os.cpu_count() or 1
    samples = {}
    for name, bit, n_rows in (("fa", 1, args.cpu_rows), ("sa", 0, 4 * args.cpu_rows)):
        o = torch.empty_like(q)
        _lib.fa_attn_prefill(q, k, v, o, cu, T,
                             torch.tensor([[bit]], dtype=torch.uint8, device=dev), 0, SINK,
                             WINDOW, BLOCK, scale, route_host=np.array([[bit]], np.uint8))
        torch.cuda.synchronize()
        rng = np.random.default_rng(5 + bit)
        rows = np.sort(rng.choice(T, size=n_rows, replace=False)).astype(np.int32)
        qh = q.view(torch.int16).cpu().numpy().view(np.uint16)
        kh = k.view(torch.int16).cpu().numpy().view(np.uint16)
        vh = v.view(torch.int16).cpu().numpy().view(np.uint16)
        t0 = time.perf_counter()
        o_ref, _ = oracle.attn_prefill(qh, kh, vh, [0, T], np.array([[bit]], np.uint8), 0,
                                       SINK, WINDOW, BLOCK, scale, rows=rows, n_threads=cores)
        dt = time.perf_counter() - t0
        log(f"oracle {name}: {len(rows)} rows in {dt:.1f} s on {cores} threads")
        # visible pairs of the sampled rows (per head)
        if bit:
            sp = int((rows + 1).sum())
        else:
            sp = 0
            for t in rows:
                i = t // BLOCK
                full = i if i < SINK // BLOCK else SINK // BLOCK + (
                    i - max(SINK // BLOCK, i - WINDOW // BLOCK + 1))
                sp += full * BLOCK + (t - i * BLOCK + 1)
        total_pairs = pairs_fa(T) if bit else pairs_sa(T)
        samples[name] = (dt, sp, total_pairs, len(rows))
        og = o[torch.from_numpy(rows.astype(np.int64)).to(dev)].float().cpu().numpy()
        errs.append(float(np.abs(og - o_ref).max()))
    n_fa = int(route_np.sum())
    t_fa_cpu = samples["fa"][0] * samples["fa"][2] / samples["fa"][1]
    t_sa_cpu = samples["sa"][0] * samples["sa"][2] / samples["sa"][1]
    t_cpu = n_fa * t_fa_cpu + (N_LAYERS - n_fa) * t_sa_cpu
    out = {
        "value": round(T / t_cpu, 4), "unit": "tok/s", "cores": cores, "kind": "oracle",
        "sample": (f"oracle (fp64, threads={cores}) on {samples['fa'][3]} random query rows x 32 "
                   f"heads of one FA layer ({samples['fa'][0]:.1f} s) and {samples['sa'][3]} "
                   f"rows of one SA layer ({samples['sa'][0]:.1f} s) at {T} tokens, scaled by "
                   f"visible-pair count to the routed 32-layer prefill ({n_fa} FA layers); "
                   f"router time ignored"),
        "gpu_over_cpu": round(t_cpu / t_prefill_gpu, 1),
    }
    parity = {"sampled_rows_max_abs_err": max(errs), "tolerance": 2e-2,
              "pass": max(errs) <= 2e-2}
    return out, parity


if __name__ == "__main__":
    main()
