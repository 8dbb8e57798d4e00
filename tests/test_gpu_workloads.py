"""Full-size workload parity on the GPU (sampled against the oracle).

Qwen3-4B-shaped mixed workload: 36 layers, 32 query / 8 KV heads, head_dim 128,
bf16, a varlen batch of 4 sequences (16384 / 32768 / 49152 / 65536 tokens), a
router 2560 -> 256 -> 36 producing per-sequence masks, SA with sink 128 /
window 4096 / block 128, prefill and then decode steps that append to the cache.
The layer checked is one whose bits differ between sequences, so the FA and SA
sequences share one prefill launch (device-route kernel) and one decode launch.
Bars: route bits bit-exact, attention max abs error <= 2e-2 (bf16 inputs),
lse <= 1e-3.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_layerrouter_amd import _lib, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
HQ, HKV, D, L, HIDDEN = 32, 8, 128, 36, 2560
SINK, WINDOW, BLOCK = 128, 4096, 128
LENGTHS = [16384, 32768, 49152, 65536]


def bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32(a):
    return synth.bf16_bits_to_f32(a)


def sample_rows(cu, per_seq=6, seed=0):
    rng = np.random.default_rng(seed)
    rows = []
    for b in range(len(cu) - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        rows += [s, s + 1, e - 2, e - 1]
        rows += rng.integers(s, e, per_seq).tolist()
    return np.array(sorted(set(rows)), np.int32)


def test_qwen3_4b_varlen_mixed_routes_prefill_and_decode():
    cu = synth.cu_seqlens_of(LENGTHS)
    total = int(cu[-1])
    cu_d = torch.tensor(cu, device=DEV)
    scale = 1 / math.sqrt(D)

    # ---- router: per-sequence 36-bit masks
    x_q = synth.device_normal((total, HIDDEN), seed=51)
    rng = np.random.default_rng(52)
    w1, b1, w2, b2 = synth.router_weights(rng, HIDDEN, 256, L)
    route = torch.zeros((4, L), dtype=torch.uint8, device=DEV)
    logits = torch.zeros((4, L), dtype=torch.float32, device=DEV)
    _lib.fa_router_decide(x_q, cu_d, 64, *(torch.from_numpy(a).to(DEV) for a in (w1, b1, w2, b2)),
                          route, logits)
    torch.cuda.synchronize()
    r_np = route.cpu().numpy()
    # oracle on the last 64 rows of each sequence only (the pool window)
    pool_rows = np.concatenate([np.arange(int(cu[b + 1]) - 64, int(cu[b + 1])) for b in range(4)])
    xs = bits(x_q[torch.from_numpy(pool_rows).to(DEV)])
    r_ref, _, l64 = oracle.router(xs, synth.cu_seqlens_of([64] * 4), 64, w1, b1, w2, b2)
    assert np.abs(l64).min() > 1e-4
    assert np.array_equal(r_np, r_ref)
    mixed = [l for l in range(L) if 0 < r_np[:, l].sum() < 4]
    assert mixed, "no layer with mixed FA/SA sequences at this seed"
    layer = mixed[0]
    del x_q

    # ---- prefill of that layer, device-route (mixed) kernel
    q = synth.device_normal((total, HQ, D), seed=53)
    k = synth.device_normal((total, HKV, D), seed=54)
    v = synth.device_normal((total, HKV, D), seed=55)
    o = torch.empty_like(q)
    lse = torch.empty((total, HQ), dtype=torch.float32, device=DEV)
    _lib.fa_attn_prefill(q, k, v, o, cu_d, max(LENGTHS), route, layer, SINK, WINDOW, BLOCK, scale,
                         lse=lse)
    torch.cuda.synchronize()
    rows = sample_rows(cu)
    qh, kh, vh = bits(q), bits(k), bits(v)
    o_ref, l_ref = oracle.attn_prefill(qh, kh, vh, cu, r_np, layer, SINK, WINDOW, BLOCK, scale,
                                       rows=rows)
    assert np.abs(f32(bits(o)[rows]) - o_ref).max() <= 2e-2
    assert np.abs(lse.cpu().numpy()[rows] - l_ref).max() <= 1e-3
    del q, o, lse

    # ---- decode: caches hold the prefill K/V, 3 steps appending fresh tokens
    steps = 3
    max_cache = max(LENGTHS) + steps
    kc = torch.zeros((4, HKV, max_cache, D), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    for b in range(4):
        s, e = int(cu[b]), int(cu[b + 1])
        kc[b, :, : e - s] = k[s:e].transpose(0, 1)
        vc[b, :, : e - s] = v[s:e].transpose(0, 1)
    del k, v
    ws = torch.empty(_lib.fa_decode_workspace_size(4, HQ, D, max_cache), dtype=torch.uint8,
                     device=DEV)
    lengths = np.array(LENGTHS, np.int32)
    for step in range(steps):
        lengths = lengths + 1
        qd = synth.device_normal((4, HQ, D), seed=60 + step)
        kn = synth.device_normal((4, HKV, D), seed=70 + step)
        vn = synth.device_normal((4, HKV, D), seed=80 + step)
        od = torch.empty_like(qd)
        lsed = torch.empty((4, HQ), dtype=torch.float32, device=DEV)
        _lib.fa_attn_decode(qd, od, kc, vc, torch.tensor(lengths, device=DEV), route, layer, SINK,
                            WINDOW, BLOCK, scale, workspace=ws, k_new=kn, v_new=vn, lse=lsed)
        torch.cuda.synchronize()
        for b in range(4):  # the new token landed at position n - 1
            assert np.array_equal(bits(kc[b, :, lengths[b] - 1]), bits(kn[b]))
            assert np.array_equal(bits(vc[b, :, lengths[b] - 1]), bits(vn[b]))
        for g in (0, HKV - 1):
            G = HQ // HKV
            o_ref, l_ref = oracle.attn_decode(
                bits(qd[:, g * G:(g + 1) * G]), bits(kc[:, g:g + 1]), bits(vc[:, g:g + 1]), lengths,
                r_np, layer, SINK, WINDOW, BLOCK, scale)
            assert np.abs(f32(bits(od[:, g * G:(g + 1) * G])) - o_ref).max() <= 2e-2
            assert np.abs(lsed[:, g * G:(g + 1) * G].cpu().numpy() - l_ref).max() <= 1e-3
