"""GPU parity of the compact SA ring cache (fa_kv_compact + fa_attn_decode_ring).

An SA layer's decode reads only sink + window tokens, so a ring of
sink + window rows replaces the full cache.  The ring decode must give exactly
the full-cache SA decode (same kept tokens in the same order: bit-identical)
and match the oracle (max abs 2e-2 for bf16, 1e-4 for fp32) over decode steps
that cross block boundaries, the sink boundary and the ring wrap-around.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_layerrouter_amd import _lib, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def dev_from(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host_of(t):
    t = t.contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def as_f32(a):
    return synth.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a


@pytest.mark.parametrize("bf16", [True, False])
def test_ring_decode_equals_full_cache_and_oracle(bf16):
    lengths = [300, 77, 20, 1000]
    B, hq, hkv, d = len(lengths), 8, 2, 128
    sink, window, block = 32, 128, 32
    steps = 70
    rng = np.random.default_rng(90 + bf16)
    cu = synth.cu_seqlens_of(lengths)
    _, k, v = synth.qkv_host(rng, int(cu[-1]), hq, hkv, d, bf16=bf16)
    max_cache = max(lengths) + steps
    # full caches from the prefill K/V (test-side layout move, no arithmetic)
    kc = np.zeros((B, hkv, max_cache, d), k.dtype)
    vc = np.zeros_like(kc)
    for b, n in enumerate(lengths):
        kc[b, :, :n] = k[cu[b]:cu[b + 1]].transpose(1, 0, 2)
        vc[b, :, :n] = v[cu[b]:cu[b + 1]].transpose(1, 0, 2)
    kc_d, vc_d = dev_from(kc), dev_from(vc)
    ring = sink + window
    kr = torch.zeros((B, hkv, ring, d), dtype=kc_d.dtype, device=DEV)
    vr = torch.zeros_like(kr)
    _lib.fa_kv_compact(dev_from(k), dev_from(v), torch.tensor(cu, device=DEV), sink, window, block,
                       kr, vr)
    route = np.zeros((B, 1), np.uint8)
    route_d = torch.tensor(route, device=DEV)
    scale = 1 / math.sqrt(d)
    lens = np.array(lengths, np.int32)
    tol = 2e-2 if bf16 else 1e-4
    for step in range(steps):
        lens = lens + 1
        q = synth.normal(rng, (B, hq, d))
        kn = synth.normal(rng, (B, hkv, d))
        vn = synth.normal(rng, (B, hkv, d))
        if bf16:
            q, kn, vn = (synth.f32_to_bf16_bits(a) for a in (q, kn, vn))
        qd, knd, vnd = dev_from(q), dev_from(kn), dev_from(vn)
        cl = torch.tensor(lens, device=DEV)
        o_full = torch.empty_like(qd)
        o_ring = torch.empty_like(qd)
        lse_full = torch.empty((B, hq), dtype=torch.float32, device=DEV)
        lse_ring = torch.empty_like(lse_full)
        _lib.fa_attn_decode(qd, o_full, kc_d, vc_d, cl, route_d, 0, sink, window, block, scale,
                            k_new=knd, v_new=vnd, lse=lse_full, route_host=route)
        _lib.fa_attn_decode_ring(qd, o_ring, kr, vr, cl, sink, window, block, scale, k_new=knd,
                                 v_new=vnd, lse=lse_ring)
        torch.cuda.synchronize()
        assert np.array_equal(host_of(o_ring), host_of(o_full)), step
        assert np.array_equal(lse_ring.cpu().numpy(), lse_full.cpu().numpy()), step
        for b in range(B):
            kc[b, :, lens[b] - 1] = kn[b]
            vc[b, :, lens[b] - 1] = vn[b]
        if step % 10 == 9 or step == steps - 1:
            o_ref, l_ref = oracle.attn_decode(q, kc, vc, lens, route, 0, sink, window, block, scale)
            assert np.abs(as_f32(host_of(o_ring)).astype(np.float64) - o_ref).max() <= tol
            assert np.abs(lse_ring.cpu().numpy() - l_ref).max() <= (1e-3 if bf16 else 1e-4)


def test_ring_decode_llama_131k_matches_full_cache():
    """Batch 8, 131072-token sequences, Llama head layout, sink 128 / window 2048 /
    block 64: the ring (2176 rows per head) decodes exactly like the full cache."""
    B, hq, hkv, d, n = 8, 32, 8, 128, 131072
    sink, window, block = 128, 2048, 64
    kc = torch.empty((B, hkv, n + 1, d), dtype=torch.bfloat16, device=DEV)
    vc = torch.empty_like(kc)
    for b in range(B):
        kc[b, :, :n] = synth.device_normal((hkv, n, d), seed=400 + b)
        vc[b, :, :n] = synth.device_normal((hkv, n, d), seed=500 + b)
    # packed prefill layout [total, hkv, d] of the same tokens for the compaction
    cu = torch.tensor(synth.cu_seqlens_of([n] * B), device=DEV)
    kr = torch.empty((B, hkv, sink + window, d), dtype=torch.bfloat16, device=DEV)
    vr = torch.empty_like(kr)
    for b in range(B):  # compact one sequence at a time to bound the packed copy
        kp = kc[b, :, :n].transpose(0, 1).contiguous()
        vp = vc[b, :, :n].transpose(0, 1).contiguous()
        _lib.fa_kv_compact(kp, vp, torch.tensor([0, n], dtype=torch.int32, device=DEV), sink,
                           window, block, kr[b:b + 1], vr[b:b + 1])
    del kp, vp
    q = synth.device_normal((B, hq, d), seed=600)
    kn = synth.device_normal((B, hkv, d), seed=601)
    vn = synth.device_normal((B, hkv, d), seed=602)
    cl = torch.full((B,), n + 1, dtype=torch.int32, device=DEV)
    route = np.zeros((B, 1), np.uint8)
    scale = 1 / math.sqrt(d)
    o_full = torch.empty_like(q)
    o_ring = torch.empty_like(q)
    _lib.fa_attn_decode(q, o_full, kc, vc, cl, torch.tensor(route, device=DEV), 0, sink, window,
                        block, scale, k_new=kn, v_new=vn, route_host=route)
    _lib.fa_attn_decode_ring(q, o_ring, kr, vr, cl, sink, window, block, scale, k_new=kn,
                             v_new=vn)
    torch.cuda.synchronize()
    assert torch.equal(o_ring, o_full)
    # and one sampled KV head against the oracle
    G = hq // hkv
    o_ref, _ = oracle.attn_decode(host_of(q[:, :G]), host_of(kc[:, :1]), host_of(vc[:, :1]),
                                  [n + 1] * B, route, 0, sink, window, block, scale)
    assert np.abs(synth.bf16_bits_to_f32(host_of(o_ring[:, :G])) - o_ref).max() <= 2e-2
