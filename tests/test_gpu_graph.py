"""A routed step captured as a HIP graph and replayed.

The library's launch path calls no allocation, memset or synchronising API, so
a caller can capture its calls (here with torch.cuda.CUDAGraph, whose capture
stream the binding picks up as the current stream).  The captured step -- the
router, two prefill layers and four decode layers with per-sequence routes --
is replayed several times, with the program's own eager work (NaN fills of the
outputs, an unrelated eager decode) and synchronisations between the replays;
every replay must reproduce the eager step bit for bit.
"""
import math

import numpy as np
import pytest
import torch

from sparse_attention_layerrouter_amd import _lib, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_routed_step_graph_replays_equal_eager():
    HQ, HKV, D, L = 8, 2, 128, 4
    SINK, WINDOW, BLOCK = 128, 1024, 64
    scale = 1 / math.sqrt(D)
    # prefill: a varlen batch of two sequences
    lengths = [1500, 700]
    cu = torch.tensor(synth.cu_seqlens_of(lengths), device=DEV)
    total, T = sum(lengths), max(lengths)
    qp = synth.device_normal((total, HQ, D), 11)
    kp = synth.device_normal((total, HKV, D), 12)
    vp = synth.device_normal((total, HKV, D), 13)
    # router over the prefill's hidden states: 4 layers, fp32 weights
    HID, RH = 256, 32
    x_q = synth.device_normal((total, HID), 14)
    w1 = synth.device_normal((RH, HID), 15, "f32", scale=0.1)
    b1 = torch.zeros(RH, device=DEV)
    w2 = synth.device_normal((L, RH), 16, "f32", scale=0.1)
    b2 = torch.tensor([1.0, -1.0, 0.5, -0.5], device=DEV)
    route = torch.empty((2, L), dtype=torch.uint8, device=DEV)
    logits = torch.empty((2, L), dtype=torch.float32, device=DEV)
    ws_r = torch.empty(max(_lib.fa_router_workspace_size(2, HID, RH), 1), dtype=torch.uint8,
                       device=DEV)
    # decode: four sequences over four layers, routes mixed within a layer
    B, NC = 4, 3000
    cache_len = torch.tensor([3000, 2049, 1, 130], dtype=torch.int32, device=DEV)
    dec_route_np = np.array([[1, 0, 1, 0], [0, 0, 1, 1], [1, 1, 0, 0], [0, 1, 0, 1]], np.uint8)
    dec_route = torch.from_numpy(dec_route_np).to(DEV)
    kc = [synth.device_normal((B, HKV, NC, D), 20 + l) for l in range(L)]
    vc = [synth.device_normal((B, HKV, NC, D), 30 + l) for l in range(L)]
    qd = synth.device_normal((B, HQ, D), 17)
    ws_d = torch.empty(_lib.fa_decode_workspace_size(B, HQ, D, NC), dtype=torch.uint8,
                       device=DEV)
    pre_route_np = np.array([[1, 0, 1, 0], [1, 0, 0, 1]], np.uint8)
    pre_route = torch.from_numpy(pre_route_np).to(DEV)

    def step(o_pre, lse_pre, o_dec):
        _lib.fa_router_decide(x_q, cu, 64, w1, b1, w2, b2, route, logits, ws_r)
        for l in range(2):
            _lib.fa_attn_prefill(qp, kp, vp, o_pre[l], cu, T, pre_route, l, SINK, WINDOW, BLOCK,
                                 scale, lse=lse_pre[l], route_host=pre_route_np)
        for l in range(L):
            _lib.fa_attn_decode(qd, o_dec[l], kc[l], vc[l], cache_len, dec_route, l, SINK,
                                WINDOW, BLOCK, scale, workspace=ws_d, route_host=dec_route_np)

    def outputs():
        return ([torch.empty_like(qp) for _ in range(2)],
                [torch.empty((total, HQ), dtype=torch.float32, device=DEV) for _ in range(2)],
                [torch.empty_like(qd) for _ in range(L)])

    ref = outputs()
    step(*ref)
    torch.cuda.synchronize()
    ref_route, ref_logits = route.clone(), logits.clone()

    got = outputs()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(*got)
    torch.cuda.synchronize()

    other_o = torch.empty_like(qd)
    for rep in range(3):
        for t in got[0] + got[1] + got[2] + [logits]:
            t.fill_(float("nan"))
        route.fill_(7)
        # unrelated eager work between the replays
        _lib.fa_attn_decode(qd, other_o, kc[rep], vc[rep], cache_len, dec_route, rep, SINK,
                            WINDOW, BLOCK, scale, workspace=ws_d)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(route, ref_route), rep
        assert torch.equal(bits(logits), bits(ref_logits)), rep
        for a, b in zip(got[0] + got[1] + got[2], ref[0] + ref[1] + ref[2]):
            assert torch.equal(bits(a), bits(b)), rep
