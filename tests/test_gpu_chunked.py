"""GPU parity of prefill over a key prefix (fa_attn_prefill_kv): chunked prefill.

The queries of sequence b are its last Tq_b tokens and attend to all Tk_b of
its keys, so the outputs must equal the oracle's full prefill restricted to
rows Tk_b - Tq_b .. Tk_b - 1 (bars: max abs 2e-2 for bf16 inputs, 1e-4 for
fp32; lse 1e-3 / 1e-4).  Processing a sequence in 64-aligned chunks visits the
same tiles in the same order as one prefill call, so the concatenated chunk
outputs must be bit-identical to it.
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


def as_f64(a):
    return (synth.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)


def i32(a):
    return torch.tensor(np.asarray(a, np.int32), device=DEV)


CASES = [
    # (Tk, Tq) per sequence, hq, hkv, d, route bits, sink, window, block, bf16
    ([(700, 700), (1000, 333), (517, 1), (300, 64), (129, 65)], 8, 2, 128, [1, 0, 1, 0, 1],
     64, 256, 64, True),
    ([(900, 200), (400, 399)], 4, 4, 128, [0, 1], 32, 128, 32, True),     # G = 1
    ([(650, 100), (200, 200)], 16, 2, 64, [1, 0], 64, 192, 64, True),     # G = 8, d = 64
    ([(600, 250), (90, 90)], 8, 2, 128, [0, 1], 32, 64, 16, False),       # fp32
]


@pytest.mark.parametrize("case", CASES)
def test_prefill_kv_matches_oracle_suffix_rows(case):
    pairs, hq, hkv, d, bits, sink, window, block, bf16 = case
    rng = np.random.default_rng(11 + hq + d)
    tk = [a for a, _ in pairs]
    tq = [b for _, b in pairs]
    cu_k = synth.cu_seqlens_of(tk)
    cu_q = synth.cu_seqlens_of(tq)
    q_full, k, v = synth.qkv_host(rng, int(cu_k[-1]), hq, hkv, d, bf16=bf16)
    rows = np.concatenate([np.arange(cu_k[b + 1] - tq[b], cu_k[b + 1]) for b in range(len(pairs))])
    q = q_full[rows]
    route = np.array(bits, np.uint8)[:, None]
    scale = 1 / math.sqrt(d)
    qd = dev_from(q)
    o = torch.empty_like(qd)
    lse = torch.empty((len(rows), hq), dtype=torch.float32, device=DEV)
    _lib.fa_attn_prefill_kv(qd, dev_from(k), dev_from(v), o, i32(cu_q), i32(cu_k), max(tq),
                            torch.tensor(route, device=DEV), 0, sink, window, block, scale,
                            lse=lse)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attn_prefill(q_full, k, v, cu_k, route, 0, sink, window, block, scale,
                                       rows=rows.astype(np.int32))
    tol, tol_lse = (2e-2, 1e-3) if bf16 else (1e-4, 1e-4)
    assert np.abs(as_f64(host_of(o)) - o_ref).max() <= tol
    assert np.abs(lse.cpu().numpy() - l_ref).max() <= tol_lse


@pytest.mark.parametrize("bit,hq", [(1, 32), (0, 32), (1, 8)])
def test_chunked_prefill_is_bit_identical_to_one_call(bit, hq):
    T, hkv, d, chunk = 4096, 8, 128, 1024
    if hq == 8:
        hkv = 8  # G = 1: 256-position workgroups, still aligned with 1024-token chunks
    q = synth.device_normal((T, hq, d), seed=21)
    k = synth.device_normal((T, hkv, d), seed=22)
    v = synth.device_normal((T, hkv, d), seed=23)
    route = torch.full((1, 1), bit, dtype=torch.uint8, device=DEV)
    rh = np.full((1, 1), bit, np.uint8)
    scale = 1 / math.sqrt(d)
    o_one = torch.empty_like(q)
    l_one = torch.empty((T, hq), dtype=torch.float32, device=DEV)
    _lib.fa_attn_prefill(q, k, v, o_one, i32([0, T]), T, route, 0, 128, 1024, 64, scale,
                         lse=l_one, route_host=rh)
    o_ch = torch.empty_like(q)
    l_ch = torch.empty_like(l_one)
    for c0 in range(0, T, chunk):
        c1 = c0 + chunk
        # keys: the whole prefix 0 .. c1-1; queries: the chunk
        _lib.fa_attn_prefill_kv(q[c0:c1], k[:c1], v[:c1], o_ch[c0:c1], i32([0, chunk]),
                                i32([0, c1]), chunk, route, 0, 128, 1024, 64, scale,
                                lse=l_ch[c0:c1], route_host=rh)
    torch.cuda.synchronize()
    assert torch.equal(o_ch, o_one)
    assert torch.equal(l_ch, l_one)


def test_prefill_kv_more_queries_than_keys_gives_nan():
    rng = np.random.default_rng(3)
    tk, tq = [100, 300], [120, 50]   # sequence 0 is invalid (Tq > Tk)
    cu_k, cu_q = synth.cu_seqlens_of(tk), synth.cu_seqlens_of(tq)
    _, k, v = synth.qkv_host(rng, int(cu_k[-1]), 8, 2, 128, bf16=True)
    q_full, _, _ = synth.qkv_host(rng, int(cu_k[-1]), 8, 2, 128, bf16=True)
    q = np.concatenate([q_full[:120], q_full[cu_k[2] - 50:cu_k[2]]])
    route = np.ones((2, 1), np.uint8)
    qd = dev_from(q)
    o = torch.zeros_like(qd)
    lse = torch.zeros((170, 8), dtype=torch.float32, device=DEV)
    _lib.fa_attn_prefill_kv(qd, dev_from(k), dev_from(v), o, i32(cu_q), i32(cu_k), 120,
                            torch.tensor(route, device=DEV), 0, 64, 128, 64, 1 / math.sqrt(128),
                            lse=lse)
    torch.cuda.synchronize()
    of = as_f64(host_of(o))
    assert np.isnan(of[:120]).all() and np.isnan(lse[:120].cpu().numpy()).all()
    rows = np.arange(cu_k[2] - 50, cu_k[2]).astype(np.int32)
    o_ref, _ = oracle.attn_prefill(q_full, k, v, cu_k, route, 0, 64, 128, 64, 1 / math.sqrt(128),
                                   rows=rows)
    assert np.abs(of[120:] - o_ref).max() <= 2e-2
