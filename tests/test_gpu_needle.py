"""Parity on inputs whose outputs are O(1) ("needle" inputs), so that the
spec bars (max abs 2e-2 on bf16 outputs, lse 1e-3) can fail at the
headline sizes.

With i.i.d. N(0,1) Q/K/V and scale 1/sqrt(d), a late FA row at T = 131072 has
|O| ~ sqrt(e/T) ~ 0.005 per element: an all-zero output, or one built from
mis-read V tiles, would pass a 2e-2 bar.  Here every query row is a copy (x2)
of one earlier key (`synth.device_needle_qkv`), so almost all of its softmax
mass sits on that one key and its output is close to that key's V row, a
vector of size O(1).  Even heads point anywhere in the causal past (every tile
of the FA layer gets tested across rows and heads); odd heads point into the
first 128 or the last 64 positions, which are kept by the SA layer (sink 128,
window 2048, block 64).  Each test asserts that its reference outputs are at
least 5x the bar on the rows it checks, so a dropped or mis-read K/V tile, or
a zero output, fails.

Layer kinds run through the per-kind kernels picked from the host route copy,
the launch configuration the benchmark times.  Bars: 2e-2 / 1e-3 (bf16).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_layerrouter_amd import _lib, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
HQ, HKV, D = 32, 8, 128
SINK, WINDOW, BLOCK = 128, 2048, 64
BAR_O, BAR_LSE = 2e-2, 1e-3


def host_bf16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def run_prefill(q, k, v, cu_np, max_len, bit):
    o = torch.empty_like(q)
    lse = torch.empty((q.shape[0], HQ), dtype=torch.float32, device=DEV)
    r = np.array([[bit]] * (len(cu_np) - 1), np.uint8)
    _lib.fa_attn_prefill(q, k, v, o, torch.tensor(cu_np, device=DEV), max_len,
                         torch.tensor(r, device=DEV), 0, SINK, WINDOW, BLOCK, 1 / math.sqrt(D),
                         lse=lse, route_host=r)
    torch.cuda.synchronize()
    return o, lse, r


def check_rows(q, k, v, o, lse, cu_np, r, rows, fa):
    o_ref, l_ref = oracle.attn_prefill(host_bf16(q), host_bf16(k), host_bf16(v), cu_np, r, 0,
                                       SINK, WINDOW, BLOCK, 1 / math.sqrt(D), rows=rows)
    got = f64(host_bf16(o)[rows])
    err = np.abs(got - o_ref).max()
    lerr = np.abs(lse.cpu().numpy()[rows] - l_ref).max()
    # the check can fail: the reference is far above the bar on the heads whose
    # needle the layer sees (every head for FA, the odd heads for SA)
    heads = slice(None) if fa else slice(1, None, 2)
    scale = np.abs(o_ref[:, heads]).max(axis=(1, 2))
    assert scale.min() >= 5 * BAR_O, f"reference |O| {scale.min()} too small to discriminate"
    assert err <= BAR_O, f"max abs err {err}"
    assert lerr <= BAR_LSE, f"lse err {lerr}"
    return err, lerr


def needle_rows(n, fa, seed, n_random):
    rng = np.random.default_rng(seed)
    if fa:
        rows = {0, 1, 63, 64, 2047, 2048, n // 2, n - 65, n - 64, n - 2, n - 1}
    else:
        rows = set(range(0, 64, 7)) | set(range(n - 64, n))
        for edge in (SINK, WINDOW, SINK + WINDOW):
            rows |= {edge - 1, edge, edge + 1}
    rows |= set(rng.integers(0, n, n_random).tolist())
    return np.array(sorted(rows), np.int32)


@pytest.mark.parametrize("bit", [1, 0])
def test_needle_prefill_varlen_every_row(bit):
    """A ragged varlen batch (1000 / 3001 / 77 tokens), every row and head."""
    lens = [1000, 3001, 77]
    parts = [synth.device_needle_qkv(n, HQ, HKV, D, seed=40 + i) for i, n in enumerate(lens)]
    q = torch.cat([p[0] for p in parts])
    k = torch.cat([p[1] for p in parts])
    v = torch.cat([p[2] for p in parts])
    cu = synth.cu_seqlens_of(lens)
    o, lse, r = run_prefill(q, k, v, cu, max(lens), bit)
    rows = np.arange(int(cu[-1]), dtype=np.int32)
    o_ref, l_ref = oracle.attn_prefill(host_bf16(q), host_bf16(k), host_bf16(v), cu, r, 0,
                                       SINK, WINDOW, BLOCK, 1 / math.sqrt(D), rows=rows)
    assert np.abs(f64(host_bf16(o)) - o_ref).max() <= BAR_O
    assert np.abs(lse.cpu().numpy() - l_ref).max() <= BAR_LSE
    assert np.abs(o_ref[:, 1::2]).max(axis=(1, 2)).min() >= 5 * BAR_O


@pytest.mark.parametrize("bit", [1, 0])
def test_needle_prefill_131k(bit):
    """One Llama-shaped layer at 131072 tokens (the benchmark's launch), FA and SA."""
    T = 131072
    q, k, v, _ = synth.device_needle_qkv(T, HQ, HKV, D, seed=300 + bit)
    cu = np.array([0, T], np.int32)
    o, lse, r = run_prefill(q, k, v, cu, T, bit)
    rows = needle_rows(T, bool(bit), 9 + bit, 14 if bit else 200)
    check_rows(q, k, v, o, lse, cu, r, rows, bool(bit))


@pytest.mark.parametrize("bit", [1, 0])
def test_needle_prefill_262k(bit):
    """The longest context the pages evaluate (262144 tokens), FA and SA."""
    T = 262144
    q, k, v, _ = synth.device_needle_qkv(T, HQ, HKV, D, seed=310 + bit)
    cu = np.array([0, T], np.int32)
    o, lse, r = run_prefill(q, k, v, cu, T, bit)
    rows = needle_rows(T, bool(bit), 19 + bit, 6 if bit else 100)
    check_rows(q, k, v, o, lse, cu, r, rows, bool(bit))


def test_needle_decode_batch8_131k():
    """The benchmark's decode launch: batch 8 over 131072-token caches, one FA and
    one SA layer through the per-kind kernels; KV heads 0 and 7 of every sequence.
    Cache lengths differ per sequence (131072 down to 130000) so the SA window
    starts at different offsets."""
    B, n_max = 8, 131072
    G = HQ // HKV
    kc = torch.empty((B, HKV, n_max, D), dtype=torch.bfloat16, device=DEV)
    vc = torch.empty_like(kc)
    for b in range(B):
        kc[b] = synth.device_normal((HKV, n_max, D), seed=900 + 2 * b)
        vc[b] = synth.device_normal((HKV, n_max, D), seed=901 + 2 * b)
    lens = [n_max - 137 * b for b in range(B)]
    cl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    r = np.array([[1, 0]] * B, np.uint8)
    scale = 1 / math.sqrt(D)
    ws = torch.empty(_lib.fa_decode_workspace_size(B, HQ, D, n_max), dtype=torch.uint8,
                     device=DEV)
    q, _ = synth.device_needle_decode_q(kc, HQ, lens, seed=77)
    for layer in (0, 1):
        o = torch.empty_like(q)
        lse = torch.empty((B, HQ), dtype=torch.float32, device=DEV)
        _lib.fa_attn_decode(q, o, kc, vc, cl, torch.tensor(r, device=DEV), layer, SINK, WINDOW,
                            BLOCK, scale, lse=lse, route_host=r, workspace=ws)
        torch.cuda.synchronize()
        for g in (0, HKV - 1):
            o_ref, l_ref = oracle.attn_decode(
                host_bf16(q[:, g * G:(g + 1) * G]), host_bf16(kc[:, g:g + 1]),
                host_bf16(vc[:, g:g + 1]), lens, r, layer, SINK, WINDOW, BLOCK, scale)
            og = f64(host_bf16(o[:, g * G:(g + 1) * G]))
            heads = slice(None) if layer == 0 else slice(1, None, 2)
            assert np.abs(o_ref[:, heads]).max(axis=2).min() >= 5 * BAR_O
            assert np.abs(og - o_ref).max() <= BAR_O
            assert np.abs(lse[:, g * G:(g + 1) * G].cpu().numpy() - l_ref).max() <= BAR_LSE
