"""NaN-poisoned memory next to every input.  A kernel that reads a row it
should not -- past a sequence's end, past a cache length -- and gives it zero
weight still turns the output into NaN (0 x NaN = NaN), so these cases catch
out-of-range reads that a clean-memory parity test can miss.  Each case also
compares with the oracle on the clean values, at the parity bars."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import triangle, xattn
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


def nan_padded(a, extra_rows=512):
    """Device copy of a [rows, ...] array at the start of a NaN-filled buffer."""
    d = dev_from(a)
    big = torch.full((a.shape[0] + extra_rows,) + tuple(a.shape[1:]), float("nan"),
                     dtype=d.dtype, device=DEV)
    big[: a.shape[0]] = d
    return big[: a.shape[0]]


@pytest.mark.parametrize("kind", ["fa", "sa", "triangle"])
@pytest.mark.parametrize("bf16", [True, False])
def test_prefill_reads_nothing_past_the_last_sequence(kind, bf16):
    rng = np.random.default_rng(31)
    lengths, hq, hkv, d = [333, 1000, 65, 1], 8, 2, 128
    block, sink, window, last_q = 64, 64, 128, 64
    cu = synth.cu_seqlens_of(lengths)
    total = int(cu[-1])
    q, k, v = synth.qkv_host(rng, total, hq, hkv, d, bf16=bf16)
    scale = 1 / math.sqrt(d)
    bit = 1 if kind == "fa" else 0
    route = np.full((len(lengths), 1), bit, np.uint8)
    qd = dev_from(q)
    o = torch.empty_like(qd)
    lse = torch.empty((total, hq), dtype=torch.float32, device=DEV)
    args = [qd, nan_padded(k), nan_padded(v), o, torch.tensor(cu, device=DEV), max(lengths),
            torch.tensor(route, device=DEV), 0, sink, window, block]
    if kind == "triangle":
        _lib.fa_attn_prefill_triangle(*args, last_q, scale, lse=lse, route_host=route)
        o_ref, l_ref = triangle.attn_prefill(q, k, v, cu, route[:, 0], block, sink, window,
                                             last_q, scale)
    else:
        _lib.fa_attn_prefill(*args, scale, lse=lse, route_host=route)
        o_ref, l_ref = oracle.attn_prefill(q, k, v, cu, route, 0, sink, window, block, scale)
    torch.cuda.synchronize()
    got, l_got = as_f64(host_of(o)), lse.cpu().numpy()
    assert np.isfinite(got).all() and np.isfinite(l_got).all()
    tol, tol_lse = (2e-2, 1e-3) if bf16 else (1e-4, 1e-4)
    assert np.abs(got - o_ref).max() <= tol
    assert np.abs(l_got - l_ref).max() <= tol_lse


@pytest.mark.parametrize("bit", [1, 0])
@pytest.mark.parametrize("bf16", [True, False])
def test_decode_reads_nothing_past_the_cache_length(bit, bf16):
    rng = np.random.default_rng(37)
    B, hq, hkv, d, max_cache = 3, 8, 2, 128, 2048
    sink, window, block = 64, 512, 64
    cache_len = np.array([2000, 317, 1], np.int32)
    q = synth.normal(rng, (B, hq, d))
    kc, vc = synth.kv_cache_host(rng, B, hkv, max_cache, d, bf16=bf16)
    if bf16:
        q = synth.f32_to_bf16_bits(q)
        nan_bits = np.uint16(0x7FC0)
    for b in range(B):  # every row at or past the cache length is NaN
        if bf16:
            kc[b, :, cache_len[b]:] = nan_bits
            vc[b, :, cache_len[b]:] = nan_bits
        else:
            kc[b, :, cache_len[b]:] = np.nan
            vc[b, :, cache_len[b]:] = np.nan
    route = np.full((B, 1), bit, np.uint8)
    scale = 1 / math.sqrt(d)
    qd = dev_from(q)
    o = torch.empty_like(qd)
    lse = torch.empty((B, hq), dtype=torch.float32, device=DEV)
    _lib.fa_attn_decode(qd, o, dev_from(kc), dev_from(vc), torch.tensor(cache_len, device=DEV),
                        torch.tensor(route, device=DEV), 0, sink, window, block, scale, lse=lse,
                        route_host=route)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attn_decode(q, kc, vc, cache_len, route, 0, sink, window, block, scale)
    got, l_got = as_f64(host_of(o)), lse.cpu().numpy()
    assert np.isfinite(got).all() and np.isfinite(l_got).all()
    tol, tol_lse = (2e-2, 1e-3) if bf16 else (1e-4, 1e-4)
    assert np.abs(got - o_ref).max() <= tol
    assert np.abs(l_got - l_ref).max() <= tol_lse


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("stride", [8, 4])
def test_xattn_scores_read_nothing_past_the_last_sequence(stride, bf16):
    rng = np.random.default_rng(41)
    lengths, hq, hkv, d = [700, 130, 1], 8, 2, 128
    block = 16 * stride
    cu = synth.cu_seqlens_of(lengths)
    q, k, _ = synth.qkv_host(rng, int(cu[-1]), hq, hkv, d, bf16=bf16)
    scale = 1 / math.sqrt(d)
    nqb = -(-max(lengths) // block)
    sc = torch.zeros((len(lengths), hq, nqb, nqb), dtype=torch.float32, device=DEV)
    _lib.fa_xattn_scores(nan_padded(q), nan_padded(k), torch.tensor(cu, device=DEV),
                         max(lengths), block, stride, scale, sc)
    torch.cuda.synchronize()
    got = sc.cpu().numpy()
    ref = xattn.block_scores(q, k, cu, block, stride, scale)
    for b, T in enumerate(lengths):
        nb = -(-T // block)
        tri = np.tril(np.ones((nb, nb), bool))
        g = got[b][:, :nb, :nb][:, tri]
        assert np.isfinite(g).all()
        assert np.abs(g - ref[b][:, :nb, :nb][:, tri]).max() <= 1e-4
