"""Full-size parity in the benchmark's own launch configuration: the router on
the benchmark's 131072 x 4096 input and seeds, and the FA and SA prefill layers
at 131072 tokens through the kernels the benchmark launches (picked from the
host copy of the route), on sampled rows the oracle computes one by one."""
import math

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_layerrouter_amd import _lib, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
T = 131072
HIDDEN, ROUTER_HIDDEN, N_LAYERS, POOL = 4096, 256, 32, 64
SINK, WINDOW, BLOCK = 128, 2048, 64


def host_bf16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def test_router_on_the_benchmark_input():
    """x_Q [131072, 4096] bf16 (seed 11), Xavier 4096 -> 256 -> 32 (rng seed 0): the
    route bits bit-exact and the logits within fp32 rounding of the oracle, which
    pools the same last 64 rows."""
    x = synth.device_normal((T, HIDDEN), seed=11)
    rng = np.random.default_rng(0)
    w1, b1, w2, b2 = synth.router_weights(rng, HIDDEN, ROUTER_HIDDEN, N_LAYERS)
    cu = torch.tensor([0, T], dtype=torch.int32, device=DEV)
    route = torch.zeros((1, N_LAYERS), dtype=torch.uint8, device=DEV)
    logits = torch.zeros((1, N_LAYERS), dtype=torch.float32, device=DEV)
    ws = torch.empty(_lib.fa_router_workspace_size(1, HIDDEN, ROUTER_HIDDEN), dtype=torch.uint8,
                     device=DEV)
    wd = [torch.from_numpy(a).to(DEV) for a in (w1, b1, w2, b2)]
    _lib.fa_router_decide(x, cu, POOL, *wd, route, logits, ws)
    torch.cuda.synchronize()
    tail = host_bf16(x[T - POOL:])  # the pooling window: the last 64 rows
    r_ref, _, l64 = oracle.router(tail, np.array([0, POOL], np.int32), POOL, w1, b1, w2, b2)
    assert np.abs(l64).min() > 1e-4, "a logit sits on the threshold: bit not determined"
    assert np.array_equal(route.cpu().numpy(), r_ref)
    assert np.abs(logits.cpu().numpy() - l64).max() < 1e-5


def sample_rows(n_random, seed, fa, n=T):
    rng = np.random.default_rng(seed)
    if fa:  # the FA oracle costs O(T) per row: a few rows at each end and at random
        rows = {0, 1, 63, 64, 2047, 2048, n - 65, n - 64, n - 2, n - 1}
    else:
        rows = set(range(64)) | set(range(n - 64, n))
        for edge in (SINK, WINDOW, SINK + WINDOW):
            rows |= {edge - 1, edge, edge + 1}
    rows |= set(rng.integers(0, n, n_random).tolist())
    return np.array(sorted(rows), np.int32)


@pytest.mark.parametrize("bit", [1, 0])
def test_prefill_131k_sampled_rows(bit):
    """One Llama-shaped layer (32 q / 8 kv heads, d 128, bf16) at 131072 tokens, run
    as FA and as SA (sink 128, window 2048, block 64) with the host route copy, so
    the per-kind kernel the benchmark times runs; every head of sampled rows."""
    hq, hkv, d = 32, 8, 128
    q = synth.device_normal((T, hq, d), seed=100)
    k = synth.device_normal((T, hkv, d), seed=101)
    v = synth.device_normal((T, hkv, d), seed=102)
    o = torch.empty_like(q)
    lse = torch.empty((T, hq), dtype=torch.float32, device=DEV)
    r = np.array([[bit]], np.uint8)
    scale = 1 / math.sqrt(d)
    _lib.fa_attn_prefill(q, k, v, o, torch.tensor([0, T], dtype=torch.int32, device=DEV), T,
                         torch.tensor(r, device=DEV), 0, SINK, WINDOW, BLOCK, scale, lse=lse,
                         route_host=r)
    torch.cuda.synchronize()
    rows = sample_rows(4 if bit else 200, seed=7 + bit, fa=bool(bit))
    o_ref, l_ref = oracle.attn_prefill(host_bf16(q), host_bf16(k), host_bf16(v), [0, T], r, 0,
                                       SINK, WINDOW, BLOCK, scale, rows=rows)
    got = synth.bf16_bits_to_f32(host_bf16(o)[rows]).astype(np.float64)
    assert np.abs(got - o_ref).max() <= 2e-2
    assert np.abs(lse.cpu().numpy()[rows] - l_ref).max() <= 1e-3


@pytest.mark.parametrize("bit", [1, 0])
def test_prefill_262k_sampled_rows(bit):
    """The longest context the pages evaluate (RULER at 256K): one Llama-shaped
    layer at 262144 tokens, FA and SA, through the per-kind kernels; every head
    of sampled rows, the last ones included."""
    hq, hkv, d, n = 32, 8, 128, 262144
    q = synth.device_normal((n, hq, d), seed=110)
    k = synth.device_normal((n, hkv, d), seed=111)
    v = synth.device_normal((n, hkv, d), seed=112)
    o = torch.empty_like(q)
    lse = torch.empty((n, hq), dtype=torch.float32, device=DEV)
    r = np.array([[bit]], np.uint8)
    scale = 1 / math.sqrt(d)
    _lib.fa_attn_prefill(q, k, v, o, torch.tensor([0, n], dtype=torch.int32, device=DEV), n,
                         torch.tensor(r, device=DEV), 0, SINK, WINDOW, BLOCK, scale, lse=lse,
                         route_host=r)
    torch.cuda.synchronize()
    rows = sample_rows(2 if bit else 100, seed=17 + bit, fa=bool(bit), n=n)
    o_ref, l_ref = oracle.attn_prefill(host_bf16(q), host_bf16(k), host_bf16(v), [0, n], r, 0,
                                       SINK, WINDOW, BLOCK, scale, rows=rows)
    got = synth.bf16_bits_to_f32(host_bf16(o)[rows]).astype(np.float64)
    assert np.abs(got - o_ref).max() <= 2e-2
    assert np.abs(lse.cpu().numpy()[rows] - l_ref).max() <= 1e-3


@pytest.mark.parametrize("bs", [32])
def test_decode_serving_batch_32k_sampled_heads(bs):
    """The batched-serving launch: batch 32 over 32768-token bf16 caches (Llama shape),
    the route copy on the host, one FA and one SA layer; KV heads 0 and 7 of every
    sequence against the oracle."""
    hq, hkv, d, n = 32, 8, 128, 32768
    G = hq // hkv
    kc = torch.empty((bs, hkv, n, d), dtype=torch.bfloat16, device=DEV)
    vc = torch.empty_like(kc)
    for b in range(bs):
        kc[b] = synth.device_normal((hkv, n, d), seed=500 + b)
        vc[b] = synth.device_normal((hkv, n, d), seed=600 + b)
    q = synth.device_normal((bs, hq, d), seed=700)
    cl = torch.full((bs,), n, dtype=torch.int32, device=DEV)
    r = np.array([[1, 0]] * bs, np.uint8)
    scale = 1 / math.sqrt(d)
    for layer in (0, 1):
        o = torch.empty_like(q)
        lse = torch.empty((bs, hq), dtype=torch.float32, device=DEV)
        _lib.fa_attn_decode(q, o, kc, vc, cl, torch.tensor(r, device=DEV), layer, SINK, WINDOW,
                            BLOCK, scale, lse=lse, route_host=r)
        torch.cuda.synchronize()
        for g in (0, hkv - 1):
            o_ref, l_ref = oracle.attn_decode(
                host_bf16(q[:, g * G:(g + 1) * G]), host_bf16(kc[:, g:g + 1]),
                host_bf16(vc[:, g:g + 1]), [n] * bs, r, layer, SINK, WINDOW, BLOCK, scale)
            og = synth.bf16_bits_to_f32(host_bf16(o[:, g * G:(g + 1) * G])).astype(np.float64)
            assert np.abs(og - o_ref).max() <= 2e-2
            assert np.abs(lse[:, g * G:(g + 1) * G].cpu().numpy() - l_ref).max() <= 1e-3
