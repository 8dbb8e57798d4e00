"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and lays them out; it holds none of the
attention or routing arithmetic.  Host inputs come from
``numpy.random.default_rng(seed)`` drawn in a fixed order; large device inputs
come from a seeded ``torch.Generator`` on the GPU.  bf16 values are produced
from fp32 by round-to-nearest-even and carried on the host as their uint16 bit
patterns.

Workload shapes: Llama-3.1-8B attention
(32 query heads, 8 KV heads, head_dim 128) and Qwen3-4B attention (same head
layout, 36 layers, hidden 2560), the model shapes the pages evaluate on
[thelatestinai paper page, Tables 1, 15, 18].
"""
from __future__ import annotations

import math

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); return the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to fp32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def xavier_uniform(rng: np.random.Generator, fan_out: int, fan_in: int) -> np.ndarray:
    """Glorot-uniform weights U(-a, a), a = sqrt(6 / (fan_in + fan_out)), shape [fan_out, fan_in]."""
    a = math.sqrt(6.0 / (fan_in + fan_out))
    return rng.uniform(-a, a, size=(fan_out, fan_in)).astype(np.float32)


def normal(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    return (rng.standard_normal(size=shape) * scale).astype(np.float32)


# ---------------------------------------------------------------------------
# Tiny case: 2 layers, 4 query heads / 2 KV heads, head_dim 64, fp32, T=256.
# ---------------------------------------------------------------------------

TINY = dict(n_layers=2, hq=4, hkv=2, d=64, seq=256, hidden=256, router_hidden=16,
            sink=16, window=64, block=16, pool=64)


def tiny_case(seed: int = 0) -> dict:
    """Tiny CPU-checkable case.

    Per layer Q [256, 4, 64], K and V [256, 2, 64] ~ N(0,1)/sqrt(64), drawn in the
    order layer0 Q, K, V, then layer1 Q, K, V.  Router: x_Q [256, 256] ~ N(0,1),
    W1 [16, 256] Xavier, b1 = 0, and logits fixed by W2 = 0, b2 = (+1, -1), which
    sends layer 0 to FA and layer 1 to SA."""
    c = TINY
    rng = np.random.default_rng(seed)
    s = 1.0 / math.sqrt(c["d"])
    layers = []
    for _ in range(c["n_layers"]):
        q = normal(rng, (c["seq"], c["hq"], c["d"]), s)
        k = normal(rng, (c["seq"], c["hkv"], c["d"]), s)
        v = normal(rng, (c["seq"], c["hkv"], c["d"]), s)
        layers.append((q, k, v))
    x_q = normal(rng, (c["seq"], c["hidden"]))
    w1 = xavier_uniform(rng, c["router_hidden"], c["hidden"])
    b1 = np.zeros(c["router_hidden"], np.float32)
    w2 = np.zeros((c["n_layers"], c["router_hidden"]), np.float32)
    b2 = np.array([1.0, -1.0], np.float32)
    cu = np.array([0, c["seq"]], np.int32)
    return dict(cfg=c, layers=layers, x_q=x_q, w1=w1, b1=b1, w2=w2, b2=b2, cu_seqlens=cu)


def router_weights(rng: np.random.Generator, hidden: int, router_hidden: int, n_layers: int):
    """Random-init Xavier router MLP hidden -> router_hidden -> n_layers, zero biases."""
    w1 = xavier_uniform(rng, router_hidden, hidden)
    b1 = np.zeros(router_hidden, np.float32)
    w2 = xavier_uniform(rng, n_layers, router_hidden)
    b2 = np.zeros(n_layers, np.float32)
    return w1, b1, w2, b2


def cu_seqlens_of(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, np.int64))
    return cu


def qkv_host(rng: np.random.Generator, total: int, hq: int, hkv: int, d: int,
             scale: float = 1.0, bf16: bool = True):
    """Packed Q [total, hq, d] and K, V [total, hkv, d] ~ N(0, scale^2).

    bf16=True returns uint16 bit patterns (RNE from fp32), else fp32."""
    q = normal(rng, (total, hq, d), scale)
    k = normal(rng, (total, hkv, d), scale)
    v = normal(rng, (total, hkv, d), scale)
    if bf16:
        return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    return q, k, v


def kv_cache_host(rng: np.random.Generator, batch: int, hkv: int, max_cache: int, d: int,
                  scale: float = 1.0, bf16: bool = True):
    """KV cache [batch, hkv, max_cache, d] ~ N(0, scale^2)."""
    k = normal(rng, (batch, hkv, max_cache, d), scale)
    v = normal(rng, (batch, hkv, max_cache, d), scale)
    if bf16:
        return f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    return k, v


# ---------------------------------------------------------------------------
# Device-side generators for the large shapes (torch is plumbing only).
# ---------------------------------------------------------------------------

def device_normal(shape, seed: int, dtype_name: str = "bf16", device: str = "cuda:0",
                  scale: float = 1.0):
    """N(0, scale^2) tensor drawn on the device from a seeded torch.Generator."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    dt = torch.bfloat16 if dtype_name == "bf16" else torch.float32
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if scale != 1.0:
        t.mul_(scale)
    return t.to(dt)


def device_positional_qkv(T: int, hq: int, hkv: int, d: int, seed: int, alpha: float,
                          device: str = "cuda:0"):
    """Locality-structured bf16 Q, K, V [T, heads, d] drawn on the device.

    Q and K are N(0,1) plus alpha times a sinusoidal position code on their first
    32 dims: [cos(t w_i), sin(t w_i)], w_i = 2 pi / (64 * 2^i), i = 0..15.  The
    code's dot product between positions t and s is alpha^2 * sum_i cos((t-s) w_i),
    largest at t = s and decaying with distance, so attention mass concentrates
    on nearby keys the way it does in trained long-context models; V is N(0,1).
    Drawn in the order Q, K, V from one seeded generator."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.arange(T, device=device, dtype=torch.float32)[:, None]
    w = 2 * math.pi / (64.0 * 2.0 ** torch.arange(16, device=device, dtype=torch.float32))
    pe = torch.cat([torch.cos(t * w), torch.sin(t * w)], dim=1)  # [T, 32]

    def draw(h, with_pe):
        x = torch.randn((T, h, d), generator=g, device=device, dtype=torch.float32)
        if with_pe:
            x[:, :, :32] += alpha * pe[:, None, :]
        return x.to(torch.bfloat16)

    q = draw(hq, True)
    k = draw(hkv, True)
    v = draw(hkv, False)
    return q, k, v


def _needle_positions(t, n_heads: int, gen, n_first: int, n_recent: int):
    """One key position per (query position, head) for the needle inputs below.

    t: int64 tensor of query positions.  Even heads draw uniformly from [0, t]
    (anywhere in the causal past); odd heads draw, with even odds, from the first
    min(t + 1, n_first) positions or from the last n_recent positions up to t.
    Returns an int64 tensor [len(t), n_heads]."""
    import torch

    dev = t.device
    n = t.numel()
    u_far = torch.rand((n, n_heads), generator=gen, device=dev, dtype=torch.float64)
    u_near = torch.rand((n, n_heads), generator=gen, device=dev, dtype=torch.float64)
    pick_first = torch.rand((n, n_heads), generator=gen, device=dev) < 0.5
    tt = t[:, None]
    far = torch.minimum(torch.floor(u_far * (tt + 1).double()).long(), tt)
    n_f = torch.clamp(tt + 1, max=n_first)
    first = torch.minimum(torch.floor(u_near * n_f.double()).long(), n_f - 1)
    lo = torch.clamp(tt - (n_recent - 1), min=0)
    recent = torch.minimum(lo + torch.floor(u_near * (tt - lo + 1).double()).long(), tt)
    near = torch.where(pick_first, first, recent)
    even = (torch.arange(n_heads, device=dev) % 2 == 0)[None, :]
    return torch.where(even, far, near)


def device_needle_qkv(T: int, hq: int, hkv: int, d: int, seed: int, beta: float = 2.0,
                      n_first: int = 128, n_recent: int = 64, device: str = "cuda:0"):
    """bf16 Q, K, V [T, heads, d] in which every query row points at one earlier key.

    K and V are N(0,1).  Query row t of head h is beta * K[g][h // G] (G = hq / hkv),
    a copy of the key at a drawn position g <= t (see _needle_positions); beta = 2
    scales bf16 values exactly.  That key's score (about beta * d / sqrt(d)) stands
    far above the others, so a row's output is close to one V row, a vector of
    size O(1): a dropped, misplaced or mis-read key/value tile moves the output by
    O(1) instead of by O(1/sqrt(T)) as with i.i.d. inputs.  Returns (q, k, v, g)
    with g the int64 positions [T, hq]."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    k = torch.randn((T, hkv, d), generator=gen, device=device, dtype=torch.float32)
    k = k.to(torch.bfloat16)
    v = torch.randn((T, hkv, d), generator=gen, device=device, dtype=torch.float32)
    v = v.to(torch.bfloat16)
    t = torch.arange(T, device=device, dtype=torch.int64)
    g = _needle_positions(t, hq, gen, n_first, n_recent)
    kvh = (torch.arange(hq, device=device) // (hq // hkv))[None, :]
    q = k[g, kvh] * beta
    return q.contiguous(), k, v, g


def device_needle_decode_q(k_cache, hq: int, cache_len, seed: int, beta: float = 2.0,
                           n_first: int = 128, n_recent: int = 64):
    """Decode queries [B, hq, d] (bf16) pointing at one cached key each.

    k_cache [B, hkv, max_cache, d] bf16; cache_len: host sequence of the cache
    lengths n_b (the query sits at position n_b - 1).  Query head h of sequence b
    is beta * k_cache[b][h // G][g], g drawn as in _needle_positions with
    t = n_b - 1.  Returns (q, g)."""
    import torch

    dev = k_cache.device
    B, hkv = k_cache.shape[0], k_cache.shape[1]
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    t = torch.tensor([int(n) - 1 for n in cache_len], device=dev, dtype=torch.int64)
    g = _needle_positions(t, hq, gen, n_first, n_recent)
    b_idx = torch.arange(B, device=dev)[:, None]
    kvh = (torch.arange(hq, device=dev) // (hq // hkv))[None, :]
    q = k_cache[b_idx, kvh, g] * beta
    return q.contiguous(), g
