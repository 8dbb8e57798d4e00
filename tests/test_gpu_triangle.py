"""GPU parity of fa_attn_prefill_triangle (Triangle Attention as the sparse
branch) against oracle/triangle.py, through the C ABI.

Bars: attention within 2e-2 max-abs for bf16 inputs and 1e-4 for fp32, lse
within 1e-3 / 1e-4 (the prefill bars).  No dense tail must reproduce the
streaming SA kernel bit for bit, a tail covering the sequence the FA kernel,
and the per-kind kernels picked from the host route copy the mixed kernel.
"""
import math

import numpy as np
import pytest
import torch

from oracle import triangle
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


def run(fn, q, k, v, cu, routes, sink, window, block, scale, last_q=None, route_host=True):
    qd, kd, vd = dev_from(q), dev_from(k), dev_from(v)
    o = torch.empty_like(qd)
    lse = torch.empty((q.shape[0], q.shape[1]), dtype=torch.float32, device=DEV)
    r = np.asarray(routes, np.uint8).reshape(-1, 1)
    args = [qd, kd, vd, o, torch.tensor(cu, device=DEV), int(np.diff(cu).max()),
            torch.tensor(r, device=DEV), 0, sink, window, block]
    if last_q is not None:
        args.append(last_q)
    fn(*args, scale, lse=lse, route_host=r if route_host else None)
    torch.cuda.synchronize()
    return host_of(o), lse.cpu().numpy()


CASES = [
    # lengths, hq, hkv, d, block, sink, window, last_q, bf16, routes
    ([1000, 333, 64, 1], 8, 2, 128, 64, 128, 256, 128, True, [0, 0, 1, 0]),  # MFMA, mixed
    ([700, 130], 8, 2, 128, 16, 16, 64, 32, True, [0, 0]),   # tail edge inside a wave's rows
    ([517], 4, 4, 128, 32, 32, 64, 64, True, [0]),           # G = 1
    ([390, 200], 16, 2, 64, 64, 64, 128, 64, True, [0, 0]),  # G = 8, d = 64
    ([300, 90], 8, 2, 128, 16, 16, 48, 48, False, [0, 1]),   # fp32: plain kernel
    ([257], 12, 4, 64, 16, 16, 32, 16, True, [0]),           # G = 3: plain bf16 kernel
    ([2048, 1500], 32, 8, 128, 64, 128, 512, 256, True, [0, 0]),  # Llama heads
]


@pytest.mark.parametrize("case", CASES)
def test_triangle_prefill_matches_oracle(case):
    lengths, hq, hkv, d, block, sink, window, last_q, bf16, routes = case
    rng = np.random.default_rng(sum(lengths) + hq + block + last_q)
    cu = synth.cu_seqlens_of(lengths)
    q, k, v = synth.qkv_host(rng, int(cu[-1]), hq, hkv, d, bf16=bf16)
    scale = 1 / math.sqrt(d)
    o, lse = run(_lib.fa_attn_prefill_triangle, q, k, v, cu, routes, sink, window, block, scale,
                 last_q)
    o_ref, l_ref = triangle.attn_prefill(q, k, v, cu, routes, block, sink, window, last_q, scale)
    tol, tol_lse = (2e-2, 1e-3) if bf16 else (1e-4, 1e-4)
    assert np.abs(as_f64(o) - o_ref).max() <= tol
    assert np.abs(lse - l_ref).max() <= tol_lse
    # the kernel picked from the host route copy equals the per-sequence-route kernel
    o2, lse2 = run(_lib.fa_attn_prefill_triangle, q, k, v, cu, routes, sink, window, block,
                   scale, last_q, route_host=False)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


@pytest.mark.parametrize("bf16", [True, False])
def test_no_tail_is_the_sa_kernel_and_covering_tail_the_fa_kernel(bf16):
    rng = np.random.default_rng(21)
    lengths, hq, hkv, d, block, sink, window = [1000, 257], 8, 2, 128, 64, 128, 256
    cu = synth.cu_seqlens_of(lengths)
    q, k, v = synth.qkv_host(rng, int(cu[-1]), hq, hkv, d, bf16=bf16)
    sa = [0, 0]
    o_t0, l_t0 = run(_lib.fa_attn_prefill_triangle, q, k, v, cu, sa, sink, window, block, 0.09, 0)
    o_sa, l_sa = run(_lib.fa_attn_prefill, q, k, v, cu, sa, sink, window, block, 0.09)
    assert np.array_equal(o_t0, o_sa) and np.array_equal(l_t0, l_sa)
    o_tf, l_tf = run(_lib.fa_attn_prefill_triangle, q, k, v, cu, sa, sink, window, block, 0.09,
                     1024)
    o_fa, l_fa = run(_lib.fa_attn_prefill, q, k, v, cu, [1, 1], sink, window, block, 0.09)
    assert np.array_equal(o_tf, o_fa) and np.array_equal(l_tf, l_fa)


def test_full_size_llama_128k_sampled():
    """A 131072-token Llama-shaped layer (32 q / 8 kv heads, d 128, bf16; sink
    128, window 2048, block 64, dense tail 128), launched as the benchmark
    launches it: sampled rows before and inside the tail against the oracle."""
    T, hq, hkv, d = 131072, 32, 8, 128
    sink, window, block, last_q = 128, 2048, 64, 128
    scale = 1 / math.sqrt(d)
    q = synth.device_normal((T, hq, d), seed=41)
    k = synth.device_normal((T, hkv, d), seed=42)
    v = synth.device_normal((T, hkv, d), seed=43)
    o = torch.empty_like(q)
    lse = torch.empty((T, hq), dtype=torch.float32, device=DEV)
    r = np.zeros((1, 1), np.uint8)
    _lib.fa_attn_prefill_triangle(q, k, v, o, torch.tensor([0, T], dtype=torch.int32, device=DEV),
                                  T, torch.tensor(r, device=DEV), 0, sink, window, block, last_q,
                                  scale, lse=lse, route_host=r)
    torch.cuda.synchronize()
    rows = [0, 2047, 70001, T - 129, T - 128, T - 65, T - 1]
    qh, kh, vh = host_of(q), host_of(k), host_of(v)
    o_ref, l_ref = triangle.attn_prefill(qh, kh, vh, [0, T], [0], block, sink, window, last_q,
                                         scale, rows=rows)
    oh = as_f64(host_of(o)[rows])
    assert np.abs(oh - o_ref).max() <= 2e-2
    assert np.abs(lse.cpu().numpy()[rows] - l_ref).max() <= 1e-3


@pytest.mark.parametrize("bf16", [True, False])
def test_empty_and_short_sequences(bf16):
    """A zero-length sequence, one shorter than the tail and one shorter than a
    block, beside a normal one."""
    rng = np.random.default_rng(29)
    lengths, hq, hkv, d = [700, 0, 40, 130], 8, 2, 128
    block, sink, window, last_q = 64, 64, 128, 128
    cu = synth.cu_seqlens_of(lengths)
    q, k, v = synth.qkv_host(rng, int(cu[-1]), hq, hkv, d, bf16=bf16)
    routes = [0, 0, 0, 0]
    o, lse = run(_lib.fa_attn_prefill_triangle, q, k, v, cu, routes, sink, window, block, 0.09,
                 last_q)
    o_ref, l_ref = triangle.attn_prefill(q, k, v, cu, routes, block, sink, window, last_q, 0.09)
    tol, tol_lse = (2e-2, 1e-3) if bf16 else (1e-4, 1e-4)
    assert np.abs(as_f64(o) - o_ref).max() <= tol
    assert np.abs(lse - l_ref).max() <= tol_lse
