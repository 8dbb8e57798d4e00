"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars (written in every test):
  - route bits and block plans: bit-exact;
  - attention outputs: max abs error <= 1e-4 for fp32 inputs and <= 2e-2 for
    bf16 inputs, against the oracle's fp64 result on the same input bytes;
  - lse: <= 1e-3 (scores are exact bf16 products summed in fp32).
Small cases run the oracle on every row; the full-size cases compare sampled
rows / heads the oracle computes one by one.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_layerrouter_amd import _lib, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL_F32 = 1e-4
TOL_BF16 = 2e-2
TOL_LSE = 1e-3


# ---------------------------------------------------------------------------
# host <-> device helpers (no method arithmetic)
# ---------------------------------------------------------------------------

def dev_from(a: np.ndarray) -> torch.Tensor:
    """numpy fp32 -> float32 tensor; numpy uint16 (bf16 bits) -> bfloat16 tensor."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host_of(t: torch.Tensor) -> np.ndarray:
    """device tensor -> numpy with the same bytes (bf16 -> uint16 bits)."""
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def as_f32(a: np.ndarray) -> np.ndarray:
    return synth.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a.astype(np.float32)


def i32(a):
    return torch.tensor(np.asarray(a, np.int32), device=DEV)


def u8(a):
    return torch.tensor(np.asarray(a, np.uint8), device=DEV)


def max_err(gpu, ref):
    return float(np.abs(as_f32(gpu).astype(np.float64) - ref).max())


# ---------------------------------------------------------------------------
# Router
# ---------------------------------------------------------------------------

def run_router(x, cu, pool, w1, b1, w2, b2):
    B, L = len(cu) - 1, w2.shape[0]
    route = torch.zeros((B, L), dtype=torch.uint8, device=DEV)
    logits = torch.zeros((B, L), dtype=torch.float32, device=DEV)
    _lib.fa_router_decide(dev_from(x), i32(cu), pool, dev_from(w1), dev_from(b1), dev_from(w2),
                          dev_from(b2), route, logits)
    torch.cuda.synchronize()
    return route.cpu().numpy(), logits.cpu().numpy()


def test_router_tiny_fixed_logits():
    """Tiny case: W2 = 0, b2 = (+1, -1) sends layer 0 to FA and layer 1 to SA."""
    c = synth.tiny_case(0)
    route, logits = run_router(c["x_q"], c["cu_seqlens"], 64, c["w1"], c["b1"], c["w2"], c["b2"])
    assert route.tolist() == [[1, 0]]
    assert logits.tolist() == [[1.0, -1.0]]


@pytest.mark.parametrize("bf16", [True, False])
def test_router_matches_oracle_bits(bf16):
    """Llama-shaped router 4096 -> 256 -> 32 on a varlen batch: bits bit-exact, logits
    within fp32 rounding of the oracle; every logit is far from the threshold."""
    rng = np.random.default_rng(21)
    lengths = [100, 7, 3000, 64]
    cu = synth.cu_seqlens_of(lengths)
    x = synth.normal(rng, (int(cu[-1]), 4096))
    if bf16:
        x = synth.f32_to_bf16_bits(x)
    w1, b1, w2, b2 = synth.router_weights(rng, 4096, 256, 32)
    route, logits = run_router(x, cu, 64, w1, b1, w2, b2)
    r_ref, l32, l64 = oracle.router(x, cu, 64, w1, b1, w2, b2)
    assert np.abs(l64).min() > 1e-4, "a logit sits on the threshold: bit not determined"
    assert np.array_equal(route, r_ref)
    assert np.abs(logits - l64).max() < 1e-5
    route2, logits2 = run_router(x, cu, 64, w1, b1, w2, b2)
    assert np.array_equal(route2, route) and np.array_equal(logits2, logits)


# ---------------------------------------------------------------------------
# Block plan
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("lengths,bits,sink,window,block", [
    ([256], [0], 16, 64, 16),
    ([32768], [0], 128, 2048, 64),
    ([32768], [1], 128, 2048, 64),
    ([16384, 32768, 49152, 65536], [0, 1, 0, 1], 128, 4096, 128),
    ([1, 17, 1000, 333], [0, 0, 1, 0], 0, 32, 32),
])
def test_block_plan_bit_exact(lengths, bits, sink, window, block):
    cu = synth.cu_seqlens_of(lengths)
    route = np.array(bits, np.uint8)[:, None]
    mq = -(-max(lengths) // block) + 3
    plan = torch.full((len(lengths), mq, 4), -7, dtype=torch.int32, device=DEV)
    _lib.fa_block_plan(i32(cu), mq, u8(route), 0, sink, window, block, plan)
    torch.cuda.synchronize()
    want = oracle.block_plan(lengths, mq, route, 0, sink, window, block)
    assert np.array_equal(plan.cpu().numpy(), want)


# ---------------------------------------------------------------------------
# Prefill
# ---------------------------------------------------------------------------

def run_prefill(q, k, v, cu, route, layer, sink, window, block, scale):
    total, hq, d = q.shape
    qd, kd, vd = dev_from(q), dev_from(k), dev_from(v)
    o = torch.empty_like(qd)
    lse = torch.empty((total, hq), dtype=torch.float32, device=DEV)
    lengths = np.diff(cu)
    _lib.fa_attn_prefill(qd, kd, vd, o, i32(cu), int(lengths.max()), u8(route), layer, sink,
                         window, block, scale, lse=lse)
    torch.cuda.synchronize()
    return host_of(o), lse.cpu().numpy()


def test_prefill_tiny_fp32_both_layers():
    """Tiny case (fp32, d 64, 4/2 heads, T 256): layer 0 FA, layer 1 SA (sink 16,
    window 64, block 16); every row against the oracle at 1e-4."""
    c = synth.tiny_case(0)
    route = np.array([[1, 0]], np.uint8)
    for layer, (q, k, v) in enumerate(c["layers"]):
        o, lse = run_prefill(q, k, v, c["cu_seqlens"], route, layer, 16, 64, 16, 1 / 8.0)
        o_ref, l_ref = oracle.attn_prefill(q, k, v, c["cu_seqlens"], route, layer, 16, 64, 16,
                                           1 / 8.0)
        assert max_err(o, o_ref) <= TOL_F32
        assert np.abs(lse - l_ref).max() <= TOL_F32


PREFILL_CASES = [
    # lengths, hq, hkv, d, bits, sink, window, block
    ([700], 8, 2, 128, [1], 128, 256, 64),
    ([700], 8, 2, 128, [0], 128, 256, 64),
    ([1000, 333, 64, 1], 8, 2, 128, [0, 1, 0, 1], 64, 128, 32),
    ([517], 4, 4, 128, [0], 32, 64, 16),            # G = 1
    ([517], 4, 2, 128, [1], 0, 128, 128),           # G = 2, no sink
    ([390], 16, 2, 128, [0], 128, 128, 64),         # G = 8
    ([450, 129], 8, 2, 64, [1, 0], 64, 192, 64),    # d = 64
    ([300], 6, 2, 128, [0], 32, 64, 32),            # G = 3: plain kernel
    ([260, 77], 32, 2, 128, [0, 1], 64, 128, 64),   # G = 16: four head groups per KV head
]


@pytest.mark.parametrize("case", PREFILL_CASES)
def test_prefill_bf16_matches_oracle(case):
    lengths, hq, hkv, d, bits, sink, window, block = case
    rng = np.random.default_rng(sum(lengths) + hq + d)
    cu = synth.cu_seqlens_of(lengths)
    q, k, v = synth.qkv_host(rng, int(cu[-1]), hq, hkv, d, bf16=True)
    route = np.array(bits, np.uint8)[:, None]
    scale = 1 / math.sqrt(d)
    o, lse = run_prefill(q, k, v, cu, route, 0, sink, window, block, scale)
    o_ref, l_ref = oracle.attn_prefill(q, k, v, cu, route, 0, sink, window, block, scale)
    assert max_err(o, o_ref) <= TOL_BF16
    assert np.abs(lse - l_ref).max() <= TOL_LSE


def test_prefill_fp32_matches_oracle_varlen():
    rng = np.random.default_rng(5)
    lengths = [300, 77]
    cu = synth.cu_seqlens_of(lengths)
    q, k, v = synth.qkv_host(rng, int(cu[-1]), 8, 2, 128, bf16=False)
    route = np.array([[0], [1]], np.uint8)
    o, lse = run_prefill(q, k, v, cu, route, 0, 32, 64, 16, 0.09)
    o_ref, l_ref = oracle.attn_prefill(q, k, v, cu, route, 0, 32, 64, 16, 0.09)
    assert max_err(o, o_ref) <= TOL_F32
    assert np.abs(lse - l_ref).max() <= TOL_F32


def test_prefill_deterministic_and_sa_full_window_equals_fa():
    rng = np.random.default_rng(9)
    T = 640
    cu = synth.cu_seqlens_of([T])
    q, k, v = synth.qkv_host(rng, T, 8, 2, 128, bf16=True)
    a, la = run_prefill(q, k, v, cu, np.ones((1, 1), np.uint8), 0, 64, 64, 64, 0.088)
    b, lb = run_prefill(q, k, v, cu, np.ones((1, 1), np.uint8), 0, 64, 64, 64, 0.088)
    assert np.array_equal(a, b) and np.array_equal(la, lb)
    c, lc = run_prefill(q, k, v, cu, np.zeros((1, 1), np.uint8), 0, 64, 640, 64, 0.088)
    assert np.array_equal(a, c) and np.array_equal(la, lc)


@pytest.mark.parametrize("bit", [1, 0])
def test_prefill_bf16_rescale_path_growing_scores(bit):
    """Key norms that grow 300x along the sequence make each row's scores climb
    by many octaves from tile to tile, so the softmax reference max has to move
    on many tiles (the rescale path, not only the first visible tile)."""
    rng = np.random.default_rng(31)
    T, hq, hkv, d = 1500, 8, 2, 128
    cu = synth.cu_seqlens_of([T])
    qf = rng.standard_normal((T, hq, d)).astype(np.float32)
    kf = rng.standard_normal((T, hkv, d)).astype(np.float32)
    kf *= (0.05 + np.arange(T, dtype=np.float32) / 100.0)[:, None, None]
    vf = rng.standard_normal((T, hkv, d)).astype(np.float32)
    q, k, v = (synth.f32_to_bf16_bits(a) for a in (qf, kf, vf))
    route = np.full((1, 1), bit, np.uint8)
    scale = 1 / math.sqrt(d)
    o, lse = run_prefill(q, k, v, cu, route, 0, 64, 256, 64, scale)
    o_ref, l_ref = oracle.attn_prefill(q, k, v, cu, route, 0, 64, 256, 64, scale)
    assert np.abs(l_ref).max() > 20.0  # the scores really are large
    assert max_err(o, o_ref) <= TOL_BF16
    assert np.abs(lse - l_ref).max() <= TOL_LSE


def test_empty_sequence_in_varlen_batch():
    """A zero-length sequence inside a varlen batch.  The router gives it route 0
    and NaN logits (the documented device behaviour), its block-plan rows are
    all (0, 0, 0, 0), prefill writes nothing for it, and every other sequence
    matches the oracle run on the batch without it (the packed rows are the
    same): route bits bit-exact, attention within the bf16 bar."""
    rng = np.random.default_rng(44)
    lengths, kept = [300, 0, 129], [300, 129]
    cu, cu_kept = synth.cu_seqlens_of(lengths), synth.cu_seqlens_of(kept)
    hidden, L = 256, 3
    x = rng.standard_normal((int(cu[-1]), hidden)).astype(np.float32)
    w1, b1, w2, b2 = synth.router_weights(rng, hidden, 16, L)
    route, logits = run_router(x, cu, 64, w1, b1, w2, b2)
    assert route[1].tolist() == [0] * L and np.isnan(logits[1]).all()
    r_ref, _, l64 = oracle.router(x, cu_kept, 64, w1, b1, w2, b2)
    assert np.abs(l64).min() > 1e-4
    assert np.array_equal(route[[0, 2]], r_ref)

    mq = 8
    plan = torch.full((3, mq, 4), -7, dtype=torch.int32, device=DEV)
    route_bits = np.array([[0], [1], [0]], np.uint8)
    _lib.fa_block_plan(i32(cu), mq, u8(route_bits), 0, 64, 128, 64, plan)
    torch.cuda.synchronize()
    plan = plan.cpu().numpy()
    assert not plan[1].any()
    assert np.array_equal(plan, oracle.block_plan(lengths, mq, route_bits, 0, 64, 128, 64))

    q, k, v = synth.qkv_host(rng, int(cu[-1]), 8, 2, 128, bf16=True)
    scale = 1 / math.sqrt(128)
    o, lse = run_prefill(q, k, v, cu, route_bits, 0, 64, 128, 64, scale)
    o_ref, l_ref = oracle.attn_prefill(q, k, v, cu_kept, route_bits[[0, 2]], 0, 64, 128, 64,
                                       scale)
    assert max_err(o, o_ref) <= TOL_BF16
    assert np.abs(lse - l_ref).max() <= TOL_LSE


# ---------------------------------------------------------------------------
# Decode
# ---------------------------------------------------------------------------

def run_decode(q, kc, vc, cache_len, route, layer, sink, window, block, scale, k_new=None,
               v_new=None, route_host=None):
    qd, kcd, vcd = dev_from(q), dev_from(kc), dev_from(vc)
    o = torch.empty_like(qd)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=DEV)
    kn = None if k_new is None else dev_from(k_new)
    vn = None if v_new is None else dev_from(v_new)
    _lib.fa_attn_decode(qd, o, kcd, vcd, i32(cache_len), u8(route), layer, sink, window, block,
                        scale, k_new=kn, v_new=vn, lse=lse, route_host=route_host)
    torch.cuda.synchronize()
    return host_of(o), lse.cpu().numpy(), host_of(kcd), host_of(vcd)


DECODE_CASES = [
    # B, hq, hkv, d, max_cache, lengths, bits, sink, window, block, bf16
    (3, 8, 2, 128, 1000, [1000, 513, 1], [1, 0, 0], 128, 256, 64, True),
    (2, 32, 8, 128, 5000, [5000, 4097], [0, 1], 128, 2048, 64, True),
    (2, 4, 4, 64, 700, [650, 700], [0, 1], 32, 64, 16, True),
    (2, 16, 2, 128, 900, [900, 31], [1, 0], 0, 128, 128, True),
    (2, 8, 2, 128, 600, [600, 250], [0, 1], 64, 128, 32, False),
    (1, 4, 2, 64, 256, [256], [0], 16, 64, 16, False),
    (2, 32, 2, 128, 1500, [1500, 700], [1, 0], 128, 512, 64, True),   # G = 16
    (2, 8, 4, 64, 900, [900, 450], [0, 1], 64, 256, 32, True),        # G = 2, d = 64
]


@pytest.mark.parametrize("case", DECODE_CASES)
@pytest.mark.parametrize("append", [False, True])
def test_decode_matches_oracle(case, append):
    B, hq, hkv, d, max_cache, lengths, bits, sink, window, block, bf16 = case
    rng = np.random.default_rng(max_cache + hq + int(append))
    kc, vc = synth.kv_cache_host(rng, B, hkv, max_cache, d, bf16=bf16)
    q = synth.normal(rng, (B, hq, d))
    q = synth.f32_to_bf16_bits(q) if bf16 else q
    route = np.array(bits, np.uint8)[:, None]
    scale = 1 / math.sqrt(d)
    k_new = v_new = None
    kc_ref, vc_ref = kc, vc
    if append:
        kn, vn = synth.kv_cache_host(rng, B, hkv, 1, d, bf16=bf16)
        k_new, v_new = kn[:, :, 0].copy(), vn[:, :, 0].copy()
        kc_ref, vc_ref = kc.copy(), vc.copy()
        for b, n in enumerate(lengths):
            kc_ref[b, :, n - 1] = k_new[b]
            vc_ref[b, :, n - 1] = v_new[b]
    o, lse, kc_after, vc_after = run_decode(q, kc, vc, lengths, route, 0, sink, window, block,
                                            scale, k_new, v_new)
    o_ref, l_ref = oracle.attn_decode(q, kc_ref, vc_ref, lengths, route, 0, sink, window, block,
                                      scale)
    assert max_err(o, o_ref) <= (TOL_BF16 if bf16 else TOL_F32)
    assert np.abs(lse - l_ref).max() <= (TOL_LSE if bf16 else TOL_F32)
    # the append writes exactly the new token into the cache, nothing else moves
    assert np.array_equal(kc_after, kc_ref) and np.array_equal(vc_after, vc_ref)


def test_decode_route_host_sizing_gives_same_result():
    """A host mirror of an all-SA mask shrinks the grid; the result must not change."""
    rng = np.random.default_rng(33)
    B, hq, hkv, d, max_cache = 2, 8, 2, 128, 8192
    kc, vc = synth.kv_cache_host(rng, B, hkv, max_cache, d)
    q = synth.f32_to_bf16_bits(synth.normal(rng, (B, hq, d)))
    route = np.zeros((B, 1), np.uint8)
    a = run_decode(q, kc, vc, [8192, 5000], route, 0, 128, 1024, 64, 0.088)
    b = run_decode(q, kc, vc, [8192, 5000], route, 0, 128, 1024, 64, 0.088, route_host=route)
    o_ref, _ = oracle.attn_decode(q, kc, vc, [8192, 5000], route, 0, 128, 1024, 64, 0.088)
    assert max_err(a[0], o_ref) <= TOL_BF16 and max_err(b[0], o_ref) <= TOL_BF16


def test_decode_equals_last_prefill_row_on_gpu():
    rng = np.random.default_rng(44)
    T, hq, hkv, d = 777, 8, 2, 128
    cu = synth.cu_seqlens_of([T])
    q, k, v = synth.qkv_host(rng, T, hq, hkv, d, bf16=True)
    for bit in (0, 1):
        route = np.array([[bit]], np.uint8)
        o_p, l_p = run_prefill(q, k, v, cu, route, 0, 64, 256, 64, 0.088)
        kc = k.transpose(1, 0, 2)[None].copy()
        vc = v.transpose(1, 0, 2)[None].copy()
        o_d, l_d, _, _ = run_decode(q[T - 1][None].copy(), kc, vc, [T], route, 0, 64, 256, 64,
                                    0.088)
        assert np.abs(as_f32(o_d[0]) - as_f32(o_p[T - 1])).max() <= TOL_BF16
        assert np.abs(l_d[0] - l_p[T - 1]).max() <= TOL_LSE


def test_decode_bad_cache_len_gives_nan_and_deterministic():
    rng = np.random.default_rng(45)
    B, hq, hkv, d, max_cache = 3, 8, 2, 128, 512
    kc, vc = synth.kv_cache_host(rng, B, hkv, max_cache, d)
    q = synth.f32_to_bf16_bits(synth.normal(rng, (B, hq, d)))
    route = np.ones((B, 1), np.uint8)
    o, lse, kc_after, _ = run_decode(q, kc, vc, [512, 0, 600], route, 0, 64, 128, 64, 0.088)
    of = as_f32(o)
    assert np.isfinite(of[0]).all()
    assert np.isnan(of[1]).all() and np.isnan(of[2]).all()
    assert np.isnan(lse[1]).all() and np.isnan(lse[2]).all()
    assert np.array_equal(kc_after, kc)
    o2, lse2, _, _ = run_decode(q, kc, vc, [512, 0, 600], route, 0, 64, 128, 64, 0.088)
    assert np.array_equal(o2, o) and np.array_equal(lse2[0], lse[0])


# ---------------------------------------------------------------------------
# Full-size workloads, sampled
# ---------------------------------------------------------------------------

def sample_rows(T, block, sink, window, n_random, seed):
    rows = set(range(64)) | set(range(T - 64, T))
    for edge in (sink, window, sink + window):
        for e in (edge - 1, edge, edge + 1):
            if 0 <= e < T:
                rows.add(e)
    rng = np.random.default_rng(seed)
    rows |= set(rng.integers(0, T, n_random).tolist())
    return np.array(sorted(rows), np.int32)


@pytest.mark.parametrize("bit", [1, 0])
def test_prefill_llama_32k_sampled_rows(bit):
    """Llama-3.1-8B attention shape, 32768 tokens, bf16, in the benchmark's launch
    configuration; sampled rows of every head against the oracle."""
    T, hq, hkv, d = 32768, 32, 8, 128
    q = synth.device_normal((T, hq, d), seed=1)
    k = synth.device_normal((T, hkv, d), seed=2)
    v = synth.device_normal((T, hkv, d), seed=3)
    o = torch.empty_like(q)
    lse = torch.empty((T, hq), dtype=torch.float32, device=DEV)
    cu = i32([0, T])
    route = u8([[bit]])
    scale = 1 / math.sqrt(d)
    _lib.fa_attn_prefill(q, k, v, o, cu, T, route, 0, 128, 2048, 64, scale, lse=lse)
    torch.cuda.synchronize()
    rows = sample_rows(T, 64, 128, 2048, 24 if bit else 200, seed=bit)
    if bit:  # the FA oracle costs O(T) per row: keep the sample small
        rows = np.concatenate([rows[:8], rows[-40:], rows[64:80]])
    qh, kh, vh = host_of(q), host_of(k), host_of(v)
    o_ref, l_ref = oracle.attn_prefill(qh, kh, vh, [0, T], np.array([[bit]], np.uint8), 0, 128,
                                       2048, 64, scale, rows=rows)
    oh = host_of(o)[rows]
    assert max_err(oh, o_ref) <= TOL_BF16
    assert np.abs(lse.cpu().numpy()[rows] - l_ref).max() <= TOL_LSE


def test_decode_llama_131k_sampled_heads():
    """Decode step, batch 8, 131072-token bf16 cache, Llama shape; one FA and one SA
    layer (sink 128, window 2048, block 64); KV heads 0 and 7 of every sequence."""
    B, hq, hkv, d, n = 8, 32, 8, 128, 131072
    G = hq // hkv
    kc = torch.empty((B, hkv, n, d), dtype=torch.bfloat16, device=DEV)
    vc = torch.empty_like(kc)
    for b in range(B):
        kc[b] = synth.device_normal((hkv, n, d), seed=100 + b)
        vc[b] = synth.device_normal((hkv, n, d), seed=200 + b)
    q = synth.device_normal((B, hq, d), seed=300)
    cl = i32([n] * B)
    route = u8([[1, 0]] * B)
    scale = 1 / math.sqrt(d)
    for layer in (0, 1):
        o = torch.empty_like(q)
        lse = torch.empty((B, hq), dtype=torch.float32, device=DEV)
        _lib.fa_attn_decode(q, o, kc, vc, cl, route, layer, 128, 2048, 64, scale, lse=lse,
                            route_host=np.array([[1, 0]] * B, np.uint8))
        torch.cuda.synchronize()
        for g in (0, hkv - 1):
            qs = host_of(q[:, g * G:(g + 1) * G].contiguous())
            ks = host_of(kc[:, g:g + 1].contiguous())
            vs = host_of(vc[:, g:g + 1].contiguous())
            o_ref, l_ref = oracle.attn_decode(qs, ks, vs, [n] * B,
                                              np.array([[1, 0]] * B, np.uint8), layer, 128, 2048,
                                              64, scale)
            og = host_of(o[:, g * G:(g + 1) * G].contiguous())
            assert max_err(og, o_ref) <= TOL_BF16
            assert np.abs(lse[:, g * G:(g + 1) * G].cpu().numpy() - l_ref).max() <= TOL_LSE


@pytest.mark.parametrize("bf16", [True, False])
def test_decode_long_cache_many_splits(bf16):
    """Caches of 600000 and 300001 tokens: the splits cap at 4096 tokens, so a
    sequence has 147 of them (more than 64, the merge walks several chunks of
    partials); FA and SA layers against the oracle on the whole row."""
    B, hq, hkv, d, n = 2, 8, 2, 128, 600000
    lengths = [n, 300001]
    dt = "bf16" if bf16 else "f32"
    kc = synth.device_normal((B, hkv, n, d), 41, dt)
    vc = synth.device_normal((B, hkv, n, d), 42, dt)
    q = synth.device_normal((B, hq, d), 43, dt)
    cl = i32(lengths)
    scale = 1 / math.sqrt(d)
    bits = np.array([[1, 0], [1, 0]], np.uint8)
    kh, vh, qh = host_of(kc), host_of(vc), host_of(q)
    for layer in (0, 1):
        o = torch.empty_like(q)
        lse = torch.empty((B, hq), dtype=torch.float32, device=DEV)
        _lib.fa_attn_decode(q, o, kc, vc, cl, u8(bits), layer, 128, 2048, 64, scale, lse=lse,
                            route_host=bits)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.attn_decode(qh, kh, vh, lengths, bits, layer, 128, 2048, 64, scale)
        assert max_err(host_of(o), o_ref) <= (TOL_BF16 if bf16 else TOL_F32), layer
        assert np.abs(lse.cpu().numpy() - l_ref).max() <= (TOL_LSE if bf16 else TOL_F32), layer


@pytest.mark.parametrize("bf16", [True, False])
def test_route_host_kernels_match_device_route(bf16):
    """A host copy of the mask selects kernels compiled for all-FA / all-SA layers;
    their outputs must equal the device-route kernel bit for bit."""
    rng = np.random.default_rng(77)
    lengths = [400, 190]
    cu = synth.cu_seqlens_of(lengths)
    q, k, v = synth.qkv_host(rng, int(cu[-1]), 8, 2, 128, bf16=bf16)
    qd, kd, vd, cud = dev_from(q), dev_from(k), dev_from(v), i32(cu)
    for bit in (0, 1):
        route = np.full((2, 1), bit, np.uint8)
        outs = []
        for rh in (None, route):
            o = torch.empty_like(qd)
            _lib.fa_attn_prefill(qd, kd, vd, o, cud, 400, u8(route), 0, 64, 128, 32, 0.09,
                                 route_host=rh)
            torch.cuda.synchronize()
            outs.append(host_of(o))
        assert np.array_equal(outs[0], outs[1])
    rng = np.random.default_rng(78)
    kc, vc = synth.kv_cache_host(rng, 2, 2, 3000, 128, bf16=bf16)
    qq = synth.normal(rng, (2, 8, 128))
    qq = synth.f32_to_bf16_bits(qq) if bf16 else qq
    for bit in (0, 1):
        route = np.full((2, 1), bit, np.uint8)
        a = run_decode(qq, kc, vc, [3000, 2500], route, 0, 64, 256, 32, 0.09)
        b = run_decode(qq, kc, vc, [3000, 2500], route, 0, 64, 256, 32, 0.09, route_host=route)
        o_ref, _ = oracle.attn_decode(qq, kc, vc, [3000, 2500], route, 0, 64, 256, 32, 0.09)
        tol = TOL_BF16 if bf16 else TOL_F32
        assert max_err(a[0], o_ref) <= tol and max_err(b[0], o_ref) <= tol
        if bit:  # same grid, same kernel body: identical bits
            assert np.array_equal(a[0], b[0])
