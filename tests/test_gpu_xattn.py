"""GPU parity of the XAttention branch (fa_xattn_scores, fa_xattn_select,
fa_attn_prefill_xattn) against oracle/xattn.py.

Bars: block scores within 1e-4 absolute of the float64 oracle (each score sums
at most 256 softmax values that carry ~1e-6 relative error from fp32 products
and exp2; scores lie in [0, 16]); the kept-block masks bit-exact against the
oracle's selection run on the GPU's own fp32 scores (where floating point
decides an integer both sides decide on the same fp32 values, in the same
order); attention within 2e-2 (bf16 inputs) and lse within 1e-3.
"""
import math

import numpy as np
import pytest
import torch

from oracle import xattn
from sparse_attention_layerrouter_amd import _lib, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def dev_from(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def unpack(mask_words, nqb):
    """[B, H, NQB, NW] int32 words -> bool [B, H, NQB, NQB] (bit j of row i)."""
    w = mask_words.astype(np.uint32)
    bits = (w[..., :, None] >> np.arange(32, dtype=np.uint32)) & 1
    return bits.reshape(*w.shape[:-1], -1)[..., :nqb].astype(bool)


def run_scores(q, k, cu, block, stride, scale, nqb):
    B, hq = len(cu) - 1, q.shape[1]
    sc = torch.full((B, hq, nqb, nqb), -1.0, dtype=torch.float32, device=DEV)
    _lib.fa_xattn_scores(dev_from(q), dev_from(k), torch.tensor(cu, device=DEV),
                         int(np.diff(cu).max()), block, stride, scale, sc)
    torch.cuda.synchronize()
    return sc


CASES = [
    # lengths, hq, hkv, d, stride
    ([1000, 333, 64, 1], 8, 2, 128, 8),
    ([700, 129], 8, 2, 128, 4),
    ([517], 4, 4, 128, 8),          # G = 1
    ([390, 200], 16, 2, 64, 8),     # G = 8, d = 64
    ([300], 4, 2, 64, 4),
    ([600, 77], 4, 2, 128, 8),      # G = 2 at block 128: two heads per workgroup
    ([260, 130], 16, 1, 128, 8),    # G = 16: eight head groups of two
]


@pytest.mark.parametrize("case", CASES)
def test_scores_and_selection_match_oracle(case):
    lengths, hq, hkv, d, stride = case
    block = 16 * stride
    rng = np.random.default_rng(sum(lengths) + d + stride)
    cu = synth.cu_seqlens_of(lengths)
    q, k, _ = synth.qkv_host(rng, int(cu[-1]), hq, hkv, d, bf16=True)
    scale = 1 / math.sqrt(d)
    nqb = -(-max(lengths) // block)
    sc = run_scores(q, k, cu, block, stride, scale, nqb)
    got = sc.cpu().numpy()
    ref = xattn.block_scores(q, k, cu, block, stride, scale)
    for b, T in enumerate(lengths):
        nb = -(-T // block)
        tri = np.tril(np.ones((nb, nb), bool))
        assert np.abs(got[b][:, :nb, :nb][:, tri] - ref[b][:, :nb, :nb][:, tri]).max() <= 1e-4
    # selection, bit-exact on the GPU's scores, at a few thresholds
    for tau in (0.5, 0.9, 0.99):
        nw = -(-nqb // 32)
        m = torch.full((len(lengths), hq, nqb, nw), -1, dtype=torch.int32, device=DEV)
        _lib.fa_xattn_select(sc, torch.tensor(cu, device=DEV), block, tau, m)
        torch.cuda.synchronize()
        keep = unpack(m.cpu().numpy(), nqb)
        want = xattn.select_blocks(np.where(got < 0, 0, got).astype(np.float32), lengths, block,
                                   tau)
        assert np.array_equal(keep, want), tau


@pytest.mark.parametrize("case", [
    ([1000, 333, 64, 1], 8, 2, 128, 8),
    ([700, 129], 8, 2, 128, 4),
    ([390, 200], 16, 2, 64, 8),
    ([300], 4, 4, 64, 4),           # G = 1
])
def test_fp32_scores_and_selection_match_oracle(case):
    """fp32 inputs take the VALU score kernel: scores within 1e-4 of the oracle,
    selection bit-exact on them, the same partial sums and finishing kernel as bf16."""
    lengths, hq, hkv, d, stride = case
    block = 16 * stride
    rng = np.random.default_rng(sum(lengths) + 3 * d + stride)
    cu = synth.cu_seqlens_of(lengths)
    q, k, _ = synth.qkv_host(rng, int(cu[-1]), hq, hkv, d, bf16=False)
    scale = 1 / math.sqrt(d)
    nqb = -(-max(lengths) // block)
    got = run_scores(q, k, cu, block, stride, scale, nqb).cpu().numpy()
    ref = xattn.block_scores(q, k, cu, block, stride, scale)
    for b, T in enumerate(lengths):
        nb = -(-T // block)
        tri = np.tril(np.ones((nb, nb), bool))
        assert np.abs(got[b][:, :nb, :nb][:, tri] - ref[b][:, :nb, :nb][:, tri]).max() <= 1e-4
    nw = -(-nqb // 32)
    m = torch.full((len(lengths), hq, nqb, nw), -1, dtype=torch.int32, device=DEV)
    sc = torch.from_numpy(np.where(got < 0, 0, got).astype(np.float32)).to(DEV)
    _lib.fa_xattn_select(sc, torch.tensor(cu, device=DEV), block, 0.9, m)
    torch.cuda.synchronize()
    want = xattn.select_blocks(np.where(got < 0, 0, got).astype(np.float32), lengths, block, 0.9)
    assert np.array_equal(unpack(m.cpu().numpy(), nqb), want)


def test_padded_block_layout():
    """n_qblocks above what the longest sequence needs (35 for 8 blocks, so the
    mask rows take two words): the padding cells are never written, the selection
    leaves their mask rows zero, and the masked prefill over the padded mask
    equals the one over the tight layout bit for bit."""
    rng = np.random.default_rng(35)
    lengths, hq, hkv, d, block = [1000, 300], 8, 2, 128, 128
    cu = synth.cu_seqlens_of(lengths)
    q, k, v = synth.qkv_host(rng, int(cu[-1]), hq, hkv, d, bf16=True)
    scale = 1 / math.sqrt(d)
    tight = -(-max(lengths) // block)
    nqb = 35
    sc_t = run_scores(q, k, cu, block, 8, scale, tight).cpu().numpy()
    sc_p = run_scores(q, k, cu, block, 8, scale, nqb)
    got = sc_p.cpu().numpy()
    for b, T in enumerate(lengths):
        nb = -(-T // block)
        tri = np.tril(np.ones((nb, nb), bool))
        assert np.array_equal(got[b][:, :nb, :nb][:, tri], sc_t[b][:, :nb, :nb][:, tri])
        assert (got[b][:, nb:] == -1.0).all()   # rows past the sequence: untouched
        assert (got[b][:, :nb, nb:] == -1.0).all()
    masks = {}
    for n in (tight, nqb):
        nw = -(-n // 32)
        m = torch.full((len(lengths), hq, n, nw), -1, dtype=torch.int32, device=DEV)
        src = sc_p if n == nqb else torch.from_numpy(sc_t).to(DEV)
        _lib.fa_xattn_select(src, torch.tensor(cu, device=DEV), block, 0.9, m)
        torch.cuda.synchronize()
        masks[n] = m.cpu().numpy()
    keep_t, keep_p = unpack(masks[tight], tight), unpack(masks[nqb], nqb)
    for b, T in enumerate(lengths):
        nb = -(-T // block)
        assert np.array_equal(keep_p[b][:, :nb, :nb], keep_t[b][:, :nb, :nb])
        assert not keep_p[b][:, nb:].any() and not keep_p[b][:, :, nb:].any()
    o_t, l_t = run_xattn_prefill(q, k, v, cu, block, masks[tight], scale)
    o_p, l_p = run_xattn_prefill(q, k, v, cu, block, masks[nqb], scale)
    assert np.array_equal(o_t, o_p) and np.array_equal(l_t, l_p)


def test_scores_are_deterministic():
    rng = np.random.default_rng(8)
    cu = synth.cu_seqlens_of([2048])
    q, k, _ = synth.qkv_host(rng, 2048, 32, 8, 128, bf16=True)
    a = run_scores(q, k, cu, 128, 8, 0.088, 16)
    b = run_scores(q, k, cu, 128, 8, 0.088, 16)
    assert torch.equal(a, b)


def pack(keep):
    """bool [B, H, NQB, NQB] -> int32 words [B, H, NQB, ceil(NQB/32)]."""
    B, H, n, _ = keep.shape
    nw = -(-n // 32)
    pad = np.zeros((B, H, n, nw * 32), bool)
    pad[..., :n] = keep
    w = (pad.reshape(B, H, n, nw, 32).astype(np.uint64) << np.arange(32, dtype=np.uint64)).sum(-1)
    return w.astype(np.uint32).view(np.int32)


def run_xattn_prefill(q, k, v, cu, block, keep_words, scale):
    qd = dev_from(q)
    o = torch.empty_like(qd)
    lse = torch.empty((q.shape[0], q.shape[1]), dtype=torch.float32, device=DEV)
    _lib.fa_attn_prefill_xattn(qd, dev_from(k), dev_from(v), o, torch.tensor(cu, device=DEV),
                               int(np.diff(cu).max()), block, torch.tensor(keep_words, device=DEV),
                               scale, lse=lse)
    torch.cuda.synchronize()
    t = o.contiguous()
    host = t.view(torch.int16).cpu().numpy().view(np.uint16) if t.dtype == torch.bfloat16 \
        else t.cpu().numpy()
    return host, lse.cpu().numpy()


def as_f64(a):
    return (synth.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)


XA_CASES = [
    # lengths, hq, hkv, d, block, bf16, mask kind
    ([1000, 333, 64, 1], 8, 2, 128, 128, True, "selected"),
    ([700, 130], 8, 2, 128, 64, True, "random"),
    ([517], 4, 4, 128, 128, True, "random"),        # G = 1: plain kernel
    ([390, 200], 16, 2, 64, 128, True, "random"),   # G = 8, d = 64
    ([300, 90], 8, 2, 128, 64, False, "random"),    # fp32: plain kernel
    ([600], 4, 2, 128, 128, True, "random"),        # G = 2, block 128: MFMA kernel
    ([260, 130], 16, 1, 128, 128, True, "random"),  # G = 16: eight head groups of two
]


@pytest.mark.parametrize("case", XA_CASES)
def test_xattn_prefill_matches_oracle(case):
    lengths, hq, hkv, d, block, bf16, kind = case
    rng = np.random.default_rng(sum(lengths) + hq + block)
    cu = synth.cu_seqlens_of(lengths)
    q, k, v = synth.qkv_host(rng, int(cu[-1]), hq, hkv, d, bf16=bf16)
    scale = 1 / math.sqrt(d)
    nqb = -(-max(lengths) // block)
    if kind == "selected":
        sc = run_scores(q, k, cu, block, block // 16, scale, nqb)
        nw = -(-nqb // 32)
        m = torch.zeros((len(lengths), hq, nqb, nw), dtype=torch.int32, device=DEV)
        _lib.fa_xattn_select(sc, torch.tensor(cu, device=DEV), block, 0.9, m)
        torch.cuda.synchronize()
        words = m.cpu().numpy()
        keep = unpack(words, nqb)
    else:
        keep = rng.random((len(lengths), hq, nqb, nqb)) < 0.45
        idx = np.arange(nqb)
        keep[..., idx, idx] = True                   # every row keeps its own block
        keep &= np.tril(np.ones((nqb, nqb), bool))   # causal blocks only
        words = pack(keep)
    o, lse = run_xattn_prefill(q, k, v, cu, block, words, scale)
    o_ref, l_ref = xattn.attn_prefill(q, k, v, cu, keep, block, scale)
    tol, tol_lse = (2e-2, 1e-3) if bf16 else (1e-4, 1e-4)
    assert np.abs(as_f64(o) - o_ref).max() <= tol
    assert np.abs(lse - l_ref).max() <= tol_lse


@pytest.mark.parametrize("block", [64, 128])
def test_xattn_prefill_with_every_block_kept_is_the_fa_kernel(block):
    rng = np.random.default_rng(12)
    lengths, hq, hkv, d = [1000, 257], 8, 2, 128
    cu = synth.cu_seqlens_of(lengths)
    q, k, v = synth.qkv_host(rng, int(cu[-1]), hq, hkv, d, bf16=True)
    nqb = -(-max(lengths) // block)
    keep = np.broadcast_to(np.tril(np.ones((nqb, nqb), bool)), (2, hq, nqb, nqb)).copy()
    o, lse = run_xattn_prefill(q, k, v, cu, block, pack(keep), 0.09)
    qd, kd, vd = dev_from(q), dev_from(k), dev_from(v)
    o_fa = torch.empty_like(qd)
    l_fa = torch.empty((q.shape[0], hq), dtype=torch.float32, device=DEV)
    route = np.ones((2, 1), np.uint8)
    _lib.fa_attn_prefill(qd, kd, vd, o_fa, torch.tensor(cu, device=DEV), max(lengths),
                         torch.tensor(route, device=DEV), 0, 0, 64, 64, 0.09, lse=l_fa,
                         route_host=route)
    torch.cuda.synchronize()
    assert np.array_equal(o, o_fa.view(torch.int16).cpu().numpy().view(np.uint16))
    assert np.array_equal(lse, l_fa.cpu().numpy())


def _tied_scores(rng, shape):
    """fp32 score rows: half continuous, half from a few values (ties, zeros)."""
    x = rng.random(shape, dtype=np.float32)
    tied = rng.choice(np.array([0.0, 0.25, 1.0], np.float32), size=shape)
    return np.where(rng.random(shape) < 0.5, tied, x).astype(np.float32)


@pytest.mark.parametrize("tau", [0.3, 0.9, 0.999, 1.5])
def test_selection_alone_matches_oracle_on_tied_scores(tau):
    """fa_xattn_select on synthetic rows of up to 600 blocks (ragged sequences,
    one of a single token): every row's kept bits equal the oracle's x6
    decision on the same fp32 scores, ties broken by block index."""
    rng = np.random.default_rng(int(tau * 1000))
    block, nqb = 64, 600
    lengths = [nqb * block - 17, 37 * block, 1]
    nw = -(-nqb // 32)
    sc = _tied_scores(rng, (len(lengths), 1, nqb, nqb))
    m = torch.full((len(lengths), 1, nqb, nw), -1, dtype=torch.int32, device=DEV)
    _lib.fa_xattn_select(dev_from(sc), torch.tensor(synth.cu_seqlens_of(lengths), device=DEV),
                         block, tau, m)
    torch.cuda.synchronize()
    got = unpack(m.cpu().numpy(), nqb)
    want = xattn.select_blocks(sc, lengths, block, tau)
    assert np.array_equal(got, want)


def test_selection_at_the_4096_block_maximum():
    """Rows of a 4096-block sequence (the largest n_qblocks the ABI takes),
    sampled where the decision's 16-value loads end at or past the last entry."""
    rng = np.random.default_rng(4096)
    block, nqb, tau = 16, 4096, 0.9
    sc = _tied_scores(rng, (1, 1, nqb, nqb))
    m = torch.full((1, 1, nqb, nqb // 32), -1, dtype=torch.int32, device=DEV)
    _lib.fa_xattn_select(dev_from(sc), torch.tensor([0, nqb * block], device=DEV,
                                                    dtype=torch.int32), block, tau, m)
    torch.cuda.synchronize()
    got = unpack(m.cpu().numpy(), nqb)
    for i in [0, 1, 2, 15, 16, 17, 2047, 4079, 4080, 4081, 4094, 4095]:
        want = xattn.select_row(sc[0, 0, i], i, tau)
        assert np.array_equal(got[0, 0, i, : i + 1], want), i
        assert not got[0, 0, i, i + 1:].any(), i


def test_full_size_llama_128k_sampled():
    """A 131072-token Llama-shaped layer (32 q / 8 kv heads, d 128, bf16; block
    128, stride 8, threshold 0.9) on locality-structured inputs, launched as the
    benchmark launches it.  Every (head, query block) row of scores must sum to
    the block's 16 reshaped rows (each row's softmax sums to 1); sampled rows
    match the oracle's per-block scores; their selections are bit-exact against
    the oracle's on the GPU's scores; sampled output rows of the masked prefill
    match the oracle over the GPU's mask."""
    T, hq, hkv, d, block, stride, tau = 131072, 32, 8, 128, 128, 8, 0.9
    scale = 1 / math.sqrt(d)
    q, k, v = synth.device_positional_qkv(T, hq, hkv, d, seed=31, alpha=3.0)
    cu = torch.tensor([0, T], dtype=torch.int32, device=DEV)
    nqb = T // block
    nw = nqb // 32
    sc = torch.empty((1, hq, nqb, nqb), dtype=torch.float32, device=DEV)
    m = torch.empty((1, hq, nqb, nw), dtype=torch.int32, device=DEV)
    o = torch.empty_like(q)
    lse = torch.empty((T, hq), dtype=torch.float32, device=DEV)
    _lib.fa_xattn_scores(q, k, cu, T, block, stride, scale, sc)
    _lib.fa_xattn_select(sc, cu, block, tau, m)
    _lib.fa_attn_prefill_xattn(q, k, v, o, cu, T, block, m, scale, lse=lse)
    torch.cuda.synchronize()
    got = sc.cpu().numpy()[0]
    tri = np.tril(np.ones((nqb, nqb), bool))
    row_sums = np.where(tri, got, 0.0).sum(axis=-1, dtype=np.float64)
    assert np.abs(row_sums - 16.0).max() <= 2e-3
    qh = q.view(torch.int16).cpu().numpy().view(np.uint16)
    kh = k.view(torch.int16).cpu().numpy().view(np.uint16)
    vh = v.view(torch.int16).cpu().numpy().view(np.uint16)
    keep = unpack(m.cpu().numpy(), nqb)
    for h, i in [(0, 0), (0, 1), (5, 300), (13, 511), (31, 1023), (22, 1022)]:
        ref = xattn.block_score_row(qh[:, h], kh[:, h // (hq // hkv)], stride, scale, block, i)
        assert np.abs(got[h, i, : i + 1] - ref).max() <= 1e-4, (h, i)
        want = xattn.select_row(got[h, i], i, tau)
        assert np.array_equal(keep[0, h, i, : i + 1], want), (h, i)
        assert not keep[0, h, i, i + 1:].any(), (h, i)
    rows = [0, 127, 128, 65537, T - 1]
    o_ref, l_ref = xattn.attn_prefill(qh, kh, vh, [0, T], keep, block, scale, rows=rows)
    oh = synth.bf16_bits_to_f32(o.view(torch.int16).cpu().numpy().view(np.uint16)[rows])
    assert np.abs(oh.astype(np.float64) - o_ref).max() <= 2e-2
    assert np.abs(lse.cpu().numpy()[rows] - l_ref).max() <= 1e-3


def test_empty_sequence_in_the_batch():
    """A zero-length sequence gets no scores, an all-zero mask row set and no
    output rows; its neighbours match the oracle as if it were absent."""
    rng = np.random.default_rng(17)
    lengths, hq, hkv, d, block, stride = [300, 0, 200], 8, 2, 128, 128, 8
    cu = synth.cu_seqlens_of(lengths)
    q, k, v = synth.qkv_host(rng, int(cu[-1]), hq, hkv, d, bf16=True)
    scale = 1 / math.sqrt(d)
    nqb = -(-max(lengths) // block)
    sc = run_scores(q, k, cu, block, stride, scale, nqb)   # filled with -1 first
    got = sc.cpu().numpy()
    assert (got[1] == -1.0).all()                           # nothing written for it
    ref = xattn.block_scores(q, k, cu, block, stride, scale)
    for b in (0, 2):
        nb = -(-lengths[b] // block)
        tri = np.tril(np.ones((nb, nb), bool))
        assert np.abs(got[b][:, :nb, :nb][:, tri] - ref[b][:, :nb, :nb][:, tri]).max() <= 1e-4
    nw = -(-nqb // 32)
    m = torch.full((3, hq, nqb, nw), -1, dtype=torch.int32, device=DEV)
    _lib.fa_xattn_select(sc, torch.tensor(cu, device=DEV), block, 0.9, m)
    torch.cuda.synchronize()
    words = m.cpu().numpy()
    assert (words[1] == 0).all()
    keep = unpack(words, nqb)
    o, lse = run_xattn_prefill(q, k, v, cu, block, words, scale)
    o_ref, l_ref = xattn.attn_prefill(q, k, v, cu, keep, block, scale)
    assert np.abs(as_f64(o) - o_ref).max() <= 2e-2
    assert np.abs(lse - l_ref).max() <= 1e-3


@pytest.mark.parametrize("bf16", [True, False])
def test_tile_past_the_sequence_end_reads_nothing(bf16):
    """The masked prefill walks a kept 128-token block as two 64-key tiles; when
    a sequence ends in the first tile, the second starts past its end and must
    read nothing.  K and V sit at the start of NaN-filled buffers, so a read past
    the last sequence would turn the (zero-weighted) V rows into NaN outputs."""
    rng = np.random.default_rng(23)
    lengths, hq, hkv, d, block = [300, 40, 1], 8, 2, 128, 128
    cu = synth.cu_seqlens_of(lengths)
    total = int(cu[-1])
    q, k, v = synth.qkv_host(rng, total, hq, hkv, d, bf16=bf16)
    nqb = -(-max(lengths) // block)
    keep = rng.random((len(lengths), hq, nqb, nqb)) < 0.6
    idx = np.arange(nqb)
    keep[..., idx, idx] = True
    keep &= np.tril(np.ones((nqb, nqb), bool))
    qd = dev_from(q)
    kd0, vd0 = dev_from(k), dev_from(v)
    kbig = torch.full((total + 512, hkv, d), float("nan"), dtype=kd0.dtype, device=DEV)
    vbig = torch.full((total + 512, hkv, d), float("nan"), dtype=vd0.dtype, device=DEV)
    kbig[:total] = kd0
    vbig[:total] = vd0
    o = torch.empty_like(qd)
    lse = torch.empty((total, hq), dtype=torch.float32, device=DEV)
    _lib.fa_attn_prefill_xattn(qd, kbig[:total], vbig[:total], o, torch.tensor(cu, device=DEV),
                               max(lengths), block, torch.tensor(pack(keep), device=DEV), 0.09,
                               lse=lse)
    torch.cuda.synchronize()
    t = o.contiguous()
    oh = t.view(torch.int16).cpu().numpy().view(np.uint16) if bf16 else t.cpu().numpy()
    o_ref, l_ref = xattn.attn_prefill(q, k, v, cu, keep, block, 0.09)
    got = as_f64(oh)
    assert np.isfinite(got).all() and np.isfinite(lse.cpu().numpy()).all()
    assert np.abs(got - o_ref).max() <= (2e-2 if bf16 else 1e-4)


def test_sequence_longer_than_the_block_layout():
    """A sequence with more blocks than n_qblocks (1400 tokens = 11 blocks of 128 in a
    9-block layout, longer than the max_seqlen the call promises), beside a short one,
    with an odd n_qblocks: the first 9 query blocks of every head match the oracle,
    the cells of the layout past each row stay unwritten, the workspace tail past its
    stated size is untouched, and the selection keeps only blocks below n_qblocks."""
    rng = np.random.default_rng(1400)
    lengths, hq, hkv, d, stride, block, nqb = [1400, 300], 8, 2, 128, 8, 128, 9
    cu = synth.cu_seqlens_of(lengths)
    q, k, _ = synth.qkv_host(rng, int(cu[-1]), hq, hkv, d, bf16=True)
    scale = 1 / math.sqrt(d)
    sc = torch.full((2, hq, nqb, nqb), -1.0, dtype=torch.float32, device=DEV)
    need = _lib.fa_xattn_workspace_size(2, hq, nqb)
    ws = torch.full((need + 4096,), 0x5A, dtype=torch.uint8, device=DEV)
    _lib.fa_xattn_scores(dev_from(q), dev_from(k), torch.tensor(cu, device=DEV),
                         nqb * block - 100, block, stride, scale, sc, workspace=ws)
    torch.cuda.synchronize()
    assert (ws[need:].cpu().numpy() == 0x5A).all()
    got = sc.cpu().numpy()
    ref = xattn.block_scores(q, k, cu, block, stride, scale)
    for b, T in enumerate(lengths):
        nb = min(-(-T // block), nqb)
        tri = np.tril(np.ones((nb, nb), bool))
        assert np.abs(got[b][:, :nb, :nb][:, tri] - ref[b][:, :nb, :nb][:, tri]).max() <= 1e-4
        assert (got[b][:, :nb, :nb][:, ~tri] == -1.0).all()
        assert (got[b][:, nb:] == -1.0).all()
    nw = -(-nqb // 32)
    m = torch.full((2, hq, nqb, nw), -1, dtype=torch.int32, device=DEV)
    _lib.fa_xattn_select(sc, torch.tensor(cu, device=DEV), block, 0.9, m)
    torch.cuda.synchronize()
    keep = unpack(m.cpu().numpy(), nqb)
    want = xattn.select_blocks(np.where(got < 0, 0, got).astype(np.float32),
                               [min(T, nqb * block) for T in lengths], block, 0.9)
    assert np.array_equal(keep, want)
