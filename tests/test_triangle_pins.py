"""Pins of the Triangle Attention oracle (oracle/triangle.py), each against
something other than that oracle: a hand-derived block table, the C oracle's
streaming block plan and its FA / SA attention layers, and closed forms."""
import math
import os

import numpy as np
import pytest

import oracle
from oracle import triangle
from sparse_attention_layerrouter_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "triangle_keep_10blocks.txt")


def golden_table():
    rows = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        i, js = line.split(":")
        rows[int(i)] = [int(x) for x in js.split()]
    return rows


@pytest.mark.parametrize("T", [160, 150])
def test_keep_table_matches_hand_derived_golden(T):
    keep = triangle.triangle_keep(T, 16, 16, 48, 32)
    table = golden_table()
    assert keep.shape == (10, 10)
    for i in range(10):
        assert list(np.nonzero(keep[i])[0]) == table[i], i


@pytest.mark.parametrize("T,block,sink,window", [(1000, 16, 16, 64), (777, 32, 0, 96),
                                                 (4096, 64, 128, 2048), (65, 64, 64, 64)])
def test_no_tail_is_the_streaming_block_plan(T, block, sink, window):
    """last_q = 0: the kept blocks are exactly the C oracle's SA block plan."""
    keep = triangle.triangle_keep(T, block, sink, window, 0)
    nb = keep.shape[0]
    plan = oracle.block_plan([T], nb, np.zeros((1, 1), np.uint8), 0, sink, window, block)[0]
    for i in range(nb):
        want = set(range(plan[i, 0], plan[i, 1])) | set(range(plan[i, 2], plan[i, 3]))
        assert set(np.nonzero(keep[i])[0]) == want, i


@pytest.mark.parametrize("T,last_q", [(1000, 1008), (1000, 4096), (64, 64)])
def test_covering_tail_is_every_causal_block(T, last_q):
    keep = triangle.triangle_keep(T, 16, 16, 64, last_q)
    nb = keep.shape[0]
    assert np.array_equal(keep, np.tril(np.ones((nb, nb), bool)))


def test_kept_block_count_closed_form():
    """Per SA row min(i + 1, ns + nw) kept blocks (the C oracle's count), plus the
    nl dense rows with i + 1 each."""
    T, block, sink, window, last_q = 4096, 64, 128, 1024, 256
    nb, ns, nw, nl = 64, 2, 16, 4
    keep = triangle.triangle_keep(T, block, sink, window, last_q)
    want = sum(min(i + 1, ns + nw) for i in range(nb - nl)) + sum(i + 1 for i in range(nb - nl, nb))
    assert int(keep.sum()) == want


def test_attention_rows_are_sa_rows_then_fa_rows():
    """Rows before the dense tail equal the C oracle's SA layer, rows in it its
    FA layer; a FA-routed sequence is the FA layer everywhere."""
    rng = np.random.default_rng(3)
    lengths = [300, 197]
    cu = synth.cu_seqlens_of(lengths)
    hq, hkv, d = 4, 2, 64
    q, k, v = synth.qkv_host(rng, int(cu[-1]), hq, hkv, d, bf16=False)
    block, sink, window, last_q = 16, 32, 64, 48
    scale = 1 / math.sqrt(d)
    o, lse = triangle.attn_prefill(q, k, v, cu, [0, 1], block, sink, window, last_q, scale)
    route_sa = np.zeros((2, 1), np.uint8)
    route_fa = np.ones((2, 1), np.uint8)
    o_sa, l_sa = oracle.attn_prefill(q, k, v, cu, route_sa, 0, sink, window, block, scale)
    o_fa, l_fa = oracle.attn_prefill(q, k, v, cu, route_fa, 0, sink, window, block, scale)
    T0 = lengths[0]
    tail0 = (-(-T0 // block) - last_q // block) * block   # 304 - 48 = 256
    assert tail0 == 256
    np.testing.assert_allclose(o[:tail0], o_sa[:tail0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[:tail0], l_sa[:tail0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(o[tail0:T0], o_fa[tail0:T0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[tail0:T0], l_fa[tail0:T0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(o[T0:], o_fa[T0:], rtol=0, atol=1e-12)   # FA-routed sequence
    # and the tail differs from SA there (the pin has power)
    assert np.abs(o[tail0:T0] - o_sa[tail0:T0]).max() > 1e-3
