"""Pins of the XAttention oracle (oracle/xattn.py), each against something
other than the oracle itself: direct antidiagonal sums of the full score
matrix, the softmax row-sum identity, brute-force minimal selections, a
planted attention pattern, and the C oracle's FA / SA attention."""
import itertools
import math

import numpy as np
import pytest

import oracle
from oracle import xattn
from sparse_attention_layerrouter_amd import synth


def test_antidiagonal_scores_are_subblock_antidiagonal_means():
    rng = np.random.default_rng(1)
    T, S, d, scale = 37, 4, 8, 0.3
    q = rng.standard_normal((T, d))
    k = rng.standard_normal((T, d))
    A = xattn.reshaped_scores(q, k, S, scale)
    M = q @ k.T  # full score matrix, positions past T are absent (zero)
    Tr = -(-T // S)
    assert A.shape == (Tr, Tr)
    for a in range(Tr):
        for b in range(Tr):
            if b > a:
                assert A[a, b] == -np.inf
                continue
            # the antidiagonal of sub-block (a, b): row + column == a*S + b*S + S - 1
            want = 0.0
            for r in range(a * S, a * S + S):
                c = a * S + b * S + S - 1 - r
                if r < T and b * S <= c < b * S + S and c < T:
                    want += M[r, c]
            assert A[a, b] == pytest.approx(want * scale / S, abs=1e-12)


@pytest.mark.parametrize("T", [512, 450])
def test_block_scores_of_a_query_block_sum_to_its_reshaped_rows(T):
    rng = np.random.default_rng(2)
    B, S, hq, hkv, d = 64, 8, 4, 2, 16
    cu = [0, T]
    q = rng.standard_normal((T, hq, d)) / 2
    k = rng.standard_normal((T, hkv, d)) / 2
    sc = xattn.block_scores(q, k, cu, B, S, 1 / math.sqrt(d))
    Tr = -(-T // S)
    nb = -(-T // B)
    for i in range(nb):
        rows = min(Tr, (i + 1) * (B // S)) - i * (B // S)
        np.testing.assert_allclose(sc[0, :, i, : i + 1].sum(axis=1), rows, rtol=1e-12)
        assert not sc[0, :, i, i + 1:].any()


def test_selection_is_the_smallest_set_reaching_the_threshold():
    rng = np.random.default_rng(3)
    for trial in range(40):
        n = 7
        s = rng.random((1, 1, n, n)).astype(np.float32)
        tau = float(rng.uniform(0.3, 0.95))
        keep = xattn.select_blocks(s, [n * 64], 64, tau)
        for i in range(n):
            row = s[0, 0, i, : i + 1].astype(np.float64)
            goal = tau * row.sum()
            forced = {0, i}
            best = None
            others = [j for j in range(1, i)]
            for r in range(len(others) + 1):  # brute force by size, then by kept mass
                for extra in itertools.combinations(others, r):
                    sel = forced | set(extra)
                    if row[list(sel)].sum() >= goal:
                        mass = row[list(sel)].sum()
                        if best is None or (len(sel), -mass) < (len(best), -row[list(best)].sum()):
                            best = sel
                if best is not None:
                    break
            got = set(np.flatnonzero(keep[0, 0, i]))
            if abs(row[list(best)].sum() - goal) < 1e-5 or abs(row[list(got)].sum() - goal) < 1e-5:
                continue  # too close to the threshold to compare fp32 with float64
            assert got == best, (trial, i, got, best)


def test_planted_block_is_found():
    rng = np.random.default_rng(4)
    T, B, S, d = 512, 64, 4, 16
    u = np.zeros(d)
    u[0] = 1.0
    q = rng.standard_normal((T, 1, d)) * 0.05
    k = rng.standard_normal((T, 1, d)) * 0.05
    q[6 * B:7 * B, 0] += 6.0 * u       # query block 6 ...
    k[2 * B:3 * B, 0] += 6.0 * u       # ... attends to key block 2
    sc = xattn.block_scores(q, k, [0, T], B, S, 1.0)
    keep = xattn.select_blocks(sc.astype(np.float32), [T], B, 0.9)
    assert set(np.flatnonzero(keep[0, 0, 6])) == {0, 2, 6}


def test_attention_with_every_block_kept_is_full_attention():
    rng = np.random.default_rng(5)
    lengths, hq, hkv, d, B, S = [300, 130], 4, 2, 32, 64, 8
    cu = synth.cu_seqlens_of(lengths)
    q, k, v = synth.qkv_host(rng, int(cu[-1]), hq, hkv, d, bf16=False)
    sc = xattn.block_scores(q, k, cu, B, S, 1 / math.sqrt(d))
    keep = xattn.select_blocks(sc.astype(np.float32), lengths, B, 1.5)  # unreachable goal
    nb = [-(-t // B) for t in lengths]
    for b, n in enumerate(nb):
        for i in range(n):
            assert keep[b, :, i, : i + 1].all() and not keep[b, :, i, i + 1:].any()
    o, lse = xattn.attn_prefill(q, k, v, cu, keep, B, 1 / math.sqrt(d))
    route = np.ones((2, 1), np.uint8)
    o_ref, l_ref = oracle.attn_prefill(q, k, v, cu, route, 0, 0, 64, 64, 1 / math.sqrt(d))
    np.testing.assert_allclose(o, o_ref, atol=1e-10)
    np.testing.assert_allclose(lse, l_ref, atol=1e-10)


def test_attention_over_the_streaming_blocks_is_the_sa_layer():
    rng = np.random.default_rng(6)
    lengths, hq, hkv, d, B = [700, 333], 8, 2, 32, 64
    sink, window = 64, 192
    cu = synth.cu_seqlens_of(lengths)
    q, k, v = synth.qkv_host(rng, int(cu[-1]), hq, hkv, d, bf16=True)
    nqb = -(-max(lengths) // B)
    keep = np.zeros((2, hq, nqb, nqb), bool)
    for b, T in enumerate(lengths):
        for i in range(-(-T // B)):
            for j in range(i + 1):
                keep[b, :, i, j] = j < sink // B or j > i - window // B
    o, lse = xattn.attn_prefill(q, k, v, cu, keep, B, 0.11)
    route = np.zeros((2, 1), np.uint8)
    o_ref, l_ref = oracle.attn_prefill(q, k, v, cu, route, 0, sink, window, B, 0.11)
    np.testing.assert_allclose(o, o_ref, atol=1e-10)
    np.testing.assert_allclose(lse, l_ref, atol=1e-10)


def test_selection_stops_exactly_at_the_threshold_and_breaks_ties_by_block():
    # total 1.0, tau 0.75: forced {0, 3} hold 0.5; block 1 (tie with block 2, the
    # smaller index goes first) brings the kept sum to exactly 0.75 = tau * total,
    # which is enough: block 2 stays out.
    s = np.zeros((1, 1, 4, 4), np.float32)
    s[0, 0, 3, :4] = 0.25
    keep = xattn.select_blocks(s, [256], 64, 0.75)
    assert set(np.flatnonzero(keep[0, 0, 3])) == {0, 1, 3}


def test_block_scores_gqa_equal_repeated_kv():
    rng = np.random.default_rng(7)
    T, hq, hkv, d, B, S = 256, 4, 2, 16, 64, 8
    q = rng.standard_normal((T, hq, d))
    k = rng.standard_normal((T, hkv, d))
    k_rep = np.repeat(k, hq // hkv, axis=1)  # head h -> KV head h // G, written out
    a = xattn.block_scores(q, k, [0, T], B, S, 0.25)
    b = xattn.block_scores(q, k_rep, [0, T], B, S, 0.25)
    np.testing.assert_array_equal(a, b)
    assert not np.allclose(a[0, 1], xattn.block_scores(q, np.repeat(k[:, ::-1], 2, axis=1),
                                                       [0, T], B, S, 0.25)[0, 1])


@pytest.mark.parametrize("T,stride,block", [(700, 8, 128), (450, 4, 64), (129, 8, 128)])
def test_single_block_row_agrees_with_the_pinned_full_scores(T, stride, block):
    """The per-block score function (used for sampled checks at full length) agrees
    with the whole-matrix scores pinned above, on every query block."""
    rng = np.random.default_rng(7)
    q = rng.standard_normal((T, 2, 16))
    k = rng.standard_normal((T, 1, 16))
    full = xattn.block_scores(q, k, [0, T], block, stride, 0.25)
    for i in range(-(-T // block)):
        for h in range(2):
            row = xattn.block_score_row(q[:, h], k[:, 0], stride, 0.25, block, i)
            np.testing.assert_allclose(row, full[0, h, i, : i + 1], rtol=1e-12, atol=1e-13)
