"""CPU oracle of the Triangle Attention branch.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: the tests and the
CPU-baseline leg of ``bench.py`` may import it, the product library never does.

The pages use TriangleMix's Triangle Attention (TA) as a sparse backend of the
router: a block-level, fixed ("triangle") topology, training-free, for prefill
[thelatestinai paper page, Table 3, Table 5 and its caption, Table 12].  They
print none of its rules, so the published topology is read as follows (readings
labelled t1..t3):

  t1  a query block i of a sequence of nb blocks keeps the streaming blocks of
      the SA rule -- the sink blocks j < ns and the window blocks j > i - nw --
      and, when i is one of the last nl query blocks (i >= nb - nl), every key
      block j <= i: the kept region is the sink column, the diagonal band and
      the dense bottom rows of the causal triangle;
  t2  ns = sink / block, nw = window / block, nl = last_q / block, all in
      tokens that are multiples of the block; inside kept blocks the token-level
      causal rule s <= t holds;
  t3  FA-routed sequences keep every causal block; decode of a TA layer is the
      FA decode, since the decoded token lies in the dense tail.

The attention itself is the exact masked softmax of ``oracle.xattn.attn_prefill``
(float64) over the kept blocks.
"""
from __future__ import annotations

import numpy as np

from . import xattn


def triangle_keep(T: int, block: int, sink: int, window: int, last_q: int) -> np.ndarray:
    """t1-t2 for one sequence of T tokens: bool [nb, nb], row i = query block i,
    column j = key block j (False above the diagonal)."""
    nb = -(-T // block)
    ns, nw, nl = sink // block, window // block, last_q // block
    keep = np.zeros((nb, nb), bool)
    for i in range(nb):
        dense_row = i >= nb - nl
        for j in range(i + 1):
            keep[i, j] = dense_row or j < ns or j > i - nw
    return keep


def keep_mask(cu_seqlens, route_bits, hq, block, sink, window, last_q) -> np.ndarray:
    """t1-t3 for a packed varlen batch: bool [B, hq, NQB, NQB] (the same for
    every head); route_bits[b] = 1 keeps every causal block of sequence b."""
    cu = np.asarray(cu_seqlens, np.int64)
    B = len(cu) - 1
    nqb = max(1, max(-(-int(cu[b + 1] - cu[b]) // block) for b in range(B)))
    keep = np.zeros((B, hq, nqb, nqb), bool)
    for b in range(B):
        T = int(cu[b + 1] - cu[b])
        if T <= 0:
            continue
        nb = -(-T // block)
        if route_bits[b]:
            m = np.tril(np.ones((nb, nb), bool))
        else:
            m = triangle_keep(T, block, sink, window, last_q)
        keep[b, :, :nb, :nb] = m
    return keep


def attn_prefill(q, k, v, cu_seqlens, route_bits, block, sink, window, last_q, sm_scale,
                 rows=None):
    """Prefill attention with Triangle Attention as the sparse branch.  q [total,
    Hq, d], k/v [total, Hkv, d] (fp32 or bf16 bits).  Returns (o float64
    [n_rows, Hq, d], lse float64 [n_rows, Hq])."""
    keep = keep_mask(cu_seqlens, route_bits, q.shape[1], block, sink, window, last_q)
    return xattn.attn_prefill(q, k, v, cu_seqlens, keep, block, sm_scale, rows=rows)
