"""CPU oracle of the XAttention sparse branch (antidiagonal block scoring).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: the tests and the
CPU-baseline leg of ``bench.py`` may import it, the product library never does.

The pages name XAttention as one of the sparse operators Flux Attention's
router can send a layer to: "XAttention: Block Sparse Attention with
Antidiagonal Scoring" in the mlsanity page's reference list; a block-level
operator with a block selection score used for prefill in the thelatestinai
paper page's Table 3; the XA columns of its Table 12; and ``find_blocks_chunked``
in an ``Xattention.py`` file of the codewithpapers function list.  They print
none of its steps.  This module writes out the published method as read here
(every point is a reading of the pages, labelled x1..x7):

  x1  block size B and stride S with B % S == 0; R = B / S reshaped rows per block.
  x2  reshaped rows: query row a stands for positions a*S + (S-1-s), key row b
      for positions b*S + s (s = 0..S-1); positions >= T are zero vectors.
  x3  antidiagonal score A[a][b] = (sm_scale / S) * sum_s <q[a*S+S-1-s], k[b*S+s]>,
      i.e. the mean of the S x S sub-block's antidiagonal (row + column is
      constant on it), for b <= a (causal on reshaped rows); query head h
      reads KV head h // G.
  x4  P = row-wise softmax of A over b <= a.
  x5  block score score[i][j] = sum of P[a][b] over the R reshaped rows of query
      block i and the R reshaped columns of key block j (j <= i).
  x6  selection for query block i: the sink block 0 and the diagonal block i
      are always kept; the other blocks j < i join in order of decreasing score
      (ties: smaller j first) while the kept sum is below tau * total, where
      total = sum_{j<=i} score[i][j].  Every sum of this step is fp32 in the
      stated order, and the kernel takes the same fp32 decision.
  x7  attention: query t sees key s iff s <= t and block s // B is kept for
      the query block t // B of t's head.

Scores and attention are float64; x6 runs in float32 on the scores it is given.
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:  # bf16 bits -> exact float
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def reshaped_scores(q_h, k_h, stride, sm_scale):
    """x2-x3 for one head of one sequence: q_h, k_h [T, d] -> A [Tr, Tr] (float64),
    entries above the reshaped diagonal set to -inf."""
    q_h, k_h = _f64(q_h), _f64(k_h)
    T, d = q_h.shape
    Tr = -(-T // stride)
    qp = np.zeros((Tr * stride, d))
    kp = np.zeros((Tr * stride, d))
    qp[:T] = q_h
    kp[:T] = k_h
    # row a of qr = [q[a*S + S-1], q[a*S + S-2], ..., q[a*S]]; row b of kr = [k[b*S], .., k[b*S+S-1]]
    qr = qp.reshape(Tr, stride, d)[:, ::-1, :].reshape(Tr, stride * d)
    kr = kp.reshape(Tr, stride * d)
    A = (qr @ kr.T) * (sm_scale / stride)
    A[np.triu_indices(Tr, 1)] = -np.inf
    return A


def block_scores(q, k, cu_seqlens, block, stride, sm_scale, heads=None):
    """x2-x5 for a packed varlen batch: q [total, Hq, d], k [total, Hkv, d] ->
    scores [B, n_heads, NQB, NQB] float64 (NQB = blocks of the longest sequence;
    entries past a sequence's blocks or above the block diagonal are 0)."""
    cu = np.asarray(cu_seqlens, np.int64)
    hq, hkv = q.shape[1], k.shape[1]
    G = hq // hkv
    heads = list(range(hq)) if heads is None else list(heads)
    R = block // stride
    nqb = max(-(-int(cu[b + 1] - cu[b]) // block) for b in range(len(cu) - 1))
    out = np.zeros((len(cu) - 1, len(heads), nqb, nqb))
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        T = s1 - s0
        if T <= 0:
            continue
        nb = -(-T // block)
        for hi, h in enumerate(heads):
            A = reshaped_scores(q[s0:s1, h], k[s0:s1, h // G], stride, sm_scale)
            m = A.max(axis=1, keepdims=True)
            P = np.exp(A - m)
            P /= P.sum(axis=1, keepdims=True)
            Tr = A.shape[0]  # the last block may hold fewer than R reshaped rows
            Pp = np.zeros((nb * R, nb * R))
            Pp[:Tr, :Tr] = P
            out[b, hi, :nb, :nb] = Pp.reshape(nb, R, nb, R).sum(axis=(1, 3))
    return out


def block_score_row(q_h, k_h, stride, sm_scale, block, i):
    """x2-x5 for query block i of one head of one sequence, computed on its own
    (for sampled checks at full length): q_h, k_h [T, d] -> score[i][0..i]
    (float64, length i + 1).  Only the reshaped rows of block i and the columns
    they can see are formed."""
    q_h, k_h = _f64(q_h), _f64(k_h)
    T, d = q_h.shape
    Tr = -(-T // stride)
    R = block // stride
    a0, a1 = R * i, min(R * i + R, Tr)
    cols = a1  # reshaped columns 0 .. a1-1 (b <= a)

    def rows_of(x, r0, r1, flip):
        out = np.zeros(((r1 - r0) * stride, d))
        p0, p1 = r0 * stride, min(r1 * stride, T)
        if p1 > p0:
            out[: p1 - p0] = x[p0:p1]
        out = out.reshape(r1 - r0, stride, d)
        if flip:
            out = out[:, ::-1, :]
        return out.reshape(r1 - r0, stride * d)

    qr = rows_of(q_h, a0, a1, True)
    kr = rows_of(k_h, 0, cols, False)
    A = (qr @ kr.T) * (sm_scale / stride)
    A[np.arange(cols)[None, :] > np.arange(a0, a1)[:, None]] = -np.inf
    m = A.max(axis=1, keepdims=True)
    P = np.exp(A - m)
    P /= P.sum(axis=1, keepdims=True)
    Pp = np.zeros((a1 - a0, (i + 1) * R))
    Pp[:, :cols] = P
    return Pp.sum(axis=0).reshape(i + 1, R).sum(axis=1)


def select_row(row32, i, threshold):
    """x6 for query block i: row32 float32 scores score[i][0..i] (entries past i
    are ignored) -> kept-block flags bool [i + 1]."""
    row = np.asarray(row32, np.float32)
    tau = np.float32(threshold)
    keep = np.zeros(i + 1, bool)
    total = np.float32(0.0)
    for j in range(i + 1):
        total = np.float32(total + row[j])
    goal = np.float32(tau * total)
    keep[0] = True
    keep[i] = True
    kept = np.float32(row[0])
    if i > 0:
        kept = np.float32(kept + row[i])
    rest = sorted(range(1, i), key=lambda j: (-float(row[j]), j))
    for j in rest:
        if not kept < goal:
            break
        keep[j] = True
        kept = np.float32(kept + row[j])
    return keep


def select_blocks(scores32, seqlens, block, threshold):
    """x6: scores float32 [B, H, NQB, NQB] (as the kernel produced them) ->
    kept-block mask bool [B, H, NQB, NQB]."""
    s = np.asarray(scores32, np.float32)
    B, H, nqb, _ = s.shape
    keep = np.zeros(s.shape, bool)
    for b in range(B):
        nb = -(-int(seqlens[b]) // block)
        for h in range(H):
            for i in range(nb):
                keep[b, h, i, : i + 1] = select_row(s[b, h, i], i, threshold)
    return keep


def attn_prefill(q, k, v, cu_seqlens, keep, block, sm_scale, rows=None):
    """x7: exact softmax attention over the kept blocks.  q [total, Hq, d], k/v
    [total, Hkv, d] (fp32 or bf16 bits), keep bool [B, Hq, NQB, NQB].
    Returns (o float64 [n_rows, Hq, d], lse float64 [n_rows, Hq])."""
    cu = np.asarray(cu_seqlens, np.int64)
    total, hq, d = q.shape
    G = hq // k.shape[1]
    rows = np.arange(total) if rows is None else np.asarray(rows)
    o = np.zeros((len(rows), hq, d))
    lse = np.zeros((len(rows), hq))
    seq_of = np.searchsorted(cu, rows, side="right") - 1
    for n, (r, b) in enumerate(zip(rows, seq_of)):
        s0 = int(cu[b])
        t = int(r) - s0
        keys = np.arange(t + 1)
        kept = keep[b, :, t // block][:, keys // block]  # [hq, t + 1]: key s visible to head h
        # widen only what row r reads: its query and the keys some head keeps
        used = keys[kept.any(axis=0)]
        qf = _f64(q[r])
        kf, vf = _f64(k[s0 + used]), _f64(v[s0 + used])
        for h in range(hq):
            vis = kept[h, used]
            sc = kf[vis, h // G] @ qf[h] * sm_scale
            m = sc.max()
            p = np.exp(sc - m)
            o[n, h] = p @ vf[vis, h // G] / p.sum()
            lse[n, h] = m + np.log(p.sum())
    return o, lse
