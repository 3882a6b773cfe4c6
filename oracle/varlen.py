"""Attention over a batch of variable-length sequences packed end to end, in
fp64 (test infrastructure).

Sources:
  * FlashAttention from Scratch (ryhuang.blog), §11.5 "Scheduling and
    implementation language matter": variable-length batches are a source of
    imbalance between work tiles, next to the causal diagonal.  Nothing about
    what a sequence attends to changes: each sequence is an attention problem
    of its own (§2), with the §5 rectangular causal rule (queries are the last
    positions of their sequence's keys) applied per sequence.
  * §12 "Programmable attention": packing several documents into one stream is
    only correct if no query attends to another document's keys; this module
    states that isolation twice, once per segment (``varlen_attention_forward``)
    and once as one materialised block-diagonal mask over the whole packed
    stream (``packed_mask_forward``), so each pins the other.
  * FlashAttention-4: Blackwell Attention Kernel Co-Design, "LPT scheduling for
    imbalanced grids", step 4: sort the batches by their maximum worktile time
    and keep the virtual-to-actual batch map.  ``lpt_schedule`` writes out that
    order for the library's work tiles (query blocks of 256 rows, KV tiles of
    64 keys), so the GPU's schedule can be compared integer for integer.

Layout (the library's varlen layout, stated here so the two can be compared):
  q : [Hq, total_q, D], k and v : [Hkv, total_k, D], sequences packed end to
  end along the row axis; sequence b owns query rows cu_q[b] .. cu_q[b+1]-1
  and key rows cu_k[b] .. cu_k[b+1]-1.  O is laid out like q and the LSE is
  [Hq, total_q].
"""
from __future__ import annotations

import numpy as np

from .attention import as_f64, dense_head


def segments(cu):
    """(start, length) of every sequence from cumulative offsets [B + 1]."""
    cu = np.asarray(as_f64(cu), dtype=np.int64)
    return [(int(cu[b]), int(cu[b + 1] - cu[b])) for b in range(len(cu) - 1)]


def sequence_view(q, k, v, cu_q, cu_k, b):
    """Sequence b of the packed batch as a batch of one: q [1, Hq, Lq_b, D],
    k and v [1, Hkv, Lk_b, D] (views of the packed rows), for the batched
    definition in ``attention``."""
    (qs, lq), (ks, lk) = segments(cu_q)[b], segments(cu_k)[b]
    return q[None, :, qs:qs + lq], k[None, :, ks:ks + lk], v[None, :, ks:ks + lk]


def varlen_attention_forward(q, k, v, cu_q, cu_k, scale, causal=False):
    """O [Hq, total_q, Dv] and LSE [Hq, total_q] (fp64): every sequence by the
    dense definition on its own rows, with its queries at key positions
    Lk_b - Lq_b + i (bottom-right, per sequence)."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    Hq, total_q = q.shape[0], q.shape[1]
    Hkv, Dv = k.shape[0], v.shape[2]
    assert Hq % Hkv == 0, "query heads must be a multiple of KV heads"
    r = Hq // Hkv
    O = np.zeros((Hq, total_q, Dv))
    lse = np.full((Hq, total_q), -np.inf)
    for b, ((qs, lq), (ks, lk)) in enumerate(zip(segments(cu_q), segments(cu_k))):
        if lq == 0:
            continue
        qb, kb, vb = sequence_view(q, k, v, cu_q, cu_k, b)
        q_pos = (lk - lq) + np.arange(lq)
        for h in range(Hq):
            g = h // r
            O[h, qs:qs + lq], lse[h, qs:qs + lq] = dense_head(
                qb[0, h], kb[0, g], vb[0, g], scale, causal, q_pos, np.arange(lk))
    return O, lse


def packed_mask_forward(q, k, v, cu_q, cu_k, scale, causal=False):
    """The same result from one materialised score matrix over the whole
    packed stream per head, with the mask allowed(i, j) = (i and j belong to
    the same sequence) and, if causal, (j's position <= i's position) -- no
    per-sequence loop over the arithmetic."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    Hq, total_q = q.shape[0], q.shape[1]
    Hkv, total_k = k.shape[0], k.shape[1]
    r = Hq // Hkv
    seg_q = np.full(total_q, -1)
    pos_q = np.zeros(total_q, dtype=np.int64)
    seg_k = np.full(total_k, -2)
    pos_k = np.zeros(total_k, dtype=np.int64)
    for b, ((qs, lq), (ks, lk)) in enumerate(zip(segments(cu_q), segments(cu_k))):
        seg_q[qs:qs + lq] = b
        pos_q[qs:qs + lq] = (lk - lq) + np.arange(lq)
        seg_k[ks:ks + lk] = b
        pos_k[ks:ks + lk] = np.arange(lk)
    allowed = seg_q[:, None] == seg_k[None, :]
    if causal:
        allowed &= pos_k[None, :] <= pos_q[:, None]
    O = np.zeros((Hq, total_q, v.shape[2]))
    lse = np.full((Hq, total_q), -np.inf)
    for h in range(Hq):
        S = np.where(allowed, scale * (q[h] @ k[h // r].T), -np.inf)
        m = S.max(axis=1) if total_k else np.full(total_q, -np.inf)
        row = np.isfinite(m)
        E = np.exp(S - np.where(row, m, 0.0)[:, None])
        ell = E.sum(axis=1)
        O[h] = np.where(row[:, None], (E @ v[h // r]) / np.where(row, ell, 1.0)[:, None], 0.0)
        lse[h] = np.where(row, m + np.log(np.where(row, ell, 1.0)), -np.inf)
    return O, lse


def lpt_schedule(cu_q, cu_k, causal, q_block=256, kv_tile=64):
    """(order, prefix): the sequences sorted by their longest work tile (the
    KV tiles the last query block of the sequence visits; ties keep the lower
    index first), and the running count of query blocks in that order
    (prefix[0] = 0, prefix[B] = all query blocks)."""
    segs_q, segs_k = segments(cu_q), segments(cu_k)
    cost, blocks = [], []
    for (_, lq), (_, lk) in zip(segs_q, segs_k):
        nqb = -(-lq // q_block)
        blocks.append(nqb)
        # The longest tile is the last query block.  Without the causal rule it
        # sees every key; with it, its last query sits at position lk - 1 (the
        # bottom-right alignment), so it sees every key too.  A sequence with
        # no query has no tile at all.  (``causal`` therefore leaves the order
        # unchanged; it is kept in the signature because the rule is per mask.)
        cost.append(-(-lk // kv_tile) if nqb else 0)
    order = sorted(range(len(cost)), key=lambda b: (-cost[b], b))
    prefix = [0]
    for b in order:
        prefix.append(prefix[-1] + blocks[b])
    return order, prefix
