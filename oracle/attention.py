"""The definition of exact attention, written out in fp64 (test infrastructure).

O = softmax(S + M) V with S = scale * Q K^T and M_ij = 0 for an allowed pair,
-inf otherwise, one softmax per query row.  Sources:
  * FlashAttention from Scratch (ryhuang.blog), §2 "Begin with one attention
    row" (the formula, the per-row softmax, the {0, -inf} mask) and
    "Stabilize softmax before doing anything clever" (subtract the row max);
  * §3 "Why straightforward attention is expensive": the materialised form
    (write S, softmax it into P, multiply P by V) is exactly what this module
    does, in fp64 on the CPU;
  * §4.4 "Handle the empty state deliberately": a row with no allowed key
    returns a zero output and log-sum-exp -inf (an API convention);
  * §5 "Run the math before writing a GPU kernel": causal pairs are allowed
    when key position <= query position, with absolute positions;
    "Rectangular causal masking is a correctness issue": with fewer queries
    than keys the queries are the last positions of the cache
    (bottom-right alignment);
  * §7.1 / FlashAttention 1-4 (noviorlu.github.io), FlashAttention-2 change 1:
    the saved row statistic is the natural-log LSE = m + log(l);
  * §9.2 "GQA changes the reuse opportunity": query head h reads KV head
    floor(h / r) with r = Hq / Hkv;
  * §12 "Programmable attention": a causal window of width w allows a key
    only at the query's position or at most w - 1 positions before it (the
    page's formula is lost in extraction; this reading makes w the number of
    keys a row sees once it is w or more positions into the sequence);
  * §12 "Programmable attention": a score may be modified before the softmax,
    S'_ij = f(S_ij, i, j); FlashAttention 1-4 (noviorlu.github.io),
    FlashAttention-4 point 4, names ALiBi and soft-capping as such
    modifiers.  Neither formula is on the pages; the readings taken are
    soft-capping S' = cap * tanh(S / cap) of the scaled score and ALiBi
    S' = S - slope_h * |pos_i - pos_j| with one slope per query head (on
    causal pairs |pos_i - pos_j| = pos_i - pos_j); a modifier acts before the
    masks, so a masked pair stays -inf;
  * FlashAttention Cheat Sheet (mxino.github.io), §1 "The whole operation":
    Q [B, Hq, Lq, D], K and V [B, Hkv, Lk, D].

Inputs are taken at their exact values (bf16 tensors are widened to fp64 with
no rounding), so the oracle answers "what is the exact attention of these
bf16 numbers", which is what the tolerances of the GPU comparison are about.
"""
from __future__ import annotations

import numpy as np


def as_f64(x) -> np.ndarray:
    """Widen a numpy array or a torch tensor (any dtype, any device) to fp64."""
    if hasattr(x, "detach"):  # torch tensor, converted without importing torch here
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def dense_head(q, k, v, scale, causal=False, q_pos=None, k_pos=None, window=0,
               alibi_slope=0.0, softcap=0.0, return_weights=False):
    """Materialised attention for one (batch, head): returns (O, LSE) in fp64
    (with ``return_weights`` also the probability matrix P and the value rows).

    q: [Lq, D]; k: [Lk, D]; v: [Lk, Dv].  q_pos / k_pos are the absolute
    token positions of the rows (default 0..L-1); with ``causal`` a pair is
    allowed iff k_pos[j] <= q_pos[i]; with ``window`` = w > 0 a pair is
    allowed iff 0 <= q_pos[i] - k_pos[j] < w (the causal window, which is
    causal by itself).  ``softcap`` > 0 caps the scaled scores at +-softcap
    (cap * tanh(S / cap)); ``alibi_slope`` subtracts slope * |q_pos - k_pos|.
    """
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    Lq, Lk, Dv = q.shape[0], k.shape[0], v.shape[1]
    q_pos = np.arange(Lq) if q_pos is None else np.asarray(q_pos)
    k_pos = np.arange(Lk) if k_pos is None else np.asarray(k_pos)
    if Lk == 0:
        if return_weights:
            return np.zeros((Lq, Dv)), np.full(Lq, -np.inf), np.zeros((Lq, 0)), v
        return np.zeros((Lq, Dv)), np.full(Lq, -np.inf)

    # Write the whole score matrix.
    S = scale * (q @ k.T)
    # Score modifiers, before any mask.
    if softcap > 0:
        S = softcap * np.tanh(S / softcap)
    if alibi_slope != 0.0:
        S = S - alibi_slope * np.abs(q_pos[:, None] - k_pos[None, :]).astype(np.float64)
    if causal:
        S = np.where(k_pos[None, :] > q_pos[:, None], -np.inf, S)
    if window > 0:
        dist = q_pos[:, None] - k_pos[None, :]
        S = np.where((dist < 0) | (dist >= window), -np.inf, S)

    # Row softmax with the max shift; masked entries give exp(-inf) = 0.
    m = S.max(axis=1)
    has_key = np.isfinite(m)
    shift = np.where(has_key, m, 0.0)
    E = np.exp(S - shift[:, None])
    ell = E.sum(axis=1)
    safe_ell = np.where(has_key, ell, 1.0)
    P = E / safe_ell[:, None]

    # Multiply the probability matrix by V.
    O = P @ v
    O[~has_key] = 0.0
    lse = np.where(has_key, shift + np.log(safe_ell), -np.inf)
    if return_weights:
        return O, lse, P, v
    return O, lse


def _kv_len(kv_lens, b, Lk):
    if kv_lens is None:
        return Lk
    return int(min(max(int(as_f64(kv_lens)[b]), 0), Lk))


def attention_rows(q, k, v, scale, causal, kv_lens, b, h, rows=None, window=0,
                   alibi_slopes=None, softcap=0.0, return_weights=False, trim_keys=False):
    """(O, LSE) of selected query rows of one (b, h) of a batched problem.

    Rows are evaluated by the same definition as ``attention_forward``; this
    lets full-size problems be checked on sampled rows or row chunks.  With
    ``trim_keys``, keys that the causal mask (or the window) removes for EVERY
    selected row are left out of the materialised S: they would be -inf
    there, add exp(-inf) = 0 to every sum and never be a row max, so the
    result is the same up to the rounding order of the matrix products, and a
    chunk of early causal rows costs what its allowed keys cost.
    ``return_weights`` also returns P and the value rows it weights.
    """
    Hq, Lq = q.shape[1], q.shape[2]
    Hkv, Lk = k.shape[1], k.shape[2]
    r = Hq // Hkv
    g = h // r
    n = _kv_len(kv_lens, b, Lk)
    rows = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    q_pos = (n - Lq) + rows          # bottom-right: the queries end the cache
    lo, hi = 0, n
    if trim_keys and (causal or window > 0) and rows.size:
        hi = int(min(n, max(q_pos.max() + 1, 0)))
        if window > 0:
            lo = int(min(hi, max(q_pos.min() - window + 1, 0)))
    q_bh = as_f64(q[b, h])[rows]
    k_bg = as_f64(k[b, g, lo:hi])
    v_bg = as_f64(v[b, g, lo:hi])
    slope = 0.0 if alibi_slopes is None else float(as_f64(alibi_slopes)[h])
    return dense_head(q_bh, k_bg, v_bg, scale, causal, q_pos, np.arange(lo, hi), window, slope, softcap,
                      return_weights)


def attention_forward(q, k, v, scale, causal=False, kv_lens=None, window=0, alibi_slopes=None,
                      softcap=0.0):
    """Batched attention over [B, H, L, D] inputs: returns O [B, Hq, Lq, Dv]
    and LSE [B, Hq, Lq], both fp64.  ``kv_lens[b]`` (clamped to [0, Lk]) is the
    number of valid keys of sequence b; None means all Lk are valid.
    ``window`` > 0 applies the causal window of that width; ``alibi_slopes``
    ([Hq], one per query head) and ``softcap`` are the score modifiers of
    ``dense_head``."""
    B, Hq, Lq = q.shape[0], q.shape[1], q.shape[2]
    Hkv, Dv = k.shape[1], v.shape[3]
    assert Hq % Hkv == 0, "query heads must be a multiple of KV heads"
    O = np.zeros((B, Hq, Lq, Dv))
    lse = np.zeros((B, Hq, Lq))
    for b in range(B):
        for h in range(Hq):
            O[b, h], lse[b, h] = attention_rows(q, k, v, scale, causal, kv_lens, b, h,
                                                window=window, alibi_slopes=alibi_slopes,
                                                softcap=softcap)
    return O, lse
