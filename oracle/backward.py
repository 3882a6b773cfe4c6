"""Gradients of exact attention, written out densely in fp64 (test
infrastructure).

Sources:
  * FlashAttention from Scratch (ryhuang.blog), §8 "Backward: spend
    arithmetic to save memory", no dropout, fixed mask: with G = dL/dO,
    O = P V gives dV = P^T G and dP = G V^T; the softmax Jacobian gives
    dS_ij = P_ij (dP_ij - delta_i) with delta_i = sum_t P_it dP_it, which
    equals G_i . O_i (the section's checkpoint); the scores are s = c q.k, so
    dQ = c dS K and dK = c dS^T Q.  (The page's equations are lost in
    extraction; these are the standard results its text describes and its
    checkpoint states.)
  * Same section: a row's probabilities are reconstructed from its saved
    normaliser, P_ij = exp(s_ij - LSE_i); a fully masked row has P = 0 and
    contributes nothing.
  * Same section: with grouped-query attention the gradients of a shared KV
    head accumulate the contributions of every query head that reads it.

This module materialises S, P, dP and dS for one (batch, query head) at a
time; it does not use a saved LSE (P comes from the definition of softmax),
so it checks the GPU path's reconstruction rather than sharing it.

``o_given`` evaluates the same formulas with delta_i = G_i . o_given_i for a
given output o_given instead of the exact O (everything else unchanged): the
gradient a backward computes when it is handed a stored, rounded forward
output, as the section's recomputation does.
"""
from __future__ import annotations

import numpy as np

from .attention import as_f64


def dense_backward_head(q, k, v, g, scale, causal=False, q_pos=None, k_pos=None, window=0,
                        o_given=None):
    """(dQ, dK, dV) of one (batch, head) in fp64 for upstream gradient g.

    q: [Lq, D]; k: [Lk, D]; v: [Lk, Dv]; g: [Lq, Dv].  Masks as in
    ``attention.dense_head``.  ``o_given`` [Lq, Dv]: form delta from it.
    """
    q, k, v, g = as_f64(q), as_f64(k), as_f64(v), as_f64(g)
    Lq, Lk = q.shape[0], k.shape[0]
    q_pos = np.arange(Lq) if q_pos is None else np.asarray(q_pos)
    k_pos = np.arange(Lk) if k_pos is None else np.asarray(k_pos)
    if Lk == 0:
        return np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    allowed = np.ones((Lq, Lk), dtype=bool)
    if causal:
        allowed &= k_pos[None, :] <= q_pos[:, None]
    if window > 0:
        dist = q_pos[:, None] - k_pos[None, :]
        allowed &= (dist >= 0) & (dist < window)

    # Forward quantities, materialised: S, P (row softmax over allowed keys), O.
    S = np.where(allowed, scale * (q @ k.T), -np.inf)
    m = S.max(axis=1)
    has_key = np.isfinite(m)
    E = np.exp(S - np.where(has_key, m, 0.0)[:, None])
    ell = E.sum(axis=1)
    P = E / np.where(has_key, ell, 1.0)[:, None]
    O = P @ v

    # Backward through O = P V, the row softmax and S = scale * Q K^T.
    dV = P.T @ g
    dP = g @ v.T
    delta = (g * (O if o_given is None else as_f64(o_given))).sum(axis=1)
    dS = P * (dP - delta[:, None])
    dQ = scale * (dS @ k)
    dK = scale * (dS.T @ q)
    return dQ, dK, dV


def attention_backward(q, k, v, g, scale, causal=False, kv_lens=None, window=0, o_given=None):
    """Batched gradients for [B, H, L, D] inputs: dQ [B, Hq, Lq, D],
    dK [B, Hkv, Lk, D], dV [B, Hkv, Lk, Dv] in fp64.  Queries sit at the end
    of each sequence's valid keys (bottom-right alignment, as in the
    forward); keys at or past kv_lens[b] get zero gradient; a KV head's
    gradients sum over the query heads h with floor(h / r) equal to it.
    ``o_given`` [B, Hq, Lq, Dv]: delta from this output (module docstring)."""
    q, k, v, g = as_f64(q), as_f64(k), as_f64(v), as_f64(g)
    B, Hq, Lq = q.shape[0], q.shape[1], q.shape[2]
    Hkv, Lk = k.shape[1], k.shape[2]
    assert Hq % Hkv == 0, "query heads must be a multiple of KV heads"
    r = Hq // Hkv
    lens = None if kv_lens is None else as_f64(kv_lens)
    og = None if o_given is None else as_f64(o_given)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        n = Lk if lens is None else int(min(max(int(lens[b]), 0), Lk))
        q_pos = (n - Lq) + np.arange(Lq)
        for h in range(Hq):
            gk = h // r
            dqh, dkh, dvh = dense_backward_head(q[b, h], k[b, gk, :n], v[b, gk, :n], g[b, h],
                                                scale, causal, q_pos, np.arange(n), window,
                                                None if og is None else og[b, h])
            dq[b, h] = dqh
            dk[b, gk, :n] += dkh
            dv[b, gk, :n] += dvh
    return dq, dk, dv
