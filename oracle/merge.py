"""fp64 models of merging attention over disjoint key partitions (test
infrastructure).

Sources:
  * FlashAttention from Scratch (ryhuang.blog), §4.3 "Merge independently
    computed partitions": the states (reference, normaliser, weighted value
    sum) of disjoint key sets combine by re-expressing each relative to the
    largest reference and adding; any merge tree gives the same exact result.
    Normalised partials combine by their natural-log normalisers: the merged
    normaliser is log sum_s e^(L_s) and the merged output is
    sum_s e^(L_s - L) O_s; a row empty in every part stays empty;
  * §9.1 "Split the long dimension that remains": split-KV decoding computes
    one normalised partial per KV partition and reduces them with that merge;
  * §4.4: the empty state is (-inf, 0, 0), finishing to O = 0 and LSE = -inf.

Each merge here takes any number of parts at once (a two-part merge is the
special case the trees in the tests nest).
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def _anchor(top):
    """The common exponent reference: the largest one, or 0 where every part
    is empty (so no -inf - (-inf) is formed)."""
    return np.where(np.isfinite(top), top, 0.0)


def partition_state(q, k, v, scale, causal=False, q_pos=None, k_pos=None):
    """State (reference, normaliser, weighted sum) of every query row over one
    key subset, with the subset's row maximum as the reference (§4.1)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    Lq, Lk, Dv = q.shape[0], k.shape[0], v.shape[1]
    if Lk == 0:
        return np.full(Lq, -np.inf), np.zeros(Lq), np.zeros((Lq, Dv))
    q_pos = np.arange(Lq) if q_pos is None else np.asarray(q_pos)
    k_pos = np.arange(Lk) if k_pos is None else np.asarray(k_pos)
    scores = scale * (q @ k.T)
    if causal:
        scores = np.where(k_pos[None, :] <= q_pos[:, None], scores, -np.inf)
    ref = scores.max(axis=1)
    terms = np.exp(scores - _anchor(ref)[:, None])
    return ref, terms.sum(axis=1), terms @ v


def merge_states(*parts):
    """Merge the states of disjoint key subsets (§4.3, first form)."""
    refs = np.stack([p[0] for p in parts])
    top = refs.max(axis=0)
    scale_to_top = np.exp(refs - _anchor(top)[None, :])      # [parts, rows]; empty parts give 0
    norm = np.einsum("pr,pr->r", scale_to_top, np.stack([p[1] for p in parts]))
    acc = np.einsum("pr,prd->rd", scale_to_top, np.stack([p[2] for p in parts]))
    return top, norm, acc


def finish_state(state):
    """(O, LSE) from a state: O = sum / normaliser and LSE = reference +
    log(normaliser), or (0, -inf) for a row with no key (§4.4 convention)."""
    ref, norm, acc = state
    seen = norm > 0
    den = np.where(seen, norm, 1.0)
    out = np.where(seen[:, None], acc / den[:, None], 0.0)
    return out, np.where(seen, ref + np.log(den), -np.inf)


def merge_normalized(*pairs):
    """Merge normalised partials given as O_1, L_1, O_2, L_2, ... by their
    natural-log normalisers (§4.3, second form; §9.1)."""
    assert len(pairs) >= 2 and len(pairs) % 2 == 0, "pass (output, lse) pairs"
    outs = np.stack([_f64(o) for o in pairs[0::2]])            # [parts, rows, dv]
    lses = np.stack([_f64(l) for l in pairs[1::2]])            # [parts, rows]
    top = lses.max(axis=0)
    with np.errstate(divide="ignore"):                       # log(0) = -inf for an all-empty row
        total = _anchor(top) + np.log(np.exp(lses - _anchor(top)[None, :]).sum(axis=0))
    total = np.where(np.isfinite(top), total, -np.inf)          # every part empty: stays empty
    weights = np.exp(lses - _anchor(total)[None, :])
    return np.einsum("pr,prd->rd", weights, outs), total
