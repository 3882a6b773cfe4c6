"""fp64 model of the online-softmax recurrence (test infrastructure).

Used only to pin the dense definition (and to be pinned by it); it shares no
code with ``attention.py``.  Sources:
  * FlashAttention from Scratch (ryhuang.blog), §4.1 "Maintain three
    quantities": every query row carries a reference exponent, a normaliser
    and a weighted sum of value rows, all relative to the reference, over the
    keys seen so far; a new tile raises the reference to its row maximum if
    larger, scales the old normaliser and sum by e^(old - new) and adds the
    tile's terms; the output is the sum over the normaliser;
  * §4.4 "Handle the empty state deliberately": the state starts empty
    (reference -inf, zero normaliser and sum), and no -inf - (-inf) is ever
    formed;
  * §11.3 "Derive conditional rescaling correctly" and "FlashAttention-4:
    Blackwell Attention Kernel Co-Design", "Conditional online-softmax
    rescaling": the reference may stay put while a tile's maximum exceeds it
    by at most tau; it is first set by the first tile that holds a valid key;
  * FlashAttention Cheat Sheet (mxino.github.io), §5 "Why online softmax is
    globally exact": the order in which tiles are visited does not change the
    result.

Structure: the state of all rows of a query block lives in one ``RowState``;
the key tiles are the outer loop (in the requested order) and each query
block absorbs every tile, so tile order and tile sizes are free parameters.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


class RowState:
    """Running state of a set of query rows: ``ref`` (the exponent every
    stored term is taken relative to), ``norm`` (sum of e^(s - ref)) and
    ``acc`` (sum of e^(s - ref) v)."""

    def __init__(self, rows: int, dv: int):
        self.ref = np.full(rows, -np.inf)
        self.norm = np.zeros(rows)
        self.acc = np.zeros((rows, dv))

    def absorb(self, scores: np.ndarray, values: np.ndarray, tau=None) -> np.ndarray:
        """Fold one tile in: ``scores`` [rows, n] (masked pairs -inf) and the
        tile's value rows [n, dv].  Returns the factor e^(old ref - new ref)
        the earlier terms were multiplied by."""
        peak = scores.max(axis=1)
        raised = np.maximum(self.ref, peak)
        if tau is not None:
            with np.errstate(invalid="ignore"):
                # -inf - (-inf) is NaN and compares false: an empty row always takes the raise
                keep = (peak - self.ref) <= tau
            raised = np.where(keep, self.ref, raised)
        anchor = np.where(np.isfinite(raised), raised, 0.0)
        factor = np.exp(self.ref - anchor)        # an empty state gives 0
        terms = np.exp(scores - anchor[:, None])
        self.norm = factor * self.norm + terms.sum(axis=1)
        self.acc = factor[:, None] * self.acc + terms @ values
        self.ref = raised
        return factor

    def result(self):
        """(O, LSE): acc / norm and ref + log(norm), or (0, -inf) for a row
        that absorbed no valid key."""
        seen = self.norm > 0
        den = np.where(seen, self.norm, 1.0)
        out = np.where(seen[:, None], self.acc / den[:, None], 0.0)
        return out, np.where(seen, self.ref + np.log(den), -np.inf)


def streaming_head(q, k, v, scale, causal=False, q_pos=None, k_pos=None,
                   block_q=32, block_k=64, kv_order=None, tau=None, trace=None):
    """Tile-by-tile forward for one head; returns (O, LSE) in fp64.

    block_q / block_k: tile sizes.  kv_order: optional permutation of the KV
    tile indices (tile t covers keys [t*block_k, (t+1)*block_k)).  tau: None
    for the plain recurrence, else the conditional-rescale threshold in
    natural-log units.  trace: optional list that receives, per visited
    (query block, tile) pair in visiting order, a dict with the state after
    it in the pages' notation (m = reference, ell = normaliser, u = sum,
    alpha = the factor applied to the earlier terms).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    Lq, Lk, Dv = q.shape[0], k.shape[0], v.shape[1]
    q_pos = np.arange(Lq) if q_pos is None else np.asarray(q_pos)
    k_pos = np.arange(Lk) if k_pos is None else np.asarray(k_pos)
    n_tiles = (Lk + block_k - 1) // block_k
    order = list(range(n_tiles)) if kv_order is None else list(kv_order)
    assert sorted(order) == list(range(n_tiles)), "kv_order must permute the tiles"

    blocks = [(r0, min(r0 + block_q, Lq)) for r0 in range(0, Lq, block_q)]
    states = [RowState(r1 - r0, Dv) for r0, r1 in blocks]
    for t in order:
        keys = slice(t * block_k, min((t + 1) * block_k, Lk))
        for (r0, r1), st in zip(blocks, states):
            tile = scale * (q[r0:r1] @ k[keys].T)
            if causal:
                tile = np.where(k_pos[keys][None, :] <= q_pos[r0:r1][:, None], tile, -np.inf)
            factor = st.absorb(tile, v[keys], tau)
            if trace is not None:
                trace.append({"q_block": r0, "tile": t, "m": st.ref.copy(), "alpha": factor.copy(),
                              "ell": st.norm.copy(), "u": st.acc.copy()})

    out = np.zeros((Lq, Dv))
    lse = np.full(Lq, -np.inf)
    for (r0, r1), st in zip(blocks, states):
        out[r0:r1], lse[r0:r1] = st.result()
    return out, lse
