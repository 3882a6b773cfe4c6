"""fp64 model of the online-softmax recurrence (test infrastructure).

Used only to pin the dense definition (and to be pinned by it); it shares no
code with ``attention.py``.  Sources:
  * FlashAttention from Scratch (ryhuang.blog), §4.1 "Maintain three
    quantities": per query row the state (m, l, u) over the keys seen so far;
    when a tile arrives, m' = max(m, tile max), alpha = exp(m - m'),
    l' = alpha l + sum exp(s - m'), u' = alpha u + sum exp(s - m') v; after the
    last tile o = u / l;
  * §4.4 "Handle the empty state deliberately": start from m = -inf, l = 0,
    u = 0, and never form -inf - (-inf);
  * §11.3 "Derive conditional rescaling correctly" and "FlashAttention-4:
    Blackwell Attention Kernel Co-Design", "Conditional online-softmax
    rescaling": keep the reference r unless a tile's max t exceeds it by more
    than tau; the reference is first set from the first tile with a valid key;
  * FlashAttention Cheat Sheet (mxino.github.io), §5 "Why online softmax is
    globally exact": tile order may change without changing the result.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def streaming_head(q, k, v, scale, causal=False, q_pos=None, k_pos=None,
                   block_q=32, block_k=64, kv_order=None, tau=None, trace=None):
    """Tile-by-tile forward for one head; returns (O, LSE) in fp64.

    block_q / block_k: tile sizes.  kv_order: optional permutation of the KV
    tile indices (tile t covers keys [t*block_k, (t+1)*block_k)).  tau: None
    for the plain recurrence, else the conditional-rescale threshold in
    natural-log units.  trace: optional list that receives, per query block
    and per visited tile, a dict with the state after that tile.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    Lq, Lk, Dv = q.shape[0], k.shape[0], v.shape[1]
    q_pos = np.arange(Lq) if q_pos is None else np.asarray(q_pos)
    k_pos = np.arange(Lk) if k_pos is None else np.asarray(k_pos)
    n_tiles = (Lk + block_k - 1) // block_k
    order = list(range(n_tiles)) if kv_order is None else list(kv_order)
    assert sorted(order) == list(range(n_tiles)), "kv_order must permute the tiles"

    out = np.zeros((Lq, Dv))
    lse = np.full(Lq, -np.inf)
    for i0 in range(0, Lq, block_q):
        qt = q[i0:i0 + block_q]
        qp = q_pos[i0:i0 + block_q]
        rows = qt.shape[0]
        m = np.full(rows, -np.inf)       # running reference (max, or stale max under tau)
        ell = np.zeros(rows)
        u = np.zeros((rows, Dv))
        for t in order:
            j0 = t * block_k
            kt, vt, kp = k[j0:j0 + block_k], v[j0:j0 + block_k], k_pos[j0:j0 + block_k]
            s = scale * (qt @ kt.T)
            if causal:
                s[kp[None, :] > qp[:, None]] = -np.inf
            tile_max = s.max(axis=1)
            if tau is None:
                new_m = np.maximum(m, tile_max)
            else:
                with np.errstate(invalid="ignore"):
                    jump = tile_max - m      # +inf (or NaN) while the row has no reference yet
                move = ~(jump <= tau)
                new_m = np.where(move, np.maximum(m, tile_max), m)
            shift = np.where(np.isfinite(new_m), new_m, 0.0)
            alpha = np.exp(m - shift)        # m = -inf gives 0, never NaN
            p = np.exp(s - shift[:, None])
            ell = alpha * ell + p.sum(axis=1)
            u = alpha[:, None] * u + p @ vt
            m = new_m
            if trace is not None:
                trace.append({"q_block": i0, "tile": t, "m": m.copy(), "alpha": alpha.copy(),
                              "ell": ell.copy(), "u": u.copy()})
        ok = ell > 0
        safe = np.where(ok, ell, 1.0)
        out[i0:i0 + rows] = np.where(ok[:, None], u / safe[:, None], 0.0)
        lse[i0:i0 + rows] = np.where(ok, m + np.log(safe), -np.inf)
    return out, lse
