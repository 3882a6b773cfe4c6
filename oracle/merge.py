"""fp64 models of merging attention over disjoint key partitions (test
infrastructure).

Sources:
  * FlashAttention from Scratch (ryhuang.blog), §4.3 "Merge independently
    computed partitions": states (m_A, l_A, u_A), (m_B, l_B, u_B) of disjoint
    key sets combine as m = max(m_A, m_B), l = e^{m_A-m} l_A + e^{m_B-m} l_B,
    u = e^{m_A-m} u_A + e^{m_B-m} u_B; any merge tree gives the same exact
    result.  With normalised outputs and natural-log normalisers
    L = log sum e^{s}: L = logaddexp(L_A, L_B) and
    O = e^{L_A-L} O_A + e^{L_B-L} O_B; a row empty in both stays empty;
  * §9.1 "Split the long dimension that remains": split-KV decoding computes
    one partial (O_s, L_s) per KV partition and reduces them with that merge;
  * §4.4: the empty state is m = -inf, l = 0, u = 0, finishing to O = 0 and
    LSE = -inf.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def partition_state(q, k, v, scale, causal=False, q_pos=None, k_pos=None):
    """State (m, l, u) of every query row over one key subset (§4.1's
    definitions: m = max s, l = sum e^{s-m}, u = sum e^{s-m} v)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    Lq, Lk, Dv = q.shape[0], k.shape[0], v.shape[1]
    if Lk == 0:
        return np.full(Lq, -np.inf), np.zeros(Lq), np.zeros((Lq, Dv))
    q_pos = np.arange(Lq) if q_pos is None else np.asarray(q_pos)
    k_pos = np.arange(Lk) if k_pos is None else np.asarray(k_pos)
    s = scale * (q @ k.T)
    if causal:
        s[k_pos[None, :] > q_pos[:, None]] = -np.inf
    m = s.max(axis=1)
    base = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(s - base[:, None])
    return m, w.sum(axis=1), w @ v


def merge_states(a, b):
    """Merge two partition states (§4.3, first form)."""
    ma, la, ua = a
    mb, lb, ub = b
    m = np.maximum(ma, mb)
    base = np.where(np.isfinite(m), m, 0.0)
    wa = np.exp(ma - base)
    wb = np.exp(mb - base)
    return m, wa * la + wb * lb, wa[:, None] * ua + wb[:, None] * ub


def finish_state(state):
    """(O, LSE) from a state: O = u / l and LSE = m + log l, or (0, -inf) for
    a row with no key (§4.4 convention)."""
    m, ell, u = state
    ok = ell > 0
    safe = np.where(ok, ell, 1.0)
    out = np.where(ok[:, None], u / safe[:, None], 0.0)
    return out, np.where(ok, m + np.log(safe), -np.inf)


def merge_normalized(oa, la, ob, lb):
    """Merge normalised partials by their natural-log normalisers (§4.3,
    second form; §9.1)."""
    oa, la, ob, lb = _f64(oa), _f64(la), _f64(ob), _f64(lb)
    L = np.logaddexp(la, lb)
    base = np.where(np.isfinite(L), L, 0.0)
    wa = np.exp(la - base)
    wb = np.exp(lb - base)
    return wa[:, None] * oa + wb[:, None] * ob, L
