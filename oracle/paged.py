"""Attention over a paged KV cache, in fp64 (test infrastructure).

Sources:
  * FlashAttention from Scratch (ryhuang.blog), §9.3 "Paging changes where
    keys live": a sequence's cache is a list of fixed-size pages instead of
    one contiguous buffer; with page size P, logical token t of sequence b is
    stored in the physical page that b's page table lists at entry
    floor(t / P), at row t mod P of that page.  (The page's formula is lost
    in extraction; this is the plain reading of the text around it.)  Paging
    changes where keys live, not what attention computes: the result is the
    attention of §2 over the logical sequence, which is how this module
    evaluates it (gather the logical rows, then ``attention.dense_head``).
  * The same section's experiment: permuting the physical pages while the
    page table follows them must leave every output unchanged.

Layout (the library's paged layout, stated here so the two can be compared):
  k_cache, v_cache : [num_pages, Hkv, P, D] -- each page holds P consecutive
                     tokens of every KV head, one head's rows contiguous;
  page_table       : [B, max_pages] integers;
  kv_lens          : [B], the number of valid logical tokens of each
                     sequence, clamped to [0, max_pages * P].
Convention (not from the pages): a table entry outside [0, num_pages) holds
no keys -- its tokens are masked but keep their logical positions for the
causal and window masks.  Entries past the last valid token are never read.
"""
from __future__ import annotations

import numpy as np

from .attention import as_f64, dense_head


def gather_sequence(cache, page_table, b, n, page_size):
    """Logical rows 0..n-1 of sequence b that live in valid pages.

    Returns (rows [Hkv, m, D] fp64, positions [m]) where positions are the
    logical token indices of the m gathered rows, in increasing order.
    """
    cache = as_f64(cache)
    table = np.asarray(as_f64(page_table), dtype=np.int64)
    num_pages, hkv, _, d = cache.shape
    rows, positions = [], []
    for t in range(n):
        page = table[b, t // page_size]
        if page < 0 or page >= num_pages:
            continue
        rows.append(cache[page, :, t % page_size, :])
        positions.append(t)
    if not rows:
        return np.zeros((hkv, 0, d)), np.zeros(0, dtype=np.int64)
    return np.stack(rows, axis=1), np.asarray(positions, dtype=np.int64)


def paged_attention_forward(q, k_cache, v_cache, page_table, kv_lens, page_size, scale,
                            causal=False, window=0):
    """O [B, Hq, Lq, Dv] and LSE [B, Hq, Lq] (fp64) of attention against a
    paged cache.  Queries of sequence b sit at logical positions
    n_b - Lq + i (bottom-right alignment, as for a contiguous cache)."""
    q = as_f64(q)
    B, Hq, Lq = q.shape[0], q.shape[1], q.shape[2]
    Hkv = k_cache.shape[1]
    Dv = v_cache.shape[3]
    assert Hq % Hkv == 0, "query heads must be a multiple of KV heads"
    r = Hq // Hkv
    lens = as_f64(kv_lens)
    capacity = page_table.shape[1] * page_size
    O = np.zeros((B, Hq, Lq, Dv))
    lse = np.zeros((B, Hq, Lq))
    for b in range(B):
        n = int(min(max(int(lens[b]), 0), capacity))
        kb, kpos = gather_sequence(k_cache, page_table, b, n, page_size)
        vb, _ = gather_sequence(v_cache, page_table, b, n, page_size)
        q_pos = (n - Lq) + np.arange(Lq)
        for h in range(Hq):
            g = h // r
            O[b, h], lse[b, h] = dense_head(q[b, h], kb[g], vb[g], scale, causal,
                                            q_pos, kpos, window)
    return O, lse
