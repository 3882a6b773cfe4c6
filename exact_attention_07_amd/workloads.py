"""Seeded synthetic workloads and work accounting for the attention forward.

This module draws inputs and counts work; it performs none of the attention
arithmetic, so both the fp64 oracle tests and the GPU path take their inputs
from here without sharing any of the method's code.

Workload shapes follow the FlashAttention Cheat Sheet, §1 "The whole
operation" (Q is [B, Hq, Lq, D], K and V are [B, Hkv, Lk, D]) and the shape
family of the FlashAttention-4 benchmark summarised in "FlashAttention-4:
Blackwell Attention Kernel Co-Design", "How we know: Blackwell benchmarks and
ablations" (bf16, sequence lengths 1K-32K, head dimensions 64 and 128, causal
and non-causal).  Inputs are iid N(0, 1) drawn in fp32 and rounded to bf16,
the illustrative assumption of FlashAttention from Scratch, §2 ("Why divide by
sqrt d?").

Generation recipe (fixed; never changed to make a comparison pass):
  * a torch CPU generator seeded with ``1000 + config index``;
  * Q, K, V drawn in that order with ``torch.randn`` in fp32, then cast to
    bf16 (round to nearest even);
  * the long-context GQA workload multiplies Q on every head h with
    h % 8 == 0 by 4 (exact in bf16) so that large row maxima arrive late;
  * the decode workload then draws ``kv_lens`` uniformly in [512, 8192] with
    ``torch.randint(512, 8193)``; K and V are allocated at the full capacity
    of 8192 rows per sequence and only the first ``kv_lens[b]`` are valid.
  * the packed variable-length workload first draws its B sequence lengths
    uniformly in [128, 8192] (``torch.randint(128, 8193)``, the same length
    for queries and keys: self-attention over packed documents), then Q
    [Hq, total, D], K and V [Hkv, total, D] as above; the offsets are the
    running sums of the lengths.

Follow-on workloads reuse the draws of a base workload (its seed index) and
change one thing: a causal window (FlashAttention from Scratch, §12) or a
paged cache layout (§9.3).  ``page_kv`` scatters contiguous K and V into a
page pool through a seeded random page table; it moves rows and computes
nothing.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Lq: int
    Lk: int
    D: int
    causal: bool
    index: int
    q_boost_every: int = 0      # multiply Q by q_boost on heads h % q_boost_every == 0
    q_boost: float = 1.0
    ragged: Optional[tuple] = None  # (lo, hi) inclusive range of kv_lens, else None
    description: str = ""
    window: int = 0             # causal window width (0 = none)
    page_size: int = 0          # > 0: K and V are served from a paged cache
    backward: bool = False      # time the backward (fa_bwd) instead of the forward
    fp8: bool = False           # FP8 scores: Q, K block-quantized after the random-sign Hadamard transform
    alibi: bool = False         # ALiBi score modifier, slopes 2^(-8 (h + 1) / Hq)
    softcap: float = 0.0        # soft-cap score modifier (0 = none)
    varlen: Optional[tuple] = None  # (lo, hi): B packed sequences, lengths uniform in [lo, hi]

    @property
    def seed(self) -> int:
        return 1000 + self.index

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


WORKLOADS = [
    Workload("tiny_b1_h2_l256_d64", 1, 2, 2, 256, 256, 64, False, 0,
             description="tiny exact-attention forward, non-causal"),
    Workload("prefill_b4_h16_l1024_d64", 4, 16, 16, 1024, 1024, 64, False, 1,
             description="prefill forward, no mask"),
    Workload("causal_b2_h16_l4096_d128", 2, 16, 16, 4096, 4096, 128, True, 2,
             description="causal prefill forward"),
    Workload("gqa_causal_b1_hq32_hkv8_l16384_d128", 1, 32, 8, 16384, 16384, 128, True, 3,
             q_boost_every=8, q_boost=4.0,
             description="long-context causal GQA forward, Q x4 on every 8th head"),
    Workload("decode_b64_hq32_hkv8_d128_ragged", 64, 32, 8, 1, 8192, 128, False, 4,
             ragged=(512, 8192),
             description="split-KV decode, ragged kv_lens in [512, 8192]"),
    # Follow-on variants (same draws as the base workload of the same index).
    Workload("gqa_window4096_b1_hq32_hkv8_l16384_d128", 1, 32, 8, 16384, 16384, 128, True, 3,
             q_boost_every=8, q_boost=4.0, window=4096,
             description="long-context GQA forward with a causal window of 4096 keys"),
    Workload("decode_paged16_b64_hq32_hkv8_d128_ragged", 64, 32, 8, 1, 8192, 128, False, 4,
             ragged=(512, 8192), page_size=16,
             description="split-KV decode from a paged cache (16-token pages, shuffled)"),
    Workload("bwd_causal_b2_h16_l4096_d128", 2, 16, 16, 4096, 4096, 128, True, 2, backward=True,
             description="backward of the causal prefill forward"),
    Workload("bwd_prefill_b4_h16_l1024_d64", 4, 16, 16, 1024, 1024, 64, False, 1, backward=True,
             description="backward of the prefill forward, no mask"),
    Workload("alibi_causal_b2_h16_l4096_d128", 2, 16, 16, 4096, 4096, 128, True, 2, alibi=True,
             description="causal prefill forward with ALiBi score biases"),
    Workload("softcap_prefill_b4_h16_l1024_d64", 4, 16, 16, 1024, 1024, 64, False, 1, softcap=20.0,
             description="prefill forward with soft-capped scores (cap 20)"),
    Workload("fp8_causal_b2_h16_l4096_d128", 2, 16, 16, 4096, 4096, 128, True, 2, fp8=True,
             description="causal prefill forward with FP8 scores (block scales, incoherent processing)"),
    Workload("fp8_gqa_causal_b1_hq32_hkv8_l16384_d128", 1, 32, 8, 16384, 16384, 128, True, 3,
             q_boost_every=8, q_boost=4.0, fp8=True,
             description="long-context causal GQA forward with FP8 scores"),
    # Packed variable-length batch: Lq and Lk are the largest possible length.
    Workload("varlen_causal_b16_hq32_hkv8_d128", 16, 32, 8, 8192, 8192, 128, True, 5,
             varlen=(128, 8192),
             description="causal GQA forward over 16 packed sequences of 128-8192 tokens"),
]
BY_NAME = {w.name: w for w in WORKLOADS}


@dataclass
class Inputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    kv_lens: Optional[torch.Tensor]
    scale: float
    causal: bool
    meta: dict = field(default_factory=dict)


def make_inputs(w: Workload) -> Inputs:
    """Draw the workload's inputs on the CPU (bf16 Q, K, V; int32 kv_lens)."""
    g = torch.Generator().manual_seed(w.seed)
    if w.varlen is not None:
        return _make_varlen(w, g)
    q = torch.randn(w.B, w.Hq, w.Lq, w.D, generator=g, dtype=torch.float32).to(torch.bfloat16)
    k = torch.randn(w.B, w.Hkv, w.Lk, w.D, generator=g, dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn(w.B, w.Hkv, w.Lk, w.D, generator=g, dtype=torch.float32).to(torch.bfloat16)
    if w.q_boost_every:
        q[:, ::w.q_boost_every] *= w.q_boost
    kv_lens = None
    if w.ragged is not None:
        lo, hi = w.ragged
        kv_lens = torch.randint(lo, hi + 1, (w.B,), generator=g, dtype=torch.int64).to(torch.int32)
    meta = {"workload": w.name, "seed": w.seed}
    if w.backward:
        # The upstream gradient dL/dO, drawn after the forward's inputs.
        meta["dout"] = torch.randn(w.B, w.Hq, w.Lq, w.D, generator=g,
                                   dtype=torch.float32).to(torch.bfloat16)
    if w.window:
        meta["window"] = w.window
    if w.alibi:
        # The geometric slopes of the ALiBi construction (not on the pages; a
        # synthetic choice), one per query head.
        meta["alibi_slopes"] = torch.tensor([2.0 ** (-8.0 * (h + 1) / w.Hq) for h in range(w.Hq)],
                                            dtype=torch.float32)
    if w.softcap:
        meta["softcap"] = w.softcap
    if w.fp8:
        # The random signs of the incoherent-processing transform, drawn after the base inputs.
        meta["signs"] = (torch.randint(0, 2, (w.D,), generator=g) * 2 - 1).to(torch.float32)
    if w.page_size:
        # The paged copy of the same K and V; the contiguous tensors stay for reference.
        meta["paged"] = page_kv(k, v, kv_lens, w.page_size, seed=w.seed + 7919)
    return Inputs(q, k, v, kv_lens, w.scale, w.causal, meta)


def _make_varlen(w: Workload, g: torch.Generator) -> Inputs:
    lo, hi = w.varlen
    lens = torch.randint(lo, hi + 1, (w.B,), generator=g, dtype=torch.int64)
    total = int(lens.sum())
    q = torch.randn(w.Hq, total, w.D, generator=g, dtype=torch.float32).to(torch.bfloat16)
    k = torch.randn(w.Hkv, total, w.D, generator=g, dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn(w.Hkv, total, w.D, generator=g, dtype=torch.float32).to(torch.bfloat16)
    cu = torch.zeros(w.B + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(lens, 0).to(torch.int32)
    meta = {"workload": w.name, "seed": w.seed, "cu_seqlens_q": cu, "cu_seqlens_k": cu.clone(),
            "lens_q": [int(x) for x in lens], "lens_k": [int(x) for x in lens]}
    return Inputs(q, k, v, None, w.scale, w.causal, meta)


def varlen_case(seed: int, lens_q, lens_k, Hq: int, Hkv: int, D: int, causal: bool = False,
                scale: Optional[float] = None) -> Inputs:
    """A seeded N(0,1) packed batch of arbitrary sequence lengths for parity
    tests: q [Hq, sum(lens_q), D], k and v [Hkv, sum(lens_k), D]."""
    g = torch.Generator().manual_seed(seed)
    tq, tk = int(sum(lens_q)), int(sum(lens_k))
    q = torch.randn(Hq, tq, D, generator=g).to(torch.bfloat16)
    k = torch.randn(Hkv, tk, D, generator=g).to(torch.bfloat16)
    v = torch.randn(Hkv, tk, D, generator=g).to(torch.bfloat16)
    cq = torch.zeros(len(lens_q) + 1, dtype=torch.int32)
    ck = torch.zeros(len(lens_k) + 1, dtype=torch.int32)
    cq[1:] = torch.cumsum(torch.tensor(list(lens_q), dtype=torch.int64), 0).to(torch.int32)
    ck[1:] = torch.cumsum(torch.tensor(list(lens_k), dtype=torch.int64), 0).to(torch.int32)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    return Inputs(q, k, v, None, scale, causal, {"seed": seed, "cu_seqlens_q": cq, "cu_seqlens_k": ck,
                                                 "lens_q": list(lens_q), "lens_k": list(lens_k)})


def page_kv(k: torch.Tensor, v: torch.Tensor, kv_lens, page_size: int, seed: int,
            spare_pages: int = 7, fill: float = float("nan")):
    """Scatter contiguous K, V [B, Hkv, Lk, D] into a page pool.

    Returns (k_cache, v_cache, page_table): caches [num_pages, Hkv, P, D] of
    k's dtype, table int32 [B, ceil(Lk / P)].  Sequence b's first kv_lens[b]
    tokens go, page by page, to physical pages in a seeded random order; the
    pool has ``spare_pages`` more pages than needed.  Unused pages and the
    tail of each sequence's last page hold ``fill``; table entries past a
    sequence's last page point at random pages of the pool (never meant to be
    read).
    """
    B, Hkv, Lk, D = k.shape
    lens = [Lk] * B if kv_lens is None else [min(max(int(x), 0), Lk) for x in kv_lens]
    max_pages = max(1, -(-Lk // page_size))
    need = [-(-n // page_size) for n in lens]
    num_pages = sum(need) + spare_pages
    g = torch.Generator().manual_seed(seed)
    order = torch.randperm(num_pages, generator=g)
    table = torch.randint(0, num_pages, (B, max_pages), generator=g, dtype=torch.int64)
    kc = torch.full((num_pages, Hkv, page_size, D), fill, dtype=torch.float32).to(k.dtype)
    vc = torch.full((num_pages, Hkv, page_size, D), fill, dtype=torch.float32).to(v.dtype)
    nxt = 0
    for b in range(B):
        m, n = need[b], lens[b]
        if m == 0:
            continue
        pages = order[nxt:nxt + m]
        nxt += m
        table[b, :m] = pages
        for src, dst in ((k, kc), (v, vc)):
            rows = torch.full((Hkv, m * page_size, D), fill, dtype=torch.float32).to(src.dtype)
            rows[:, :n] = src[b, :, :n]
            dst[pages] = rows.view(Hkv, m, page_size, D).transpose(0, 1)
    return kc, vc, table.to(torch.int32)


def random_case(seed: int, B: int, Hq: int, Hkv: int, Lq: int, Lk: int, D: int,
                causal: bool = False, kv_lens=None, scale: Optional[float] = None,
                q_mult: float = 1.0, k_mult: float = 1.0) -> Inputs:
    """A seeded N(0,1) case of arbitrary shape for parity tests.

    ``kv_lens`` may be None, a list of ints, or the string "ragged" (drawn
    uniformly in [0, Lk] after Q, K, V from the same generator).
    """
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn(B, Hq, Lq, D, generator=g) * q_mult).to(torch.bfloat16)
    k = (torch.randn(B, Hkv, Lk, D, generator=g) * k_mult).to(torch.bfloat16)
    v = torch.randn(B, Hkv, Lk, D, generator=g).to(torch.bfloat16)
    if isinstance(kv_lens, str) and kv_lens == "ragged":
        kv_lens = torch.randint(0, Lk + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)
    elif kv_lens is not None:
        kv_lens = torch.tensor(list(kv_lens), dtype=torch.int32)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return Inputs(q, k, v, kv_lens, scale, causal, {"seed": seed})


# ---------------------------------------------------------------------------
# Work accounting (algorithmic FLOPs and compulsory bytes)
# ---------------------------------------------------------------------------

def valid_lengths(w_or_shape, kv_lens=None):
    """Per-sequence valid key counts n_b (kv_lens clamped to [0, Lk], else Lk)."""
    B, Lk = w_or_shape.B, w_or_shape.Lk
    if kv_lens is None:
        return [Lk] * B
    return [min(max(int(x), 0), Lk) for x in kv_lens]


def allowed_pairs(Lq: int, n: int, causal: bool, window: int = 0) -> int:
    """Number of allowed (query, key) pairs in one head.

    Causal masking is bottom-right aligned: query i sits at absolute position
    n - Lq + i and sees keys j <= that position (FlashAttention from Scratch,
    §5 "Rectangular causal masking is a correctness issue"); a causal window
    of width w also drops keys j <= position - w (§12).
    """
    if not causal and window <= 0:
        return Lq * n
    tot = 0
    off = n - Lq
    # rows with position p = off + i see keys max(0, p - w + 1) .. min(p, n - 1)
    for i in range(Lq):
        p = off + i
        hi = min(p + 1, n)
        lo = max(p - window + 1, 0) if window > 0 else 0
        tot += max(hi - lo, 0)
    return tot


def algorithmic_flops(w, kv_lens=None, lens=None) -> int:
    """4 * D FLOPs per allowed pair for the forward: two matrix products with
    multiply and add counted separately (FlashAttention from Scratch, §11.1
    counts 4MNd per tile); 10 * D for the backward's five products (§8).
    A packed batch passes its (Lq_b, Lk_b) pairs as ``lens``."""
    if lens is not None:
        return sum(4 * w.D * allowed_pairs(lq, lk, w.causal) * w.Hq for lq, lk in lens)
    ns = valid_lengths(w, kv_lens)
    per_pair = 10 * w.D if w.backward else 4 * w.D
    return sum(per_pair * allowed_pairs(w.Lq, n, w.causal, w.window) * w.Hq for n in ns)


def compulsory_bytes(w, kv_lens=None, lens=None) -> int:
    """Bytes that must cross HBM once: Q read, the K and V rows some query can
    see read once per KV head, O written (bf16) and the LSE written (fp32);
    with a paged cache also the page-table entries of those rows (int32);
    with FP8 scores Q and K are one byte per element plus their block scales.
    A packed batch passes its (Lq_b, Lk_b) pairs as ``lens`` (plus its two
    offset arrays, int32)."""
    if lens is not None:
        total = 0
        for lq, lk in lens:
            # every key of a sequence is seen by its last query (bottom-right
            # alignment), unless the sequence has no query at all
            seen = lk if lq > 0 else 0
            total += 2 * w.Hq * lq * w.D * 2 + w.Hq * lq * 4 + 2 * w.Hkv * seen * w.D * 2
        return total + 2 * 4 * (len(lens) + 1)
    ns = valid_lengths(w, kv_lens)
    if w.fp8:
        q = w.B * w.Hq * w.Lq * w.D + w.B * w.Hq * -(-w.Lq // 256) * 4
        o = w.B * w.Hq * w.Lq * w.D * 2
        kv = sum(w.Hkv * n * w.D * (1 + 2) + w.Hkv * -(-n // 64) * 4 for n in ns)
        return q + o + w.B * w.Hq * w.Lq * 4 + kv
    qo = 2 * w.B * w.Hq * w.Lq * w.D * 2
    lse = w.B * w.Hq * w.Lq * 4
    seen = [min(n, w.window + w.Lq - 1) if w.window > 0 else n for n in ns]
    kv = sum(2 * w.Hkv * m * w.D * 2 for m in seen)
    table = sum(4 * -(-n // w.page_size) for n in ns) if w.page_size > 0 else 0
    if w.backward:
        # Reads Q, O, dO and the LSE, K and V; writes dQ, dK and dV.
        return 2 * qo + lse + 2 * kv
    return qo + lse + kv + table


def paper_tiled_traffic_bytes(N: int, d: int, tile: int, elem_bytes: int = 2) -> int:
    """Forward HBM traffic of the tiled schedule for one head: Q read once, O
    written once, K and V re-read N / tile times, i.e. 2Nd + 2N^2 d / tile
    numbers (FlashAttention visualisation, giaicuuthegioi.com, "Tiling: one S
    tile at a time")."""
    return (2 * N * d + 2 * N * N * d // tile) * elem_bytes


def paper_naive_traffic_bytes(N: int, d: int, elem_bytes: int = 2) -> int:
    """Three-kernel materialised attention: 4N^2 + 4Nd numbers in total
    (same page, "Naive attention: three kernels" table)."""
    return (4 * N * N + 4 * N * d) * elem_bytes


def paper_tile_live_numbers(tile: int, d: int) -> int:
    """On-chip numbers live for one tile: Q, K, V, O tiles (4Bd), the S tile
    (B^2) and m, l (2B) (same page, "Tile size and SRAM")."""
    return 4 * tile * d + tile * tile + 2 * tile
