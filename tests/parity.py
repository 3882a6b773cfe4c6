"""Comparison of GPU outputs with the fp64 oracle (test infrastructure).

Forward bar (the stated tolerances, for the bf16 output O and the fp32 LSE):
  * max-abs |O_gpu - O_ref| <= 1e-2 on EVERY compared element;
  * relative L2 ||O_gpu - O_ref|| / ||O_ref|| <= 4e-3 over the whole tensor;
  * max |LSE_gpu - LSE_ref| <= 1e-3 over rows with a finite reference LSE;
  * a row with no allowed key must give exactly O = 0 and LSE = -inf;
  * no NaN anywhere.
The one exception is an element the bar cannot be met at by ANY bf16 value:
for |O_ref| >= 4 the bf16 spacing is 2^-5, and where O_ref lies more than
1e-2 from both of its bf16 neighbours (``floor_over_1e-2`` counts them:
|bf16(O_ref) - O_ref| > 1e-2) no bf16 output is within 1e-2.  There the
output must be one of those two neighbours (error below one bf16 spacing of
O_ref), and the count is reported as ``unrepresentable``; everywhere else the
1e-2 bar holds as stated, and ``max_abs_representable`` reports the largest
error over those elements.  The seeded long-context GQA workload has two such
elements (its x4 heads give |O| up to 4.3); no other workload has any.
``bf16_floor_max`` = max |bf16(O_ref) - O_ref| is reported beside max-abs.

Variant bar (``compare(..., pbound=...)``), used only for the causal window,
the score modifiers and random shapes of those paths, where rows may be
dominated by a few keys.  The kernels round each probability to bf16 before
the PV product and normalise by the sum of the rounded values.  With
p~_j = p_j (1 + e_j), |e_j| <= u = 2^-8 (round to nearest, 8 significant
bits) and sum_j P_j (v_j - O) = 0,
    O_fp32 - O = sum_j P_j e_j (v_j - O) / (1 + sum_j P_j e_j),
so |O_fp32 - O| <= u / (1 - u) * A with A = sum_j P_j |v_j - O| per element,
and the bf16 output adds at most half a bf16 spacing of O_fp32.  An element
above 1e-2 passes on these paths only when its error is within
    1.0040 * 2^-8 * A + half_spacing(|O_ref| + 2^-8 A) + 2e-4
(the last term covers the fp32 scores, exponentials and accumulation), with A
computed from the oracle's own P for exactly those elements.  The count of
such elements is reported (``pbound``).  Relative L2, LSE and empty-row
checks are unchanged.
"""
from __future__ import annotations

import math

import numpy as np
import torch

MAX_ABS = 1e-2
REL_L2 = 4e-3
MAX_DLSE = 1e-3
U_BF16 = 2.0 ** -8          # unit roundoff of bf16 (8 significant bits)

# Metrics of named comparisons, collected for the end-of-session summary
# (tests/conftest.py prints them as JSON lines, which survive ``pytest -q``).
RECORDED: dict = {}


def record(name: str, metrics: dict) -> None:
    RECORDED[name] = metrics


def bf16_half_spacing(x: np.ndarray) -> np.ndarray:
    """Half the distance between adjacent bf16 numbers at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float64).tiny)
    e = np.floor(np.log2(ax))
    return 0.5 * np.exp2(e - 7)


def pbound_limit(ref_o: np.ndarray, spread: np.ndarray) -> np.ndarray:
    """Per-element error bound of the bf16-probability arithmetic (module doc)."""
    return (1.0040 * U_BF16 * spread + bf16_half_spacing(np.abs(ref_o) + U_BF16 * spread) + 2e-4)


def _np64(x):
    if hasattr(x, "detach"):
        return x.detach().float().cpu().numpy().astype(np.float64)
    return np.asarray(x, np.float64)


class Stats:
    """Accumulates the forward bar over chunks of a large comparison.

    ``add`` takes chunks shaped [..., L, D] / [..., L] plus a label for the
    (b, h) they belong to; ``finish`` asserts the bar and returns the metrics,
    including the worst (b, h) by max-abs and by relative L2.
    """

    def __init__(self, variant: bool = False):
        self.variant = variant          # False: the strict forward bar; True: the variant bar
        self.max_abs = 0.0
        self.err2 = 0.0
        self.ref2 = 0.0
        self.dlse = 0.0
        self.floor_max = 0.0
        self.floor_over = 0
        self.over = 0
        self.unrep = 0
        self.max_abs_rep = 0.0
        self.pbound_count = 0
        self.elements = 0
        self.empty_rows = 0
        self.rows = 0
        self.per_bh: dict = {}
        self.failures: list = []

    def add(self, go, gl, ro, rl, bh=None, spread=None):
        """Compare one chunk.  On the variant bar ``spread`` is a callable that
        takes flat element indices of the chunk's O (only those above 1e-2)
        and returns A = sum_j P_j |v_j - O| for each."""
        go, gl, ro, rl = _np64(go), _np64(gl), np.asarray(ro, np.float64), np.asarray(rl, np.float64)
        assert go.shape == ro.shape and gl.shape == rl.shape, (go.shape, ro.shape, gl.shape, rl.shape)
        if np.isnan(go).any():
            self.failures.append(f"NaN in O at {bh}")
        if np.isnan(gl).any():
            self.failures.append(f"NaN in LSE at {bh}")
        empty = ~np.isfinite(rl)
        if not np.all(gl[empty] == -np.inf):
            self.failures.append(f"an empty row did not get LSE = -inf at {bh}")
        if not np.all(go[empty] == 0.0):
            self.failures.append(f"an empty row did not get O = 0 at {bh}")
        if not np.all(np.isfinite(gl[~empty])):
            self.failures.append(f"a non-empty row got a non-finite LSE at {bh}")
        err = np.abs(go - ro)
        e2 = float(np.sum((go - ro) ** 2))
        r2 = float(np.sum(ro ** 2))
        mx = float(err.max()) if err.size else 0.0
        self.max_abs = max(self.max_abs, mx)
        self.err2 += e2
        self.ref2 += r2
        if (~empty).any():
            self.dlse = max(self.dlse, float(np.abs(gl[~empty] - rl[~empty]).max()))
        floor = np.abs(torch.from_numpy(np.ascontiguousarray(ro)).to(torch.bfloat16).double().numpy() - ro)
        if floor.size:
            self.floor_max = max(self.floor_max, float(floor.max()))
        unrep = floor > MAX_ABS               # no bf16 value lies within 1e-2 of O_ref
        self.floor_over += int(unrep.sum())
        if unrep.any():
            # one of the two bf16 neighbours of O_ref: within one spacing of it
            near = err[unrep] < 2.0 * bf16_half_spacing(ro[unrep])
            self.unrep += int(unrep.sum())
            if not near.all():
                self.failures.append(f"an element with no bf16 value within 1e-2 of O_ref is not one of "
                                     f"its bf16 neighbours at {bh}")
        rep_err = err[~unrep]
        if rep_err.size:
            self.max_abs_rep = max(self.max_abs_rep, float(rep_err.max()))
        over = (err > MAX_ABS) & ~unrep
        n_over = int(over.sum())
        self.over += n_over
        if n_over:
            if not self.variant or spread is None:
                self.failures.append(f"max-abs {float(err[over].max()):.5g} above {MAX_ABS} at {bh} "
                                     f"({n_over} elements)")
            else:
                idx = np.flatnonzero(over)
                a = np.asarray(spread(idx), np.float64)
                lim = pbound_limit(ro.reshape(-1)[idx], a)
                bad = err.reshape(-1)[idx] > lim
                self.pbound_count += int((~bad).sum())
                if bad.any():
                    j = int(np.flatnonzero(bad)[0])
                    self.failures.append(
                        f"error {err.reshape(-1)[idx[j]]:.5g} above 1e-2 and above the bf16-P bound "
                        f"{lim[j]:.5g} (A = {a[j]:.4g}) at {bh}")
        self.elements += int(err.size)
        self.empty_rows += int(empty.sum())
        self.rows += int(rl.size)
        if bh is not None:
            a = self.per_bh.setdefault(bh, [0.0, 0.0, 0.0])
            a[0] = max(a[0], mx)
            a[1] += e2
            a[2] += r2
        return self

    def metrics(self) -> dict:
        rel = math.sqrt(self.err2 / self.ref2) if self.ref2 > 0 else math.sqrt(self.err2)
        m = {
            "max_abs": self.max_abs, "rel_l2": rel, "max_dlse": self.dlse,
            "max_abs_representable": self.max_abs_rep,
            "bf16_floor_max": self.floor_max, "floor_over_1e-2": self.floor_over,
            "unrepresentable": self.unrep, "over_1e-2": self.over, "elements": self.elements, "rows": self.rows,
            "empty_rows": self.empty_rows,
        }
        if self.variant:
            m["pbound"] = self.pbound_count
        if self.per_bh:
            wa = max(self.per_bh.items(), key=lambda kv: kv[1][0])
            wr = max(self.per_bh.items(),
                     key=lambda kv: math.sqrt(kv[1][1] / kv[1][2]) if kv[1][2] > 0 else 0.0)
            m["worst_bh_max_abs"] = [list(wa[0]), wa[1][0]]
            m["worst_bh_rel_l2"] = [list(wr[0]),
                                    math.sqrt(wr[1][1] / wr[1][2]) if wr[1][2] > 0 else 0.0]
        return m

    def finish(self, name: str | None = None) -> dict:
        m = self.metrics()
        if name is not None:
            record(name, m)
        assert not self.failures, f"{self.failures[:5]}; {m}"
        assert m["rel_l2"] <= REL_L2, f"relative L2 above {REL_L2}: {m}"
        assert m["max_dlse"] <= MAX_DLSE, f"|dLSE| above {MAX_DLSE}: {m}"
        return m


def compare(got_o, got_lse, ref_o, ref_lse, name: str | None = None, spread=None):
    """Return a metrics dict; raise AssertionError when the bar fails.

    Strict forward bar by default.  With ``spread`` (the variant bar, see the
    module docstring) a callable that receives the flat indices of the
    elements of O above 1e-2 and returns A = sum_j P_j |v_j - O| for each.
    ``variant_spread`` builds it for a batched problem.
    """
    return Stats(variant=spread is not None).add(got_o, got_lse, ref_o, ref_lse,
                                                spread=spread).finish(name)


def variant_spread(case, rows=None, window: int = 0, alibi_slopes=None, softcap: float = 0.0,
                   q=None, k=None):
    """The ``spread`` callable of ``compare`` for O of shape [B, Hq, len(rows), D]
    (all rows when ``rows`` is None): A = sum_j P_j |v_j - O| from the
    oracle's P of the element's row.  ``q``/``k`` replace the case's Q/K (the
    FP8 path compares against the attention of the dequantized values)."""
    import oracle

    qq = case.q if q is None else q
    kk = case.k if k is None else k
    B, Hq, Lq, D = qq.shape
    rows = np.arange(Lq) if rows is None else np.asarray(rows, np.int64)
    nr = rows.size

    def fn(idx):
        out = []
        for i in np.asarray(idx, np.int64):
            d = int(i % D); rest = int(i // D)
            ri = rest % nr; rest //= nr
            h = rest % Hq; b = rest // Hq
            ro, _, P, vv = oracle.attention_rows(qq, kk, case.v, case.scale, case.causal, case.kv_lens,
                                                 b, h, rows[ri:ri + 1], window=window,
                                                 alibi_slopes=alibi_slopes, softcap=softcap,
                                                 return_weights=True)
            out.append(float(np.sum(P[0] * np.abs(vv[:, d] - ro[0, d]))))
        return out
    return fn


def sample_rows(Lq: int, seed: int, block: int = 256, wave: int = 32, extra: int = 64):
    """Rows to check on a full-size problem: both ends, the rows on each side
    of every ``block`` boundary (the prefill workgroup's query block) and of
    every ``wave`` boundary inside every block (a wavefront's 32 rows), and
    seeded random rows.  Every (query block, wavefront) slot is covered."""
    rows = set(range(min(Lq, 40))) | set(range(max(0, Lq - 40), Lq))
    for b0 in range(0, Lq, block):
        rows |= {b0 - 1, b0}
        for w0 in range(b0 + wave, min(b0 + block, Lq), wave):
            rows |= {w0 - 1, w0}
    r = np.random.default_rng(seed)
    rows |= set(int(x) for x in r.integers(0, Lq, extra))
    return np.array(sorted(x for x in rows if 0 <= x < Lq), dtype=np.int64)


def host_threads() -> int:
    """Threads for host-side oracle work: the cores this process may run on,
    at most 16 (a GPU machine's CPU share)."""
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def compare_all_rows(case, got_o, got_lse, name: str | None = None, chunk: int = 512,
                     window: int = 0, alibi_slopes=None, softcap: float = 0.0, pbound: bool = False,
                     heads=None):
    """Compare EVERY query row of every (b, h) (or of the listed ``heads``)
    with the oracle, in row chunks evaluated on a thread pool (numpy releases
    the interpreter lock in its matrix products and elementwise loops; BLAS is
    held to one thread per worker).  Each chunk is compared as soon as the
    oracle has produced it, so the full fp64 output never has to be held."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover - threadpoolctl is part of the image
        threadpool_limits = None
    B, Hq, Lq = case.q.shape[0], case.q.shape[1], case.q.shape[2]
    go = got_o.detach().cpu() if hasattr(got_o, "detach") else got_o
    gl = got_lse.detach().cpu() if hasattr(got_lse, "detach") else got_lse
    heads = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else list(heads)
    tasks = [(b, h, r0, min(r0 + chunk, Lq)) for (b, h) in heads for r0 in range(0, Lq, chunk)]

    def work(t):
        b, h, r0, r1 = t
        rows = np.arange(r0, r1)
        ro, rl = oracle.attention_rows(case.q, case.k, case.v, case.scale, case.causal, case.kv_lens,
                                       b, h, rows, window=window, alibi_slopes=alibi_slopes,
                                       softcap=softcap, trim_keys=True)
        return t, ro, rl

    st = Stats(variant=pbound)
    ctx = threadpool_limits(limits=1, user_api="blas") if threadpool_limits else None
    try:
        with ThreadPoolExecutor(max_workers=host_threads()) as ex:
            for (b, h, r0, r1), ro, rl in ex.map(work, tasks):
                spread = None
                if pbound:
                    one = variant_spread(case, rows=np.arange(r0, r1), window=window,
                                         alibi_slopes=alibi_slopes, softcap=softcap)
                    nr = r1 - r0
                    D = case.q.shape[3]
                    # flat index of the chunk [nr, D] -> flat index in a [B, Hq, nr, D] view
                    spread = (lambda f, b=b, h=h, nr=nr, D=D:
                              lambda idx: f([((b * Hq + h) * nr) * D + int(i) for i in idx]))(one)
                st.add(go[b, h, r0:r1], gl[b, h, r0:r1], ro, rl, bh=(b, h), spread=spread)
    finally:
        if ctx is not None:
            ctx.restore_original_limits()
    return st.finish(name)


def compare_varlen(case, got_o, got_lse, name: str | None = None, chunk: int = 512, sequences=None):
    """Compare EVERY query row of every head of the packed batch's sequences
    (or of the listed ``sequences``) with the oracle, on the strict bar.
    Sequence b is taken as a batch of one (``oracle.varlen.sequence_view``)
    and its rows evaluated in chunks by ``oracle.attention_rows`` on a thread
    pool, as in ``compare_all_rows``.  got_o [Hq, total_q, D], got_lse
    [Hq, total_q]."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover - threadpoolctl is part of the image
        threadpool_limits = None
    cq, ck = case.meta["cu_seqlens_q"], case.meta["cu_seqlens_k"]
    B = cq.numel() - 1
    Hq = case.q.shape[0]
    go = got_o.detach().cpu() if hasattr(got_o, "detach") else got_o
    gl = got_lse.detach().cpu() if hasattr(got_lse, "detach") else got_lse
    seqs = list(range(B)) if sequences is None else list(sequences)
    views = {b: oracle.varlen.sequence_view(case.q, case.k, case.v, cq, ck, b) for b in seqs}
    tasks = [(b, h, r0, min(r0 + chunk, views[b][0].shape[2]))
             for b in seqs for h in range(Hq) for r0 in range(0, views[b][0].shape[2], chunk)]

    def work(t):
        b, h, r0, r1 = t
        qb, kb, vb = views[b]
        ro, rl = oracle.attention_rows(qb, kb, vb, case.scale, case.causal, None, 0, h, np.arange(r0, r1),
                                       trim_keys=True)
        return t, ro, rl

    st = Stats()
    ctx = threadpool_limits(limits=1, user_api="blas") if threadpool_limits else None
    try:
        with ThreadPoolExecutor(max_workers=host_threads()) as ex:
            for (b, h, r0, r1), ro, rl in ex.map(work, tasks):
                s0 = int(cq[b])
                st.add(go[h, s0 + r0:s0 + r1], gl[h, s0 + r0:s0 + r1], ro, rl, bh=(b, h))
    finally:
        if ctx is not None:
            ctx.restore_original_limits()
    return st.finish(name)
