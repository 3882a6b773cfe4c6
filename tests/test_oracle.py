"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Every pin is a ``check_*`` function of an oracle namespace, so the same pins
run against the real oracle (the ordinary tests) and against copies of it
with a plausible mistake planted on the CPU (``test_pins_catch_mutants``),
which shows that a dropped term, a wrong sign, index or alignment, or a
transposed operand anywhere in the oracle fails at least one pin.

Pins used (none of them retypes the oracle's own formula):
  * values the pages print: the worked row (FlashAttention from Scratch,
    §2 and §4.2), the two-tile example (FlashAttention Cheat Sheet, §6), the
    rectangular causal mask table (FlashAttention from Scratch, §5);
  * the page's own fp64 experiments re-derived with the same seeds and
    shapes (§5 streaming vs dense, §9.1 split-KV merge);
  * invariances the pages state (+1000 shift, §2 checkpoint; tile size and
    tile order, Cheat Sheet §5; merge trees, §4.3);
  * closed forms (one key, identical keys, zero query, causal row 0);
  * brute force on tiny inputs: sum of e^s v over sum of e^s with no max
    shift, evaluated with math.fsum in pure Python;
  * a library routine: torch's CPU scaled_dot_product_attention in fp64 with
    an explicit boolean mask, GQA by repeating KV heads;
  * causal window (FlashAttention from Scratch, §12): width 1 returns each
    row's own value row, a window as long as the sequence is plain causal
    attention, and brute force over the allowed pairs;
  * paged KV (§9.3): through random page tables over NaN-filled pools the
    result equals the contiguous cache's; the section's own experiment
    (permute the physical pages, the table follows, the output stays
    identical); out-of-range entries against brute force;
  * variable-length packed batches: torch SDPA over the whole packed stream
    with a block-diagonal mask built here from the lengths, a single sequence
    against the batched definition, reordering the sequences, empty ones; the
    LPT order against a worked example and its defining properties.
"""
from __future__ import annotations

import itertools
import json
import math
import os
import types

import numpy as np
import pytest
import torch

import oracle as real_oracle

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden")
ORACLE_DIR = os.path.join(os.path.dirname(HERE), "oracle")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def oracle_namespace(mutations=()):
    """Load fresh copies of the oracle modules, optionally with textual
    mutations (module, old, new) applied, and expose their functions."""
    mods = {}
    for name in ("attention", "streaming", "merge", "paged", "backward", "fp8", "varlen"):
        path = os.path.join(ORACLE_DIR, name + ".py")
        with open(path) as f:
            src = f.read()
        for mname, old, new in mutations:
            if mname == name:
                assert old in src, f"mutation target not found in {name}.py: {old!r}"
                src = src.replace(old, new, 1)
        mod = types.ModuleType(f"_oracle_copy_{name}")
        if name == "paged":
            # The paged module evaluates through the (possibly mutated) copy
            # of the dense definition instead of the package's.
            imp = "from .attention import as_f64, dense_head\n"
            assert imp in src
            src = src.replace(imp, "")
            mod.as_f64, mod.dense_head = mods["attention"].as_f64, mods["attention"].dense_head
        if name == "varlen":
            imp = "from .attention import as_f64, dense_head\n"
            assert imp in src
            src = src.replace(imp, "")
            mod.as_f64, mod.dense_head = mods["attention"].as_f64, mods["attention"].dense_head
        if name == "backward":
            imp = "from .attention import as_f64\n"
            assert imp in src
            src = src.replace(imp, "")
            mod.as_f64 = mods["attention"].as_f64
        if name == "fp8":
            imp = "from .attention import as_f64, attention_forward\n"
            assert imp in src
            src = src.replace(imp, "")
            mod.as_f64, mod.attention_forward = mods["attention"].as_f64, mods["attention"].attention_forward
        exec(compile(src, path, "exec"), mod.__dict__)
        mods[name] = mod
    a, s, m, pg, bw, f8 = (mods["attention"], mods["streaming"], mods["merge"], mods["paged"],
                           mods["backward"], mods["fp8"])
    return types.SimpleNamespace(
        dense_head=a.dense_head, attention_forward=a.attention_forward,
        attention_rows=a.attention_rows, streaming_head=s.streaming_head,
        partition_state=m.partition_state, merge_states=m.merge_states,
        finish_state=m.finish_state, merge_normalized=m.merge_normalized,
        gather_sequence=pg.gather_sequence,
        paged_attention_forward=pg.paged_attention_forward,
        dense_backward_head=bw.dense_backward_head, attention_backward=bw.attention_backward,
        fp8=f8, varlen=mods["varlen"])


def row_inputs(scores, values):
    """One query whose scores against the keys are ``scores`` at scale 1:
    q = e0, k_j = s_j e0; scalar values v_j (Dv = 1)."""
    n = len(scores)
    q = np.zeros((1, 2))
    q[0, 0] = 1.0
    k = np.zeros((n, 2))
    k[:, 0] = scores
    v = np.asarray(values, dtype=np.float64).reshape(n, 1)
    return q, k, v


def rng_case(seed, Lq, Lk, D, Dv=None, mult=1.0):
    r = np.random.default_rng(seed)
    Dv = D if Dv is None else Dv
    return (r.standard_normal((Lq, D)) * mult, r.standard_normal((Lk, D)) * mult,
            r.standard_normal((Lk, Dv)))


def close(a, b, tol=1e-10):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    fin_a, fin_b = np.isfinite(a), np.isfinite(b)
    assert np.array_equal(fin_a, fin_b), "finite/non-finite pattern differs"
    assert np.array_equal(a[~fin_a], b[~fin_b]), "non-finite values differ"
    if fin_a.any():
        err = np.abs(a[fin_a] - b[fin_b])
        lim = tol * (1.0 + np.abs(b[fin_b]))
        assert np.all(err <= lim), f"max err {err.max():.3e}"


# ---------------------------------------------------------------------------
# The checks
# ---------------------------------------------------------------------------

def check_worked_row(orc):
    g = golden("worked_row.json")
    q, k, v = row_inputs(g["scores"], g["values"])
    out, lse = orc.dense_head(q, k, v, 1.0)
    assert abs(out[0, 0] - g["output"]["value"]) <= g["output"]["abs_tol"], out
    # LSE closed form, evaluated without any shift: log(e^1 + e^2 + e^3).
    assert abs(lse[0] - math.log(sum(math.exp(s) for s in g["scores"]))) < 1e-12
    # Streamed as [1, 2] then [3] (§4.2): alpha = e^-1 on the second tile.
    trace = []
    o2, l2 = orc.streaming_head(q, k, v, 1.0, block_q=1, block_k=2, trace=trace)
    assert len(trace) == 2
    t1, t2 = trace
    assert t1["m"][0] == 2.0
    assert abs(t1["ell"][0] - (1.0 + math.exp(-1.0))) < 1e-14          # e^{1-2} + e^{2-2}
    assert abs(t1["u"][0, 0] - (10.0 * math.exp(-1.0) + 20.0)) < 1e-12
    assert abs(t2["alpha"][0] - g["alpha_second_tile"]["value"]) < 1e-15
    assert abs(o2[0, 0] - g["output"]["value"]) <= g["output"]["abs_tol"]
    assert abs(l2[0] - lse[0]) < 1e-12


def check_shift_invariance(orc):
    g = golden("worked_row.json")
    c = g["shift_invariance_offset"]
    q, k, v = row_inputs(g["scores"], g["values"])
    qs, ks, vs = row_inputs([s + c for s in g["scores"]], g["values"])
    o, l = orc.dense_head(q, k, v, 1.0)
    os_, ls = orc.dense_head(qs, ks, vs, 1.0)
    assert np.all(np.isfinite(os_)), "shifted scores overflowed"
    assert abs(os_[0, 0] - o[0, 0]) < 1e-12
    assert abs(ls[0] - (l[0] + c)) < 1e-9
    ot, lt = orc.streaming_head(qs, ks, vs, 1.0, block_k=1)
    assert abs(ot[0, 0] - o[0, 0]) < 1e-12
    assert abs(lt[0] - (l[0] + c)) < 1e-9


def check_mask_renormalises(orc):
    # §2 checkpoint: mask the third key; the remaining two weights renormalise.
    g = golden("worked_row.json")
    q, k, v = row_inputs(g["scores"], g["values"])
    out, lse = orc.dense_head(q, k, v, 1.0, causal=True, q_pos=[1], k_pos=[0, 1, 2])
    e = math.e
    expected = 10.0 / (1.0 + e) + 20.0 * e / (1.0 + e)
    assert abs(out[0, 0] - expected) < 1e-12
    assert abs(lse[0] - math.log(e + e * e)) < 1e-12
    zeroed = sum(math.exp(s) * v for s, v in zip(g["scores"][:2], g["values"][:2])) / \
        sum(math.exp(s) for s in g["scores"])
    assert abs(out[0, 0] - zeroed) > 1.0


def check_two_tile(orc):
    g = golden("two_tile_example.json")
    q, k, v = row_inputs(g["scores"], g["values"])
    trace = []
    out, lse = orc.streaming_head(q, k, v, 1.0, block_q=1, block_k=g["tile_size"], trace=trace)
    t1, t2 = trace
    a1, a2 = g["after_tile_1"], g["after_tile_2"]
    assert t1["m"][0] == a1["m"] and t2["m"][0] == a2["m"]
    assert abs(t1["ell"][0] - a1["ell"]) <= 1e-4
    assert abs(t1["u"][0, 0] - a1["A"]) <= 1e-3
    assert abs(t2["alpha"][0] - a2["alpha"]) <= 1e-4
    assert abs(t2["ell"][0] - a2["ell"]) <= 1e-4
    assert abs(t2["u"][0, 0] - a2["A"]) <= 1e-3
    assert abs(out[0, 0] - g["output"]) <= 1e-2
    od, ld = orc.dense_head(q, k, v, 1.0)
    assert abs(od[0, 0] - g["output"]) <= 1e-2
    assert abs(od[0, 0] - out[0, 0]) < 1e-12 and abs(ld[0] - lse[0]) < 1e-12


def check_mask_table(orc):
    # All scores 0 and V = identity: a row's output is uniform over its allowed keys.
    g = golden("rectangular_causal_mask.json")
    nq, nk = g["n_queries"], g["n_keys"]
    q = np.zeros((1, 1, nq, 1))
    k = np.zeros((1, 1, nk, 1))
    v = np.eye(nk).reshape(1, 1, nk, nk)
    out, lse = orc.attention_forward(q, k, v, 1.0, causal=True)
    allowed = (out[0, 0] > 0).astype(int).tolist()
    assert allowed == g["allowed"], allowed
    counts = np.asarray(g["allowed"]).sum(axis=1)
    close(lse[0, 0], np.log(counts), 1e-14)


def check_streaming_vs_dense(orc):
    cases = [(11, 5, 13, 16, 8, 8), (12, 33, 70, 8, 8, 0), (13, 64, 64, 4, 3, -5),
             (14, 7, 19, 5, 5, 12)]
    for seed, Lq, Lk, D, Dv, q_start in cases:
        q, k, v = rng_case(seed, Lq, Lk, D, Dv)
        scale = 1.0 / math.sqrt(D)
        for causal in (False, True):
            qp = q_start + np.arange(Lq)
            od, ld = orc.dense_head(q, k, v, scale, causal, q_pos=qp)
            for bq, bk in [(1, 1), (3, 4), (4, 7), (64, 64), (Lq, Lk), (7, 3)]:
                nt = (Lk + bk - 1) // bk
                orders = [None, list(range(nt))[::-1],
                          list(np.random.default_rng(seed + bk).permutation(nt))]
                for order in orders:
                    for tau in (None, 0.0, 8 * math.log(2.0), 1e3):
                        os_, ls = orc.streaming_head(q, k, v, scale, causal, q_pos=qp,
                                                     block_q=bq, block_k=bk,
                                                     kv_order=order, tau=tau)
                        close(os_, od)
                        close(ls, ld)


def check_merge_trees(orc):
    q, k, v = rng_case(21, 6, 13, 8, 5)
    scale = 0.3
    qp = np.array([-1, 2, 5, 7, 11, 12])        # row 0 sees no key at all
    kp = np.arange(13)
    od, ld = orc.dense_head(q, k, v, scale, True, q_pos=qp, k_pos=kp)
    assert np.all(od[0] == 0.0) and ld[0] == -np.inf
    bounds = [(0, 3), (3, 3), (3, 7), (7, 13)]   # includes an empty partition
    states = [orc.partition_state(q, k[a:b], v[a:b], scale, True, qp, kp[a:b]) for a, b in bounds]
    A, B_, C, D_ = states
    trees = [
        orc.merge_states(orc.merge_states(orc.merge_states(A, B_), C), D_),
        orc.merge_states(A, orc.merge_states(B_, orc.merge_states(C, D_))),
        orc.merge_states(orc.merge_states(D_, B_), orc.merge_states(C, A)),
    ]
    for st in trees:
        o, l = orc.finish_state(st)
        close(o, od)
        close(l, ld)
    parts = [orc.finish_state(s) for s in states]
    (oa, la), (ob, lb), (oc, lc), (oe, le) = parts
    o1, l1 = orc.merge_normalized(*orc.merge_normalized(*orc.merge_normalized(oa, la, ob, lb), oc, lc), oe, le)
    o2, l2 = orc.merge_normalized(oe, le, *orc.merge_normalized(oc, lc, *orc.merge_normalized(ob, lb, oa, la)))
    for o, l in ((o1, l1), (o2, l2)):
        close(o, od)
        close(l, ld)


def check_page_streaming_experiment(orc):
    # FlashAttention from Scratch §5: seed 7, q 5x16, k 13x16, v 13x8, causal,
    # queries are the last five positions of a 13-token cache, blocks 3 / 4, 1e-10.
    torch.manual_seed(7)
    q = torch.randn(5, 16)
    k = torch.randn(13, 16)
    v = torch.randn(13, 8)
    scale = 1.0 / math.sqrt(16)
    qp = 8 + np.arange(5)
    ref, ref_lse = orc.dense_head(q, k, v, scale, True, q_pos=qp)
    out, lse = orc.streaming_head(q, k, v, scale, True, q_pos=qp, block_q=3, block_k=4)
    close(out, ref)
    close(lse, ref_lse)


def check_page_split_experiment(orc):
    # FlashAttention from Scratch §9.1: seed 9, q 2x8, k 11x8, v 11x5; partitions
    # [0, 4) and [4, 11) with absolute key offsets; causal from position 9.
    torch.manual_seed(9)
    q = torch.randn(2, 8)
    k = torch.randn(11, 8)
    v = torch.randn(11, 5)
    scale = 1.0 / math.sqrt(8)
    qp = 9 + np.arange(2)
    oa, la = orc.streaming_head(q, k[:4], v[:4], scale, True, q_pos=qp, k_pos=np.arange(4))
    ob, lb = orc.streaming_head(q, k[4:], v[4:], scale, True, q_pos=qp, k_pos=4 + np.arange(7))
    merged, mlse = orc.merge_normalized(oa, la, ob, lb)
    ref, ref_lse = orc.dense_head(q, k, v, scale, True, q_pos=qp)
    close(merged, ref)
    close(mlse, ref_lse)


def _brute_row(qi, K, V, scale, allowed):
    """sum_j e^{s_j} v_j / sum_j e^{s_j} over allowed j, with no max shift."""
    idx = [j for j in range(len(K)) if allowed[j]]
    if not idx:
        return [0.0] * len(V[0]), -math.inf
    s = {j: scale * math.fsum(a * b for a, b in zip(qi, K[j])) for j in idx}
    den = math.fsum(math.exp(s[j]) for j in idx)
    out = [math.fsum(math.exp(s[j]) * V[j][c] for j in idx) / den for c in range(len(V[0]))]
    return out, math.log(den)


def check_brute_force(orc):
    r = np.random.default_rng(5)
    for trial in range(60):
        Lq, Lk = int(r.integers(1, 7)), int(r.integers(1, 7))
        D, Dv = int(r.integers(1, 5)), int(r.integers(1, 4))
        q = r.integers(-3, 4, (Lq, D)).astype(float)
        k = r.integers(-3, 4, (Lk, D)).astype(float)
        v = r.integers(-5, 6, (Lk, Dv)).astype(float)
        scale = 0.5
        for causal in (False, True):
            for q_start in range(-Lk, Lk + 1):
                qp = q_start + np.arange(Lq)
                out, lse = orc.dense_head(q, k, v, scale, causal, q_pos=qp)
                for i in range(Lq):
                    allowed = [(not causal) or j <= qp[i] for j in range(Lk)]
                    bo, bl = _brute_row(q[i].tolist(), k.tolist(), v.tolist(), scale, allowed)
                    if bl == -math.inf:
                        assert lse[i] == -math.inf and np.all(out[i] == 0.0)
                    else:
                        assert abs(lse[i] - bl) <= 1e-12 * (1 + abs(bl))
                        for c in range(Dv):
                            assert abs(out[i, c] - bo[c]) <= 1e-12 * (1 + abs(bo[c]))
                if not causal:
                    break


def check_closed_forms(orc):
    r = np.random.default_rng(3)
    # One key: the output is that key's value row exactly; LSE is its score.
    q, k, v = r.standard_normal((4, 8)), r.standard_normal((1, 8)), r.standard_normal((1, 6))
    out, lse = orc.dense_head(q, k, v, 0.25)
    assert np.array_equal(out, np.repeat(v, 4, axis=0))
    close(lse, 0.25 * (q @ k[0]), 1e-14)
    # Identical keys: the output is mean(V); LSE = s + ln n.
    n = 9
    k = np.repeat(r.standard_normal((1, 8)), n, axis=0)
    v = r.standard_normal((n, 5))
    out, lse = orc.dense_head(q, k, v, 0.25)
    close(out, np.repeat(v.mean(axis=0, keepdims=True), 4, axis=0), 1e-13)
    close(lse, 0.25 * (q @ k[0]) + math.log(n), 1e-13)
    # Zero query: uniform weights.
    k = r.standard_normal((n, 8))
    out, lse = orc.dense_head(np.zeros((2, 8)), k, v, 0.7)
    close(out, np.repeat(v.mean(axis=0, keepdims=True), 2, axis=0), 1e-13)
    close(lse, np.full(2, math.log(n)), 1e-14)
    # Causal row 0 (query at position 0) sees only key 0: output is v_0 exactly.
    q = r.standard_normal((n, 8))
    out, lse = orc.dense_head(q, k, v, 0.7, causal=True)
    assert np.array_equal(out[0], v[0])
    close(lse[0], 0.7 * (q[0] @ k[0]), 1e-14)


def _sdpa_reference(q, k, v, scale, causal, kv_lens):
    """torch CPU SDPA in fp64 with an explicit boolean mask (True = allowed)."""
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    r = Hq // Hkv
    qd, kd, vd = q.double(), k.double().repeat_interleave(r, dim=1), v.double().repeat_interleave(r, dim=1)
    mask = torch.zeros(B, 1, Lq, Lk, dtype=torch.bool)
    for b in range(B):
        n = Lk if kv_lens is None else int(kv_lens[b])
        for i in range(Lq):
            hi = n if not causal else min(n, n - Lq + i + 1)
            mask[b, 0, i, :max(hi, 0)] = True
    out = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd, attn_mask=mask,
                                                           dropout_p=0.0, scale=scale)
    return out.numpy(), mask


def check_vs_sdpa(orc):
    g = torch.Generator().manual_seed(17)
    B, Hq, Hkv, Lq, Lk, D = 2, 6, 2, 5, 9, 8
    q = torch.randn(B, Hq, Lq, D, generator=g)
    k = torch.randn(B, Hkv, Lk, D, generator=g)
    v = torch.randn(B, Hkv, Lk, D, generator=g)
    scale = 1.0 / math.sqrt(D)
    for causal, lens in ((False, None), (True, None), (False, [9, 6]), (True, [9, 7])):
        ref, mask = _sdpa_reference(q, k, v, scale, causal, lens)
        out, lse = orc.attention_forward(q, k, v, scale, causal, lens)
        close(out, ref)
        # LSE against an independent evaluation: torch.logsumexp over masked scores.
        s = scale * (q.double() @ k.double().repeat_interleave(Hq // Hkv, 1).transpose(-1, -2))
        s = s.masked_fill(~mask, -math.inf)
        close(lse, torch.logsumexp(s, dim=-1).numpy())


def check_gqa_vs_repeated(orc):
    r = np.random.default_rng(8)
    B, Hq, Hkv, L, D = 1, 6, 2, 7, 4
    q = r.standard_normal((B, Hq, L, D))
    k = r.standard_normal((B, Hkv, L, D))
    v = r.standard_normal((B, Hkv, L, D))
    for causal in (False, True):
        o1, l1 = orc.attention_forward(q, k, v, 0.5, causal)
        o2, l2 = orc.attention_forward(q, np.repeat(k, Hq // Hkv, axis=1),
                                       np.repeat(v, Hq // Hkv, axis=1), 0.5, causal)
        close(o1, o2, 1e-15)
        close(l1, l2, 1e-15)


def check_kv_lens(orc):
    r = np.random.default_rng(9)
    B, H, Lq, Lk, D = 3, 2, 4, 10, 4
    q = r.standard_normal((B, H, Lq, D))
    k = r.standard_normal((B, H, Lk, D))
    v = r.standard_normal((B, H, Lk, D))
    lens = [10, 6, 0]
    for causal in (False, True):
        o, l = orc.attention_forward(q, k, v, 0.5, causal, lens)
        for b, n in enumerate(lens):
            if n == 0:
                assert np.all(o[b] == 0.0) and np.all(l[b] == -np.inf)
                continue
            ob, lb = orc.attention_forward(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n], 0.5, causal)
            close(o[b], ob[0], 1e-15)
            close(l[b], lb[0], 1e-15)


def check_fully_masked_rows(orc):
    # §5 experiment: q_start = -2 masks the first two rows entirely; the rest
    # must equal the rows computed on their own.  Also Q and K multiplied by 20.
    q, k, v = rng_case(31, 6, 8, 8, 3, mult=20.0)
    qp = -2 + np.arange(6)
    out, lse = orc.dense_head(q, k, v, 0.125, True, q_pos=qp)
    assert np.all(out[:2] == 0.0) and np.all(lse[:2] == -np.inf)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse[2:]))
    o2, l2 = orc.dense_head(q[2:], k, v, 0.125, True, q_pos=qp[2:])
    close(out[2:], o2, 1e-15)
    close(lse[2:], l2, 1e-15)
    os_, ls = orc.streaming_head(q, k, v, 0.125, True, q_pos=qp, block_q=4, block_k=3)
    close(os_, out)
    close(ls, lse)
    # Fewer keys than queries under bottom-right causal alignment: leading rows empty.
    Q = q.reshape(1, 1, 6, 8)
    K = k[:4].reshape(1, 1, 4, 8)
    V = v[:4].reshape(1, 1, 4, 3)
    o, l = orc.attention_forward(Q, K, V, 0.125, True)
    assert np.all(o[0, 0, :2] == 0.0) and np.all(l[0, 0, :2] == -np.inf)
    assert np.all(np.isfinite(l[0, 0, 2:]))


# ---------------------------------------------------------------------------
# Causal window (FlashAttention from Scratch, §12) and paged KV (§9.3)
# ---------------------------------------------------------------------------

def check_window_closed_forms(orc):
    q, k, v = rng_case(41, 9, 9, 8, 5)
    # Width 1: every row sees only the key at its own position, so O is that
    # value row exactly and the LSE is that one score -- with or without the
    # causal flag, since the window is causal by itself.
    for causal in (True, False):
        out, lse = orc.dense_head(q, k, v, 0.3, causal, window=1)
        assert np.array_equal(out, v)
        close(lse, 0.3 * np.einsum("id,id->i", q, k), 1e-14)
    # Width 3: row i is plain (unmasked) attention over keys max(0, i-2)..i.
    out, lse = orc.dense_head(q, k, v, 0.3, True, window=3)
    for i in range(9):
        lo = max(0, i - 2)
        o1, l1 = orc.dense_head(q[i:i + 1], k[lo:i + 1], v[lo:i + 1], 0.3)
        close(out[i:i + 1], o1, 1e-15)
        close(lse[i:i + 1], l1, 1e-15)
    # A window at least as long as the sequence is plain causal attention.
    oc, lc = orc.dense_head(q, k, v, 0.3, True)
    for w in (9, 10, 100):
        ow, lw = orc.dense_head(q, k, v, 0.3, True, window=w)
        assert np.array_equal(ow, oc) and np.array_equal(lw, lc)


def check_window_brute_force(orc):
    r = np.random.default_rng(43)
    for trial in range(25):
        Lq, Lk = int(r.integers(1, 6)), int(r.integers(1, 7))
        D, Dv = int(r.integers(1, 4)), int(r.integers(1, 3))
        q = r.integers(-3, 4, (1, 1, Lq, D)).astype(float)
        k = r.integers(-3, 4, (1, 1, Lk, D)).astype(float)
        v = r.integers(-5, 6, (1, 1, Lk, Dv)).astype(float)
        n = int(r.integers(0, Lk + 1))
        for w in range(1, Lk + 2):
            out, lse = orc.attention_forward(q, k, v, 0.5, True, [n], window=w)
            for i in range(Lq):
                qp = n - Lq + i
                allowed = [j < n and 0 <= qp - j < w for j in range(Lk)]
                bo, bl = _brute_row(q[0, 0, i].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), 0.5, allowed)
                if bl == -math.inf:
                    assert lse[0, 0, i] == -math.inf and np.all(out[0, 0, i] == 0.0)
                else:
                    assert abs(lse[0, 0, i] - bl) <= 1e-12 * (1 + abs(bl))
                    for c in range(Dv):
                        assert abs(out[0, 0, i, c] - bo[c]) <= 1e-12 * (1 + abs(bo[c]))


def _page_out(k, v, lens, page_size, num_pages, seed):
    """Scatter contiguous [B, Hkv, Lk, D] K and V into a NaN-filled page pool
    with a random page table; returns (k_cache, v_cache, table)."""
    r = np.random.default_rng(seed)
    B, Hkv, Lk, D = k.shape
    max_pages = -(-Lk // page_size)
    table = np.full((B, max_pages), -7, dtype=np.int64)   # unused entries hold garbage
    order = r.permutation(num_pages)
    kc = np.full((num_pages, Hkv, page_size, D), np.nan)
    vc = np.full((num_pages, Hkv, page_size, v.shape[3]), np.nan)
    nxt = 0
    for b in range(B):
        for slot in range(-(-lens[b] // page_size)):
            page = order[nxt]
            nxt += 1
            table[b, slot] = page
            t0, t1 = slot * page_size, min(lens[b], (slot + 1) * page_size)
            kc[page, :, :t1 - t0] = k[b, :, t0:t1]
            vc[page, :, :t1 - t0] = v[b, :, t0:t1]
    return kc, vc, table


def check_paged_matches_contiguous(orc):
    # Paging changes only where keys live: through any page table, the
    # result equals the contiguous cache's.  Unused pages, unused table
    # entries and the tail of the last page hold NaN or garbage.
    r = np.random.default_rng(47)
    B, Hq, Hkv, Lq, Lk, D = 3, 4, 2, 3, 20, 4
    q = r.standard_normal((B, Hq, Lq, D))
    k = r.standard_normal((B, Hkv, Lk, D))
    v = r.standard_normal((B, Hkv, Lk, D))
    lens = [20, 13, 0]
    for P in (4, 3, 20):
        kc, vc, table = _page_out(k, v, lens, P, 12, seed=P)
        for causal, w in ((False, 0), (True, 0), (True, 5)):
            o1, l1 = orc.paged_attention_forward(q, kc, vc, table, lens, P, 0.5, causal, w)
            o2, l2 = orc.attention_forward(q, k, v, 0.5, causal, lens, window=w)
            assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def check_paged_permutation(orc):
    # §9.3's experiment: permute the physical pages and let the table follow;
    # every output must stay exactly the same.
    r = np.random.default_rng(53)
    B, Hq, Hkv, Lq, D, P, NP = 2, 2, 1, 1, 8, 4, 9
    q = r.standard_normal((B, Hq, Lq, D))
    kc = r.standard_normal((NP, Hkv, P, D))
    vc = r.standard_normal((NP, Hkv, P, D))
    table = np.array([[3, 0, 7, 5], [8, 1, 2, 6]])
    lens = [15, 11]
    o1, l1 = orc.paged_attention_forward(q, kc, vc, table, lens, P, 0.4)
    perm = r.permutation(NP)              # physical page p moves to perm[p]
    kp, vp = np.empty_like(kc), np.empty_like(vc)
    kp[perm], vp[perm] = kc, vc
    o2, l2 = orc.paged_attention_forward(q, kp, vp, perm[table], lens, P, 0.4)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # Without the table following, the result changes.
    o3, _ = orc.paged_attention_forward(q, kp, vp, table, lens, P, 0.4)
    assert not np.allclose(o1, o3)


def check_paged_invalid_entries(orc):
    # Tokens whose table entry is out of range are masked but keep their
    # logical positions: brute force over the remaining allowed keys.
    r = np.random.default_rng(59)
    B, Hq, Hkv, Lq, D, P, NP = 1, 1, 1, 3, 2, 2, 5
    q = r.integers(-3, 4, (B, Hq, Lq, D)).astype(float)
    kc = r.integers(-3, 4, (NP, Hkv, P, D)).astype(float)
    vc = r.integers(-5, 6, (NP, Hkv, P, 2)).astype(float)
    table = np.array([[4, -1, 0, NP, 2]])
    n = 9
    logical_k, logical_v, valid = [], [], []
    for t in range(n):
        page = table[0, t // P]
        ok = 0 <= page < NP
        logical_k.append(kc[page, 0, t % P].tolist() if ok else [0.0] * D)
        logical_v.append(vc[page, 0, t % P].tolist() if ok else [0.0, 0.0])
        valid.append(ok)
    for causal, w in ((False, 0), (True, 0), (True, 4)):
        out, lse = orc.paged_attention_forward(q, kc, vc, table, [n], P, 0.5, causal, w)
        for i in range(Lq):
            qp = n - Lq + i
            allowed = [valid[j] and (not causal or j <= qp) and (w == 0 or qp - j < w)
                       for j in range(n)]
            bo, bl = _brute_row(q[0, 0, i].tolist(), logical_k, logical_v, 0.5, allowed)
            assert abs(lse[0, 0, i] - bl) <= 1e-12 * (1 + abs(bl))
            for c in range(2):
                assert abs(out[0, 0, i, c] - bo[c]) <= 1e-12 * (1 + abs(bo[c]))


# ---------------------------------------------------------------------------
# Backward (FlashAttention from Scratch, §8)
# ---------------------------------------------------------------------------

def _torch_masked_attention(q, k, v, scale, allowed):
    """Dense softmax attention in torch fp64 with a boolean allowed mask
    (no empty rows), for autograd."""
    s = scale * (q @ k.transpose(-1, -2))
    s = s.masked_fill(~allowed, -math.inf)
    return torch.softmax(s, dim=-1) @ v


def check_backward_page_experiment(orc):
    # §8's own check, re-derived: seed 8, q 5x7, k 9x7, v 9x3, causal with
    # the queries at positions 4..8; the gradients must match autograd
    # through a dense softmax to 1e-10.
    torch.manual_seed(8)
    qg = torch.randn(5, 7, dtype=torch.float64, requires_grad=True)
    kg = torch.randn(9, 7, dtype=torch.float64, requires_grad=True)
    vg = torch.randn(9, 3, dtype=torch.float64, requires_grad=True)
    qp, kp = torch.arange(4, 9), torch.arange(9)
    allowed = kp[None, :] <= qp[:, None]
    scale = 1.0 / math.sqrt(7)
    og = _torch_masked_attention(qg, kg, vg, scale, allowed)
    g = torch.randn_like(og)
    expected = torch.autograd.grad(og, (qg, kg, vg), g)
    got = orc.dense_backward_head(qg.detach(), kg.detach(), vg.detach(), g, scale, True,
                                  q_pos=qp.numpy(), k_pos=kp.numpy())
    for a, b in zip(got, expected):
        close(a, b.numpy(), 1e-10)


def check_backward_vs_autograd(orc):
    # Batched, GQA, kv_lens, causal / window, against torch autograd through
    # a dense masked softmax (every row keeps at least one key).
    g0 = torch.Generator().manual_seed(61)
    B, Hq, Hkv, Lq, Lk, D = 2, 6, 2, 4, 9, 5
    q = torch.randn(B, Hq, Lq, D, generator=g0, dtype=torch.float64)
    k = torch.randn(B, Hkv, Lk, D, generator=g0, dtype=torch.float64)
    v = torch.randn(B, Hkv, Lk, D, generator=g0, dtype=torch.float64)
    gout = torch.randn(B, Hq, Lq, D, generator=g0, dtype=torch.float64)
    lens = [9, 6]
    scale = 0.4
    for causal, w in ((False, 0), (True, 0), (True, 3)):
        qq, kk, vv = (t.clone().requires_grad_(True) for t in (q, k, v))
        r = Hq // Hkv
        outs = []
        for b in range(B):
            n = lens[b]
            qp, kp = torch.arange(n - Lq, n), torch.arange(n)
            allowed = torch.ones(Lq, n, dtype=torch.bool)
            if causal:
                allowed &= kp[None, :] <= qp[:, None]
            if w:
                allowed &= (qp[:, None] - kp[None, :]) < w
            for h in range(Hq):
                outs.append(_torch_masked_attention(qq[b, h], kk[b, h // r, :n], vv[b, h // r, :n],
                                                    scale, allowed))
        o = torch.stack(outs).view(B, Hq, Lq, D)
        expected = torch.autograd.grad(o, (qq, kk, vv), gout)
        got = orc.attention_backward(q, k, v, gout, scale, causal, lens, window=w)
        for a, e in zip(got, expected):
            close(a, e.numpy(), 1e-12)


def check_backward_finite_differences(orc):
    # Central differences of L = sum(G * O) through the forward definition
    # (attention.dense_head), on a tiny causal case with an empty row.
    r = np.random.default_rng(67)
    Lq, Lk, D = 3, 4, 2
    q, k, v = r.standard_normal((Lq, D)), r.standard_normal((Lk, D)), r.standard_normal((Lk, D))
    g = r.standard_normal((Lq, D))
    qp = np.array([-1, 1, 3])           # row 0 sees no key
    scale, eps = 0.7, 1e-6

    def loss(qq, kk, vv):
        o, _ = orc.dense_head(qq, kk, vv, scale, True, q_pos=qp)
        return float((g * o).sum())

    got = orc.dense_backward_head(q, k, v, g, scale, True, q_pos=qp)
    for idx, x in enumerate((q, k, v)):
        num = np.zeros_like(x)
        for pos in np.ndindex(*x.shape):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[idx][pos] += eps
            args_m[idx][pos] -= eps
            num[pos] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        close(got[idx], num, 1e-7)
    assert np.all(got[0][0] == 0.0)     # the empty row has no gradient


def check_backward_gqa_and_lengths(orc):
    # A shared KV head's gradient is the sum of the gradients each query head
    # gives it; keys at or past kv_lens get zero gradient and the rest equal
    # the gradients of the truncated problem.
    r = np.random.default_rng(71)
    B, Hq, Hkv, L, D = 1, 4, 2, 6, 3
    q, k, v, g = (r.standard_normal((B, h, L, D)) for h in (Hq, Hkv, Hkv, Hq))
    dq, dk, dv = orc.attention_backward(q, k, v, g, 0.5, True)
    kr, vr = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
    dq2, dk2, dv2 = orc.attention_backward(q, kr, vr, g, 0.5, True)
    close(dq, dq2, 1e-14)
    close(dk, dk2.reshape(B, Hkv, 2, L, D).sum(axis=2), 1e-14)
    close(dv, dv2.reshape(B, Hkv, 2, L, D).sum(axis=2), 1e-14)
    dq3, dk3, dv3 = orc.attention_backward(q, k, v, g, 0.5, True, kv_lens=[4])
    assert np.all(dk3[:, :, 4:] == 0.0) and np.all(dv3[:, :, 4:] == 0.0)
    dq4, dk4, dv4 = orc.attention_backward(q, k[:, :, :4], v[:, :, :4], g, 0.5, True)
    close(dq3, dq4, 1e-15)
    close(dk3[:, :, :4], dk4, 1e-15)
    close(dv3[:, :, :4], dv4, 1e-15)


def _bf16(x):
    return torch.tensor(np.asarray(x), dtype=torch.float32).to(torch.bfloat16).double().numpy()


def check_score_modifiers(orc):
    # Zero slope / no cap is plain attention, bit for bit.
    rng = np.random.default_rng(41)
    q, k, v = rng.standard_normal((6, 8)), rng.standard_normal((11, 8)), rng.standard_normal((11, 3))
    qp = np.arange(5, 11)
    O0, l0 = orc.dense_head(q, k, v, 0.3, True, qp)
    O1, l1 = orc.dense_head(q, k, v, 0.3, True, qp, alibi_slope=0.0, softcap=0.0)
    assert np.array_equal(O0, O1) and np.array_equal(l0, l1)
    # ALiBi closed form: identical keys give equal raw scores, so the weights
    # are exp(-slope * distance) alone.
    slope, pos = 0.37, 9
    kk = np.tile(rng.standard_normal((1, 4)), (pos + 1, 1))
    qq = rng.standard_normal((1, 4))
    s0 = 0.5 * float(qq[0] @ kk[0])
    w = [math.exp(-slope * (pos - j)) for j in range(pos + 1)]
    vv = rng.standard_normal((pos + 1, 2))
    O, lse = orc.dense_head(qq, kk, vv, 0.5, True, [pos], alibi_slope=slope)
    exp_o = [sum(w[j] * vv[j, c] for j in range(pos + 1)) / math.fsum(w) for c in range(2)]
    assert np.allclose(O[0], exp_o, rtol=0, atol=1e-13)
    assert abs(lse[0] - (s0 + math.log(math.fsum(w)))) < 1e-13
    # ALiBi against torch's SDPA with an additive bias (GQA, kv_lens, causal):
    # query head h uses slopes[h].
    B, Hq, Hkv, Lq, Lk, D = 2, 4, 2, 5, 9, 6
    g0 = torch.Generator().manual_seed(43)
    qt = torch.randn(B, Hq, Lq, D, generator=g0, dtype=torch.float64)
    kt = torch.randn(B, Hkv, Lk, D, generator=g0, dtype=torch.float64)
    vt = torch.randn(B, Hkv, Lk, D, generator=g0, dtype=torch.float64)
    slopes = np.array([0.5, 0.25, 0.125, 0.0625])
    lens = [9, 6]
    O, _ = orc.attention_forward(qt, kt, vt, 0.4, True, np.array(lens), alibi_slopes=slopes)
    for b in range(B):
        n = lens[b]
        qpos = torch.arange(Lq, dtype=torch.float64) + (n - Lq)
        kpos = torch.arange(n, dtype=torch.float64)
        dist = qpos[:, None] - kpos[None, :]
        for h in range(Hq):
            bias = -slopes[h] * dist.abs()
            bias = bias.masked_fill(dist < 0, float("-inf"))
            ref = torch.nn.functional.scaled_dot_product_attention(
                qt[b, h][None], kt[b, h // 2, :n][None], vt[b, h // 2, :n][None], attn_mask=bias, scale=0.4)[0]
            assert np.allclose(O[b, h], ref.numpy(), rtol=0, atol=1e-12)
    # Soft-capping against pure-Python brute force (scalar tanh and exp), on
    # large scores so the cap bites, and its limit: a huge cap is plain attention.
    q2, k2, v2 = 3 * rng.standard_normal((3, 4)), 3 * rng.standard_normal((7, 4)), rng.standard_normal((7, 2))
    cap = 2.5
    O, lse = orc.dense_head(q2, k2, v2, 0.7, True, [4, 5, 6], softcap=cap)
    for i, p_i in enumerate([4, 5, 6]):
        sc = [cap * math.tanh(0.7 * sum(q2[i, d] * k2[j, d] for d in range(4)) / cap) for j in range(p_i + 1)]
        m = max(sc)
        e = [math.exp(x - m) for x in sc]
        z = math.fsum(e)
        assert abs(lse[i] - (m + math.log(z))) < 1e-12
        for c in range(2):
            assert abs(O[i, c] - math.fsum(e[j] * v2[j, c] for j in range(p_i + 1)) / z) < 1e-12
        assert lse[i] <= cap + math.log(p_i + 1) + 1e-12
    Oh, lh = orc.dense_head(q2, k2, v2, 0.7, True, [4, 5, 6], softcap=1e9)
    Op, lp = orc.dense_head(q2, k2, v2, 0.7, True, [4, 5, 6])
    assert np.allclose(Oh, Op, rtol=0, atol=1e-12) and np.allclose(lh, lp, rtol=0, atol=1e-12)


def check_fp8_format(orc):
    # OCP E4M3 facts (FP8 formats for deep learning, OCP 8-bit floating point
    # specification): 0x7E = 448 is the largest finite value, 0x7F / 0xFF are
    # NaN, 0x08 = 2^-6 the smallest normal, 0x01 = 2^-9 the smallest
    # subnormal, 0x38 = 1, 0x80 = -0.
    f = orc.fp8
    assert f.e4m3_value(0x7E) == 448.0 and f.e4m3_value(0xFE) == -448.0
    assert np.isnan(f.e4m3_value(0x7F)) and np.isnan(f.e4m3_value(0xFF))
    assert f.e4m3_value(0x08) == 2.0 ** -6 and f.e4m3_value(0x01) == 2.0 ** -9
    assert f.e4m3_value(0x38) == 1.0 and f.e4m3_value(0x30) == 0.5 and f.e4m3_value(0x3C) == 1.5
    assert f.e4m3_value(0x80) == 0.0 and np.signbit(f.e4m3_value(0x80))
    table = np.array([f.e4m3_value(c) for c in range(256)])
    finite = ~np.isnan(table)
    assert finite.sum() == 254 and len(set(table[finite])) == 253    # +-0 share a value
    # Rounding against brute force: the nearest finite value, a tie going to
    # the even code; exact values map to themselves; the sign of a zero result
    # follows x.
    rng = np.random.default_rng(31)
    pos = np.sort(table[finite & (table >= 0)])
    mids = (pos[1:] + pos[:-1]) / 2
    xs = np.concatenate([rng.uniform(-448, 448, 3000), rng.standard_normal(3000) * 2.0 ** rng.integers(-12, 6, 3000),
                         mids, -mids, pos, -pos, [2.0 ** -11, -2.0 ** -11, 0.0]])
    xs = np.clip(xs, -448, 448)
    vals, codes = f.round_e4m3(xs)
    for x, val, c in zip(xs, vals, codes):
        d = np.abs(table - x)
        d[~finite] = np.inf
        best = d.min()
        assert abs(val - x) == best and table[c] == val, (x, val, c)
        tied = [cc for cc in range(256) if d[cc] == best and table[cc] != 0.0]
        if len({table[cc] for cc in tied}) > 1:
            assert c % 2 == 0, ("tie to even", x, c)
        if val == 0.0:
            assert bool(c & 0x80) == bool(np.signbit(x)), ("zero sign", x, c)


def check_fp8_hadamard(orc):
    # The transform: scipy's Hadamard matrix (Sylvester's construction), H H^T
    # = D I, and the pages' invariance: with M = diag(sigma) H / sqrt(D),
    # (Q M)(K M)^T = Q K^T before any rounding.
    import scipy.linalg
    f = orc.fp8
    for D in (1, 2, 8, 64, 128):
        H = f.sylvester_hadamard(D)
        assert np.array_equal(H, scipy.linalg.hadamard(D))
        assert np.array_equal(H @ H.T, D * np.eye(D))
    rng = np.random.default_rng(33)
    q, k = rng.standard_normal((7, 64)), rng.standard_normal((9, 64))
    sig = rng.choice([-1.0, 1.0], 64)
    S = f.incoherent(q, sig) @ f.incoherent(k, sig).T / 64
    assert np.allclose(S, q @ k.T, rtol=0, atol=1e-12)
    # The matrix of the transform, read off the unit vectors, is diag(sigma) H
    # (the random sign flips, then the Hadamard transform).
    assert np.array_equal(f.incoherent(np.eye(64), sig), np.diag(sig) @ scipy.linalg.hadamard(64))
    # Exactness on small integers (every partial sum representable).
    qi = rng.integers(-50, 50, (5, 128)).astype(np.float64)
    assert np.array_equal(f.incoherent(qi, np.ones(128)), qi @ scipy.linalg.hadamard(128))


def check_fp8_block_scale(orc):
    f = orc.fp8
    rng = np.random.default_rng(35)
    amaxes = np.concatenate([rng.uniform(1e-6, 1e6, 200), [448.0, 449.0, 224.0, 0.875, 0.875 * 2 ** -3, 1.0, 2.0 ** -20]])
    for a in amaxes:
        k = f.block_scale_exponent(float(a))
        assert a * 2.0 ** -k <= 448.0 and a * 2.0 ** -(k - 1) > 448.0, (a, k)
    assert f.block_scale_exponent(0.0) == 0
    # Per-block scales: powers of two, every block within half an E4M3 step,
    # and one block's outlier leaves the other blocks' codes alone.
    x = _bf16(rng.standard_normal((2, 300, 64)))
    codes, scales, values = f.quantize_rows(x, 64)
    assert scales.shape == (2, 5) and np.all(np.log2(scales) == np.round(np.log2(scales)))
    for j in range(5):
        blk, vb = x[:, 64 * j:64 * (j + 1)], values[:, 64 * j:64 * (j + 1)]
        sc = scales[:, j][:, None, None]
        assert np.all(np.abs(vb - blk) <= np.maximum(np.abs(blk) * 2.0 ** -4, sc * 2.0 ** -10) + 1e-300)
        assert np.all(np.abs(vb / sc) <= 448.0)
    y = x.copy()
    y[0, 5, 3] = 3000.0
    c2, s2, _ = f.quantize_rows(y, 64)
    assert s2[0, 0] > scales[0, 0] and np.array_equal(s2[:, 1:], scales[:, 1:])
    assert np.array_equal(c2[:, 64:], codes[:, 64:]) and np.array_equal(c2[1], codes[1])


def check_fp8_attention(orc):
    f = orc.fp8
    rng = np.random.default_rng(37)
    # Values already on the E4M3 grid of their block (small integers, every
    # block reaching 448 after scaling) pass through the quantizer unchanged,
    # so the FP8 attention equals the exact one.
    B, H, L, D = 1, 2, 96, 16
    q = rng.integers(-7, 8, (B, H, L, D)).astype(np.float64)
    k = rng.integers(-7, 8, (B, H, L, D)).astype(np.float64)
    v = rng.standard_normal((B, H, L, D))
    O, lse, qc, qs, kc, ks = f.fp8_attention_forward(q, k, v, 0.05, causal=True, q_block=32, k_block=16)
    O0, l0 = orc.attention_forward(q, k, v, 0.05, True)
    assert np.array_equal(O, O0) and np.array_equal(lse, l0)
    # With the transform, the pages' experiment: Q and K sharing outlier
    # channels; block scales and incoherent processing cut the RMSE of O
    # against the exact attention well below that of one per-tensor scale
    # (the pages report 2.6x on FA3's inputs; this seed gives ~4x).
    B, H, L, D = 1, 2, 512, 64
    q, k, v = (rng.standard_normal((B, H, L, D)) for _ in range(3))
    ch = rng.choice(D, 2, replace=False)
    q[..., ch] *= 10.0
    k[..., ch] *= 10.0
    q, k, v = _bf16(q), _bf16(k), _bf16(v)
    scale = 1.0 / np.sqrt(D) / 10.0
    O0, _ = orc.attention_forward(q, k, v, scale)
    Ot, _ = orc.attention_forward(f.quantize_per_tensor(q), f.quantize_per_tensor(k), v, scale)
    sig = rng.choice([-1.0, 1.0], D)
    Oi, *_ = f.fp8_attention_forward(q, k, v, scale, signs=sig)
    rmse = lambda o: float(np.sqrt(np.mean((o - O0) ** 2)))
    assert rmse(Oi) * 2.0 < rmse(Ot), (rmse(Oi), rmse(Ot))
    # and the quantized attention stays close to the exact one
    assert rmse(Oi) < 0.02


def check_trimmed_rows(orc):
    # Leaving out the keys that the causal mask (or window) removes for every
    # selected row changes nothing but rounding order: chunks of rows with
    # trimming against the untrimmed rows, for causal, windowed and ragged
    # problems, including chunks that end before the first key.
    r = np.random.default_rng(53)
    B, Hq, Hkv, Lq, Lk, D = 2, 4, 2, 37, 45, 8
    q = r.standard_normal((B, Hq, Lq, D))
    k = r.standard_normal((B, Hkv, Lk, D))
    v = r.standard_normal((B, Hkv, Lk, D))
    for causal, w, lens in ((True, 0, None), (True, 6, None), (True, 0, [45, 20]), (True, 9, [30, 3]),
                            (False, 0, [45, 11])):
        for b in range(B):
            for h in (0, 3):
                for r0, r1 in ((0, 5), (5, 19), (19, 37), (0, 37), (36, 37)):
                    rows = np.arange(r0, r1)
                    o1, l1 = orc.attention_rows(q, k, v, 0.4, causal, lens, b, h, rows, window=w,
                                                trim_keys=True)
                    o2, l2 = orc.attention_rows(q, k, v, 0.4, causal, lens, b, h, rows, window=w)
                    close(o1, o2, 1e-12)
                    close(l1, l2, 1e-12)
    # weights returned with the rows: P sums to one over the kept keys and
    # reproduces O from the returned value rows
    o, l, P, vv = orc.attention_rows(q, k, v, 0.4, True, None, 1, 2, np.arange(3, 9), window=4,
                                     trim_keys=True, return_weights=True)
    close(P.sum(axis=1), np.ones(6), 1e-12)
    close(P @ vv, o, 1e-12)


def check_backward_o_given(orc):
    # delta formed from a given output: with the exact O it is the ordinary
    # gradient; a perturbation e of row i's output moves delta_i by g_i . e,
    # so dV is unchanged, dQ_i moves by -c (g_i . e) sum_j P_ij k_j and dK_j by
    # -c sum_i P_ij (g_i . e_i) q_i (closed forms of dS = P (dP - delta)).
    r = np.random.default_rng(59)
    Lq, Lk, D, c = 5, 7, 3, 0.7
    q, k, v = r.standard_normal((Lq, D)), r.standard_normal((Lk, D)), r.standard_normal((Lk, D))
    g = r.standard_normal((Lq, D))
    O, _ = orc.dense_head(q, k, v, c)
    base = orc.dense_backward_head(q, k, v, g, c)
    same = orc.dense_backward_head(q, k, v, g, c, o_given=O)
    for a, b in zip(base, same):
        close(a, b, 1e-12)
    e = r.standard_normal((Lq, D)) * 1e-3
    pert = orc.dense_backward_head(q, k, v, g, c, o_given=O + e)
    S = c * (q @ k.T)
    P = np.exp(S - S.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    dd = (g * e).sum(axis=1)
    close(pert[2], base[2], 1e-12)
    close(pert[0] - base[0], -c * dd[:, None] * (P @ k), 1e-9)
    close(pert[1] - base[1], -c * (P * dd[:, None]).T @ q, 1e-9)
    # batched form passes the given output through per (b, h)
    qb, kb, vb, gb = (x[None, None] for x in (q, k, v, g))
    ob = (O + e)[None, None]
    dq, dk, dv = orc.attention_backward(qb, kb, vb, gb, c, o_given=ob)
    close(dq[0, 0], pert[0], 1e-12)
    close(dk[0, 0], pert[1], 1e-12)


# ---------------------------------------------------------------------------
# Variable-length packed batches (FlashAttention from Scratch, §11.5 and §12;
# FlashAttention-4, "LPT scheduling for imbalanced grids")
# ---------------------------------------------------------------------------

def _packed_case(seed, lens_q, lens_k, Hq=4, Hkv=2, D=6):
    r = np.random.default_rng(seed)
    tq, tk = sum(lens_q), sum(lens_k)
    q = r.standard_normal((Hq, tq, D))
    k = r.standard_normal((Hkv, tk, D))
    v = r.standard_normal((Hkv, tk, D))
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    return q, k, v, cu_q, cu_k


def _sdpa_packed(q, k, v, lens_q, lens_k, scale, causal):
    """torch SDPA in fp64 over the whole packed stream with a mask built from
    the lengths: query i of sequence b may see key j of sequence b at position
    p_j <= (Lk_b - Lq_b) + i under the causal rule; rows with no key are
    reported as None (SDPA gives NaN there)."""
    Hq, Hkv = q.shape[0], k.shape[0]
    tq, tk = q.shape[1], k.shape[1]
    mask = torch.zeros(tq, tk, dtype=torch.bool)
    row, col = 0, 0
    for lq, lk in zip(lens_q, lens_k):
        for i in range(lq):
            last = lk if not causal else min(lk, lk - lq + i + 1)
            mask[row + i, col:col + max(last, 0)] = True
        row, col = row + lq, col + lk
    qt = torch.from_numpy(q)[None]
    kt = torch.from_numpy(k).repeat_interleave(Hq // Hkv, 0)[None]
    vt = torch.from_numpy(v).repeat_interleave(Hq // Hkv, 0)[None]
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, dropout_p=0.0, scale=scale)
    s = scale * (qt @ kt.transpose(-1, -2))
    lse = torch.logsumexp(s.masked_fill(~mask, -math.inf), dim=-1)
    return out[0].numpy(), lse[0].numpy(), mask.any(dim=1).numpy()


def check_varlen_vs_sdpa(orc):
    # both routes of the module (per sequence, one block-diagonal mask) against
    # the library routine, with queries shorter, equal and longer than keys,
    # a sequence with no key and a sequence with no query
    lens_q = [5, 1, 7, 3, 0, 4]
    lens_k = [9, 1, 4, 0, 2, 4]
    q, k, v, cu_q, cu_k = _packed_case(61, lens_q, lens_k)
    for causal in (False, True):
        ref_o, ref_l, seen = _sdpa_packed(q, k, v, lens_q, lens_k, 0.45, causal)
        for fn in (orc.varlen.varlen_attention_forward, orc.varlen.packed_mask_forward):
            o, l = fn(q, k, v, cu_q, cu_k, 0.45, causal)
            close(o[:, seen], ref_o[:, seen])
            close(l[:, seen], ref_l[:, seen])
            assert np.all(o[:, ~seen] == 0.0) and np.all(l[:, ~seen] == -np.inf)


def check_varlen_single_and_order(orc):
    # one sequence is the batched definition; reordering the sequences in the
    # packing reorders the rows of the result and nothing else
    lens_q, lens_k = [6, 3, 8], [6, 10, 5]
    q, k, v, cu_q, cu_k = _packed_case(67, lens_q, lens_k)
    for causal in (False, True):
        o, l = orc.varlen.varlen_attention_forward(q, k, v, cu_q, cu_k, 0.6, causal)
        for b in range(3):
            qs, qe, ks, ke = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
            ob, lb = orc.attention_forward(q[None, :, qs:qe], k[None, :, ks:ke], v[None, :, ks:ke], 0.6, causal)
            close(o[:, qs:qe], ob[0], 1e-15)
            close(l[:, qs:qe], lb[0], 1e-15)
        perm = [2, 0, 1]
        qp = np.concatenate([q[:, cu_q[b]:cu_q[b + 1]] for b in perm], axis=1)
        kp = np.concatenate([k[:, cu_k[b]:cu_k[b + 1]] for b in perm], axis=1)
        vp = np.concatenate([v[:, cu_k[b]:cu_k[b + 1]] for b in perm], axis=1)
        cq = np.concatenate([[0], np.cumsum([lens_q[b] for b in perm])])
        ck = np.concatenate([[0], np.cumsum([lens_k[b] for b in perm])])
        op, lp = orc.varlen.varlen_attention_forward(qp, kp, vp, cq, ck, 0.6, causal)
        for j, b in enumerate(perm):
            close(op[:, cq[j]:cq[j + 1]], o[:, cu_q[b]:cu_q[b + 1]], 1e-15)
            close(lp[:, cq[j]:cq[j + 1]], l[:, cu_q[b]:cu_q[b + 1]], 1e-15)


def check_lpt_schedule(orc):
    # worked example: query lengths 300, 40, 1000, 0, 513 with key lengths
    # 300, 700, 1000, 900, 513 -> longest tiles ceil(Lk / 64) = 5, 11, 16, 0 (no
    # query, however many keys), 9; descending: 2 (16), 1 (11), 4 (9), 0 (5), 3 (0); query blocks
    # of 256 rows: 4, 1, 3, 2, 0 -> prefix 0, 4, 5, 8, 10, 10
    cu_q = np.cumsum([0, 300, 40, 1000, 0, 513])
    cu_k = np.cumsum([0, 300, 700, 1000, 900, 513])
    for causal in (False, True):
        order, prefix = orc.varlen.lpt_schedule(cu_q, cu_k, causal)
        assert list(order) == [2, 1, 4, 0, 3], order
        assert list(prefix) == [0, 4, 5, 8, 10, 10], prefix
    # properties on random batches: a permutation, longest tile non-increasing
    # along it, equal tiles in index order, prefix counting ceil(Lq / 256)
    r = np.random.default_rng(71)
    for _ in range(20):
        B = int(r.integers(1, 40))
        lq = r.integers(0, 3000, B)
        lk = r.integers(0, 3000, B)
        lk[r.random(B) < 0.3] = 640            # force ties
        order, prefix = orc.varlen.lpt_schedule(np.cumsum(np.r_[0, lq]), np.cumsum(np.r_[0, lk]), True)
        assert sorted(order) == list(range(B))
        cost = [(-(-int(lk[b]) // 64)) if lq[b] > 0 else 0 for b in order]
        assert all(cost[i] >= cost[i + 1] for i in range(B - 1))
        assert all(order[i] < order[i + 1] for i in range(B - 1) if cost[i] == cost[i + 1])
        assert list(prefix) == list(np.cumsum(np.r_[0, [-(-int(lq[b]) // 256) for b in order]]))


CHECKS = [check_worked_row, check_shift_invariance, check_mask_renormalises, check_two_tile,
          check_mask_table, check_streaming_vs_dense, check_merge_trees,
          check_page_streaming_experiment, check_page_split_experiment, check_brute_force,
          check_closed_forms, check_vs_sdpa, check_gqa_vs_repeated, check_kv_lens,
          check_fully_masked_rows, check_window_closed_forms, check_window_brute_force,
          check_paged_matches_contiguous, check_paged_permutation, check_paged_invalid_entries,
          check_backward_page_experiment, check_backward_vs_autograd, check_backward_finite_differences,
          check_backward_gqa_and_lengths, check_score_modifiers, check_fp8_format, check_fp8_hadamard, check_fp8_block_scale,
          check_fp8_attention, check_trimmed_rows, check_backward_o_given, check_varlen_vs_sdpa,
          check_varlen_single_and_order, check_lpt_schedule]


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_oracle_pin(check):
    check(oracle_namespace())


def test_package_exports_match_copies():
    # The pins run on fresh copies of the modules; the package must export those same functions.
    ns = oracle_namespace()
    for name in ("dense_head", "attention_forward", "streaming_head", "merge_normalized"):
        assert getattr(real_oracle, name).__code__.co_code == getattr(ns, name).__code__.co_code


# Plausible mistakes; each must make at least one pin fail.
MUTANTS = {
    "scale_dropped": [("attention", "S = scale * (q @ k.T)", "S = (q @ k.T)")],
    "causal_off_by_one": [("attention", "k_pos[None, :] > q_pos[:, None]", "k_pos[None, :] >= q_pos[:, None]")],
    "causal_top_left": [("attention", "q_pos = (n - Lq) + rows", "q_pos = rows")],
    "gqa_modulo_map": [("attention", "g = h // r", "g = h % Hkv")],
    "lse_without_max": [("attention", "shift + np.log(safe_ell)", "np.log(safe_ell)")],
    "no_max_shift": [("attention", "E = np.exp(S - shift[:, None])", "E = np.exp(S)")],
    "no_normalisation": [("attention", "P = E / safe_ell[:, None]", "P = E")],
    "scores_transposed": [("attention", "S = scale * (q @ k.T)", "S = scale * (k @ q.T).T[::-1, ::-1]")],
    "empty_row_lse_zero": [("attention", "shift + np.log(safe_ell), -np.inf)", "shift + np.log(safe_ell), 0.0)")],
    "kv_len_ignored": [("attention", "n = _kv_len(kv_lens, b, Lk)", "n = Lk")],
    "alpha_sign": [("streaming", "factor = np.exp(self.ref - anchor)", "factor = np.exp(anchor - self.ref)")],
    "ell_not_rescaled": [("streaming", "self.norm = factor * self.norm + terms.sum(axis=1)",
                          "self.norm = self.norm + terms.sum(axis=1)")],
    "acc_not_rescaled": [("streaming", "self.acc = factor[:, None] * self.acc + terms @ values",
                          "self.acc = self.acc + terms @ values")],
    "tau_inverted": [("streaming", "keep = (peak - self.ref) <= tau", "keep = ~((peak - self.ref) <= tau)")],
    "stream_mask_dropped": [("streaming", "tile = np.where(k_pos[keys][None, :] <= q_pos[r0:r1][:, None], tile, -np.inf)",
                             "pass")],
    "merge_unweighted_ell": [("merge", 'norm = np.einsum("pr,pr->r", scale_to_top, np.stack([p[1] for p in parts]))',
                              'norm = np.stack([p[1] for p in parts]).sum(axis=0)')],
    "merge_lse_max": [("merge", "total = _anchor(top) + np.log(np.exp(lses - _anchor(top)[None, :]).sum(axis=0))",
                       "total = top")],
    "merge_weight_swapped": [("merge", 'return np.einsum("pr,prd->rd", weights, outs), total',
                              'return np.einsum("pr,prd->rd", weights[::-1], outs), total')],
    "window_off_by_one": [("attention", "(dist >= window)", "(dist > window)")],
    "window_not_causal": [("attention", "(dist < 0) | (dist >= window)", "(dist >= window)")],
    "window_not_passed": [("attention", "np.arange(lo, hi), window, slope, softcap,", "np.arange(lo, hi), 0, slope, softcap,")],
    "trim_past_last_row": [("attention", "hi = int(min(n, max(q_pos.max() + 1, 0)))", "hi = int(min(n, max(q_pos.max(), 0)))")],
    "trim_window_start": [("attention", "lo = int(min(hi, max(q_pos.min() - window + 1, 0)))",
                           "lo = int(min(hi, max(q_pos.min() - window + 2, 0)))")],
    "bwd_o_given_ignored": [("backward", "delta = (g * (O if o_given is None else as_f64(o_given))).sum(axis=1)",
                             "delta = (g * O).sum(axis=1)")],
    "page_offset_swapped": [("paged", "cache[page, :, t % page_size, :]", "cache[page, :, t // page_size, :]")],
    "page_index_mod": [("paged", "page = table[b, t // page_size]", "page = table[b, t % page_size]")],
    "paged_positions_compacted": [("paged", "positions.append(t)", "positions.append(len(positions))")],
    "paged_invalid_kept": [("paged", "if page < 0 or page >= num_pages:\n            continue",
                            "if page < 0 or page >= num_pages:\n            page = 0")],
    "paged_head_map": [("paged", "g = h // r", "g = h % Hkv")],
    "paged_queries_top_left": [("paged", "q_pos = (n - Lq) + np.arange(Lq)", "q_pos = np.arange(Lq)")],
    "bwd_delta_dropped": [("backward", "dS = P * (dP - delta[:, None])", "dS = P * dP")],
    "bwd_delta_wrong": [("backward", "delta = (g * (O if o_given is None else as_f64(o_given))).sum(axis=1)",
                         "delta = g.sum(axis=1)")],
    "bwd_dq_unscaled": [("backward", "dQ = scale * (dS @ k)", "dQ = (dS @ k)")],
    "bwd_dk_sign": [("backward", "dK = scale * (dS.T @ q)", "dK = -scale * (dS.T @ q)")],
    "bwd_dv_from_ds": [("backward", "dV = P.T @ g", "dV = dS.T @ g")],
    "bwd_gqa_not_summed": [("backward", "dk[b, gk, :n] += dkh", "dk[b, gk, :n] = dkh")],
    "bwd_causal_dropped": [("backward", "allowed &= k_pos[None, :] <= q_pos[:, None]", "allowed &= True")],
    "bwd_top_left": [("backward", "q_pos = (n - Lq) + np.arange(Lq)", "q_pos = np.arange(Lq)")],
    "bwd_window_off_by_one": [("backward", "(dist < window)", "(dist <= window)")],
    "alibi_sign": [("attention", "S = S - alibi_slope * np.abs", "S = S + alibi_slope * np.abs")],
    "alibi_signed_distance": [("attention", "np.abs(q_pos[:, None] - k_pos[None, :])", "(k_pos[None, :] - q_pos[:, None])")],
    "alibi_head_map": [("attention", "float(as_f64(alibi_slopes)[h])", "float(as_f64(alibi_slopes)[h // r])")],
    "softcap_unscaled": [("attention", "S = softcap * np.tanh(S / softcap)", "S = np.tanh(S / softcap)")],
    "softcap_dropped": [("attention", "S = softcap * np.tanh(S / softcap)", "S = S")],
    "fp8_ties_away": [("fp8", "mag = np.rint(a / spacing) * spacing", "mag = np.floor(a / spacing + 0.5) * spacing")],
    "fp8_no_subnormals": [("fp8", "binade = np.maximum(E - 1, -6)", "binade = E - 1")],
    "fp8_bias_off": [("fp8", "return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)", "return sign * (1.0 + m / 8.0) * 2.0 ** (e - 8)")],
    "fp8_scale_loose": [("fp8", "return int(E - 9) if amax <= 0.875 * 2.0 ** E else int(E - 8)", "return int(E - 8)")],
    "fp8_scale_overflow": [("fp8", "return int(E - 9) if amax <= 0.875 * 2.0 ** E else int(E - 8)", "return int(E - 9)")],
    "fp8_no_signs": [("fp8", "return (x * s) @ H", "return x @ H")],
    "fp8_unnormalised": [("fp8", "eff = scale / D if signs is not None else scale", "eff = scale")],
    "fp8_one_scale": [("fp8", "blk = x32[idx][j * block_rows:(j + 1) * block_rows]\n            k = block_scale_exponent(float(np.abs(blk).max()) if blk.size else 0.0)",
                       "blk = x32[idx][j * block_rows:(j + 1) * block_rows]\n            k = block_scale_exponent(float(np.abs(x32).max()))")],
    "fp8_code_sign_dropped": [("fp8", "codes = np.where(normal, code_norm, code_sub) + np.where(neg, 0x80, 0)", "codes = np.where(normal, code_norm, code_sub)")],
    "varlen_top_left": [("varlen", "q_pos = (lk - lq) + np.arange(lq)", "q_pos = np.arange(lq)")],
    "varlen_keys_at_query_offset": [("varlen", "k[None, :, ks:ks + lk], v[None, :, ks:ks + lk]",
                                     "k[None, :, qs:qs + lk], v[None, :, qs:qs + lk]")],
    "varlen_head_map": [("varlen", "g = h // r", "g = h % Hkv")],
    "varlen_segment_short": [("varlen", "(int(cu[b]), int(cu[b + 1] - cu[b]))", "(int(cu[b]), int(cu[b + 1] - cu[b]) - 1)")],
    "packed_leak": [("varlen", "allowed = seg_q[:, None] == seg_k[None, :]", "allowed = seg_q[:, None] >= seg_k[None, :]")],
    "packed_top_left": [("varlen", "pos_q[qs:qs + lq] = (lk - lq) + np.arange(lq)", "pos_q[qs:qs + lq] = np.arange(lq)")],
    "lpt_ascending": [("varlen", "key=lambda b: (-cost[b], b)", "key=lambda b: (cost[b], b)")],
    "lpt_ties_reversed": [("varlen", "key=lambda b: (-cost[b], b)", "key=lambda b: (-cost[b], -b)")],
    "lpt_prefix_unsorted": [("varlen", "prefix.append(prefix[-1] + blocks[b])", "prefix.append(prefix[-1] + blocks[len(prefix) - 1])")],
    "lpt_cost_from_queries": [("varlen", "cost.append(-(-lk // kv_tile) if nqb else 0)", "cost.append(-(-lq // kv_tile) if nqb else 0)")],
    "lpt_empty_costs": [("varlen", "cost.append(-(-lk // kv_tile) if nqb else 0)", "cost.append(-(-lk // kv_tile))")],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutants(name):
    orc = oracle_namespace(MUTANTS[name])
    failed = []
    for check in CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(orc)
        except Exception:  # an assertion or a crash both count as caught
            failed.append(check.__name__)
    assert failed, f"mutant {name} survived every pin"
