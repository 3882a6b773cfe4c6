"""GPU parity of the packed variable-length forward (fa_fwd_varlen) and of
its longest-tile-first schedule (fa_varlen_schedule) against the fp64
oracle (``oracle.varlen``), on the strict forward bar.

Covered: sequences of every length class (empty, one row, shorter than a
wavefront, ragged tails past 256-row blocks, more queries than keys and the
reverse), GQA with every head mapping (Hq a multiple of 8 with whole KV heads
per block, and not), D = 64 and 128, causal and not; the schedule against the
oracle's order integer for integer (including batches of more than one
schedule workgroup); a precomputed schedule, the library's own and schedules
in other orders giving identical bits; reordering the sequences, and the batched forward on
equal-length sequences, giving identical bits; the packed workload of the
benchmark on every row."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
from exact_attention_07_amd import binding, workloads as W
from tests.parity import compare, compare_varlen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    if not os.path.exists(binding.LIB_PATH):
        from exact_attention_07_amd import build
        build.build()
    binding.load_library()
    return torch.device("cuda:0")


def run(case, dev, schedule=None):
    cq = case.meta["cu_seqlens_q"].to(dev)
    ck = case.meta["cu_seqlens_k"].to(dev)
    o, lse = binding.fa_fwd_varlen(case.q.to(dev), case.k.to(dev), case.v.to(dev), cq, ck,
                                   schedule=schedule, causal=case.causal, scale=case.scale)
    torch.cuda.synchronize()
    return o, lse


CASES = [
    # lens_q, lens_k, Hq, Hkv, D, causal
    ([64], [64], 2, 2, 64, False),
    ([300, 17, 1, 513, 0, 256], [300, 17, 1, 513, 40, 256], 4, 2, 128, True),
    ([300, 17, 1, 513, 0, 256], [300, 17, 1, 513, 40, 256], 4, 2, 64, False),
    ([100, 260, 33], [60, 400, 33], 8, 2, 128, True),         # more queries than keys, and fewer
    ([129, 700, 5, 31], [129, 700, 0, 64], 16, 4, 64, True),  # Hq / 8 = 2 < r: plain head order
    ([257, 90, 640], [257, 190, 640], 16, 2, 128, True),      # Hq / 8 = 2, r = 8
    ([384, 200, 1000, 77], [384, 200, 1000, 77], 32, 8, 128, True),   # whole KV heads per block
    ([384, 200, 1000, 77], [500, 300, 1000, 77], 32, 4, 64, False),
    ([1] * 20, [300] * 20, 8, 8, 128, False),                 # one query per sequence
    ([0, 0, 50], [10, 0, 50], 6, 3, 64, True),                # sequences without queries or keys
]


@pytest.mark.parametrize("shape", CASES, ids=lambda s: f"B{len(s[0])}_h{s[2]}x{s[3]}_d{s[4]}_{'c' if s[5] else 'n'}")
def test_varlen_matches_oracle(dev, shape):
    lq, lk, Hq, Hkv, D, causal = shape
    case = W.varlen_case(2200 + sum(lq) + D + Hq, lq, lk, Hq, Hkv, D, causal)
    o, lse = run(case, dev)
    ref_o, ref_l = oracle.varlen.varlen_attention_forward(case.q, case.k, case.v, case.meta["cu_seqlens_q"],
                                                          case.meta["cu_seqlens_k"], case.scale, causal)
    compare(o, lse, ref_o, ref_l)


def test_schedule_matches_oracle_order(dev):
    r = np.random.default_rng(2301)
    for B in (1, 2, 16, 255, 256, 257, 700):
        lq = r.integers(0, 5000, B)
        lk = r.integers(0, 5000, B)
        lk[r.random(B) < 0.3] = 1280             # equal costs: ties resolved by index
        lq[r.random(B) < 0.05] = 0
        cq = torch.tensor(np.r_[0, np.cumsum(lq)], dtype=torch.int32)
        ck = torch.tensor(np.r_[0, np.cumsum(lk)], dtype=torch.int32)
        got = binding.fa_varlen_schedule(cq.to(dev), ck.to(dev), int(lq.sum()), int(lk.sum()))
        torch.cuda.synchronize()
        order, prefix = oracle.varlen.lpt_schedule(cq, ck, True)
        want = np.array(list(order) + list(prefix), dtype=np.int32)
        assert np.array_equal(got.cpu().numpy(), want), B


def test_precomputed_schedule_is_bitwise_the_same(dev):
    case = W.varlen_case(2311, [700, 64, 1500, 3, 300], [700, 64, 1500, 3, 300], 16, 4, 128, True)
    cq = case.meta["cu_seqlens_q"].to(dev)
    ck = case.meta["cu_seqlens_k"].to(dev)
    sched = binding.fa_varlen_schedule(cq, ck, case.q.shape[1], case.k.shape[1])
    o1, l1 = run(case, dev)
    o2, l2 = run(case, dev, schedule=sched)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_any_sequence_order_is_bitwise_the_same(dev):
    # A schedule in the given order (no sort) and one in the reverse of the
    # longest-tile-first order: same bits as the library's own schedule.
    lens_q = [700, 64, 1500, 3, 300, 0, 260]
    lens_k = [700, 90, 1500, 3, 300, 12, 900]
    case = W.varlen_case(2315, lens_q, lens_k, 32, 8, 128, True)
    o1, l1 = run(case, dev)
    order, _ = oracle.varlen.lpt_schedule(case.meta["cu_seqlens_q"], case.meta["cu_seqlens_k"], True)
    for seq in (list(range(len(lens_q))), list(order)[::-1]):
        blocks = [-(-lens_q[b] // 256) for b in seq]
        sched = torch.tensor(seq + [0] + list(np.cumsum(blocks)), dtype=torch.int32, device=dev)
        o2, l2 = run(case, dev, schedule=sched)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), seq


def test_reordering_sequences_is_bitwise_the_same(dev):
    # Each sequence's arithmetic does not depend on where it is packed or on
    # the order its blocks are scheduled in.
    lens = [900, 40, 1300, 256, 511]
    case = W.varlen_case(2321, lens, lens, 32, 8, 128, True)
    o, lse = run(case, dev)
    perm = [3, 0, 4, 2, 1]
    cu = case.meta["cu_seqlens_q"]
    pick = lambda t: torch.cat([t[:, int(cu[b]):int(cu[b + 1])] for b in perm], dim=1).contiguous()
    lp = [lens[b] for b in perm]
    cp = torch.zeros(len(lp) + 1, dtype=torch.int32)
    cp[1:] = torch.cumsum(torch.tensor(lp), 0)
    pc = W.Inputs(pick(case.q), pick(case.k), pick(case.v), None, case.scale, True,
                  {"cu_seqlens_q": cp, "cu_seqlens_k": cp.clone()})
    op, lp_ = run(pc, dev)
    for j, b in enumerate(perm):
        a0, a1 = int(cu[b]), int(cu[b + 1])
        p0, p1 = int(cp[j]), int(cp[j + 1])
        assert torch.equal(op[:, p0:p1], o[:, a0:a1]), b
        assert torch.equal(lp_[:, p0:p1], lse[:, a0:a1]), b


@pytest.mark.parametrize("D,causal", [(128, True), (64, False)])
def test_equal_lengths_match_the_batched_forward_bitwise(dev, D, causal):
    # Three sequences of 600 queries over 600 / 450 / 0 valid keys: the packed
    # call and fa_fwd with kv_lens compute the same rows the same way.
    B, Hq, Hkv, L = 3, 16, 4, 600
    lens_k = [600, 450, 0]
    c = W.random_case(2331 + D, B, Hq, Hkv, L, L, D, causal, lens_k)
    o_b, l_b = binding.fa_fwd(c.q.to(dev), c.k.to(dev), c.v.to(dev), causal=causal, scale=c.scale,
                              kv_lens=c.kv_lens.to(dev))
    q = c.q.permute(1, 0, 2, 3).reshape(Hq, B * L, D).contiguous()
    k = torch.cat([c.k[b, :, :n] for b, n in enumerate(lens_k)], dim=1).contiguous()
    v = torch.cat([c.v[b, :, :n] for b, n in enumerate(lens_k)], dim=1).contiguous()
    cq = torch.tensor([0, L, 2 * L, 3 * L], dtype=torch.int32)
    ck = torch.tensor(np.r_[0, np.cumsum(lens_k)], dtype=torch.int32)
    pc = W.Inputs(q, k, v, None, c.scale, causal, {"cu_seqlens_q": cq, "cu_seqlens_k": ck})
    o_v, l_v = run(pc, dev)
    assert torch.equal(o_v.reshape(Hq, B, L, D).permute(1, 0, 2, 3), o_b)
    assert torch.equal(l_v.reshape(Hq, B, L).permute(1, 0, 2), l_b)


def test_offsets_past_the_totals_are_clamped(dev):
    # The last offsets point past the packed rows: the device clamps them, so
    # the last sequence ends at the packed total and nothing outside the
    # tensors is touched.  The rows of the well-formed sequences are exact.
    lens = [300, 200]
    case = W.varlen_case(2341, lens, lens, 8, 2, 64, True)
    cq = torch.tensor([0, 300, 900], dtype=torch.int32)      # 900 > total_q = 500
    ck = torch.tensor([0, 300, 1 << 30], dtype=torch.int32)
    o, lse = binding.fa_fwd_varlen(case.q.to(dev), case.k.to(dev), case.v.to(dev), cq.to(dev), ck.to(dev),
                                   causal=True, scale=case.scale)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.varlen.varlen_attention_forward(case.q, case.k, case.v, case.meta["cu_seqlens_q"],
                                                          case.meta["cu_seqlens_k"], case.scale, True)
    compare(o, lse, ref_o, ref_l)


def test_no_queries_leaves_outputs_alone(dev):
    case = W.varlen_case(2351, [0, 0], [30, 0], 2, 1, 64, False)
    o = torch.full((2, 0, 64), 0.0, dtype=torch.bfloat16, device=dev)
    out, lse = binding.fa_fwd_varlen(case.q.to(dev), case.k.to(dev), case.v.to(dev),
                                     case.meta["cu_seqlens_q"].to(dev), case.meta["cu_seqlens_k"].to(dev), o=o)
    torch.cuda.synchronize()
    assert out.shape == (2, 0, 64) and lse.shape == (2, 0)


def test_packed_workload_every_row(dev):
    w = W.BY_NAME["varlen_causal_b16_hq32_hkv8_d128"]
    case = W.make_inputs(w)
    print(f"[varlen] {w.name}: lengths {case.meta['lens_q']}", flush=True)
    o, lse = run(case, dev)
    m = compare_varlen(case, o, lse, name=f"workload:{w.name}")
    assert m["rows"] == w.Hq * case.q.shape[1]
