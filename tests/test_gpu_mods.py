"""GPU parity of the score modifiers (fa_fwd_mod: ALiBi, soft-capping)
against the fp64 oracle.  Soft-capping uses the forward's bar; ALiBi, whose
steep slopes leave rows dominated by a few keys, uses the variant bar of
tests/parity.py (an element above 1e-2 must lie within the derived
bf16-probability bound).  The two modifier workloads are compared on every
row at full size."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
from exact_attention_07_amd import binding, workloads as W
from tests.parity import compare, compare_all_rows, variant_spread

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    if not os.path.exists(binding.LIB_PATH):
        from exact_attention_07_amd import build
        build.build()
    binding.load_library()
    return torch.device("cuda:0")


def slopes_for(Hq, seed):
    # Distinct slopes per query head (query heads sharing a KV head differ).
    g = torch.Generator().manual_seed(seed)
    return (torch.rand(Hq, generator=g) * 0.3 + 0.01).to(torch.float32)


CASES = [
    # B, Hq, Hkv, Lq, Lk, D, causal, kv_lens
    (1, 2, 2, 64, 64, 64, False, None),
    (2, 4, 2, 300, 333, 64, True, None),
    (2, 4, 2, 300, 333, 128, False, None),
    (2, 4, 2, 257, 300, 128, True, "ragged"),
    (3, 8, 2, 129, 190, 64, False, "ragged"),
    (2, 4, 4, 1, 500, 128, False, "ragged"),       # one query per head
    (1, 2, 2, 100, 60, 64, True, None),            # more queries than keys: empty rows
    (1, 2, 2, 300, 20, 64, True, None),            # a whole query block before the first key
    (3, 2, 2, 40, 50, 128, False, [0, 50, 7]),     # a sequence of length 0
]


@pytest.mark.parametrize("shape", CASES, ids=lambda s: "x".join(map(str, s[:7])) + f"_{s[7] is not None}")
def test_alibi_matches_oracle(dev, shape):
    B, Hq, Hkv, Lq, Lk, D, causal, lens = shape
    c = W.random_case(1600 + Lq + Lk + D, B, Hq, Hkv, Lq, Lk, D, causal, lens)
    sl = slopes_for(Hq, 1601 + Lq)
    kl = None if c.kv_lens is None else c.kv_lens.to(dev)
    o, lse = binding.fa_fwd_mod(c.q.to(dev), c.k.to(dev), c.v.to(dev), causal=causal, scale=c.scale,
                                kv_lens=kl, alibi_slopes=sl.to(dev))
    torch.cuda.synchronize()
    ro, rl = oracle.attention_forward(c.q, c.k, c.v, c.scale, causal, c.kv_lens, alibi_slopes=sl.numpy())
    m = compare(o, lse, ro, rl, spread=variant_spread(c, alibi_slopes=sl.numpy()))
    print(f"[parity] alibi {shape}: {m}", flush=True)


@pytest.mark.parametrize("cap", [2.0, 5.0])
@pytest.mark.parametrize("shape", CASES, ids=lambda s: "x".join(map(str, s[:7])) + f"_{s[7] is not None}")
def test_softcap_matches_oracle(dev, shape, cap):
    # Q x 3 so that the cap bites (scaled scores well beyond the cap).
    B, Hq, Hkv, Lq, Lk, D, causal, lens = shape
    c = W.random_case(1700 + Lq + Lk + D, B, Hq, Hkv, Lq, Lk, D, causal, lens)
    q = (c.q.float() * 3).to(torch.bfloat16)
    kl = None if c.kv_lens is None else c.kv_lens.to(dev)
    o, lse = binding.fa_fwd_mod(q.to(dev), c.k.to(dev), c.v.to(dev), causal=causal, scale=c.scale,
                                kv_lens=kl, softcap=cap)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_forward(q, c.k, c.v, c.scale, causal, c.kv_lens, softcap=cap)
    m = compare(o, lse, ro, rl)
    print(f"[parity] softcap {cap} {shape}: {m}", flush=True)


def test_no_modifier_is_the_plain_forward(dev):
    c = W.random_case(1800, 2, 4, 2, 300, 333, 128, True, "ragged")
    kl = c.kv_lens.to(dev)
    a = binding.fa_fwd_mod(c.q.to(dev), c.k.to(dev), c.v.to(dev), causal=True, scale=c.scale, kv_lens=kl)
    b = binding.fa_fwd(c.q.to(dev), c.k.to(dev), c.v.to(dev), causal=True, scale=c.scale, kv_lens=kl)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_masked_keys_stay_masked_under_softcap(dev):
    # The cap acts before the mask: future keys with huge values must not
    # leak in (their capped score would be finite).
    B, H, L, D = 1, 2, 96, 64
    c = W.random_case(1900, B, H, H, L, L, D, True, None)
    v = c.v.clone()
    v[..., 50:, :] = 1e4
    o, lse = binding.fa_fwd_mod(c.q.to(dev), c.k.to(dev), v.to(dev), causal=True, scale=c.scale, softcap=1.0)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_forward(c.q, c.k, v, c.scale, True, softcap=1.0)
    assert float(o[0, :, :50].abs().max()) < 10.0     # rows before 50 see no 1e4 value
    compare(o[:, :, :50], lse[:, :, :50], ro[:, :, :50], rl[:, :, :50])


@pytest.mark.parametrize("name", ["alibi_causal_b2_h16_l4096_d128", "softcap_prefill_b4_h16_l1024_d64"])
def test_modifier_workloads_every_row(dev, name):
    # The benchmark's workloads at full size, every row of every head.
    w = W.BY_NAME[name]
    inp = W.make_inputs(w)
    sl = inp.meta.get("alibi_slopes")
    o, lse = binding.fa_fwd_mod(inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), causal=w.causal, scale=w.scale,
                                alibi_slopes=None if sl is None else sl.to(dev), softcap=w.softcap)
    torch.cuda.synchronize()
    m = compare_all_rows(inp, o, lse, name=f"variant:{w.name}",
                         alibi_slopes=None if sl is None else sl.numpy(), softcap=w.softcap,
                         pbound=sl is not None)
    assert m["rows"] == w.B * w.Hq * w.Lq
