"""Seeded random shapes through every entry point (forward, window, split
path, paged cache, modifiers, FP8, backward), each against the fp64
oracle at the bar of its own tests (tests/parity.py for forwards; the
backward bar of test_gpu_backward).

The shapes are drawn from a fixed seed: head dimension, batch, KV heads and
query heads per KV head, query and key lengths from 1 to a few hundred (so
tiles, query blocks and split partitions end raggedly), causal or not,
ragged or full lengths, windows, ALiBi slopes or a soft-cap.  Each case is
small enough for the oracle to finish in well under a second.  Window and
ALiBi cases use the variant bar of tests/parity.py.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
from exact_attention_07_amd import binding, workloads as W
from tests.parity import compare, variant_spread

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    if not os.path.exists(binding.LIB_PATH):
        from exact_attention_07_amd import build
        build.build()
    binding.load_library()
    return torch.device("cuda:0")


def draw(seed):
    """One random configuration: (B, Hq, Hkv, Lq, Lk, D, causal, lens)."""
    r = np.random.default_rng(seed)
    D = int(r.choice([64, 128]))
    B = int(r.integers(1, 4))
    Hkv = int(r.integers(1, 4))
    Hq = Hkv * int(r.choice([1, 2, 4]))
    Lk = int(r.integers(1, 400))
    Lq = int(r.choice([1, int(r.integers(1, 400)), Lk]))
    causal = bool(r.integers(0, 2))
    lens = "ragged" if r.integers(0, 2) else None
    return B, Hq, Hkv, Lq, Lk, D, causal, lens


SEEDS = list(range(7000, 7024))


@pytest.mark.parametrize("seed", SEEDS)
def test_random_forward(dev, seed):
    B, Hq, Hkv, Lq, Lk, D, causal, lens = draw(seed)
    c = W.random_case(seed, B, Hq, Hkv, Lq, Lk, D, causal, lens)
    kl = None if c.kv_lens is None else c.kv_lens.to(dev)
    o, lse = binding.fa_fwd(c.q.to(dev), c.k.to(dev), c.v.to(dev), causal=causal, scale=c.scale, kv_lens=kl)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_forward(c.q, c.k, c.v, c.scale, causal, c.kv_lens)
    m = compare(o, lse, ro, rl)
    print(f"[parity] random fwd {seed} {(B, Hq, Hkv, Lq, Lk, D, causal, lens)}: {m}", flush=True)


@pytest.mark.parametrize("seed", SEEDS[:12])
def test_random_window(dev, seed):
    B, Hq, Hkv, Lq, Lk, D, _, lens = draw(seed)
    w = int(np.random.default_rng(seed + 1).integers(1, Lk + 40))
    c = W.random_case(seed, B, Hq, Hkv, Lq, Lk, D, True, lens)
    kl = None if c.kv_lens is None else c.kv_lens.to(dev)
    o, lse = binding.fa_fwd_window(c.q.to(dev), c.k.to(dev), c.v.to(dev), w, scale=c.scale, kv_lens=kl)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_forward(c.q, c.k, c.v, c.scale, True, c.kv_lens, window=w)
    compare(o, lse, ro, rl, spread=variant_spread(c, window=w))


@pytest.mark.parametrize("seed", SEEDS[:12])
def test_random_modifiers(dev, seed):
    B, Hq, Hkv, Lq, Lk, D, causal, lens = draw(seed)
    c = W.random_case(seed, B, Hq, Hkv, Lq, Lk, D, causal, lens)
    kl = None if c.kv_lens is None else c.kv_lens.to(dev)
    g = torch.Generator().manual_seed(seed)
    if seed % 2:
        sl = (torch.rand(Hq, generator=g) * 0.5 + 0.005).to(torch.float32)
        o, lse = binding.fa_fwd_mod(c.q.to(dev), c.k.to(dev), c.v.to(dev), causal=causal, scale=c.scale,
                                    kv_lens=kl, alibi_slopes=sl.to(dev))
        torch.cuda.synchronize()
        ro, rl = oracle.attention_forward(c.q, c.k, c.v, c.scale, causal, c.kv_lens, alibi_slopes=sl.numpy())
        spread = variant_spread(c, alibi_slopes=sl.numpy())
    else:
        cap = float(1.0 + 9.0 * torch.rand(1, generator=g))
        q = (c.q.float() * 3).to(torch.bfloat16)
        o, lse = binding.fa_fwd_mod(q.to(dev), c.k.to(dev), c.v.to(dev), causal=causal, scale=c.scale,
                                    kv_lens=kl, softcap=cap)
        torch.cuda.synchronize()
        ro, rl = oracle.attention_forward(q, c.k, c.v, c.scale, causal, c.kv_lens, softcap=cap)
        spread = None
    compare(o, lse, ro, rl, spread=spread)


@pytest.mark.parametrize("seed", SEEDS[:12])
def test_random_fp8(dev, seed):
    B, Hq, Hkv, Lq, Lk, _, causal, lens = draw(seed)
    D = 128
    c = W.random_case(seed, B, Hq, Hkv, Lq, Lk, D, causal, lens)
    kl = None if c.kv_lens is None else c.kv_lens.to(dev)
    g = torch.Generator().manual_seed(seed)
    sg = (torch.randint(0, 2, (D,), generator=g) * 2 - 1).to(torch.float32) if seed % 3 else None
    o, lse = binding.attention_fp8(c.q.to(dev), c.k.to(dev), c.v.to(dev), causal=causal, scale=c.scale,
                                   kv_lens=kl, signs=None if sg is None else sg.to(dev))
    torch.cuda.synchronize()
    ro, rl, *_ = oracle.fp8.fp8_attention_forward(c.q, c.k, c.v, c.scale, causal, c.kv_lens,
                                                  None if sg is None else sg.numpy())
    compare(o, lse, ro, rl)


@pytest.mark.parametrize("seed", SEEDS[:12])
def test_random_backward(dev, seed):
    from tests.test_gpu_backward import compare_grad, run_case, untouched
    B, Hq, Hkv, Lq, Lk, D, causal, lens = draw(seed)
    Lq, Lk = min(Lq, 200), min(Lk, 200)
    w = int(np.random.default_rng(seed + 2).integers(1, Lk + 20)) if (causal and seed % 2) else 0
    c = W.random_case(seed, B, Hq, Hkv, Lq, Lk, D, causal, lens)
    g = torch.Generator().manual_seed(seed + 3)
    dout = torch.randn(B, Hq, Lq, D, generator=g).to(torch.bfloat16)
    dq, dk, dv = run_case(dev, c, dout, causal, w)
    rq, rk, rv = oracle.attention_backward(c.q, c.k, c.v, dout, c.scale, causal, c.kv_lens, window=w)
    zq, zk = untouched(c, causal, w)
    compare_grad("dq", dq, rq, exact_zero=zq)
    compare_grad("dk", dk, rk, exact_zero=zk)
    compare_grad("dv", dv, rv, exact_zero=zk)


@pytest.mark.parametrize("seed", SEEDS[:12])
def test_random_split_path(dev, seed):
    # Decode and short query chunks through fa_fwd_splits at a random
    # partition count (1 to 40).
    B, Hq, Hkv, _, Lk, D, causal, lens = draw(seed)
    r = np.random.default_rng(seed + 4)
    Lq = int(r.choice([1, 2, 5]))
    splits = int(r.integers(1, 41))
    c = W.random_case(seed, B, Hq, Hkv, Lq, Lk, D, causal, lens)
    kl = None if c.kv_lens is None else c.kv_lens.to(dev)
    o, lse = binding.fa_fwd_splits(c.q.to(dev), c.k.to(dev), c.v.to(dev), splits, causal=causal,
                                   scale=c.scale, kv_lens=kl)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_forward(c.q, c.k, c.v, c.scale, causal, c.kv_lens)
    compare(o, lse, ro, rl)


@pytest.mark.parametrize("seed", SEEDS[:12])
def test_random_paged(dev, seed):
    # A shuffled paged cache with a random page size (a multiple of 16),
    # decode or a short causal chunk, optionally under a window.
    B, Hq, Hkv, _, Lk, D, causal, _ = draw(seed)
    r = np.random.default_rng(seed + 5)
    P = 16 * int(r.integers(1, 9))
    Lq = 1 if not causal else int(r.choice([1, 3, 8]))
    w = int(r.integers(1, Lk + 30)) if (causal and r.integers(0, 2)) else 0
    c = W.random_case(seed, B, Hq, Hkv, Lq, Lk, D, causal, "ragged")
    kc, vc, table = W.page_kv(c.k, c.v, c.kv_lens, P, seed=seed)
    o, lse = binding.fa_fwd_paged(c.q.to(dev), kc.to(dev), vc.to(dev), table.to(dev), c.kv_lens.to(dev),
                                  causal=causal, window=w, scale=c.scale)
    torch.cuda.synchronize()
    ro, rl = oracle.paged_attention_forward(c.q, kc, vc, table, c.kv_lens, P, c.scale, causal, w)
    compare(o, lse, ro, rl, spread=variant_spread(c, window=w) if w else None)
