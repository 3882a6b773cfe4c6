"""GPU parity of the backward (fa_bwd) against the fp64 dense-gradient oracle.

The GPU forward provides o and lse (the backward's inputs); the oracle takes
only q, k, v and the upstream gradient and computes dQ, dK, dV from the
definition in fp64.

Tolerance, per gradient tensor (derived from the arithmetic): every output is
rounded to bf16 (relative 2^-9 at worst), the recomputed P and dS are rounded
to bf16 before their products, and delta uses the forward's bf16 output; with
independent roundings the relative L2 error is a small multiple of 2^-9 / 3^0.5
(about 2.3e-3 measured).  The bar is
  * relative L2 <= 5e-3;
  * max |error| <= 1e-2 * max |reference| + 1e-5 (the largest elements
    carry the largest absolute rounding; the floor covers gradients that are
    zero by cancellation, e.g. dQ with a single valid key, where P = 1 and
    dP = delta exactly, which the kernel reaches only up to the rounding of
    delta from the bf16 output, ~1e-6);
  * no NaN; exact zeros where the reference is exactly zero because no
    allowed pair touches the element (keys past the valid length, rows with no
    allowed key).
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
from exact_attention_07_amd import binding, workloads as W

pytestmark = pytest.mark.gpu

REL_L2 = 5e-3
MAX_REL = 1e-2
ABS_FLOOR = 1e-5


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    if not os.path.exists(binding.LIB_PATH):
        from exact_attention_07_amd import build
        build.build()
    binding.load_library()
    return torch.device("cuda:0")


def untouched(case, causal, window):
    """Boolean masks of the dQ rows [B, Hq, Lq, D] and dK/dV rows
    [B, Hkv, Lk, D] that no allowed pair touches (their gradient is exactly
    zero): rows with no allowed key, keys no query may see (past the valid
    length, or outside every query's window)."""
    B, Hq, Lq, D = case.q.shape
    Hkv, Lk = case.k.shape[1], case.k.shape[2]
    zq = np.zeros((B, Hq, Lq, D), dtype=bool)
    zk = np.zeros((B, Hkv, Lk, D), dtype=bool)
    for b in range(B):
        n = Lk if case.kv_lens is None else min(max(int(case.kv_lens[b]), 0), Lk)
        pos = (n - Lq) + np.arange(Lq)
        key = np.arange(Lk)
        allowed = np.broadcast_to(key[None, :] < n, (Lq, Lk)).copy()
        if causal:
            allowed &= key[None, :] <= pos[:, None]
        if window:
            allowed &= (pos[:, None] - key[None, :]) < window
        zq[b] = (~allowed.any(axis=1))[None, :, None]
        zk[b] = (~allowed.any(axis=0))[None, :, None]
    return zq, zk


def compare_grad(name, got, ref, exact_zero=None, rel_bar=REL_L2, abs_extra=0.0):
    g = got.float().cpu().numpy().astype(np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (name, g.shape, r.shape)
    assert not np.isnan(g).any(), f"NaN in {name}"
    if exact_zero is not None:
        assert np.all(g[exact_zero] == 0.0), f"{name}: nonzero where no pair contributes"
    err = np.abs(g - r)
    nr = np.linalg.norm(r)
    rel = float(np.linalg.norm(g - r) / nr) if nr > 0 else float(np.linalg.norm(g))
    mref = float(np.abs(r).max()) if r.size else 0.0
    mx = float(err.max()) if err.size else 0.0
    print(f"[parity] {name}: rel_l2={rel:.3g} max_abs={mx:.3g} max_ref={mref:.3g}", flush=True)
    assert rel <= rel_bar, f"{name}: relative L2 {rel:.3g} > {rel_bar:.3g}"
    lim = MAX_REL * mref + ABS_FLOOR + abs_extra
    assert mx <= lim, f"{name}: max abs {mx:.3g} > {MAX_REL} * {mref:.3g} + {ABS_FLOOR} + {abs_extra:.3g}"
    return rel, mx


def run_case(dev, case, dout, causal, window=0, k=None, v=None):
    q = case.q.to(dev)
    kd = (case.k if k is None else k).to(dev)
    vd = (case.v if v is None else v).to(dev)
    kl = None if case.kv_lens is None else case.kv_lens.to(dev)
    if window:
        o, lse = binding.fa_fwd_window(q, kd, vd, window, kv_lens=kl, scale=case.scale)
    else:
        o, lse = binding.fa_fwd(q, kd, vd, causal=causal, kv_lens=kl, scale=case.scale)
    dq, dk, dv = binding.fa_bwd(q, kd, vd, o, lse, dout.to(dev), causal=causal, window=window,
                                kv_lens=kl, scale=case.scale)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def upstream(seed, shape):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g).to(torch.bfloat16)


CASES = [
    # B, Hq, Hkv, Lq, Lk, D, causal, window, kv_lens
    (1, 2, 2, 64, 64, 64, False, 0, None),
    (2, 4, 2, 300, 333, 64, False, 0, None),
    (2, 4, 2, 300, 333, 64, True, 0, None),
    (2, 4, 2, 300, 333, 128, False, 0, None),
    (2, 4, 2, 300, 333, 128, True, 0, None),
    (2, 4, 2, 257, 300, 128, True, 0, "ragged"),
    (3, 8, 2, 129, 190, 64, False, 0, "ragged"),
    (1, 8, 2, 200, 200, 128, True, 50, None),
    (2, 4, 2, 150, 170, 64, True, 33, "ragged"),
    (2, 4, 4, 1, 500, 64, False, 0, "ragged"),     # one query per head (decode shape)
    (1, 2, 2, 100, 60, 64, True, 0, None),         # more queries than keys: empty rows
    (1, 2, 1, 520, 777, 128, False, 0, None),      # 25 KV tiles: a ragged end of the four-stage unroll
    (1, 4, 2, 600, 650, 128, True, 100, "ragged"),  # GQA, window, ragged, several query blocks
    (2, 4, 4, 1, 500, 128, False, 0, "ragged"),    # one query per head at D = 128
    (1, 2, 2, 100, 60, 128, True, 0, None),        # more queries than keys at D = 128
    (1, 12, 3, 87, 1, 128, False, 0, None),        # one key: dQ is zero by cancellation
]


@pytest.mark.parametrize("shape", CASES, ids=lambda s: "x".join(map(str, s[:8])) + f"_{s[8] is not None}")
def test_backward_small_cases(dev, shape):
    B, Hq, Hkv, Lq, Lk, D, causal, w, lens = shape
    case = W.random_case(900 + Lq + Lk + D + w, B, Hq, Hkv, Lq, Lk, D, causal, lens)
    dout = upstream(5 + Lq + w, (B, Hq, Lq, D))
    dq, dk, dv = run_case(dev, case, dout, causal, w)
    rq, rk, rv = oracle.attention_backward(case.q, case.k, case.v, dout, case.scale, causal,
                                           case.kv_lens, window=w)
    zq, zk = untouched(case, causal, w)
    compare_grad("dq", dq, rq, exact_zero=zq)
    compare_grad("dk", dk, rk, exact_zero=zk)
    compare_grad("dv", dv, rv, exact_zero=zk)


def test_backward_zero_length_and_nan_padding(dev):
    # Sequences of length 0 give all-zero gradients; NaN in K and V rows past
    # a sequence's length is never read.
    B, H, L, D = 3, 2, 96, 128
    case = W.random_case(950, B, H, H, L, L, D, True, [96, 0, 41])
    k, v = case.k.clone(), case.v.clone()
    k[2, :, 41:] = float("nan")
    v[2, :, 41:] = float("nan")
    dout = upstream(951, (B, H, L, D))
    dq, dk, dv = run_case(dev, case, dout, True, k=k, v=v)
    rq, rk, rv = oracle.attention_backward(case.q, case.k, case.v, dout, case.scale, True, case.kv_lens)
    assert torch.all(dq[1] == 0) and torch.all(dk[1] == 0) and torch.all(dv[1] == 0)
    assert torch.all(dk[2, :, 41:] == 0) and torch.all(dv[2, :, 41:] == 0)
    compare_grad("dq", dq, rq)
    compare_grad("dk", dk, rk)
    compare_grad("dv", dv, rv)


def test_backward_is_deterministic(dev):
    case = W.random_case(960, 2, 8, 2, 200, 230, 128, True, "ragged")
    dout = upstream(961, (2, 8, 200, 128))
    a = run_case(dev, case, dout, True)
    b = run_case(dev, case, dout, True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("D", [64, 128])
def test_backward_full_size_sampled_heads(dev, D):
    # The causal 4K workload's shape at D = 128 (and its D = 64 counterpart),
    # in the launch configuration the benchmark times; the oracle evaluates
    # whole heads densely, so a few (b, h) are checked (Hq = Hkv: each KV
    # head's gradient depends on its one query head only).
    B, H, L = 2, 16, 4096
    g = torch.Generator().manual_seed(970 + D)
    q = torch.randn(B, H, L, D, generator=g).to(torch.bfloat16)
    k = torch.randn(B, H, L, D, generator=g).to(torch.bfloat16)
    v = torch.randn(B, H, L, D, generator=g).to(torch.bfloat16)
    dout = torch.randn(B, H, L, D, generator=g).to(torch.bfloat16)
    scale = 1.0 / np.sqrt(D)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o, lse = binding.fa_fwd(qd, kd, vd, causal=True)
    dq, dk, dv = binding.fa_bwd(qd, kd, vd, o, lse, dout.to(dev), causal=True)
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    for (b, h) in ((0, 0), (1, 11)):
        rq, rk, rv = oracle.dense_backward_head(q[b, h], k[b, h], v[b, h], dout[b, h], scale, True)
        compare_grad(f"dq[{b},{h}]", dq[b, h], rq)
        compare_grad(f"dk[{b},{h}]", dk[b, h], rk)
        compare_grad(f"dv[{b},{h}]", dv[b, h], rv)
