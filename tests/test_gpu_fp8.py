"""GPU tests of the FP8 path: fa_quantize_fp8 and fa_fwd_fp8 against the
fp64 oracle (oracle/fp8.py).

* Quantization is integer work decided on exact values (the transform is
  exact in fp64, the scales are powers of two), so codes and scales must
  match the oracle bit for bit.
* The forward must match the oracle's attention of the same quantized Q and
  K (the dense definition on the dequantized values, V as given) within the
  forward's bar (tests/parity.py): the FP8 rounding is in both sides; what is
  left is the kernel's fp32 accumulation and bf16 probabilities, as for
  fa_fwd.
* Accuracy against the unquantized attention is reported, and the pages'
  experiment is repeated on the GPU: with outlier channels shared by Q and
  K, incoherent processing must cut the error well below block scales alone.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
from exact_attention_07_amd import binding, workloads as W
from tests.parity import compare, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    if not os.path.exists(binding.LIB_PATH):
        from exact_attention_07_amd import build
        build.build()
    binding.load_library()
    return torch.device("cuda:0")


def signs_of(seed, D):
    g = torch.Generator().manual_seed(seed)
    return (torch.randint(0, 2, (D,), generator=g) * 2 - 1).to(torch.float32)


def rows(seed, shape, outliers=0, mult=10.0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(*shape, generator=g)
    if outliers:
        ch = torch.randperm(shape[-1], generator=g)[:outliers]
        x[..., ch] *= mult
    return x.to(torch.bfloat16)


QUANT_CASES = [
    # B, H, L, D, block_rows, transform, outlier channels
    (1, 2, 300, 128, 64, False, 0),
    (1, 2, 300, 128, 64, True, 0),
    (2, 3, 513, 128, 256, True, 2),
    (1, 1, 77, 64, 64, True, 0),
    (2, 2, 130, 64, 256, False, 3),
    (1, 2, 700, 128, 300, True, 1),   # 19 slices of 16 rows: more than the registers hold
    (1, 1, 1300, 64, 600, True, 0),   # 19 slices of 32 rows
]


@pytest.mark.parametrize("case", QUANT_CASES, ids=lambda c: "x".join(map(str, c)))
def test_quantizer_matches_oracle(dev, case):
    B, H, L, D, R, tr, nout = case
    x = rows(40 + L + D, (B, H, L, D), nout)
    if L > 100:                           # an all-zero block and a block of tiny values
        x[0, 0, :min(R, L)] = 0
        x[-1, -1, -min(R, L):] = x[-1, -1, -min(R, L):] * 2.0 ** -30
    sg = signs_of(7 + D, D) if tr else None
    codes, scales = binding.quantize_fp8(x.to(dev), R, None if sg is None else sg.to(dev))
    torch.cuda.synchronize()
    rc, rs, _ = oracle.fp8.quantize_rows(x, R, None if sg is None else sg.numpy())
    assert np.array_equal(scales.cpu().numpy().astype(np.float64), rs), "block scales differ"
    got = codes.cpu().numpy()
    bad = np.argwhere(got != rc)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:4].tolist()}"


@pytest.mark.parametrize("D,R", [(128, 256), (128, 64), (64, 256)])
def test_quantizer_several_blocks_per_workgroup(dev, D, R):
    # The quantizer's workgroups take every grid-th block, each block's copy
    # in flight during the previous one and its codes stored during the next:
    # enough blocks that every workgroup runs at least three, the last block
    # of each head partial, bit for bit against the oracle.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    slices = -(-R // (64 // (D // 64)))
    grid = cus * (8 // min(slices, 8))
    H = 16
    nblk = -(-3 * grid // H) + 1                 # blocks per head
    L = nblk * R - R // 3                        # the last block of each head partial
    x = rows(2351 + D + R, (1, H, L, D), 1)
    sg = signs_of(31 + D, D)
    codes, scales = binding.quantize_fp8(x.to(dev), R, sg.to(dev))
    torch.cuda.synchronize()
    print(f"[fp8] quantizer D={D} block_rows={R}: {H * nblk} blocks on a grid of {grid}", flush=True)
    rc, rs, _ = oracle.fp8.quantize_rows(x, R, sg.numpy())
    assert np.array_equal(scales.cpu().numpy().astype(np.float64), rs), "block scales differ"
    bad = np.argwhere(codes.cpu().numpy() != rc)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:4].tolist()}"


FWD_CASES = [
    # B, Hq, Hkv, Lq, Lk, causal, kv_lens, transform
    (1, 2, 2, 64, 64, False, None, False),
    (2, 4, 2, 300, 333, False, None, True),
    (2, 4, 2, 300, 333, True, None, True),
    (2, 4, 2, 257, 300, True, "ragged", False),
    (3, 8, 2, 129, 190, False, "ragged", True),
    (2, 4, 4, 1, 500, False, "ragged", True),       # one query per head
    (1, 2, 2, 100, 60, True, None, True),           # more queries than keys: empty rows
]


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: "x".join(map(str, c[:6])) + f"_{c[6] is not None}_{c[7]}")
def test_fp8_forward_matches_oracle(dev, case, D):
    B, Hq, Hkv, Lq, Lk, causal, lens, tr = case
    c = W.random_case(1200 + Lq + Lk + (D == 64), B, Hq, Hkv, Lq, Lk, D, causal, lens)
    sg = signs_of(11, D) if tr else None
    kl = None if c.kv_lens is None else c.kv_lens.to(dev)
    o, lse = binding.attention_fp8(c.q.to(dev), c.k.to(dev), c.v.to(dev), causal=causal, scale=c.scale,
                                   kv_lens=kl, signs=None if sg is None else sg.to(dev))
    torch.cuda.synchronize()
    ro, rl, *_ = oracle.fp8.fp8_attention_forward(c.q, c.k, c.v, c.scale, causal, c.kv_lens,
                                                  None if sg is None else sg.numpy())
    m = compare(o, lse, ro, rl)
    print(f"[parity] fp8 D={D} {case}: {m}", flush=True)


@pytest.mark.parametrize("D", [128, 64])
def test_fp8_zero_length_and_nan_padding(dev, D):
    # Zero-length sequences give O = 0 and LSE = -inf; NaN in V rows past a
    # sequence's length is never read.  (K is quantized whole, padding rows
    # included, on both sides.)
    B, H, L = 3, 2, 96
    c = W.random_case(1300, B, H, H, L, L, D, True, [96, 0, 41])
    v = c.v.clone()
    v[2, :, 41:] = float("nan")
    sg = signs_of(13, D)
    o, lse = binding.attention_fp8(c.q.to(dev), c.k.to(dev), v.to(dev), causal=True, scale=c.scale,
                                   kv_lens=c.kv_lens.to(dev), signs=sg.to(dev))
    torch.cuda.synchronize()
    ro, rl, *_ = oracle.fp8.fp8_attention_forward(c.q, c.k, c.v, c.scale, True, c.kv_lens, sg.numpy())
    assert torch.all(o[1] == 0) and torch.all(torch.isneginf(lse[1]))
    compare(o, lse, ro, rl)


def test_fp8_accuracy_and_incoherent_processing(dev):
    # Against the unquantized attention of the same bf16 inputs; with outlier
    # channels shared by Q and K, the transform must cut the error at least
    # in half (FA3 reports 2.6x against per-tensor scales on its inputs).
    B, H, L, D = 1, 4, 1024, 128
    g = torch.Generator().manual_seed(1401)
    q, k, v = (torch.randn(B, H, L, D, generator=g) for _ in range(3))
    ch = torch.randperm(D, generator=g)[:2]
    q[..., ch] *= 10.0
    k[..., ch] *= 10.0
    q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    scale = 1.0 / np.sqrt(D) / 10.0
    ref, _ = oracle.attention_forward(q, k, v, scale, True)
    sg = signs_of(15, D)
    out = {}
    for name, s in (("block", None), ("block+incoherent", sg)):
        o, _ = binding.attention_fp8(q.to(dev), k.to(dev), v.to(dev), causal=True, scale=scale,
                                     signs=None if s is None else s.to(dev))
        torch.cuda.synchronize()
        out[name] = float(np.sqrt(np.mean((o.float().cpu().numpy() - ref) ** 2)))
    print(f"[accuracy] rmse vs unquantized attention: {out}", flush=True)
    assert out["block+incoherent"] * 2.0 < out["block"], out
    assert out["block+incoherent"] < 2e-2, out


@pytest.mark.parametrize("name", ["fp8_causal_b2_h16_l4096_d128", "fp8_gqa_causal_b1_hq32_hkv8_l16384_d128"])
def test_fp8_full_size_sampled_rows(dev, name):
    # The FP8 workloads at full size in the benchmark's launch configuration:
    # quantize with the transform, run the forward, and check sampled rows of
    # a few heads against the oracle on the same quantized values.
    w = W.BY_NAME[name]
    inp = W.make_inputs(w)
    sg = inp.meta["signs"]
    q8, qs = binding.quantize_fp8(inp.q.to(dev), binding.FP8_Q_BLOCK, sg.to(dev))
    k8, ks = binding.quantize_fp8(inp.k.to(dev), binding.FP8_K_BLOCK, sg.to(dev))
    eff = w.scale / w.D
    o, lse = binding.fa_fwd_fp8(q8, k8, inp.v.to(dev), qs, ks, causal=True, scale=eff)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    r = w.Hq // w.Hkv
    for (b, h) in ((0, 0), (w.B - 1, 9)):
        g = h // r
        rc, rsq, qv = oracle.fp8.quantize_rows(inp.q[b:b + 1, h:h + 1], binding.FP8_Q_BLOCK, sg.numpy())
        kc, rsk, kv = oracle.fp8.quantize_rows(inp.k[b:b + 1, g:g + 1], binding.FP8_K_BLOCK, sg.numpy())
        assert np.array_equal(q8[b, h].cpu().numpy(), rc[0, 0]) and np.array_equal(k8[b, g].cpu().numpy(), kc[0, 0])
        rr = sample_rows(w.Lq, 1500 + b * 16 + h)
        ro, rl = oracle.attention_rows(qv, kv, inp.v[b:b + 1, g:g + 1], eff, True, None, 0, 0, rows=rr)
        compare(o[b, h][rr], lse[b, h][rr], ro, rl)


def test_fp8_d64_long_causal_sampled_rows(dev):
    # D = 64 at a long causal shape (16 query blocks, 64 key tiles per
    # block at the end): codes of the checked heads bit-exact, sampled rows
    # (every query block and wavefront slot) against the oracle.
    B, H, L, D = 2, 4, 4096, 64
    c = W.random_case(1600, B, H, H, L, L, D, True, None)
    sg = signs_of(17, D)
    q8, qs = binding.quantize_fp8(c.q.to(dev), binding.FP8_Q_BLOCK, sg.to(dev))
    k8, ks = binding.quantize_fp8(c.k.to(dev), binding.FP8_K_BLOCK, sg.to(dev))
    eff = c.scale / D
    o, lse = binding.fa_fwd_fp8(q8, k8, c.v.to(dev), qs, ks, causal=True, scale=eff)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    for (b, h) in ((0, 0), (1, 3)):
        rc, _, qv = oracle.fp8.quantize_rows(c.q[b:b + 1, h:h + 1], binding.FP8_Q_BLOCK, sg.numpy())
        kc, _, kv = oracle.fp8.quantize_rows(c.k[b:b + 1, h:h + 1], binding.FP8_K_BLOCK, sg.numpy())
        assert np.array_equal(q8[b, h].cpu().numpy(), rc[0, 0]) and np.array_equal(k8[b, h].cpu().numpy(), kc[0, 0])
        rr = sample_rows(L, 1610 + b * 8 + h)
        ro, rl = oracle.attention_rows(qv, kv, c.v[b:b + 1, h:h + 1], eff, True, None, 0, 0, rows=rr)
        m = compare(o[b, h][rr], lse[b, h][rr], ro, rl)
        print(f"[parity] fp8 D=64 long causal (b={b}, h={h}): {m}", flush=True)


FUSED_CASES = [
    # B, Hq, Hkv, Lq, Lk, causal, kv_lens, transform
    (1, 2, 2, 64, 64, False, None, False),
    (2, 4, 2, 300, 333, True, None, True),
    (2, 4, 2, 257, 300, True, "ragged", False),
    (3, 8, 2, 129, 190, False, "ragged", True),
    (2, 4, 4, 1, 500, False, "ragged", True),       # one query per head
    (1, 2, 2, 100, 60, True, None, True),           # more queries than keys: empty rows
    (1, 4, 1, 700, 650, True, None, True),          # three query blocks, the last partial
]


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: "x".join(map(str, c[:6])) + f"_{c[6] is not None}_{c[7]}")
def test_fused_q_equals_quantize_then_forward(dev, case, D):
    # fa_fwd_fp8_q quantizes Q inside the forward with the block quantizer's
    # recipe (256-row blocks, the same transform and scale rule): outputs and
    # LSE equal bit for bit those of fa_quantize_fp8 on Q followed by
    # fa_fwd_fp8.  Q blocks of every scale regime: outlier channels, an
    # all-zero block (scale 1), a block of tiny values and one of large ones.
    B, Hq, Hkv, Lq, Lk, causal, lens, tr = case
    c = W.random_case(1500 + Lq + Lk + (D == 64), B, Hq, Hkv, Lq, Lk, D, causal, lens)
    q = rows(1600 + Lq + D, (B, Hq, Lq, D), 2)
    if Lq > 512:
        q[0, 0, :256] = 0
        q[0, 1, 256:512] = q[0, 1, 256:512] * 2.0 ** -40
        q[0, 2, 512:] = q[0, 2, 512:] * 2.0 ** 12      # scores within the documented range
    sg = signs_of(17 + D, D).to(dev) if tr else None
    q, k, v = q.to(dev), c.k.to(dev), c.v.to(dev)
    kl = None if c.kv_lens is None else c.kv_lens.to(dev)
    eff = c.scale / D if tr else c.scale
    q8, qs = binding.quantize_fp8(q, binding.FP8_Q_BLOCK, sg)
    k8, ks = binding.quantize_fp8(k, binding.FP8_K_BLOCK, sg)
    o1, l1 = binding.fa_fwd_fp8(q8, k8, v, qs, ks, causal=causal, scale=eff, kv_lens=kl)
    o2 = torch.full_like(q, float("nan"))
    l2 = torch.full((B, Hq, Lq), float("nan"), dtype=torch.float32, device=dev)
    binding.fa_fwd_fp8_q(q, k8, v, ks, sg, o2, l2, causal=causal, scale=eff, kv_lens=kl)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2), (o1 - o2).abs().max().item()
    assert torch.equal(l1.isnan(), l2.isnan()) and torch.equal(l1.nan_to_num(), l2.nan_to_num())
    if case == FUSED_CASES[1]:
        ro, rl, *_ = oracle.fp8.fp8_attention_forward(q.cpu(), c.k, c.v, c.scale, causal, c.kv_lens,
                                                      None if sg is None else sg.cpu().numpy())
        m = compare(o2.cpu(), l2.cpu(), ro, rl)
        print(f"[parity] fused-Q fp8 D={D} {case}: {m}", flush=True)


@pytest.mark.parametrize("D", [128, 64])
def test_fused_q_edge_cases(dev, D):
    # No keys at all (Lk = 0), and sequences of zero length beside full ones:
    # O = 0 and LSE = -inf on rows with no allowed key, from both paths alike;
    # attention_fp8's two forms agree bit for bit.
    sg = signs_of(19 + D, D).to(dev)
    q = rows(1700 + D, (2, 4, 40, D)).to(dev)
    k = torch.zeros(2, 2, 0, D, dtype=torch.bfloat16, device=dev)
    k8 = torch.zeros(2, 2, 0, D, dtype=torch.uint8, device=dev)
    ks = torch.zeros(2, 2, 0, dtype=torch.float32, device=dev)
    o, lse = binding.fa_fwd_fp8_q(q, k8, k.clone(), ks, sg, causal=False, scale=0.1)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    c = W.random_case(1710 + D, 3, 4, 2, 70, 90, D, True, [90, 0, 33])
    kl = c.kv_lens.to(dev)
    outs = [binding.attention_fp8(c.q.to(dev), c.k.to(dev), c.v.to(dev), causal=True, scale=c.scale, kv_lens=kl,
                                  signs=sg, quantize_q_in_kernel=f) for f in (False, True)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert torch.all(outs[1][0][1] == 0) and torch.all(torch.isneginf(outs[1][1][1]))


@pytest.mark.parametrize("name", ["fp8_causal_b2_h16_l4096_d128", "fp8_gqa_causal_b1_hq32_hkv8_l16384_d128"])
def test_fused_q_full_size_equals_quantize_then_forward(dev, name):
    # The FP8 workloads at full size: the fused-Q forward equals the two-step
    # path bit for bit (the two-step path is checked against the oracle above).
    w = W.BY_NAME[name]
    inp = W.make_inputs(w)
    sg = inp.meta["signs"].to(dev)
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    eff = w.scale / w.D
    q8, qs = binding.quantize_fp8(q, binding.FP8_Q_BLOCK, sg)
    k8, ks = binding.quantize_fp8(k, binding.FP8_K_BLOCK, sg)
    o1, l1 = binding.fa_fwd_fp8(q8, k8, v, qs, ks, causal=True, scale=eff)
    o2, l2 = binding.fa_fwd_fp8_q(q, k8, v, ks, sg, causal=True, scale=eff)
    torch.cuda.synchronize()
    print(f"[fp8] fused-Q {name}: max |dO| {(o1.float() - o2.float()).abs().max().item()}", flush=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
