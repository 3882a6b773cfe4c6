"""C-ABI checks that need no GPU: every declared symbol is exported, and host
validation rejects bad arguments with the documented status before any HIP
call (the pointers passed here are never dereferenced)."""
import ctypes
import os
import re

import pytest

from exact_attention_07_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from exact_attention_07_amd import build
        build.build()
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_binding_entry_points():
    assert declared_functions() == sorted(binding.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} missing from libfa.so"


P = ctypes.c_void_p(1 << 20)   # 16-byte aligned, never dereferenced: validation fails first
MIS = ctypes.c_void_p((1 << 20) + 2)


def call(lib, q=P, k=P, v=P, o=P, lse=None, B=1, Hq=2, Hkv=1, Lq=4, Lk=8, D=64, causal=0,
         scale=0.125, kv_lens=None, splits=None):
    args = [q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, causal, ctypes.c_float(scale), kv_lens, None]
    if splits is None:
        return lib.fa_fwd(*args)
    return lib.fa_fwd_splits(*args, splits)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), binding.FA_ERR_INVALID_ARG),
    (dict(o=None), binding.FA_ERR_INVALID_ARG),
    (dict(k=None), binding.FA_ERR_INVALID_ARG),
    (dict(B=0), binding.FA_ERR_INVALID_ARG),
    (dict(Lq=-1), binding.FA_ERR_INVALID_ARG),
    (dict(Lk=-1), binding.FA_ERR_INVALID_ARG),
    (dict(Hq=3, Hkv=2), binding.FA_ERR_INVALID_ARG),
    (dict(D=96), binding.FA_ERR_UNSUPPORTED),
    (dict(D=256), binding.FA_ERR_UNSUPPORTED),
    (dict(scale=float("nan")), binding.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), binding.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), binding.FA_ERR_INVALID_ARG),
    (dict(scale=-0.5), binding.FA_ERR_INVALID_ARG),
    (dict(q=MIS), binding.FA_ERR_INVALID_ARG),
    (dict(v=MIS), binding.FA_ERR_INVALID_ARG),
    (dict(lse=ctypes.c_void_p((1 << 20) + 1)), binding.FA_ERR_INVALID_ARG),
    (dict(causal=2), binding.FA_ERR_INVALID_ARG),
    (dict(splits=-1, D=96), binding.FA_ERR_UNSUPPORTED),
    (dict(Lq=1 << 20, D=128, Lk=1 << 15, B=1 << 12), binding.FA_ERR_INVALID_ARG),
])
def test_validation_rejects_before_any_launch(lib, kw, status):
    got = call(lib, **kw)
    assert got == status, (kw, got, lib.fa_last_error())
    assert lib.fa_last_error().decode() != ""


def test_negative_split_count_is_rejected(lib):
    # Sizes are valid, so validation reaches the split-count check; it fails before launching.
    assert call(lib, splits=-3) == binding.FA_ERR_INVALID_ARG


def test_split_path_rejects_packed_rows_past_32_bit_offsets(lib):
    # 32 query heads per KV head x 2^19 queries x 128 x 2 bytes = 2^32: the
    # packed rows of one KV head no longer fit the split kernels' 32-bit
    # buffer offsets, so the split path refuses before any launch.
    st = call(lib, B=1, Hq=32, Hkv=1, Lq=1 << 19, Lk=8, D=128, splits=1)
    assert st == binding.FA_ERR_INVALID_ARG
    assert b"32-bit" in lib.fa_last_error()


def test_status_strings(lib):
    assert lib.fa_status_string(0).decode() == "FA_OK"
    for s in (1, 2, 3):
        assert lib.fa_status_string(s).decode().startswith("FA_ERR_")
    assert lib.fa_status_string(99).decode() == "unknown fa_status"


def test_workspace_bytes(lib):
    # Prefill shapes use no workspace; invalid shapes report 0.
    assert lib.fa_workspace_bytes(4, 16, 16, 1024, 1024, 64) == 0
    assert lib.fa_workspace_bytes(1, 3, 2, 1, 8, 64) == 0
    # Decode: rows * splits * (D + 1) * 4 bytes, splits >= 1.
    ws = lib.fa_workspace_bytes(64, 32, 8, 1, 8192, 128)
    rows = 64 * 32
    assert ws > 0 and ws % (rows * 129 * 4) == 0
    assert ws // (rows * 129 * 4) <= 8192 // 32


def test_binding_requires_gpu_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        binding._prepare(q, q, q, None, None, None, True)


def call_window(lib, window, q=P, k=P, v=P, o=P, lse=None, B=1, Hq=2, Hkv=1, Lq=4, Lk=8, D=64,
                scale=0.125, kv_lens=None, splits=0):
    return lib.fa_fwd_window(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, window,
                             ctypes.c_float(scale), kv_lens, None, splits)


@pytest.mark.parametrize("kw,status", [
    (dict(window=-1), binding.FA_ERR_INVALID_ARG),
    (dict(window=4, D=96), binding.FA_ERR_UNSUPPORTED),
    (dict(window=4, splits=-1), binding.FA_ERR_INVALID_ARG),
    (dict(window=4, q=None), binding.FA_ERR_INVALID_ARG),
    (dict(window=4, scale=0.0), binding.FA_ERR_INVALID_ARG),
])
def test_window_validation(lib, kw, status):
    got = call_window(lib, **kw)
    assert got == status, (kw, got, lib.fa_last_error())
    assert lib.fa_last_error().decode() != ""


def call_paged(lib, q=P, kc=P, vc=P, o=P, lse=None, B=1, Hq=2, Hkv=1, Lq=1, D=64, table=P,
               max_pages=4, num_pages=8, page_size=16, kv_lens=P, causal=0, window=0,
               scale=0.125, splits=0):
    return lib.fa_fwd_paged(q, kc, vc, o, lse, B, Hq, Hkv, Lq, D, table, max_pages, num_pages,
                            page_size, kv_lens, causal, window, ctypes.c_float(scale), None, splits)


@pytest.mark.parametrize("kw,status", [
    (dict(table=None), binding.FA_ERR_INVALID_ARG),
    (dict(kv_lens=None), binding.FA_ERR_INVALID_ARG),
    (dict(kc=None), binding.FA_ERR_INVALID_ARG),
    (dict(page_size=8), binding.FA_ERR_INVALID_ARG),
    (dict(page_size=24), binding.FA_ERR_INVALID_ARG),
    (dict(page_size=0), binding.FA_ERR_INVALID_ARG),
    (dict(num_pages=0), binding.FA_ERR_INVALID_ARG),
    (dict(max_pages=0), binding.FA_ERR_INVALID_ARG),
    (dict(max_pages=1 << 20, page_size=1 << 12), binding.FA_ERR_INVALID_ARG),
    (dict(window=8), binding.FA_ERR_INVALID_ARG),            # a window needs causal
    (dict(window=-2, causal=1), binding.FA_ERR_INVALID_ARG),
    (dict(table=ctypes.c_void_p((1 << 20) + 2)), binding.FA_ERR_INVALID_ARG),
    (dict(kc=MIS), binding.FA_ERR_INVALID_ARG),
    (dict(D=80), binding.FA_ERR_UNSUPPORTED),
    (dict(Hq=3, Hkv=2), binding.FA_ERR_INVALID_ARG),
])
def test_paged_validation(lib, kw, status):
    got = call_paged(lib, **kw)
    assert got == status, (kw, got, lib.fa_last_error())
    assert lib.fa_last_error().decode() != ""


def test_paged_binding_requires_gpu_tensors():
    import torch
    q = torch.zeros(1, 1, 1, 64, dtype=torch.bfloat16)
    kc = torch.zeros(4, 1, 16, 64, dtype=torch.bfloat16)
    t = torch.zeros(1, 4, dtype=torch.int32)
    with pytest.raises(ValueError):
        binding._prepare_paged(q, kc, kc, t, t[0, :1], None, None, True)


def call_bwd(lib, q=P, k=P, v=P, o=P, lse=P, dout=P, dq=P, dk=P, dv=P, B=1, Hq=2, Hkv=1, Lq=4, Lk=8,
             D=64, causal=0, window=0, scale=0.125, kv_lens=None):
    return lib.fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Lq, Lk, D, causal, window,
                      ctypes.c_float(scale), kv_lens, None)


@pytest.mark.parametrize("kw,status", [
    (dict(o=None), binding.FA_ERR_INVALID_ARG),
    (dict(lse=None), binding.FA_ERR_INVALID_ARG),
    (dict(dout=None), binding.FA_ERR_INVALID_ARG),
    (dict(dq=None), binding.FA_ERR_INVALID_ARG),
    (dict(dk=None), binding.FA_ERR_INVALID_ARG),
    (dict(dv=MIS), binding.FA_ERR_INVALID_ARG),
    (dict(dout=MIS), binding.FA_ERR_INVALID_ARG),
    (dict(lse=ctypes.c_void_p((1 << 20) + 2)), binding.FA_ERR_INVALID_ARG),
    (dict(window=4), binding.FA_ERR_INVALID_ARG),
    (dict(window=-1, causal=1), binding.FA_ERR_INVALID_ARG),
    (dict(D=96), binding.FA_ERR_UNSUPPORTED),
    (dict(Hq=3, Hkv=2), binding.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), binding.FA_ERR_INVALID_ARG),
    (dict(causal=3), binding.FA_ERR_INVALID_ARG),
])
def test_backward_validation(lib, kw, status):
    got = call_bwd(lib, **kw)
    assert got == status, (kw, got, lib.fa_last_error())
    assert lib.fa_last_error().decode() != ""


def call_quant(lib, x=P, x8=P, scales=P, heads=2, L=100, D=128, block_rows=64, signs=None):
    return lib.fa_quantize_fp8(x, x8, scales, heads, L, D, block_rows, signs, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), binding.FA_ERR_INVALID_ARG),
    (dict(x8=None), binding.FA_ERR_INVALID_ARG),
    (dict(scales=None), binding.FA_ERR_INVALID_ARG),
    (dict(x8=MIS), binding.FA_ERR_INVALID_ARG),
    (dict(signs=ctypes.c_void_p((1 << 20) + 2)), binding.FA_ERR_INVALID_ARG),
    (dict(signs=ctypes.c_void_p((1 << 20) + 4)), binding.FA_ERR_INVALID_ARG),   # 4-byte aligned is not enough
    (dict(block_rows=0), binding.FA_ERR_INVALID_ARG),
    (dict(L=0), binding.FA_ERR_INVALID_ARG),
    (dict(heads=-1), binding.FA_ERR_INVALID_ARG),
    (dict(D=96), binding.FA_ERR_UNSUPPORTED),
])
def test_quantize_fp8_validation(lib, kw, status):
    got = call_quant(lib, **kw)
    assert got == status, (kw, got, lib.fa_last_error())
    assert lib.fa_last_error().decode() != ""


def call_fp8(lib, q8=P, k8=P, v=P, o=P, lse=P, qs=P, ks=P, B=1, Hq=2, Hkv=1, Lq=4, Lk=8, D=128,
             causal=0, scale=0.125, kv_lens=None):
    return lib.fa_fwd_fp8(q8, k8, v, o, lse, qs, ks, B, Hq, Hkv, Lq, Lk, D, causal,
                          ctypes.c_float(scale), kv_lens, None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=32), binding.FA_ERR_UNSUPPORTED),
    (dict(D=96), binding.FA_ERR_UNSUPPORTED),
    (dict(qs=None), binding.FA_ERR_INVALID_ARG),
    (dict(ks=None), binding.FA_ERR_INVALID_ARG),
    (dict(qs=ctypes.c_void_p((1 << 20) + 2)), binding.FA_ERR_INVALID_ARG),
    (dict(q8=None), binding.FA_ERR_INVALID_ARG),
    (dict(k8=MIS), binding.FA_ERR_INVALID_ARG),
    (dict(Hq=3, Hkv=2), binding.FA_ERR_INVALID_ARG),
    (dict(scale=-1.0), binding.FA_ERR_INVALID_ARG),
    (dict(causal=2), binding.FA_ERR_INVALID_ARG),
])
def test_fwd_fp8_validation(lib, kw, status):
    got = call_fp8(lib, **kw)
    assert got == status, (kw, got, lib.fa_last_error())
    assert lib.fa_last_error().decode() != ""


def call_fp8_q(lib, q=P, signs=None, k8=P, v=P, o=P, lse=P, ks=P, B=1, Hq=2, Hkv=1, Lq=4, Lk=8, D=128,
               causal=0, scale=0.125, kv_lens=None):
    return lib.fa_fwd_fp8_q(q, signs, k8, v, o, lse, ks, B, Hq, Hkv, Lq, Lk, D, causal,
                            ctypes.c_float(scale), kv_lens, None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=32), binding.FA_ERR_UNSUPPORTED),
    (dict(D=96), binding.FA_ERR_UNSUPPORTED),
    (dict(ks=None), binding.FA_ERR_INVALID_ARG),
    (dict(ks=ctypes.c_void_p((1 << 20) + 2)), binding.FA_ERR_INVALID_ARG),
    (dict(signs=ctypes.c_void_p((1 << 20) + 4)), binding.FA_ERR_INVALID_ARG),   # 16-byte alignment
    (dict(q=None), binding.FA_ERR_INVALID_ARG),
    (dict(q=MIS), binding.FA_ERR_INVALID_ARG),
    (dict(k8=None), binding.FA_ERR_INVALID_ARG),
    (dict(o=None), binding.FA_ERR_INVALID_ARG),
    (dict(Hq=3, Hkv=2), binding.FA_ERR_INVALID_ARG),
    (dict(scale=-1.0), binding.FA_ERR_INVALID_ARG),
    (dict(causal=2), binding.FA_ERR_INVALID_ARG),
])
def test_fwd_fp8_q_validation(lib, kw, status):
    got = call_fp8_q(lib, **kw)
    assert got == status, (kw, got, lib.fa_last_error())
    assert lib.fa_last_error().decode() != ""


def test_fp8_binding_requires_gpu_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        binding.quantize_fp8(x, 64)
    with pytest.raises(ValueError):
        binding._prepare_fp8(x.to(torch.uint8), x.to(torch.uint8), x, torch.zeros(1, 1, 1), torch.zeros(1, 1, 1),
                             None, None, None, True)
    with pytest.raises(ValueError):
        binding._prepare_fp8_q(x, x.to(torch.uint8), x, torch.zeros(1, 1, 1), None, None, None, None, True)


def call_mod(lib, q=P, k=P, v=P, o=P, lse=None, B=1, Hq=2, Hkv=1, Lq=4, Lk=8, D=64, causal=0,
             scale=0.125, kv_lens=None, slopes=None, softcap=0.0):
    return lib.fa_fwd_mod(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, causal, ctypes.c_float(scale),
                          kv_lens, slopes, ctypes.c_float(softcap), None)


@pytest.mark.parametrize("kw,status", [
    (dict(slopes=P, softcap=2.0), binding.FA_ERR_INVALID_ARG),     # both modifiers
    (dict(softcap=-1.0), binding.FA_ERR_INVALID_ARG),
    (dict(softcap=float("nan")), binding.FA_ERR_INVALID_ARG),
    (dict(softcap=float("inf")), binding.FA_ERR_INVALID_ARG),
    (dict(slopes=ctypes.c_void_p((1 << 20) + 2)), binding.FA_ERR_INVALID_ARG),
    (dict(slopes=P, D=96), binding.FA_ERR_UNSUPPORTED),
    (dict(softcap=1.0, q=None), binding.FA_ERR_INVALID_ARG),
    (dict(softcap=1.0, scale=0.0), binding.FA_ERR_INVALID_ARG),
])
def test_fwd_mod_validation(lib, kw, status):
    got = call_mod(lib, **kw)
    assert got == status, (kw, got, lib.fa_last_error())
    assert lib.fa_last_error().decode() != ""


def test_prefill_grid_past_32_bit_work_items_is_rejected(lib):
    # 2^17 sequences x 64 heads x one 256-row block = 2^23 workgroups of 512
    # threads = 2^32 work-items: more than the dispatch packet's 32-bit grid.
    st = call(lib, B=1 << 17, Hq=64, Hkv=64, Lq=2, Lk=8, D=64)
    assert st == binding.FA_ERR_INVALID_ARG
    assert b"grid" in lib.fa_last_error()


def call_varlen(lib, q=P, k=P, v=P, o=P, lse=None, cu_q=P, cu_k=P, schedule=None, B=2, Hq=2, Hkv=1,
                total_q=16, total_k=32, D=64, causal=0, scale=0.125):
    return lib.fa_fwd_varlen(q, k, v, o, lse, cu_q, cu_k, schedule, B, Hq, Hkv, total_q, total_k, D, causal,
                             ctypes.c_float(scale), None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), binding.FA_ERR_INVALID_ARG),
    (dict(B=(1 << 16) + 1), binding.FA_ERR_INVALID_ARG),
    (dict(total_q=-1), binding.FA_ERR_INVALID_ARG),
    (dict(total_k=-1), binding.FA_ERR_INVALID_ARG),
    (dict(cu_q=None), binding.FA_ERR_INVALID_ARG),
    (dict(cu_k=ctypes.c_void_p((1 << 20) + 2)), binding.FA_ERR_INVALID_ARG),
    (dict(schedule=ctypes.c_void_p((1 << 20) + 2)), binding.FA_ERR_INVALID_ARG),
    (dict(Hq=3, Hkv=2), binding.FA_ERR_INVALID_ARG),
    (dict(Hkv=0), binding.FA_ERR_INVALID_ARG),
    (dict(D=96), binding.FA_ERR_UNSUPPORTED),
    (dict(causal=2), binding.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), binding.FA_ERR_INVALID_ARG),
    (dict(q=None), binding.FA_ERR_INVALID_ARG),
    (dict(k=None), binding.FA_ERR_INVALID_ARG),
    (dict(o=MIS), binding.FA_ERR_INVALID_ARG),
    (dict(lse=ctypes.c_void_p((1 << 20) + 1)), binding.FA_ERR_INVALID_ARG),
    (dict(total_q=1 << 24, D=128), binding.FA_ERR_INVALID_ARG),          # 32-bit byte offsets
    (dict(total_k=1 << 24, D=128), binding.FA_ERR_INVALID_ARG),
    (dict(Hq=256, Hkv=256, total_q=1 << 23), binding.FA_ERR_INVALID_ARG),  # packed rows past int32
])
def test_varlen_validation(lib, kw, status):
    got = call_varlen(lib, **kw)
    assert got == status, (kw, got, lib.fa_last_error())
    assert lib.fa_last_error().decode() != ""


def test_varlen_without_queries_enqueues_nothing(lib):
    # total_q = 0: valid, nothing to compute; returns before any HIP call
    # and before the tensor pointers are looked at.
    assert call_varlen(lib, total_q=0) == binding.FA_OK
    assert call_varlen(lib, total_q=0, total_k=0, q=None, k=None, v=None, o=None) == binding.FA_OK
    # sizes are still validated first
    assert call_varlen(lib, total_q=0, D=96) == binding.FA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(B=0), dict(total_q=-1), dict(cu_q=None), dict(schedule=None),
                                dict(schedule=ctypes.c_void_p((1 << 20) + 2))])
def test_varlen_schedule_validation(lib, kw):
    args = dict(cu_q=P, cu_k=P, B=2, total_q=16, total_k=32, schedule=P)
    args.update(kw)
    got = lib.fa_varlen_schedule(args["cu_q"], args["cu_k"], args["B"], args["total_q"], args["total_k"],
                                 args["schedule"], None)
    assert got == binding.FA_ERR_INVALID_ARG, (kw, got)


def test_varlen_schedule_ints(lib):
    assert lib.fa_varlen_schedule_ints(1) == 3
    assert lib.fa_varlen_schedule_ints(16) == 33
    assert lib.fa_varlen_schedule_ints(0) == 0
    assert lib.fa_varlen_schedule_ints(1 << 17) == 0


def test_varlen_binding_requires_gpu_tensors():
    import torch
    x = torch.zeros(2, 8, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 8], dtype=torch.int32)
    with pytest.raises(ValueError):
        binding.fa_fwd_varlen(x, x, x, cu, cu)
