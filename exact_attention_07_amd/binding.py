"""ctypes binding of libfa.so: argument marshalling only.

Every step of the attention forward runs in the library's HIP kernels; this
module checks tensor properties, allocates outputs with torch when the caller
does not pass them, and forwards raw device pointers and sizes to the C ABI
declared in include/fa.h.  There is no fallback: if the library is missing
or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, 1, 2, 3

# Every entry point declared in include/fa.h.
EXPORTED = ("fa_fwd", "fa_fwd_splits", "fa_fwd_noalloc", "fa_noalloc_scratch_bytes",
            "fa_fwd_window", "fa_fwd_paged", "fa_bwd",
            "fa_fwd_mod", "fa_quantize_fp8", "fa_fwd_fp8", "fa_fwd_fp8_q",
            "fa_fwd_varlen", "fa_varlen_schedule", "fa_varlen_schedule_ints",
            "fa_workspace_bytes", "fa_status_string", "fa_last_error")

# Block sizes of the FP8 forward's scales (query rows, keys).
FP8_Q_BLOCK, FP8_K_BLOCK = 256, 64


class FaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lib = None


def load_library(path: Optional[str] = None):
    """Load libfa.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise FaError(-1, f"{path} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    fwd_args = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, vp, vp]
    lib.fa_fwd.argtypes = fwd_args
    lib.fa_fwd.restype = i32
    lib.fa_fwd_splits.argtypes = fwd_args + [i32]
    lib.fa_fwd_splits.restype = i32
    lib.fa_fwd_noalloc.argtypes = fwd_args + [i32]
    lib.fa_fwd_noalloc.restype = i32
    lib.fa_noalloc_scratch_bytes.argtypes = []
    lib.fa_noalloc_scratch_bytes.restype = ctypes.c_size_t
    # q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, window, scale, kv_lens, stream, num_splits
    lib.fa_fwd_window.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, vp, vp, i32]
    lib.fa_fwd_window.restype = i32
    # q, k_cache, v_cache, o, lse, B, Hq, Hkv, Lq, D, page_table, max_pages, num_pages,
    # page_size, kv_lens, causal, window, scale, stream, num_splits
    lib.fa_fwd_paged.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, i32, i32, i32,
                                 vp, i32, i32, f32, vp, i32]
    lib.fa_fwd_paged.restype = i32
    # q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Lq, Lk, D, causal, window, scale, kv_lens, stream
    lib.fa_bwd.argtypes = [vp] * 9 + [i32] * 8 + [f32, vp, vp]
    lib.fa_bwd.restype = i32
    # q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, causal, scale, kv_lens, alibi_slopes, softcap, stream
    lib.fa_fwd_mod.argtypes = fwd_args[:14] + [vp, f32, vp]
    lib.fa_fwd_mod.restype = i32
    # x, x8, scales, heads, L, D, block_rows, signs, stream
    lib.fa_quantize_fp8.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp]
    lib.fa_quantize_fp8.restype = i32
    # q8, k8, v, o, lse, q_scales, k_scales, B, Hq, Hkv, Lq, Lk, D, causal, scale, kv_lens, stream
    lib.fa_fwd_fp8.argtypes = [vp] * 7 + [i32] * 7 + [f32, vp, vp]
    lib.fa_fwd_fp8.restype = i32
    # q, signs, k8, v, o, lse, k_scales, B, Hq, Hkv, Lq, Lk, D, causal, scale, kv_lens, stream
    lib.fa_fwd_fp8_q.argtypes = [vp] * 7 + [i32] * 7 + [f32, vp, vp]
    lib.fa_fwd_fp8_q.restype = i32
    # q, k, v, o, lse, cu_q, cu_k, schedule, B, Hq, Hkv, total_q, total_k, D, causal, scale, stream
    lib.fa_fwd_varlen.argtypes = [vp] * 8 + [i32] * 7 + [f32, vp]
    lib.fa_fwd_varlen.restype = i32
    lib.fa_varlen_schedule.argtypes = [vp, vp, i32, i32, i32, vp, vp]
    lib.fa_varlen_schedule.restype = i32
    lib.fa_varlen_schedule_ints.argtypes = [i32]
    lib.fa_varlen_schedule_ints.restype = ctypes.c_size_t
    lib.fa_workspace_bytes.argtypes = [i32] * 6
    lib.fa_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_status_string.argtypes = [i32]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_last_error.argtypes = []
    lib.fa_last_error.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = lib
    return lib


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(status).decode()


def fa_workspace_bytes(B, Hq, Hkv, Lq, Lk, D) -> int:
    return int(load_library().fa_workspace_bytes(B, Hq, Hkv, Lq, Lk, D))


def _check(status: int):
    if status != FA_OK:
        lib = load_library()
        raise FaError(status, f"{lib.fa_status_string(status).decode()}: {lib.fa_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _prepare(q, k, v, o, lse, kv_lens, want_lse):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-D bfloat16 tensor [B, H, L, D]")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on the GPU")
    B, Hq, Lq, D = q.shape
    Bk, Hkv, Lk, Dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or Dk != D:
        raise ValueError("k and v must be [B, Hkv, Lk, D] with the batch and D of q")
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty(B, Hq, Lq, dtype=torch.float32, device=q.device)
    if kv_lens is not None:
        if kv_lens.dtype != torch.int32 or kv_lens.device != q.device or kv_lens.numel() != B \
                or not kv_lens.is_contiguous():
            raise ValueError("kv_lens must be a contiguous int32 device tensor of B entries")
    return o, lse, (B, Hq, Hkv, Lq, Lk, D)


def fa_fwd(q, k, v, o=None, lse=None, *, causal=False, scale=None, kv_lens=None,
           stream=None, want_lse=True):
    """O, LSE = attention(q, k, v) through ``fa_fwd``; returns (o, lse)."""
    o, lse, (B, Hq, Hkv, Lq, Lk, D) = _prepare(q, k, v, o, lse, kv_lens, want_lse)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    s = torch.cuda.current_stream(q.device).cuda_stream if stream is None else stream
    lib = load_library()
    _check(lib.fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Lq, Lk, D,
                      int(bool(causal)), scale, _ptr(kv_lens), s))
    return o, lse


class PreparedCall:
    """fa_fwd (or fa_fwd_splits, or fa_fwd_window when ``window`` is given)
    with its arguments checked and marshalled once.

    Calling the object enqueues the same forward again with no per-call
    Python checks (one ctypes call), for timing loops and serving loops where
    host overhead would otherwise exceed the kernel time.  The caller keeps
    the tensors alive and unchanged in shape."""

    def __init__(self, q, k, v, o=None, lse=None, *, causal=False, scale=None, kv_lens=None,
                 stream=None, want_lse=True, num_splits=None, window=None):
        o, lse, (B, Hq, Hkv, Lq, Lk, D) = _prepare(q, k, v, o, lse, kv_lens, want_lse)
        scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
        s = torch.cuda.current_stream(q.device).cuda_stream if stream is None else stream
        self.o, self.lse = o, lse
        self._keep = (q, k, v, o, lse, kv_lens)
        lib = load_library()
        if window is not None:
            self._fn = lib.fa_fwd_window
            self._args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Lq, Lk, D,
                          int(window), ctypes.c_float(scale), _ptr(kv_lens), s,
                          int(num_splits or 0))
        else:
            args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Lq, Lk, D,
                    int(bool(causal)), ctypes.c_float(scale), _ptr(kv_lens), s)
            if num_splits is None:
                self._fn, self._args = lib.fa_fwd, args
            else:
                self._fn, self._args = lib.fa_fwd_splits, args + (int(num_splits),)
        self()                                   # validate now: raises on a bad argument

    def __call__(self):
        status = self._fn(*self._args)
        if status != FA_OK:
            _check(status)
        return self.o, self.lse


def fa_fwd_splits(q, k, v, num_splits, o=None, lse=None, *, causal=False, scale=None,
                  kv_lens=None, stream=None, want_lse=True):
    """Same as fa_fwd through the split-KV path with at most ``num_splits`` partitions."""
    o, lse, (B, Hq, Hkv, Lq, Lk, D) = _prepare(q, k, v, o, lse, kv_lens, want_lse)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    s = torch.cuda.current_stream(q.device).cuda_stream if stream is None else stream
    lib = load_library()
    _check(lib.fa_fwd_splits(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Lq, Lk,
                             D, int(bool(causal)), scale, _ptr(kv_lens), s, int(num_splits)))
    return o, lse


def fa_fwd_noalloc(q, k, v, o, lse, *, num_splits=0, causal=False, scale=None, kv_lens=None,
                   stream=None):
    """fa_fwd_splits through ``fa_fwd_noalloc``: the split-KV workspace is the
    library's static scratch.  The caller passes ``o`` (and ``lse`` or None);
    nothing is allocated here or in the library."""
    if o is None:
        raise ValueError("fa_fwd_noalloc needs the output tensor o (it allocates nothing)")
    o, lse, (B, Hq, Hkv, Lq, Lk, D) = _prepare(q, k, v, o, lse, kv_lens, lse is not None)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    s = torch.cuda.current_stream(q.device).cuda_stream if stream is None else stream
    lib = load_library()
    _check(lib.fa_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Lq, Lk,
                              D, int(bool(causal)), scale, _ptr(kv_lens), s, int(num_splits)))
    return o, lse


def fa_noalloc_scratch_bytes() -> int:
    return int(load_library().fa_noalloc_scratch_bytes())


def fa_fwd_window(q, k, v, window, o=None, lse=None, *, scale=None, kv_lens=None, stream=None,
                  want_lse=True, num_splits=0):
    """Causal attention with a window of ``window`` keys (0 = plain causal)
    through ``fa_fwd_window``; returns (o, lse)."""
    o, lse, (B, Hq, Hkv, Lq, Lk, D) = _prepare(q, k, v, o, lse, kv_lens, want_lse)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    s = torch.cuda.current_stream(q.device).cuda_stream if stream is None else stream
    lib = load_library()
    _check(lib.fa_fwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Lq, Lk,
                             D, int(window), scale, _ptr(kv_lens), s, int(num_splits)))
    return o, lse


def _prepare_paged(q, k_cache, v_cache, page_table, kv_lens, o, lse, want_lse):
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        if t.dtype != torch.bfloat16 or t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-D bfloat16 tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on the GPU")
    B, Hq, Lq, D = q.shape
    num_pages, Hkv, page_size, Dk = k_cache.shape
    if tuple(v_cache.shape) != tuple(k_cache.shape) or Dk != D:
        raise ValueError("k_cache and v_cache must be [num_pages, Hkv, page_size, D] with the D of q")
    for name, t in (("page_table", page_table), ("kv_lens", kv_lens)):
        if t is None or t.dtype != torch.int32 or t.device != q.device or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 device tensor")
    if page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("page_table must be [B, max_pages]")
    if kv_lens.numel() != B:
        raise ValueError("kv_lens must hold B entries")
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty(B, Hq, Lq, dtype=torch.float32, device=q.device)
    return o, lse, (B, Hq, Hkv, Lq, D, page_table.shape[1], num_pages, page_size)


def fa_fwd_paged(q, k_cache, v_cache, page_table, kv_lens, o=None, lse=None, *, causal=False,
                 window=0, scale=None, stream=None, want_lse=True, num_splits=0):
    """Attention against a paged cache [num_pages, Hkv, page_size, D] through
    ``fa_fwd_paged``; ``page_table`` is int32 [B, max_pages]; returns (o, lse)."""
    o, lse, (B, Hq, Hkv, Lq, D, max_pages, num_pages, page_size) = _prepare_paged(
        q, k_cache, v_cache, page_table, kv_lens, o, lse, want_lse)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    s = torch.cuda.current_stream(q.device).cuda_stream if stream is None else stream
    lib = load_library()
    _check(lib.fa_fwd_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse), B, Hq, Hkv,
                            Lq, D, _ptr(page_table), max_pages, num_pages, page_size,
                            _ptr(kv_lens), int(bool(causal)), int(window), scale, s,
                            int(num_splits)))
    return o, lse


class PreparedPagedCall:
    """fa_fwd_paged with its arguments checked and marshalled once (see
    PreparedCall)."""

    def __init__(self, q, k_cache, v_cache, page_table, kv_lens, o=None, lse=None, *,
                 causal=False, window=0, scale=None, stream=None, want_lse=True, num_splits=0):
        o, lse, (B, Hq, Hkv, Lq, D, max_pages, num_pages, page_size) = _prepare_paged(
            q, k_cache, v_cache, page_table, kv_lens, o, lse, want_lse)
        scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
        s = torch.cuda.current_stream(q.device).cuda_stream if stream is None else stream
        self.o, self.lse = o, lse
        self._keep = (q, k_cache, v_cache, page_table, kv_lens, o, lse)
        self._fn = load_library().fa_fwd_paged
        self._args = (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse), B, Hq, Hkv, Lq,
                      D, _ptr(page_table), max_pages, num_pages, page_size, _ptr(kv_lens),
                      int(bool(causal)), int(window), ctypes.c_float(scale), s, int(num_splits))
        self()

    def __call__(self):
        status = self._fn(*self._args)
        if status != FA_OK:
            _check(status)
        return self.o, self.lse


def fa_bwd(q, k, v, o, lse, dout, dq=None, dk=None, dv=None, *, causal=False, window=0, scale=None,
           kv_lens=None, stream=None):
    """dQ, dK, dV of the attention forward through ``fa_bwd``; ``o`` and ``lse``
    are the forward's outputs for the same arguments.  Returns (dq, dk, dv)."""
    _, _, (B, Hq, Hkv, Lq, Lk, D) = _prepare(q, k, v, o, lse, kv_lens, True)
    for name, t in (("o", o), ("dout", dout)):
        if t is None or t.dtype != torch.bfloat16 or tuple(t.shape) != tuple(q.shape) \
                or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous bf16 device tensor shaped like q")
    if lse is None or lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Lq) \
            or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous fp32 device tensor [B, Hq, Lq]")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    s = torch.cuda.current_stream(q.device).cuda_stream if stream is None else stream
    _check(load_library().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                 _ptr(dq), _ptr(dk), _ptr(dv), B, Hq, Hkv, Lq, Lk, D,
                                 int(bool(causal)), int(window), scale, _ptr(kv_lens), s))
    return dq, dk, dv


class PreparedBwdCall:
    """fa_bwd with its arguments checked and marshalled once (see PreparedCall)."""

    def __init__(self, q, k, v, o, lse, dout, *, causal=False, window=0, scale=None, kv_lens=None,
                 stream=None):
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, causal=causal, window=window, scale=scale,
               kv_lens=kv_lens, stream=stream)               # validates; raises on a bad argument
        D = q.shape[3]
        scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
        s = torch.cuda.current_stream(q.device).cuda_stream if stream is None else stream
        self.grads = (dq, dk, dv)
        self._keep = (q, k, v, o, lse, dout, dq, dk, dv, kv_lens)
        self._fn = load_library().fa_bwd
        self._args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                      _ptr(dv), q.shape[0], q.shape[1], k.shape[1], q.shape[2], k.shape[2], D,
                      int(bool(causal)), int(window), ctypes.c_float(scale), _ptr(kv_lens), s)

    def __call__(self):
        status = self._fn(*self._args)
        if status != FA_OK:
            _check(status)
        return self.grads


def quantize_fp8(x, block_rows, signs=None, stream=None):
    """E4M3 codes and block scales of the rows of ``x`` [B, H, L, D] (bf16)
    through ``fa_quantize_fp8``; ``signs`` (D values +-1, fp32 device tensor)
    applies the Hadamard transform with those sign flips first.  Returns
    (codes uint8 [B, H, L, D], scales fp32 [B, H, ceil(L / block_rows)])."""
    if x.dtype != torch.bfloat16 or x.dim() != 4 or not x.is_contiguous() or x.device.type != "cuda":
        raise ValueError("x must be a contiguous 4-D bfloat16 GPU tensor [B, H, L, D]")
    B, H, L, D = x.shape
    if signs is not None and (signs.dtype != torch.float32 or signs.numel() != D
                              or signs.device != x.device or not signs.is_contiguous()):
        raise ValueError("signs must be a contiguous fp32 device tensor of D entries")
    codes = torch.empty(B, H, L, D, dtype=torch.uint8, device=x.device)
    scales = torch.empty(B, H, -(-L // block_rows), dtype=torch.float32, device=x.device)
    s = torch.cuda.current_stream(x.device).cuda_stream if stream is None else stream
    _check(load_library().fa_quantize_fp8(_ptr(x), _ptr(codes), _ptr(scales), B * H, L, D,
                                          int(block_rows), _ptr(signs), s))
    return codes, scales


def _prepare_fp8(q8, k8, v, q_scales, k_scales, o, lse, kv_lens, want_lse):
    for name, t in (("q8", q8), ("k8", k8)):
        if t.dtype != torch.uint8 or t.dim() != 4 or not t.is_contiguous() or t.device.type != "cuda":
            raise ValueError(f"{name} must be a contiguous 4-D uint8 GPU tensor of E4M3 codes")
    if v.dtype != torch.bfloat16 or not v.is_contiguous() or v.device != q8.device:
        raise ValueError("v must be a contiguous bf16 device tensor")
    B, Hq, Lq, D = q8.shape
    _, Hkv, Lk, _ = k8.shape
    if tuple(v.shape) != tuple(k8.shape) or k8.shape[0] != B or k8.shape[3] != D:
        raise ValueError("k8 and v must be [B, Hkv, Lk, D] with the batch and D of q8")
    for name, t, shape in (("q_scales", q_scales, (B, Hq, -(-Lq // FP8_Q_BLOCK))),
                           ("k_scales", k_scales, (B, Hkv, -(-Lk // FP8_K_BLOCK)))):
        if t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous() \
                or t.device != q8.device:
            raise ValueError(f"{name} must be a contiguous fp32 device tensor {shape}")
    if kv_lens is not None and (kv_lens.dtype != torch.int32 or kv_lens.numel() != B
                                or kv_lens.device != q8.device or not kv_lens.is_contiguous()):
        raise ValueError("kv_lens must be a contiguous int32 device tensor of B entries")
    o = torch.empty(B, Hq, Lq, D, dtype=torch.bfloat16, device=q8.device) if o is None else o
    if lse is None and want_lse:
        lse = torch.empty(B, Hq, Lq, dtype=torch.float32, device=q8.device)
    return o, lse, (B, Hq, Hkv, Lq, Lk, D)


def fa_fwd_fp8(q8, k8, v, q_scales, k_scales, o=None, lse=None, *, causal=False, scale=None,
               kv_lens=None, stream=None, want_lse=True):
    """Attention with FP8 scores through ``fa_fwd_fp8``: q8, k8 are E4M3 codes
    with block scales (256 query rows, 64 keys) as from ``quantize_fp8``;
    S = scale * (q8 sq)(k8 sk)^T.  Returns (o, lse)."""
    o, lse, (B, Hq, Hkv, Lq, Lk, D) = _prepare_fp8(q8, k8, v, q_scales, k_scales, o, lse, kv_lens,
                                                   want_lse)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    s = torch.cuda.current_stream(q8.device).cuda_stream if stream is None else stream
    _check(load_library().fa_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v), _ptr(o), _ptr(lse), _ptr(q_scales),
                                      _ptr(k_scales), B, Hq, Hkv, Lq, Lk, D, int(bool(causal)), scale,
                                      _ptr(kv_lens), s))
    return o, lse


def attention_fp8(q, k, v, *, causal=False, scale=None, kv_lens=None, signs=None, stream=None,
                  quantize_q_in_kernel=False):
    """bf16 Q, K, V -> FP8 attention: Q and K block-quantized (after the
    Hadamard transform with ``signs`` when given, whose factor D in the
    scores is divided out of the scale), then ``fa_fwd_fp8``; with
    ``quantize_q_in_kernel`` K alone is quantized first and
    ``fa_fwd_fp8_q`` quantizes Q inside the forward (the same result, bit
    for bit).  Returns (o, lse)."""
    D = q.shape[3]
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    k8, ks = quantize_fp8(k, FP8_K_BLOCK, signs, stream)
    eff = scale / D if signs is not None else scale
    if quantize_q_in_kernel:
        return fa_fwd_fp8_q(q, k8, v, ks, signs, causal=causal, scale=eff, kv_lens=kv_lens, stream=stream)
    q8, qs = quantize_fp8(q, FP8_Q_BLOCK, signs, stream)
    return fa_fwd_fp8(q8, k8, v, qs, ks, causal=causal, scale=eff, kv_lens=kv_lens, stream=stream)


class PreparedFp8Call:
    """fa_fwd_fp8 with its arguments checked and marshalled once (see PreparedCall)."""

    def __init__(self, q8, k8, v, q_scales, k_scales, *, causal=False, scale=None, kv_lens=None,
                 stream=None):
        o, lse, (B, Hq, Hkv, Lq, Lk, D) = _prepare_fp8(q8, k8, v, q_scales, k_scales, None, None,
                                                       kv_lens, True)
        scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
        s = torch.cuda.current_stream(q8.device).cuda_stream if stream is None else stream
        self.o, self.lse = o, lse
        self._keep = (q8, k8, v, q_scales, k_scales, kv_lens)
        self._fn = load_library().fa_fwd_fp8
        self._args = (_ptr(q8), _ptr(k8), _ptr(v), _ptr(o), _ptr(lse), _ptr(q_scales), _ptr(k_scales),
                      B, Hq, Hkv, Lq, Lk, D, int(bool(causal)), ctypes.c_float(scale), _ptr(kv_lens), s)
        self()

    def __call__(self):
        status = self._fn(*self._args)
        if status != FA_OK:
            _check(status)
        return self.o, self.lse


def _prepare_fp8_q(q, k8, v, k_scales, signs, o, lse, kv_lens, want_lse):
    if q.dtype != torch.bfloat16 or q.dim() != 4 or not q.is_contiguous() or q.device.type != "cuda":
        raise ValueError("q must be a contiguous 4-D bfloat16 GPU tensor [B, Hq, Lq, D]")
    if k8.dtype != torch.uint8 or k8.dim() != 4 or not k8.is_contiguous() or k8.device != q.device:
        raise ValueError("k8 must be a contiguous 4-D uint8 device tensor of E4M3 codes")
    if v.dtype != torch.bfloat16 or not v.is_contiguous() or v.device != q.device:
        raise ValueError("v must be a contiguous bf16 device tensor")
    B, Hq, Lq, D = q.shape
    _, Hkv, Lk, _ = k8.shape
    if tuple(v.shape) != tuple(k8.shape) or k8.shape[0] != B or k8.shape[3] != D:
        raise ValueError("k8 and v must be [B, Hkv, Lk, D] with the batch and D of q")
    shape = (B, Hkv, -(-Lk // FP8_K_BLOCK))
    if (k_scales.dtype != torch.float32 or tuple(k_scales.shape) != shape or not k_scales.is_contiguous()
            or k_scales.device != q.device):
        raise ValueError(f"k_scales must be a contiguous fp32 device tensor of shape {shape}")
    if signs is not None and (signs.dtype != torch.float32 or signs.numel() != D
                              or signs.device != q.device or not signs.is_contiguous()):
        raise ValueError("signs must be a contiguous fp32 device tensor of D entries")
    if kv_lens is not None and (kv_lens.dtype != torch.int32 or kv_lens.device != q.device):
        raise ValueError("kv_lens must be an int32 device tensor")
    o = torch.empty_like(q) if o is None else o
    if lse is None and want_lse:
        lse = torch.empty(B, Hq, Lq, dtype=torch.float32, device=q.device)
    return o, lse, (B, Hq, Hkv, Lq, Lk, D)


def fa_fwd_fp8_q(q, k8, v, k_scales, signs=None, o=None, lse=None, *, causal=False, scale=None,
                 kv_lens=None, stream=None, want_lse=True):
    """Attention with FP8 scores and Q quantized in the kernel through
    ``fa_fwd_fp8_q``: q is bf16; k8 and k_scales come from ``quantize_fp8``
    with 64-row blocks and the same ``signs``.  Equal bit for bit to
    ``quantize_fp8(q, 256, signs)`` followed by ``fa_fwd_fp8``.  Returns (o, lse)."""
    o, lse, (B, Hq, Hkv, Lq, Lk, D) = _prepare_fp8_q(q, k8, v, k_scales, signs, o, lse, kv_lens, want_lse)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    s = torch.cuda.current_stream(q.device).cuda_stream if stream is None else stream
    _check(load_library().fa_fwd_fp8_q(_ptr(q), _ptr(signs), _ptr(k8), _ptr(v), _ptr(o), _ptr(lse),
                                        _ptr(k_scales), B, Hq, Hkv, Lq, Lk, D, int(bool(causal)), scale,
                                        _ptr(kv_lens), s))
    return o, lse


class PreparedFp8QCall:
    """fa_fwd_fp8_q with its arguments checked and marshalled once (see PreparedCall)."""

    def __init__(self, q, k8, v, k_scales, signs=None, *, causal=False, scale=None, kv_lens=None,
                 stream=None):
        o, lse, (B, Hq, Hkv, Lq, Lk, D) = _prepare_fp8_q(q, k8, v, k_scales, signs, None, None, kv_lens, True)
        scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
        s = torch.cuda.current_stream(q.device).cuda_stream if stream is None else stream
        self.o, self.lse = o, lse
        self._keep = (q, k8, v, k_scales, signs, kv_lens)
        self._fn = load_library().fa_fwd_fp8_q
        self._args = (_ptr(q), _ptr(signs), _ptr(k8), _ptr(v), _ptr(o), _ptr(lse), _ptr(k_scales),
                      B, Hq, Hkv, Lq, Lk, D, int(bool(causal)), ctypes.c_float(scale), _ptr(kv_lens), s)
        self()

    def __call__(self):
        status = self._fn(*self._args)
        if status != FA_OK:
            _check(status)
        return self.o, self.lse


def _mod_args(q, alibi_slopes, softcap):
    Hq = q.shape[1]
    if alibi_slopes is not None and (alibi_slopes.dtype != torch.float32 or alibi_slopes.numel() != Hq
                                     or alibi_slopes.device != q.device or not alibi_slopes.is_contiguous()):
        raise ValueError("alibi_slopes must be a contiguous fp32 device tensor of Hq entries")
    return _ptr(alibi_slopes), float(softcap)


def fa_fwd_mod(q, k, v, o=None, lse=None, *, causal=False, scale=None, kv_lens=None, alibi_slopes=None,
               softcap=0.0, stream=None, want_lse=True):
    """Attention with a score modifier through ``fa_fwd_mod``: ALiBi
    (``alibi_slopes``, [Hq] fp32) or soft-capping (``softcap`` > 0).
    Returns (o, lse)."""
    o, lse, (B, Hq, Hkv, Lq, Lk, D) = _prepare(q, k, v, o, lse, kv_lens, want_lse)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    sp, cap = _mod_args(q, alibi_slopes, softcap)
    s = torch.cuda.current_stream(q.device).cuda_stream if stream is None else stream
    _check(load_library().fa_fwd_mod(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Lq, Lk, D,
                                      int(bool(causal)), scale, _ptr(kv_lens), sp, cap, s))
    return o, lse


class PreparedModCall:
    """fa_fwd_mod with its arguments checked and marshalled once (see PreparedCall)."""

    def __init__(self, q, k, v, o=None, lse=None, *, causal=False, scale=None, kv_lens=None,
                 alibi_slopes=None, softcap=0.0, stream=None):
        o, lse = fa_fwd_mod(q, k, v, o, lse, causal=causal, scale=scale, kv_lens=kv_lens,
                            alibi_slopes=alibi_slopes, softcap=softcap, stream=stream)
        B, Hq, Lq, D = q.shape
        scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
        sp, cap = _mod_args(q, alibi_slopes, softcap)
        s = torch.cuda.current_stream(q.device).cuda_stream if stream is None else stream
        self.o, self.lse = o, lse
        self._keep = (q, k, v, o, lse, kv_lens, alibi_slopes)
        self._fn = load_library().fa_fwd_mod
        self._args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, k.shape[1], Lq, k.shape[2], D,
                      int(bool(causal)), ctypes.c_float(scale), _ptr(kv_lens), sp, ctypes.c_float(cap), s)

    def __call__(self):
        status = self._fn(*self._args)
        if status != FA_OK:
            _check(status)
        return self.o, self.lse


def _check_offsets(cu, name, device):
    if cu.dtype != torch.int32 or cu.dim() != 1 or not cu.is_contiguous() or cu.device != device:
        raise ValueError(f"{name} must be a contiguous 1-D int32 tensor on the device of q")
    if cu.numel() < 2:
        raise ValueError(f"{name} must hold B + 1 >= 2 offsets")


def _prepare_varlen(q, k, v, cu_q, cu_k, o, lse, want_lse):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or t.dim() != 3 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 3-D bfloat16 tensor [H, total, D]")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on the GPU")
    Hq, total_q, D = q.shape
    Hkv, total_k, Dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Dk != D:
        raise ValueError("k and v must be [Hkv, total_k, D] with the D of q")
    _check_offsets(cu_q, "cu_seqlens_q", q.device)
    _check_offsets(cu_k, "cu_seqlens_k", q.device)
    if cu_q.numel() != cu_k.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length B + 1")
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty(Hq, total_q, dtype=torch.float32, device=q.device)
    return o, lse, (cu_q.numel() - 1, Hq, Hkv, total_q, total_k, D)


def fa_varlen_schedule_ints(B: int) -> int:
    return int(load_library().fa_varlen_schedule_ints(B))


def fa_varlen_schedule(cu_seqlens_q, cu_seqlens_k, total_q, total_k, schedule=None, stream=None):
    """The longest-tile-first order of a packed batch through
    ``fa_varlen_schedule``: an int32 device tensor [2B + 1] (the sequence
    order, then the prefix of query blocks).  ``schedule`` may be passed in."""
    _check_offsets(cu_seqlens_q, "cu_seqlens_q", cu_seqlens_q.device)
    _check_offsets(cu_seqlens_k, "cu_seqlens_k", cu_seqlens_q.device)
    B = cu_seqlens_q.numel() - 1
    if schedule is None:
        schedule = torch.empty(2 * B + 1, dtype=torch.int32, device=cu_seqlens_q.device)
    s = torch.cuda.current_stream(cu_seqlens_q.device).cuda_stream if stream is None else stream
    _check(load_library().fa_varlen_schedule(_ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B, int(total_q),
                                             int(total_k), _ptr(schedule), s))
    return schedule


def fa_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, o=None, lse=None, *, schedule=None, causal=False,
                  scale=None, stream=None, want_lse=True):
    """Attention over a packed variable-length batch through ``fa_fwd_varlen``:
    q [Hq, total_q, D], k and v [Hkv, total_k, D], int32 offsets [B + 1];
    ``schedule`` from ``fa_varlen_schedule`` or None (computed by the
    library).  Returns (o, lse) with o like q and lse [Hq, total_q]."""
    o, lse, (B, Hq, Hkv, tq, tk, D) = _prepare_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, o, lse, want_lse)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    s = torch.cuda.current_stream(q.device).cuda_stream if stream is None else stream
    _check(load_library().fa_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens_q),
                                        _ptr(cu_seqlens_k), _ptr(schedule), B, Hq, Hkv, tq, tk, D,
                                        int(bool(causal)), scale, s))
    return o, lse


class PreparedVarlenCall:
    """fa_fwd_varlen with its arguments checked and marshalled once (see
    PreparedCall); the schedule is computed once here unless given."""

    def __init__(self, q, k, v, cu_seqlens_q, cu_seqlens_k, o=None, lse=None, *, schedule=None,
                 causal=False, scale=None, stream=None, want_lse=True):
        o, lse, (B, Hq, Hkv, tq, tk, D) = _prepare_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, o, lse,
                                                          want_lse)
        scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
        s = torch.cuda.current_stream(q.device).cuda_stream if stream is None else stream
        if schedule is None:
            schedule = fa_varlen_schedule(cu_seqlens_q, cu_seqlens_k, tq, tk, stream=s)
        self.o, self.lse, self.schedule = o, lse, schedule
        self._keep = (q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, schedule)
        self._fn = load_library().fa_fwd_varlen
        self._args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                      _ptr(schedule), B, Hq, Hkv, tq, tk, D, int(bool(causal)), ctypes.c_float(scale), s)
        self()

    def __call__(self):
        status = self._fn(*self._args)
        if status != FA_OK:
            _check(status)
        return self.o, self.lse
