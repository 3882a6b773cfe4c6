"""MI355X (gfx950) FlashAttention forward: hand-written HIP kernels behind a C ABI.

``fa_fwd`` and friends are thin ctypes wrappers over ``libfa.so`` (module
``exact_attention_07_amd.binding``).  Importing the package loads nothing;
the first call into the library loads it and raises if it has not been built.
"""
_EXPORTS = ("fa_fwd", "fa_fwd_splits", "fa_fwd_noalloc", "fa_noalloc_scratch_bytes", "fa_fwd_window",
            "fa_fwd_paged", "fa_bwd", "fa_workspace_bytes", "fa_status_string", "load_library", "FaError",
            "PreparedCall", "PreparedPagedCall", "PreparedBwdCall", "fa_fwd_mod", "PreparedModCall",
            "quantize_fp8", "fa_fwd_fp8", "attention_fp8", "PreparedFp8Call",
            "fa_fwd_varlen", "fa_varlen_schedule", "fa_varlen_schedule_ints", "PreparedVarlenCall")


def __getattr__(name):
    if name in _EXPORTS:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
