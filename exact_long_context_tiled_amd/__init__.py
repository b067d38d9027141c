"""Exact long-context attention for AMD MI355X (gfx950).

Python binding of ``libattn.so`` (C ABI: ``include/attn.h``).  The functions
here only marshal arguments: they take torch tensors (device memory for the
device calls, pinned host memory for the streaming call), pass raw pointers,
sizes and the current HIP stream to the library, and raise ``AttnError`` on a
non-OK status.  Every step of the computation runs in the library's HIP
kernels; there is no fallback path.  If the library is not built, importing
works but the first call raises.
"""
from ._binding import (  # noqa: F401
    ATTN_BF16,
    ATTN_F32,
    ATTN_FP8_E4M3,
    ATTN_INT8,
    AttnError,
    decode_multi,
    decode_multi_workspace_size,
    decode_set_tuning,
    decode_splitkv,
    decode_workspace_size,
    last_error,
    lib,
    lib_path,
    merge_partials,
    prefill,
    prefill_fp8,
    stream_budgeted,
    stream_cqs,
    stream_cqs_plan,
    stream_plan,
)

__all__ = [
    "AttnError", "prefill", "prefill_fp8", "decode_splitkv", "decode_workspace_size", "decode_multi",
    "decode_multi_workspace_size", "decode_set_tuning", "merge_partials", "stream_budgeted",
    "stream_plan", "stream_cqs", "stream_cqs_plan", "last_error", "lib", "lib_path",
]
