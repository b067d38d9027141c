"""ctypes binding of libattn.so: argument marshalling only."""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "lib", "libattn.so")

ATTN_F32, ATTN_BF16, ATTN_FP8_E4M3, ATTN_INT8, ATTN_INT4 = 0, 1, 2, 3, 4
_STATUS = {0: "ATTN_OK", 1: "ATTN_E_INVALID", 2: "ATTN_E_UNSUPPORTED", 3: "ATTN_E_BUDGET", 4: "ATTN_E_DEVICE"}


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class StreamReport(ctypes.Structure):
    _fields_ = [("tasks", ctypes.c_int64), ("h2d_bytes", ctypes.c_int64), ("d2h_bytes", ctypes.c_int64),
                ("peak_device_bytes", ctypes.c_int64), ("block_q", ctypes.c_int64), ("block_k", ctypes.c_int64),
                ("wall_s", ctypes.c_double), ("kernel_s", ctypes.c_double)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class CqsInfo(ctypes.Structure):
    _fields_ = [("n_blocks", ctypes.c_int64), ("quorum_size", ctypes.c_int64), ("pairs", ctypes.c_int64),
                ("base", ctypes.c_int64 * 128)]

    def as_dict(self):
        return {"n_blocks": self.n_blocks, "quorum_size": self.quorum_size, "pairs": self.pairs,
                "base": list(self.base[:self.quorum_size])}


_lib = None


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """Load libattn.so (built in-tree by exact_long_context_tiled_amd/build.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"libattn.so is not built ({_LIB_PATH}); run __graft_entry__.build()")
        L = ctypes.CDLL(_LIB_PATH)
        P, I, I64, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        L.attn_prefill.argtypes = [I, P, P, P, I, I, I, I64, I64, I, I, F, P, P, P]
        L.attn_prefill.restype = I
        L.attn_prefill_fp8.argtypes = [P, P, P, P, P, P, I, I, I, I64, I64, I, I, F, P, P, P]
        L.attn_prefill_fp8.restype = I
        L.attn_decode_workspace_size.argtypes = [I, I, I, I, I, I]
        L.attn_decode_workspace_size.restype = SZ
        L.attn_decode_splitkv.argtypes = [I, P, P, P, P, P, P, I, I, I, P, I, I, I, I, I, F, I, P, SZ, P, P, P]
        L.attn_decode_splitkv.restype = I
        L.attn_decode_multi_workspace_size.argtypes = [I, I, I, I, I, I, I]
        L.attn_decode_multi_workspace_size.restype = SZ
        L.attn_decode_multi.argtypes = [I, P, P, P, P, P, P, I, I, I, P, I, I, I, I, I, I, F, I, P, SZ, P, P, P]
        L.attn_decode_multi.restype = I
        L.attn_merge_partials.argtypes = [I, P, P, I64, I, P, P, P]
        L.attn_merge_partials.restype = I
        L.attn_stream_budgeted.argtypes = [I, P, P, P, I, I, I, I64, I64, I, I, F, SZ, I64, I64, P, P,
                                           ctypes.POINTER(StreamReport)]
        L.attn_stream_budgeted.restype = I
        L.attn_stream_plan.argtypes = [I, I, I, I, I64, I64, I, I, SZ, I64, I64, P, I64,
                                       ctypes.POINTER(StreamReport)]
        L.attn_stream_plan.restype = I
        L.attn_stream_cqs.argtypes = [I, P, P, P, I, I, I, I64, I64, I, I, F, SZ, I64, P, P,
                                      ctypes.POINTER(CqsInfo), ctypes.POINTER(StreamReport)]
        L.attn_stream_cqs.restype = I
        L.attn_stream_cqs_plan.argtypes = [I, I, I, I, I64, I64, I, I, SZ, I64, P, I64, ctypes.POINTER(CqsInfo),
                                           ctypes.POINTER(StreamReport)]
        L.attn_stream_cqs_plan.restype = I
        L.attn_decode_splitkv_noalloc.argtypes = [I, P, P, P, P, P, P, I, I, I, P, I, I, I, I, I, F, I, P, P, P]
        L.attn_decode_splitkv_noalloc.restype = I
        L.attn_decode_noalloc_max_scratch.argtypes = []
        L.attn_decode_noalloc_max_scratch.restype = SZ
        L.attn_decode_set_tuning.argtypes = [I, I, I64]
        L.attn_decode_set_tuning.restype = I
        L.attn_last_error.argtypes = []
        L.attn_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def last_error() -> str:
    return lib().attn_last_error().decode()


def _check(status: int):
    if status != 0:
        raise AttnError(status, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dt(t: torch.Tensor) -> int:
    return {torch.float32: ATTN_F32, torch.bfloat16: ATTN_BF16, torch.float8_e4m3fn: ATTN_FP8_E4M3,
            torch.int8: ATTN_INT8}[t.dtype]


def _need(t, name, device=True):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def prefill(q, k, v, *, causal=True, scale=None, out=None, lse=None, return_lse=True):
    """Tiled prefill.  q [B,S,Hq,D], k/v [B,T,Hkv,D] (bf16 or fp32, device).
    Returns (o [B,S,Hq,D] fp32, lse [B,Hq,S] fp32 or None)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n)
    B, S, Hq, D = q.shape
    T, Hkv = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, S, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    _check(lib().attn_prefill(_dt(q), _ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, S, T, D, int(causal), scale,
                              _ptr(out), _ptr(lse), _stream()))
    return out, lse


def prefill_fp8(q, k, v, q_scale, k_scale, v_scale, *, causal=True, scale=None, out=None, lse=None,
                return_lse=True):
    """fp8 prefill.  q [B,S,Hq,D], k/v [B,T,Hkv,D] float8_e4m3fn (or uint8 bytes)
    device tensors; q_scale [Hq], k_scale / v_scale [Hkv] fp32 device tensors.
    Returns (o [B,S,Hq,D] fp32, lse [B,Hq,S] fp32 or None)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (q_scale, "q_scale"), (k_scale, "k_scale"), (v_scale, "v_scale")):
        _need(t, n)
    B, S, Hq, D = q.shape
    T, Hkv = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, S, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    _check(lib().attn_prefill_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale), B, Hq,
                                  Hkv, S, T, D, int(causal), scale, _ptr(out), _ptr(lse), _stream()))
    return out, lse


def decode_set_tuning(*, path="auto", units=0, piece_bytes=-1):
    """Process-wide decode tuning (attn_decode_set_tuning): path 'auto'
    (matrix cores where supported) or 'valu'; units 0 = one per CU;
    piece_bytes < 0 = the default charge per segment."""
    _check(lib().attn_decode_set_tuning({"auto": 0, "valu": 1}[path], int(units), int(piece_bytes)))


def decode_workspace_size(B, Hq, Hkv, D, max_kv_len, num_splits=0) -> int:
    return int(lib().attn_decode_workspace_size(B, Hq, Hkv, D, max_kv_len, num_splits))


def _cache_dtype(k_cache, kv_dtype):
    if kv_dtype == "int4":
        if k_cache.dtype != torch.uint8:
            raise ValueError("int4 caches are uint8 tensors of packed nibble pairs")
        return ATTN_INT4
    if kv_dtype == "fp8" or k_cache.dtype == torch.float8_e4m3fn:
        return ATTN_FP8_E4M3
    if k_cache.dtype == torch.int8:
        return ATTN_INT8
    if k_cache.dtype == torch.bfloat16:
        return ATTN_BF16
    raise ValueError(f"unsupported cache dtype {k_cache.dtype}")


def decode_splitkv(q, k_cache, v_cache, kv_lens, max_kv_len, *, page_table=None, k_scale=None, v_scale=None,
                   kv_dtype=None, scale=None, num_splits=0, workspace=None, out=None, lse=None, return_lse=True):
    """Split-KV decode.  q [B,Hq,D] bf16; caches [P,Hkv,page,D] (paged) or
    [B,Hkv,page,D] (contiguous) of bf16 / int8 / float8_e4m3fn (uint8 bytes
    with kv_dtype='fp8'), or uint8 [..., D/2] packed int4 with kv_dtype='int4'
    (scales [..., page, D/32]).  Returns (o [B,Hq,D] fp32, lse [B,Hq] or None)."""
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (kv_lens, "kv_lens")):
        _need(t, n)
    kdt = _cache_dtype(k_cache, kv_dtype)
    B, Hq, D = q.shape
    num_pages, Hkv, page_size = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    max_pages = page_table.shape[1] if page_table is not None else 0
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = decode_workspace_size(B, Hq, Hkv, D, max_kv_len, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _check(lib().attn_decode_splitkv(kdt, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                     _ptr(page_table), max_pages, page_size, num_pages, _ptr(kv_lens), max_kv_len,
                                     B, Hq, Hkv, D, scale, num_splits, _ptr(workspace), workspace.numel(),
                                     _ptr(out), _ptr(lse), _stream()))
    return out, lse


def decode_multi_workspace_size(B, n_q, Hq, Hkv, D, max_kv_len, num_splits=0) -> int:
    return int(lib().attn_decode_multi_workspace_size(B, n_q, Hq, Hkv, D, max_kv_len, num_splits))


def decode_multi(q, k_cache, v_cache, kv_lens, max_kv_len, *, page_table=None, k_scale=None, v_scale=None,
                 kv_dtype=None, scale=None, num_splits=0, workspace=None, out=None, lse=None, return_lse=True):
    """Multi-token decode: q [B,n_q,Hq,D] bf16 = the last n_q tokens of each
    sequence (causal among themselves); caches as decode_splitkv.
    Returns (o [B,n_q,Hq,D] fp32, lse [B,Hq,n_q] or None)."""
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (kv_lens, "kv_lens")):
        _need(t, n)
    kdt = _cache_dtype(k_cache, kv_dtype)
    B, n_q, Hq, D = q.shape
    num_pages, Hkv, page_size = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    max_pages = page_table.shape[1] if page_table is not None else 0
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = decode_multi_workspace_size(B, n_q, Hq, Hkv, D, max_kv_len, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, n_q, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, n_q), dtype=torch.float32, device=q.device)
    _check(lib().attn_decode_multi(kdt, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                   _ptr(page_table), max_pages, page_size, num_pages, _ptr(kv_lens), max_kv_len,
                                   B, n_q, Hq, Hkv, D, scale, num_splits, _ptr(workspace), workspace.numel(),
                                   _ptr(out), _ptr(lse), _stream()))
    return out, lse


def merge_partials(o_parts, lse_parts, out=None, lse=None, return_lse=True):
    """LSE merge.  o_parts [n,R,D] fp32, lse_parts [n,R] fp32 (device)."""
    _need(o_parts, "o_parts")
    _need(lse_parts, "lse_parts")
    n, R, D = o_parts.shape
    if out is None:
        out = torch.empty((R, D), dtype=torch.float32, device=o_parts.device)
    if lse is None and return_lse:
        lse = torch.empty((R,), dtype=torch.float32, device=o_parts.device)
    _check(lib().attn_merge_partials(n, _ptr(o_parts), _ptr(lse_parts), R, D, _ptr(out), _ptr(lse), _stream()))
    return out, lse


def stream_budgeted(q_host, k_host, v_host, *, causal=True, scale=None, budget, block_q=0, block_k=0,
                    o_host=None, lse_host=None, return_lse=True):
    """Budgeted streaming prefill from pinned host memory (synchronous).
    q_host [B,S,Hq,D], k/v_host [B,T,Hkv,D] pinned CPU tensors (bf16/fp32).
    Returns (o_host, lse_host, report dict)."""
    for t, n in ((q_host, "q_host"), (k_host, "k_host"), (v_host, "v_host")):
        _need(t, n, device=False)
    B, S, Hq, D = q_host.shape
    T, Hkv = k_host.shape[1], k_host.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if o_host is None:
        o_host = torch.empty((B, S, Hq, D), dtype=torch.float32, pin_memory=True)
    if lse_host is None and return_lse:
        lse_host = torch.empty((B, Hq, S), dtype=torch.float32, pin_memory=True)
    rep = StreamReport()
    _check(lib().attn_stream_budgeted(_dt(q_host), _ptr(q_host), _ptr(k_host), _ptr(v_host), B, Hq, Hkv, S, T, D,
                                      int(causal), scale, int(budget), int(block_q), int(block_k), _ptr(o_host),
                                      _ptr(lse_host), ctypes.byref(rep)))
    return o_host, lse_host, rep.as_dict()


def stream_plan(dtype, B, Hq, Hkv, S, T, D, *, causal=True, budget, block_q=0, block_k=0, with_tasks=True):
    """The plan stream_budgeted would run (host only).  dtype: 'bf16'|'f32'.
    Returns (tasks int64 [n,3] of (b, q block, k block; -1 = empty) or None, report dict)."""
    import numpy as np

    dt = {"bf16": ATTN_BF16, "f32": ATTN_F32}.get(dtype, dtype)
    rep = StreamReport()
    _check(lib().attn_stream_plan(dt, B, Hq, Hkv, S, T, D, int(causal), int(budget), block_q, block_k, None, 0,
                                  ctypes.byref(rep)))
    tasks = None
    if with_tasks:
        tasks = np.zeros((max(rep.tasks, 1), 3), dtype=np.int64)
        _check(lib().attn_stream_plan(dt, B, Hq, Hkv, S, T, D, int(causal), int(budget), block_q, block_k,
                                      tasks.ctypes.data_as(ctypes.c_void_p), rep.tasks, ctypes.byref(rep)))
        tasks = tasks[:rep.tasks]
    return tasks, rep.as_dict()


def stream_cqs(q_host, k_host, v_host, *, causal=True, scale=None, budget, n_blocks=0, o_host=None, lse_host=None,
               return_lse=True):
    """Budgeted streaming prefill over cyclic quorums (synchronous).  Arguments
    as stream_budgeted; n_blocks 0 = chosen from the budget.
    Returns (o_host, lse_host or None, info dict, report dict)."""
    for t, n in ((q_host, "q_host"), (k_host, "k_host"), (v_host, "v_host")):
        _need(t, n, device=False)
    B, S, Hq, D = q_host.shape
    T, Hkv = k_host.shape[1], k_host.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if o_host is None:
        o_host = torch.empty((B, S, Hq, D), dtype=torch.float32, pin_memory=True)
    if lse_host is None and return_lse:
        lse_host = torch.empty((B, Hq, S), dtype=torch.float32, pin_memory=True)
    info, rep = CqsInfo(), StreamReport()
    _check(lib().attn_stream_cqs(_dt(q_host), _ptr(q_host), _ptr(k_host), _ptr(v_host), B, Hq, Hkv, S, T, D,
                                 int(causal), scale, int(budget), int(n_blocks), _ptr(o_host), _ptr(lse_host),
                                 ctypes.byref(info), ctypes.byref(rep)))
    return o_host, lse_host, info.as_dict(), rep.as_dict()


def stream_cqs_plan(dtype, B, Hq, Hkv, S, T, D, *, causal=True, budget, n_blocks=0, with_pairs=True):
    """The plan stream_cqs would run (host only).  Returns (pairs int64 [n,4] of
    (b, quorum, q block, k block; -1 = empty) or None, info dict, report dict)."""
    import numpy as np

    dt = {"bf16": ATTN_BF16, "f32": ATTN_F32}.get(dtype, dtype)
    info, rep = CqsInfo(), StreamReport()
    _check(lib().attn_stream_cqs_plan(dt, B, Hq, Hkv, S, T, D, int(causal), int(budget), int(n_blocks), None, 0,
                                      ctypes.byref(info), ctypes.byref(rep)))
    pairs = None
    if with_pairs:
        pairs = np.zeros((max(info.pairs, 1), 4), dtype=np.int64)
        _check(lib().attn_stream_cqs_plan(dt, B, Hq, Hkv, S, T, D, int(causal), int(budget), int(n_blocks),
                                          pairs.ctypes.data_as(ctypes.c_void_p), info.pairs, ctypes.byref(info),
                                          ctypes.byref(rep)))
        pairs = pairs[:info.pairs]
    return pairs, info.as_dict(), rep.as_dict()
