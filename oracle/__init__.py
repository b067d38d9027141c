"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the bench's ``cpu_baseline`` leg may import
this package.  The product library (``exact_long_context_tiled_amd``) never
imports, loads or calls it, and the two share no code.

``attn_oracle.c`` (plain loops, fp64, OpenMP over independent query rows) is
compiled with gcc into ``liboracle.so`` next to this file; this module only
marshals numpy arrays into it.  ``brute.py`` is a second, independent
implementation built from numpy/scipy/torch library routines, used to pin the
C code on small shapes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DT = {"f32": 0, "bf16": 1, "fp8": 2, "int8": 3, "int4": 4}

_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (fp64, -O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
                               "-fno-fast-math", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oracle_attention.argtypes = [ctypes.c_int, P, P, ctypes.c_int, ctypes.c_int, P, P, P, P, P, I64, I64, P,
                                         I64, I64, I64, I64, I64, I64, ctypes.c_int, ctypes.c_double, P, I64, P, P]
        lib.oracle_attention.restype = ctypes.c_int
        lib.oracle_merge.argtypes = [I64, P, P, I64, I64, P, P]
        lib.oracle_merge.restype = ctypes.c_int
        lib.oracle_e4m3fn_value.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3fn_value.restype = ctypes.c_double
        lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_value.restype = ctypes.c_double
        lib.oracle_threads.argtypes = []
        lib.oracle_threads.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_threads.restype = None
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _elem_kind(a: np.ndarray) -> str:
    return {np.dtype(np.float32): "f32", np.dtype(np.uint16): "bf16", np.dtype(np.uint8): "fp8",
            np.dtype(np.int8): "int8"}[a.dtype]


def attention(q, k, v, *, B, Hq, Hkv, S, T, D, causal, scale, layout=0, k_scale=None, v_scale=None,
              page_table=None, page_size=0, kv_lens=None, rows=None, kv_kind=None, q_scale=None):
    """Exact attention in fp64 on host arrays.

    Element type follows the numpy dtype: float32 -> f32, uint16 -> bf16 bits,
    uint8 -> OCP e4m3fn bytes, int8 -> int8 codes; kv_kind="int4" reads uint8
    K/V as packed int4 pairs (last dimension D/2 bytes) with per-32-element
    group scales [.., D/32].  q_scale [Hq] (optional) multiplies query head h;
    k_scale / v_scale [Hkv] are per-KV-head scales of e4m3 K/V in either
    layout.  Returns (o, lse):
    o [B, n_rows, Hq, D], lse [B, Hq, n_rows] (float64)."""
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    assert k.dtype == v.dtype
    ks = None if k_scale is None else np.ascontiguousarray(k_scale, dtype=np.float32)
    vs = None if v_scale is None else np.ascontiguousarray(v_scale, dtype=np.float32)
    pt = None if page_table is None else np.ascontiguousarray(page_table, dtype=np.int32)
    lens = None if kv_lens is None else np.ascontiguousarray(kv_lens, dtype=np.int64)
    rws = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n_rows = S if rws is None else len(rws)
    o = np.empty((B, n_rows, Hq, D), dtype=np.float64)
    lse = np.empty((B, Hq, n_rows), dtype=np.float64)
    max_pages = 0 if pt is None else pt.shape[1]
    kvk = kv_kind if kv_kind is not None else _elem_kind(k)
    qsc = None if q_scale is None else np.ascontiguousarray(q_scale, dtype=np.float32)
    rc = load().oracle_attention(DT[_elem_kind(q)], _p(q), _p(qsc), DT[kvk], layout, _p(k), _p(v), _p(ks), _p(vs),
                                 _p(pt), max_pages, page_size, _p(lens), B, Hq, Hkv, S, T, D, int(causal),
                                 float(scale), _p(rws), n_rows if rws is not None else 0, _p(o), _p(lse))
    if rc:
        raise RuntimeError(f"oracle_attention failed ({rc})")
    return o, lse


def prefill(case, causal=True, rows=None):
    """Oracle for a dense prefill case built by attn_inputs.prefill_inputs
    (e4m3 cases carry per-head q/k/v scales)."""
    c = case
    return attention(c["q"], c["k"], c["v"], B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], S=c["S"], T=c["T"], D=c["D"],
                     causal=causal, scale=c["scale"], rows=rows, q_scale=c.get("q_scale"),
                     k_scale=c.get("k_scale"), v_scale=c.get("v_scale"))


def decode(case):
    """Oracle for a decode case built by attn_inputs.decode_inputs: (o [B,Hq,D], lse [B,Hq]);
    with n_q query tokens per sequence (the last n_q positions, causal among
    themselves, bottom-right aligned to each sequence's length):
    (o [B,n_q,Hq,D], lse [B,Hq,n_q])."""
    c = case
    n_q = c.get("n_q")
    S = 1 if n_q is None else n_q
    o, lse = attention(c["q"].reshape(c["B"], S, c["Hq"], c["D"]), c["k"], c["v"], B=c["B"], Hq=c["Hq"],
                       Hkv=c["Hkv"], S=S, T=0, D=c["D"], causal=n_q is not None, scale=c["scale"], layout=1,
                       k_scale=c.get("k_scale"), v_scale=c.get("v_scale"), page_table=c["page_table"],
                       page_size=c["page_size"], kv_lens=c["lengths"], kv_kind=c["kv"] if c["kv"] == "int4" else None)
    if n_q is None:
        return o[:, 0], lse[:, :, 0]
    return o, lse


def merge(o_parts, lse_parts):
    """LSE merge: o_parts [n, R, D], lse_parts [n, R] -> (o [R, D], lse [R]) in fp64."""
    op = np.ascontiguousarray(o_parts, dtype=np.float64)
    lp = np.ascontiguousarray(lse_parts, dtype=np.float64)
    n, R, D = op.shape
    o = np.empty((R, D), dtype=np.float64)
    lse = np.empty((R,), dtype=np.float64)
    rc = load().oracle_merge(n, _p(op), _p(lp), R, D, _p(o), _p(lse))
    if rc:
        raise RuntimeError("oracle_merge failed")
    return o, lse


def e4m3fn_value(code: int) -> float:
    return load().oracle_e4m3fn_value(code)


def threads() -> int:
    """OpenMP threads the oracle uses."""
    return load().oracle_threads()


def set_threads(n: int) -> None:
    """OpenMP threads of later oracle calls (timing only; results do not depend on it)."""
    load().oracle_set_threads(int(n))


def bf16_value(bits: int) -> float:
    return load().oracle_bf16_value(bits)
