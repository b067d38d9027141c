"""Second, independent reference for small shapes -- TEST INFRASTRUCTURE ONLY.

Written with library routines instead of loops so that it shares no logic with
``attn_oracle.c``: stored bytes are decoded by torch's own bfloat16 /
float8_e4m3fn conversions, pages are gathered with numpy fancy indexing, the
full S x T score matrix is materialised with an explicit mask, and the softmax
and log-sum-exp come from scipy.special.  Used only to pin the C oracle.
"""
from __future__ import annotations

import numpy as np
import torch
from scipy.special import logsumexp, softmax


def decode_elems(a: np.ndarray) -> np.ndarray:
    """Stored element bytes -> float64 via torch's dtype conversions."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a.astype(np.float64)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
        return t.to(torch.float64).numpy()
    if a.dtype == np.uint8:
        t = torch.from_numpy(a).view(torch.float8_e4m3fn)
        return t.to(torch.float64).numpy()
    if a.dtype == np.int8:
        return a.astype(np.float64)
    raise TypeError(a.dtype)


def int4_values(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Packed int4 bytes [..., D/2] and group scales [..., D/32] -> float64 [..., D]:
    low nibble first, 4-bit two's complement, numpy bit operations."""
    b = np.asarray(packed, dtype=np.uint8)
    nib = np.stack([b & 0x0F, b >> 4], axis=-1).reshape(*b.shape[:-1], b.shape[-1] * 2).astype(np.int64)
    codes = np.where(nib >= 8, nib - 16, nib).astype(np.float64)
    group = codes.shape[-1] // np.asarray(scales).shape[-1]
    return codes * np.repeat(np.asarray(scales, dtype=np.float64), group, axis=-1)


def dense_kv_from_cache(case):
    """Gather a decode case's cache into dense fp64 K, V [B, Tmax, Hkv, D] plus lengths."""
    c = case
    B, Hkv, D, ps = c["B"], c["Hkv"], c["D"], c["page_size"]
    lens = np.asarray(c["lengths"], dtype=np.int64)
    tmax = int(lens.max()) if lens.size else 0
    if c["kv"] == "int4":
        k, v = (int4_values(c[n], c[n + "_scale"]) for n in "kv")
    else:
        k = decode_elems(c["k"])  # [P, Hkv, ps, D]
        v = decode_elems(c["v"])
    if c["kv"] == "int8":
        k = k * c["k_scale"].astype(np.float64)[..., None]
        v = v * c["v_scale"].astype(np.float64)[..., None]
    elif c["kv"] == "fp8":
        k = k * c["k_scale"].astype(np.float64)[None, :, None, None]
        v = v * c["v_scale"].astype(np.float64)[None, :, None, None]
    K = np.zeros((B, tmax, Hkv, D))
    V = np.zeros((B, tmax, Hkv, D))
    for b in range(B):
        t = np.arange(int(lens[b]))
        if c["paged"]:
            page = c["page_table"][b, t // ps]
        else:
            page = np.full_like(t, b)
        K[b, t] = k[page, :, t % ps, :]
        V[b, t] = v[page, :, t % ps, :]
    return K, V, lens


def attention(Q, K, V, *, causal, scale, lens=None):
    """Q [B,S,Hq,D], K/V [B,T,Hkv,D] float64 -> (O [B,S,Hq,D], lse [B,Hq,S])."""
    B, S, Hq, D = Q.shape
    T, Hkv = K.shape[1], K.shape[2]
    G = Hq // Hkv
    O = np.zeros((B, S, Hq, D))
    L = np.full((B, Hq, S), -np.inf)
    for b in range(B):
        Tb = T if lens is None else int(lens[b])
        for h in range(Hq):
            hk = h // G
            s = scale * (Q[b, :, h, :] @ K[b, :Tb, hk, :].T)  # [S, Tb]
            mask = np.ones((S, Tb), dtype=bool)
            if causal:
                i = np.arange(S)[:, None]
                j = np.arange(Tb)[None, :]
                mask = j <= i + Tb - S
            s = np.where(mask, s, -np.inf)
            live = mask.any(axis=1)
            if live.any():
                p = softmax(s[live], axis=1)
                O[b, live, h, :] = p @ V[b, :Tb, hk, :]
                L[b, h, live] = logsumexp(s[live], axis=1)
    return O, L
