"""Seeded synthetic inputs for exact attention: the only module shared by the
fp64 oracle side and the HIP side.

It draws i.i.d. N(0,1) tensors, rounds them to bf16, encodes quantised KV
caches (symmetric int8 with one scale per token and KV head; OCP e4m3fn with
one scale per KV head), lays out random page tables, draws ragged KV lengths
and samples query rows.  It computes no attention: scores, softmax, merges and
decoding of stored bytes live on each side separately.

Every array is produced from ``numpy.random.SeedSequence`` streams keyed by
(workload seed, tensor id, chunk index), so the bytes are identical for any
thread count and on any host.  Large tensors are drawn in fixed-size chunks by
a thread pool (numpy releases the GIL while filling).

Recipe (the pages fix shapes but print no data):
  * Q, K, V: N(0,1) float32 draws, rounded to bf16 with round-to-nearest-even
    (or kept as float32 for the fp32 workload).
  * int8 KV: per (sequence, token, KV head) row ``s = max|x| / 127``,
    ``q = clamp(rne(x / s), -127, 127)``; an all-zero row gets ``s = 1``.
  * fp8 KV: per KV head ``s = amax / 448`` over every stored element of that
    head, bytes = OCP e4m3fn(rne(clamp(x / s, -448, 448))).
  * page tables: the pages of all sequences are a seeded permutation of the
    physical pool, which also holds spare pages; unused slots are poisoned
    (bf16 NaN, fp8 NaN, int8 with NaN scales) so a stray read shows up.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22  # elements per independently seeded chunk

# tensor ids inside one workload seed
TID_Q, TID_K, TID_V, TID_LENS, TID_PAGES, TID_ROWS, TID_MISC = range(7)

BF16_NAN = np.uint16(0x7FC0)
E4M3_NAN = np.uint8(0x7F)
E4M3_MAX = 448.0


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _rng(seed: int, tid: int, chunk: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tid, chunk))))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _fill_chunks(out_flat: np.ndarray, seed: int, tid: int, kind: str) -> None:
    n = out_flat.size
    nchunks = (n + CHUNK - 1) // CHUNK

    def work(c: int) -> None:
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        x = _rng(seed, tid, c).standard_normal(hi - lo, dtype=np.float32)
        if kind == "bf16":
            out_flat[lo:hi] = f32_to_bf16_bits(x)
        else:
            out_flat[lo:hi] = x

    if nchunks <= 1:
        for c in range(nchunks):
            work(c)
        return
    with ThreadPoolExecutor(max_workers=_threads()) as ex:
        list(ex.map(work, range(nchunks)))


def normal(shape, seed: int, tid: int, kind: str = "bf16", out: np.ndarray | None = None) -> np.ndarray:
    """N(0,1) tensor of ``shape``; kind 'bf16' -> uint16 bits, 'f32' -> float32.

    ``out`` may be a preallocated C-contiguous array (e.g. a view of pinned
    host memory) of the right dtype and size."""
    dt = np.uint16 if kind == "bf16" else np.float32
    if out is None:
        out = np.empty(shape, dtype=dt)
    assert out.dtype == dt and out.flags["C_CONTIGUOUS"] and out.size == math.prod(shape)
    _fill_chunks(out.reshape(-1), seed, tid, kind)
    return out.reshape(shape)


def normal_f32(shape, seed: int, tid: int) -> np.ndarray:
    return normal(shape, seed, tid, "f32")


# ----------------------------------------------------------------- encoders
def quantize_int8(x: np.ndarray):
    """Symmetric int8 along the last axis: returns (int8 codes, float32 scales)
    with one scale per row (all leading indices)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    s = (amax / np.float32(127.0)).astype(np.float32)
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    q = np.rint(x / s[..., None])  # numpy rint rounds half to even
    q = np.clip(q, -127, 127).astype(np.int8)
    return q, s


INT4_GROUP = 32  # elements per int4 scale group


def quantize_int4(x: np.ndarray):
    """Symmetric int4 in groups of 32 along the last axis (D): returns (uint8
    [..., D/2] packed codes, float32 [..., D/32] scales) with
    code = clamp(rne(x / s), -7, 7) and s = group amax / 7 (1 for an all-zero
    group); element 2i sits in the low nibble of byte i, 2i+1 in its high
    nibble, as 4-bit two's complement."""
    x = np.asarray(x, dtype=np.float32)
    *lead, D = x.shape
    g = x.reshape(*lead, D // INT4_GROUP, INT4_GROUP)
    amax = np.max(np.abs(g), axis=-1)
    s = np.where(amax == 0, np.float32(1.0), amax / np.float32(7.0)).astype(np.float32)
    q = np.clip(np.rint(g / s[..., None]), -7, 7).astype(np.int8).reshape(*lead, D)
    u = q.view(np.uint8) & np.uint8(15)
    packed = (u[..., 0::2] | (u[..., 1::2] << np.uint8(4))).astype(np.uint8)
    return packed, s


def _e4m3_grid() -> np.ndarray:
    """Non-negative finite OCP e4m3fn values for codes 0x00..0x7E, increasing."""
    vals = np.empty(127, dtype=np.float64)
    for code in range(127):
        e = code >> 3
        m = code & 7
        vals[code] = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3_GRID = _e4m3_grid()


def encode_e4m3fn(y: np.ndarray) -> np.ndarray:
    """Encode float values (already divided by their scale) as OCP e4m3fn bytes:
    saturate to +-448, round to nearest, ties to the even code."""
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), E4M3_MAX)
    hi = np.searchsorted(_E4M3_GRID, a, side="left")  # first grid value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _E4M3_GRID[lo]
    dhi = _E4M3_GRID[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(_E4M3_GRID[hi] == a, hi, code).astype(np.uint8)
    sign = np.signbit(y).astype(np.uint8) << 7  # negative values that round to 0 keep -0
    return (code | sign).astype(np.uint8)


# ----------------------------------------------------------------- workloads
def quantize_e4m3_per_head(x: np.ndarray, head_axis: int):
    """e4m3fn bytes with one fp32 scale per head: s = amax / 448 over the
    head's elements (1 for an all-zero head)."""
    x = np.asarray(x, dtype=np.float32)
    axes = tuple(a for a in range(x.ndim) if a != head_axis)
    amax = np.max(np.abs(x), axis=axes) if x.size else np.zeros(x.shape[head_axis], np.float32)
    s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    shape = [1] * x.ndim
    shape[head_axis] = -1
    return encode_e4m3fn(x / s.reshape(shape)), s


def prefill_inputs(B, Hq, Hkv, S, T, D, kind="bf16", seed=0x5EED):
    """Dense prefill operands: Q [B,S,Hq,D], K,V [B,T,Hkv,D].  kind 'fp8':
    e4m3fn bytes with per-head scales q_scale [Hq], k_scale / v_scale [Hkv]."""
    if kind == "fp8":
        out = {"B": B, "Hq": Hq, "Hkv": Hkv, "S": S, "T": T, "D": D, "kind": kind, "scale": 1.0 / math.sqrt(D)}
        for name, shape, tid in (("q", (B, S, Hq, D), TID_Q), ("k", (B, T, Hkv, D), TID_K),
                                 ("v", (B, T, Hkv, D), TID_V)):
            out[name], out[name + "_scale"] = quantize_e4m3_per_head(normal(shape, seed, tid, "f32"), 2)
        return out
    q = normal((B, S, Hq, D), seed, TID_Q, kind)
    k = normal((B, T, Hkv, D), seed, TID_K, kind)
    v = normal((B, T, Hkv, D), seed, TID_V, kind)
    return {"q": q, "k": k, "v": v, "B": B, "Hq": Hq, "Hkv": Hkv, "S": S, "T": T, "D": D,
            "kind": kind, "scale": 1.0 / math.sqrt(D)}


def ragged_lengths(B, lo, hi, seed):
    """KV lengths drawn uniformly from the integers lo..hi inclusive."""
    return _rng(seed, TID_LENS).integers(lo, hi + 1, size=B).astype(np.int32)


def page_table(lengths, page_size, spare, seed):
    """Random placement of each sequence's pages in one physical pool.

    Returns (table int32 [B, max_pages] with -1 in unused slots, num_pages)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    need = [(int(t) + page_size - 1) // page_size for t in lengths]
    max_pages = max(1, max(need) if need else 1)
    total = sum(need) + spare
    perm = _rng(seed, TID_PAGES).permutation(total).astype(np.int32)
    table = np.full((len(lengths), max_pages), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[pos:pos + n]
        pos += n
    return table, total


def decode_inputs(B, Hq, Hkv, D, lengths, kv="bf16", page_size=512, paged=True, spare=8,
                  seed=0x5EED, t_alloc=None, n_q=None):
    """Decode operands: q [B,Hq,D] bf16 (or [B,n_q,Hq,D] for multi-token
    decode when n_q is given) and a KV cache.

    paged:  caches [P, Hkv, page_size, D] addressed through a page table.
    contiguous: caches [B, Hkv, t_alloc, D] (t_alloc defaults to max length).
    kv: 'bf16' | 'int8' (scales shaped like the cache minus D) | 'fp8'
        (scales [Hkv] for K and for V) | 'int4' (uint8 caches with D/2 bytes
        per row, scales [.., page_size, D/32]).
    Unused cache slots are poisoned so that any stray read is visible."""
    lengths = np.asarray(lengths, dtype=np.int32)
    q = normal((B, Hq, D) if n_q is None else (B, n_q, Hq, D), seed, TID_Q, "bf16")
    maxlen = int(lengths.max()) if lengths.size else 0
    if paged:
        table, P = page_table(lengths, page_size, spare, seed)
        cache_shape = (P, Hkv, page_size, D)
        max_pages = table.shape[1]
    else:
        table, P = None, B
        page_size = int(t_alloc if t_alloc is not None else max(maxlen, 1))
        cache_shape = (B, Hkv, page_size, D)
        max_pages = 1
    # valid[p, t]: slot t of physical page p holds a real token
    valid = np.zeros((P, page_size), dtype=bool)
    for b in range(B):
        L = int(lengths[b])
        for j in range((L + page_size - 1) // page_size):
            p = int(table[b, j]) if paged else b
            n = min(page_size, L - j * page_size)
            valid[p, :n] = True
    out = {"q": q, "B": B, "Hq": Hq, "Hkv": Hkv, "D": D, "lengths": lengths, "kv": kv, "n_q": n_q,
           "page_table": table, "page_size": page_size, "num_pages": P, "max_pages": max_pages,
           "paged": paged, "scale": 1.0 / math.sqrt(D), "valid": valid}
    kf = normal(cache_shape, seed, TID_K, "f32")
    vf = normal(cache_shape, seed, TID_V, "f32")
    vmask = valid[:, None, :]  # [P,1,ps]
    if kv == "bf16":
        for name, x in (("k", kf), ("v", vf)):
            bits = f32_to_bf16_bits(x)
            bits[~np.broadcast_to(vmask, cache_shape[:3])] = BF16_NAN
            out[name] = bits
        out["k_scale"] = out["v_scale"] = None
    elif kv == "int8":
        for name, x in (("k", kf), ("v", vf)):
            qv, s = quantize_int8(x)  # s: [P,Hkv,ps]
            bad = ~np.broadcast_to(vmask, cache_shape[:3])
            qv[bad] = 127
            s[bad] = np.float32("nan")
            out[name] = qv
            out[name + "_scale"] = s
    elif kv == "int4":
        for name, x in (("k", kf), ("v", vf)):
            qv, s = quantize_int4(x)  # [P,Hkv,ps,D/2], [P,Hkv,ps,D/32]
            bad = ~np.broadcast_to(vmask, cache_shape[:3])
            qv[bad] = 0x77
            s[bad] = np.float32("nan")
            out[name] = qv
            out[name + "_scale"] = s
    elif kv == "fp8":
        for name, x in (("k", kf), ("v", vf)):
            m = np.broadcast_to(vmask[..., None], cache_shape)
            amax = np.array([np.max(np.abs(x[:, h][m[:, 0]])) if m.any() else 0.0
                             for h in range(Hkv)], dtype=np.float32)
            s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
            codes = encode_e4m3fn(x / s[None, :, None, None])
            codes[~np.broadcast_to(vmask[..., None], cache_shape)] = E4M3_NAN
            out[name] = codes
            out[name + "_scale"] = s
    else:
        raise ValueError(kv)
    return out


def sample_rows(S, n, seed):
    """Query rows for sampled checks: 0 and S-1 plus n-2 distinct others."""
    if S <= n:
        return np.arange(S, dtype=np.int64)
    inner = _rng(seed, TID_ROWS).choice(np.arange(1, S - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, S - 1], inner]).astype(np.int64))


# The benchmark and parity workloads by name (shapes from the pages' LLaMa-13B / 512-token-page settings)
WORKLOADS = {
    "tiny_gqa_causal_f32": dict(B=1, Hq=4, Hkv=2, S=256, T=256, D=64, kind="f32", causal=True),
    "llama13b_gqa_causal_bf16": dict(B=4, Hq=40, Hkv=8, S=4096, T=4096, D=128, kind="bf16", causal=True),
    "paged_splitkv_decode_bf16": dict(B=8, Hq=32, Hkv=8, D=128, lo=1024, hi=32768, page_size=512),
    "quant_decode": dict(B=4, Hq=32, Hkv=8, D=128, T=(4096, 65536)),
    # speculative verification: the last n_q tokens of each sequence against a paged cache
    "multi_token_decode": dict(B=8, Hq=32, Hkv=8, D=128, n_q=4, lo=1024, hi=32768, page_size=512),
    "stream_cqsa_causal_1m": dict(B=1, Hq=32, Hkv=8, S=1 << 20, T=1 << 20, D=128, kind="bf16",
                                  causal=True, budget=4_000_000_000),
}
