"""CPU-only checks of libattn.so: it loads, exports every symbol declared in
include/attn.h, validates arguments before touching a device, and its
host-only stream planner covers every causally visible (query, key) pair
exactly once within the device budget."""
import os
import re

import numpy as np
import pytest

import exact_long_context_tiled_amd as attn
from exact_long_context_tiled_amd import AttnError

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    txt = open(os.path.join(ROOT, "include", "attn.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    L = attn.lib()
    syms = _declared_symbols()
    assert set(syms) >= {"attn_prefill", "attn_decode_splitkv", "attn_merge_partials", "attn_stream_budgeted",
                         "attn_stream_plan", "attn_decode_workspace_size", "attn_last_error", "attn_stream_cqs",
                         "attn_stream_cqs_plan", "attn_decode_multi", "attn_decode_multi_workspace_size",
                         "attn_prefill_fp8", "attn_decode_set_tuning"}
    for s in syms:
        assert hasattr(L, s), s


def _status(fn, *args):
    return fn(*args)


def test_prefill_validation_before_any_launch():
    L = attn.lib()
    # unsupported head dim
    assert L.attn_prefill(1, None, None, None, 1, 4, 2, 8, 8, 96, 1, 0.1, None, None, None) == 2
    assert "D must be 64 or 128" in attn.last_error()
    # Hq not a multiple of Hkv
    assert L.attn_prefill(1, None, None, None, 1, 5, 2, 8, 8, 64, 1, 0.1, None, None, None) == 1
    # unsupported dtype for prefill
    assert L.attn_prefill(3, None, None, None, 1, 4, 2, 8, 8, 64, 1, 0.1, None, None, None) == 2
    # non-finite scale
    assert L.attn_prefill(1, None, None, None, 1, 4, 2, 8, 8, 64, 1, float("nan"), None, None, None) == 1
    # null pointers with real work
    assert L.attn_prefill(1, None, None, None, 1, 4, 2, 8, 8, 64, 1, 0.1, None, None, None) == 1
    # empty work is a no-op even with null pointers
    assert L.attn_prefill(1, None, None, None, 0, 4, 2, 8, 8, 64, 1, 0.1, None, None, None) == 0
    assert L.attn_prefill(1, None, None, None, 2, 4, 2, 0, 8, 64, 1, 0.1, None, None, None) == 0
    # the kernels scale each row's raw maximum: scale must be positive
    assert L.attn_prefill(1, None, None, None, 1, 4, 2, 8, 8, 64, 1, 0.0, None, None, None) == 1
    assert L.attn_prefill(1, None, None, None, 1, 4, 2, 8, 8, 64, 1, -0.5, None, None, None) == 1
    assert "> 0" in attn.last_error()


def test_prefill_fp8_validation_before_any_launch():
    L = attn.lib()
    f = L.attn_prefill_fp8
    dummy = 256  # never dereferenced: validation fails or returns first
    assert f(None, None, None, None, None, None, 1, 4, 2, 8, 8, 96, 1, 0.1, None, None, None) == 2  # D
    assert f(None, None, None, None, None, None, 1, 5, 2, 8, 8, 64, 1, 0.1, None, None, None) == 1  # Hq % Hkv
    assert f(None, None, None, None, None, None, 1, 4, 2, 8, 8, 64, 1, -1.0, None, None, None) == 1  # scale
    assert f(None, None, None, None, None, None, 1, 4, 2, 8, 8, 64, 1, 0.1, None, None, None) == 1  # null q
    assert f(dummy, dummy, dummy, None, dummy, dummy, 1, 4, 2, 8, 8, 64, 1, 0.1, dummy, None, None) == 1
    assert "scale" in attn.last_error()
    assert f(None, None, None, None, None, None, 0, 4, 2, 8, 8, 64, 1, 0.1, None, None, None) == 0  # no work


def test_decode_and_merge_validation():
    L = attn.lib()
    args = dict(q=None, k=None, v=None, ks=None, vs=None, pt=None, maxp=0, ps=512, npg=0, lens=None, maxlen=100,
                B=2, Hq=32, Hkv=8, D=128, scale=0.1, ns=0, ws=None, wsb=0, o=None, lse=None, st=None)

    def call(**kw):
        a = dict(args, **kw)
        return L.attn_decode_splitkv(kw.get("dt", 1), a["q"], a["k"], a["v"], a["ks"], a["vs"], a["pt"], a["maxp"],
                                     a["ps"], a["npg"], a["lens"], a["maxlen"], a["B"], a["Hq"], a["Hkv"], a["D"],
                                     a["scale"], a["ns"], a["ws"], a["wsb"], a["o"], a["lse"], a["st"])

    assert call(dt=0) == 2  # fp32 caches are not a decode dtype
    assert call(D=80) == 2
    assert call(Hq=36, Hkv=4) == 2  # G = 9 > 8
    assert call(Hq=30) == 1
    assert call() == 1  # null pointers
    assert call(B=0) == 0
    # merge
    assert L.attn_merge_partials(2, None, None, 10, 0, None, None, None) == 2
    assert L.attn_merge_partials(2, None, None, 10, 64, None, None, None) == 1
    assert L.attn_merge_partials(2, None, None, 0, 64, None, None, None) == 0
    assert call(B=4096) == 2  # more sequences than the on-chip length prefix holds

    def multi(n_q, **kw):
        a = dict(args, **kw)
        return L.attn_decode_multi(1, a["q"], a["k"], a["v"], a["ks"], a["vs"], a["pt"], a["maxp"], a["ps"],
                                   a["npg"], a["lens"], a["maxlen"], a["B"], n_q, a["Hq"], a["Hkv"], a["D"],
                                   a["scale"], a["ns"], a["ws"], a["wsb"], a["o"], a["lse"], a["st"])

    assert multi(0) == 1 and multi(-1) == 1
    assert multi(65) == 2  # more query tokens than supported
    assert multi(4) == 1  # null pointers
    assert multi(4, B=0) == 0
    assert call(ns=65536) == 2  # more work units than one grid dimension
    # workspace sizing is pure host arithmetic: one record of G*D outputs plus
    # a 16-float lse line per (work unit + segment), then two ints per segment
    a = attn.decode_workspace_size(8, 32, 8, 128, 4096)
    b = attn.decode_workspace_size(8, 32, 8, 128, 32768)
    assert 0 < a <= b and a % 256 == 0

    def rnd(x):
        return (x + 255) // 256 * 256

    assert attn.decode_workspace_size(8, 32, 8, 128, 32768, num_splits=4) == (
        rnd((4 + 64) * (4 * 128 + 16) * 4) + rnd(64 * 8))
    assert attn.decode_workspace_size(3, 10, 2, 64, 100, num_splits=7) == (
        rnd((7 + 6) * (5 * 64 + 16) * 4) + rnd(6 * 8))
    # multi-token: a record holds n_q * G rows, the lse line padded to 16 floats
    assert attn.decode_multi_workspace_size(8, 4, 32, 8, 128, 32768, num_splits=4) == (
        rnd((4 + 64) * (16 * 128 + 16) * 4) + rnd(64 * 8))
    assert attn.decode_multi_workspace_size(3, 7, 10, 2, 64, 100, num_splits=7) == (
        rnd((7 + 6) * (35 * 64 + 48) * 4) + rnd(6 * 8))
    assert attn.decode_multi_workspace_size(8, 1, 32, 8, 128, 32768) == attn.decode_workspace_size(8, 32, 8, 128,
                                                                                                   32768)
    assert attn.decode_multi_workspace_size(8, 0, 32, 8, 128, 32768) == 0


def _coverage(tasks, rep, S, T, causal, B):
    bq, bk = rep["block_q"], rep["block_k"]
    nqb = (S + bq - 1) // bq
    cover = np.zeros((B, S, max(T, 1)), dtype=np.int32)
    per_block = np.zeros((B, nqb), dtype=np.int32)
    empty_block = np.zeros((B, nqb), dtype=np.int32)
    for b, qb, kb in tasks:
        per_block[b, qb] += 1
        q0, q1 = qb * bq, min(S, (qb + 1) * bq)
        if kb < 0:
            empty_block[b, qb] += 1
            continue
        k0, k1 = kb * bk, min(T, (kb + 1) * bk)
        i = np.arange(q0, q1)[:, None]
        j = np.arange(k0, k1)[None, :]
        vis = (j <= i + T - S) if causal else np.ones((q1 - q0, k1 - k0), bool)
        assert vis.any(), "a scheduled task must contain at least one visible pair"
        cover[b, q0:q1, k0:k1] += 1
    i = np.arange(S)[:, None]
    j = np.arange(max(T, 1))[None, :]
    vis = ((j <= i + T - S) if causal else np.ones((S, max(T, 1)), bool)) & (j < T)
    for b in range(B):
        # every visible pair lies in exactly one task's rectangle; no rectangle overlaps another
        assert np.all(cover[b][vis] == 1)
        assert np.all(cover[b] <= 1)
        # every query block is written by at least one task; a block gets an empty task
        # exactly when none of its rows sees any key, and then it has no other task
        assert np.all(per_block[b] >= 1)
        for qb in range(nqb):
            sees = vis[qb * bq:min(S, (qb + 1) * bq)].any()
            assert empty_block[b, qb] == (0 if sees else 1)
            if not sees:
                assert per_block[b, qb] == 1


@pytest.mark.parametrize("S,T,causal,bq,bk", [(300, 300, True, 64, 32), (100, 260, True, 32, 64),
                                                (260, 100, True, 64, 32), (97, 131, False, 32, 64),
                                                (50, 0, True, 16, 16), (1, 500, True, 128, 64)])
def test_stream_plan_covers_visible_pairs_exactly_once(S, T, causal, bq, bk):
    B = 2
    tasks, rep = attn.stream_plan("bf16", B, 8, 2, S, T, 64, causal=causal, budget=1 << 40, block_q=bq,
                                  block_k=bk)
    assert rep["tasks"] == len(tasks)
    _coverage(tasks, rep, S, T, causal, B)


@pytest.mark.parametrize("budget", [2 ** 22, 2 ** 24, 2 ** 26, 2 ** 30])
def test_stream_plan_fits_budget_and_covers(budget):
    S = T = 3000
    tasks, rep = attn.stream_plan("bf16", 1, 8, 2, S, T, 128, causal=True, budget=budget)
    assert rep["peak_device_bytes"] <= budget
    _coverage(tasks, rep, S, T, True, 1)


def test_stream_plan_memory_tracks_block_size_not_length():
    """Device bytes depend on the chosen blocks, not on the sequence length."""
    reps = [attn.stream_plan("bf16", 1, 32, 8, n, n, 128, causal=True, budget=4_000_000_000, block_q=8192,
                             block_k=4096, with_tasks=False)[1] for n in (1 << 16, 1 << 18, 1 << 20)]
    assert len({r["peak_device_bytes"] for r in reps}) == 1
    small = attn.stream_plan("bf16", 1, 32, 8, 1 << 20, 1 << 20, 128, budget=4_000_000_000, block_q=4096,
                             block_k=4096, with_tasks=False)[1]
    assert small["peak_device_bytes"] < reps[0]["peak_device_bytes"]


def test_stream_plan_million_token_workload():
    S = T = 1 << 20
    budget = 4_000_000_000
    _, rep = attn.stream_plan("bf16", 1, 32, 8, S, T, 128, causal=True, budget=budget, with_tasks=False)
    assert rep["peak_device_bytes"] <= budget
    assert rep["block_q"] >= 32768 and rep["block_k"] >= 4096
    # every Q byte goes up once; O + lse come back once
    assert rep["d2h_bytes"] == S * 32 * 128 * 4 + S * 32 * 4
    assert rep["h2d_bytes"] >= S * 32 * 128 * 2 + 2 * T * 8 * 128 * 2


def test_stream_budget_errors():
    with pytest.raises(AttnError) as e:
        attn.stream_plan("bf16", 1, 32, 8, 1 << 20, 1 << 20, 128, budget=1 << 16)
    assert e.value.status == 3
    with pytest.raises(AttnError) as e:
        attn.stream_plan("bf16", 1, 32, 8, 4096, 4096, 128, budget=1 << 22, block_q=4096, block_k=4096)
    assert e.value.status == 3
    with pytest.raises(AttnError) as e:
        attn.stream_plan("bf16", 1, 32, 8, 4096, 4096, 96, budget=1 << 30)
    assert e.value.status == 2


def test_library_has_no_undefined_internal_symbols():
    """Every kernel the library launches is defined in it (a kernel whose host
    stub is silently not emitted shows up as an undefined attn:: symbol)."""
    import shutil
    import subprocess

    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-C", "--undefined-only", attn.lib_path()], capture_output=True, text=True).stdout
    bad = [l for l in out.splitlines() if "attn::" in l]
    assert not bad, bad


def test_misaligned_pointers_rejected_before_any_launch():
    """The kernels move 16-byte vectors: misaligned device pointers are refused
    with ATTN_E_INVALID by the argument checks, before anything is launched
    (the fake addresses below are never dereferenced)."""
    L = attn.lib()
    A, M = 4096, 4096 + 4  # 16-byte aligned, and only 4-byte aligned
    # prefill: q, k, v, o need 16 bytes
    for q, k, v, o in ((M, A, A, A), (A, M, A, A), (A, A, M, A), (A, A, A, M)):
        assert L.attn_prefill(1, q, k, v, 1, 4, 2, 8, 8, 64, 1, 0.1, o, None, None) == 1
        assert "16-byte aligned" in attn.last_error()
        assert L.attn_prefill_fp8(q, k, v, A, A, A, 1, 4, 2, 8, 8, 64, 1, 0.1, o, None, None) == 1
    # lse needs 4 bytes
    assert L.attn_prefill(1, A, A, A, 1, 4, 2, 8, 8, 64, 1, 0.1, A, A + 2, None) == 1
    assert "4-byte" in attn.last_error()
    # fp8 scales need 4 bytes
    assert L.attn_prefill_fp8(A, A, A, A + 1, A, A, 1, 4, 2, 8, 8, 64, 1, 0.1, A, None, None) == 1
    # decode: q and caches need 16 bytes, the rest 4
    ws = 1 << 20
    base = dict(q=A, k=A, v=A, ks=None, vs=None, pt=None, maxp=0, ps=512, npg=0, lens=A, maxlen=100, B=2, Hq=32,
                Hkv=8, D=128, scale=0.1, ns=0, ws=1 << 24, wsb=ws, o=A, lse=None, st=None)

    def call(**kw):
        a = dict(base, **kw)
        return L.attn_decode_splitkv(1, a["q"], a["k"], a["v"], a["ks"], a["vs"], a["pt"], a["maxp"], a["ps"],
                                     a["npg"], a["lens"], a["maxlen"], a["B"], a["Hq"], a["Hkv"], a["D"],
                                     a["scale"], a["ns"], a["ws"], a["wsb"], a["o"], a["lse"], a["st"])

    for kw in (dict(q=M), dict(k=M), dict(v=M)):
        assert call(**kw) == 1 and "16-byte aligned" in attn.last_error()
    for kw in (dict(o=A + 2), dict(lse=A + 1), dict(lens=A + 2)):
        assert call(**kw) == 1 and "4-byte aligned" in attn.last_error()
    # merge: 4 bytes
    assert L.attn_merge_partials(2, A + 1, A, 10, 64, A, None, None) == 1
    assert L.attn_merge_partials(2, A, A, 10, 64, A + 3, None, None) == 1


def test_decode_tuning_validation():
    L = attn.lib()
    assert L.attn_decode_set_tuning(2, 0, -1) == 1
    assert L.attn_decode_set_tuning(0, -1, -1) == 1
    assert L.attn_decode_set_tuning(0, 2049, -1) == 1
    assert L.attn_decode_set_tuning(1, 64, 1 << 20) == 0
    assert L.attn_decode_set_tuning(0, 0, -1) == 0


def test_noalloc_decode_rejects_sizes_beyond_its_scratch():
    """The allocation-free decode refuses, before touching a device, sizes whose
    workspace exceeds its static scratch (addresses below are never dereferenced)."""
    L = attn.lib()
    cap = int(L.attn_decode_noalloc_max_scratch())
    assert cap == 8 << 20
    A = 4096
    f = L.attn_decode_splitkv_noalloc
    # B=4095 sequences x 8 KV heads x (4 rows x 128 + 16) floats per record: far beyond 8 MiB
    assert attn.decode_workspace_size(4095, 32, 8, 128, 1000) > cap
    assert f(1, A, A, A, None, None, None, 0, 1000, 0, A, 1000, 4095, 32, 8, 128, 0.1, 0, A, None, None) == 2
    assert "scratch" in attn.last_error()
    # validation still comes first
    assert f(1, A, A, A, None, None, None, 0, 1000, 0, A, 1000, 2, 32, 8, 80, 0.1, 0, A, None, None) == 2
    assert f(1, None, A, A, None, None, None, 0, 1000, 0, A, 1000, 2, 32, 8, 128, 0.1, 0, A, None, None) == 1
    assert f(1, None, None, None, None, None, None, 0, 1000, 0, None, 1000, 0, 32, 8, 128, 0.1, 0, None, None,
             None) == 0
