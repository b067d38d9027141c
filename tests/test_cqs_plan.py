"""CPU-only checks of the cyclic-quorum (CQS) streaming planner.

The pins come from the definition of the decomposition, not from the
library's own arithmetic: the base quorum must be a planar difference set
(every nonzero residue mod N is a difference of exactly one ordered pair of
members, checked here by enumerating the differences), the N quorums D + i
must pairwise intersect, and the pair list must cover every causally visible
(query position, key position) pair exactly once with both blocks of each
pair inside the quorum that computes it.  The host<->device byte counts are
recounted here from the pair list."""
import itertools

import numpy as np
import pytest

import exact_long_context_tiled_amd as attn
from exact_long_context_tiled_amd import AttnError


def _primes(hi):
    return [p for p in range(2, hi + 1) if all(p % d for d in range(2, int(p ** 0.5) + 1))]


SUPPORTED = [1, 3] + [p * p + p + 1 for p in _primes(127)]


@pytest.mark.parametrize("n", SUPPORTED)
def test_base_quorum_is_a_planar_difference_set(n):
    _, info, _ = attn.stream_cqs_plan("bf16", 1, 2, 1, 1, 1, 64, causal=False, budget=1 << 50, n_blocks=n,
                                      with_pairs=False)
    d = info["base"]
    k = info["quorum_size"]
    assert info["n_blocks"] == n and len(d) == k
    assert d[0] == 0 and d == sorted(set(d)) and all(0 <= e < n for e in d)
    # k(k-1) = N - 1 ordered differences, each nonzero residue exactly once
    assert k * (k - 1) == n - 1
    diffs = np.bincount([(a - b) % n for a in d for b in d if a != b], minlength=n)
    assert diffs[0] == 0 and np.all(diffs[1:] == 1)


@pytest.mark.parametrize("n", [7, 13, 31, 57])
def test_quorums_pairwise_intersect(n):
    _, info, _ = attn.stream_cqs_plan("bf16", 1, 2, 1, n, n, 64, causal=False, budget=1 << 50, n_blocks=n,
                                      with_pairs=False)
    quorums = [{(e + i) % n for e in info["base"]} for i in range(n)]
    for a, b in itertools.combinations(quorums, 2):
        assert len(a & b) == 1  # planar: two quorums meet in exactly one block


def _check_pairs(pairs, info, rep, S, T, causal, B):
    n, base = info["n_blocks"], info["base"]
    bq, bk = rep["block_q"], rep["block_k"]
    assert bq == -(-S // n) and bk == (-(-T // n) if T else 0)
    cover = np.zeros((B, S, max(T, 1)), dtype=np.int32)
    empty = np.zeros((B, n), dtype=np.int32)
    seen_pairs = set()
    for b, i, x, y in pairs:
        members = {(e + i) % n for e in base}
        assert x in members, "the query block of a pair belongs to the quorum computing it"
        q0, q1 = x * bq, min(S, (x + 1) * bq)
        assert q1 > q0
        if y < 0:
            empty[b, x] += 1
            assert i == x  # the empty pair of block x sits with its diagonal, in quorum x
            continue
        assert y in members, "the key block of a pair belongs to the quorum computing it"
        assert (b, x, y) not in seen_pairs
        seen_pairs.add((b, x, y))
        if x == y:
            assert i == x, "the diagonal (x, x) is computed by quorum x"
        k0, k1 = y * bk, min(T, (y + 1) * bk)
        assert k1 > k0
        ii = np.arange(q0, q1)[:, None]
        jj = np.arange(k0, k1)[None, :]
        vis = (jj <= ii + T - S) if causal else np.ones((q1 - q0, k1 - k0), bool)
        assert vis.any(), "a scheduled pair holds at least one visible (query, key) pair"
        cover[b, q0:q1, k0:k1] += 1
    ii = np.arange(S)[:, None]
    jj = np.arange(max(T, 1))[None, :]
    vis = ((jj <= ii + T - S) if causal else np.ones((S, max(T, 1)), bool)) & (jj < T)
    for b in range(B):
        assert np.all(cover[b][vis] == 1), "every visible (query, key) pair is computed exactly once"
        assert np.all(cover[b] <= 1)
        for x in range(n):
            q0, q1 = x * bq, min(S, (x + 1) * bq)
            if q1 <= q0:
                continue
            sees = vis[q0:q1].any()
            assert empty[b, x] == (0 if sees else 1)
    # execution order: sequence by sequence, quorum by quorum
    assert all(tuple(p[:2]) <= tuple(q[:2]) for p, q in zip(pairs[:-1], pairs[1:]))
    assert info["pairs"] == len(pairs)
    assert rep["tasks"] == len({(b, i) for b, i, _, _ in pairs})


def _recount(pairs, info, rep, S, T, Hq, Hkv, D, es):
    """H2D / D2H bytes of executing the pair list: per sub-task, its key blocks
    and query blocks go in; a query block's running (O, lse) goes in when a
    sub-task before the previous one wrote it last (the previous sub-task's
    is copied on the device); every query block it touched goes out."""
    n = info["n_blocks"]
    bq, bk = rep["block_q"], rep["block_k"]
    h2d = d2h = 0
    writer = {}  # (sequence, block) -> index of the sub-task that last wrote it
    for t, ((b, i), grp) in enumerate(itertools.groupby(pairs.tolist(), key=lambda r: (r[0], r[1]))):
        grp = list(grp)
        xs = sorted({x for _, _, x, _ in grp})
        ys = sorted({y for _, _, _, y in grp if y >= 0})
        for y in ys:
            h2d += 2 * (min(T, (y + 1) * bk) - y * bk) * Hkv * D * es
        for x in xs:
            nq = min(S, (x + 1) * bq) - x * bq
            h2d += nq * Hq * D * es
            if writer.get((b, x), t - 1) < t - 1:
                h2d += nq * Hq * (D + 1) * 4
            d2h += nq * Hq * (D + 1) * 4
            writer[(b, x)] = t
    return h2d, d2h


@pytest.mark.parametrize("S,T,causal,n", [(300, 300, True, 7), (300, 300, False, 13), (100, 260, True, 7),
                                          (260, 100, True, 13), (97, 131, False, 3), (50, 0, True, 7),
                                          (1, 500, True, 3), (20, 20, True, 31), (5, 5, True, 1),
                                          (64, 64, True, 57)])
def test_cqs_plan_covers_visible_pairs_exactly_once(S, T, causal, n):
    B, Hq, Hkv, D = 2, 8, 2, 64
    pairs, info, rep = attn.stream_cqs_plan("bf16", B, Hq, Hkv, S, T, D, causal=causal, budget=1 << 40, n_blocks=n)
    assert info["n_blocks"] == n
    _check_pairs(pairs, info, rep, S, T, causal, B)
    h2d, d2h = _recount(pairs, info, rep, S, T, Hq, Hkv, D, 2)
    assert (rep["h2d_bytes"], rep["d2h_bytes"]) == (h2d, d2h)


@pytest.mark.parametrize("budget", [2 ** 22, 2 ** 24, 2 ** 26])
def test_cqs_plan_fits_budget_with_the_smallest_quorum_size(budget):
    S = T = 3000
    pairs, info, rep = attn.stream_cqs_plan("bf16", 1, 8, 2, S, T, 128, causal=True, budget=budget)
    assert rep["peak_device_bytes"] <= budget
    _check_pairs(pairs, info, rep, S, T, True, 1)
    smaller = [m for m in SUPPORTED if m < info["n_blocks"]]
    if smaller:  # the next smaller N does not fit
        with pytest.raises(AttnError) as e:
            attn.stream_cqs_plan("bf16", 1, 8, 2, S, T, 128, causal=True, budget=budget, n_blocks=smaller[-1],
                                 with_pairs=False)
        assert e.value.status == 3


def test_cqs_plan_traffic_vs_rectangular_plan_at_a_million_tokens():
    """At the 2^20-token causal GQA shape under 4e9 bytes, the quorum plan moves
    far more bytes than the rectangular plan: each block's Q and running O
    travel once per quorum holding it (k = 18 of N = 307), while the
    rectangular plan sends each query block once and streams K/V past it."""
    S = T = 1 << 20
    _, info, rep = attn.stream_cqs_plan("bf16", 1, 32, 8, S, T, 128, causal=True, budget=4_000_000_000,
                                        with_pairs=False)
    _, rect = attn.stream_plan("bf16", 1, 32, 8, S, T, 128, causal=True, budget=4_000_000_000, with_tasks=False)
    assert rep["peak_device_bytes"] <= 4_000_000_000
    assert (info["n_blocks"], info["quorum_size"]) == (307, 18)
    assert info["pairs"] == 307 * 308 // 2  # the causal triangle of block pairs, diagonal included
    assert rep["h2d_bytes"] > 10 * rect["h2d_bytes"]
    assert rep["d2h_bytes"] > 10 * rect["d2h_bytes"]


def test_cqs_plan_errors():
    with pytest.raises(AttnError) as e:  # no planar difference set of that size is built in
        attn.stream_cqs_plan("bf16", 1, 8, 2, 100, 100, 64, budget=1 << 30, n_blocks=5)
    assert e.value.status == 2
    with pytest.raises(AttnError) as e:
        attn.stream_cqs_plan("bf16", 1, 32, 8, 1 << 20, 1 << 20, 128, budget=1 << 16)
    assert e.value.status == 3
    with pytest.raises(AttnError) as e:
        attn.stream_cqs_plan("bf16", 1, 32, 8, 4096, 4096, 96, budget=1 << 30)
    assert e.value.status == 2
    with pytest.raises(AttnError) as e:
        attn.stream_cqs_plan("bf16", 1, 30, 8, 4096, 4096, 128, budget=1 << 30)
    assert e.value.status == 1
    # empty work is a no-op
    pairs, info, rep = attn.stream_cqs_plan("bf16", 0, 8, 2, 100, 100, 64, budget=1 << 30)
    assert len(pairs) == 0 and info["n_blocks"] == 0 and rep["tasks"] == 0
