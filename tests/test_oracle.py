"""Pins of the fp64 oracle against things other than itself (CPU only).

Closed forms, invariants of the definition, the format definitions of the
stored encodings, library decoders, hand-derived golden fixtures, and an
independent brute force (numpy/scipy/torch) on tiny shapes."""
import math
import os

import numpy as np
import pytest
import torch

import attn_inputs as gen
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.txt")


def _f32(shape, rng):
    return rng.standard_normal(shape).astype(np.float32)


# ------------------------------------------------------------------ encodings
def test_e4m3_fixed_points(orc):
    v = orc.e4m3fn_value
    assert v(0x38) == 1.0
    assert v(0x40) == 2.0
    assert v(0x7E) == 448.0
    assert v(0xFE) == -448.0
    assert v(0x08) == 2.0 ** -6  # smallest normal
    assert v(0x07) == 7 / 8 * 2.0 ** -6  # largest subnormal
    assert v(0x01) == 2.0 ** -9  # smallest subnormal
    assert v(0x00) == 0.0 and math.copysign(1.0, v(0x80)) == -1.0 and v(0x80) == 0.0
    assert math.isnan(v(0x7F)) and math.isnan(v(0xFF))
    assert v(0x3C) == 1.5 and v(0x39) == 1.125


def test_e4m3_all_codes_match_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = np.array([orc.e4m3fn_value(int(c)) for c in codes])
    assert np.array_equal(np.isnan(ref), np.isnan(mine))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], mine[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(mine[ok]))


def test_bf16_decode_matches_torch(orc):
    rng = np.random.default_rng(1)
    bits = np.concatenate([rng.integers(0, 1 << 16, 2000), [0, 0x8000, 0x3F80, 0xBF80, 0x7F7F, 0x0001]])
    bits = bits.astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    for b, r in zip(bits, ref):
        m = orc.bf16_value(int(b))
        assert (math.isnan(m) and math.isnan(r)) or m == r


def test_input_encoders_match_libraries():
    """The shared generators' bf16 rounding and e4m3 encoding agree with torch."""
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(20000) * rng.choice([1e-3, 1, 30, 500], 20000)).astype(np.float32)
    bits = gen.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    codes = gen.encode_e4m3fn(x)
    ref8 = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref8)


def test_int8_quantizer_roundtrip():
    rng = np.random.default_rng(3)
    x = _f32((5, 7, 64), rng)
    x[0, 0] = 0
    q, s = gen.quantize_int8(x)
    assert q.dtype == np.int8 and s.shape == (5, 7)
    err = np.abs(q.astype(np.float64) * s[..., None] - x)
    assert np.all(err <= s[..., None] / 2 + 1e-7)
    assert s[0, 0] == 1.0 and np.all(q[0, 0] == 0)
    assert q.min() >= -127


# ------------------------------------------------------------------ golden
def _parse_rows(txt):
    return np.array([[float(x) for x in r.split(",")] for r in txt.split(";")], dtype=np.float64)


def test_golden_closed_forms(orc):
    n = 0
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, scale, causal, qs, ks, vs, os_, ls = [f.strip() for f in line.split("|")]
        q, k, v, o_exp = map(_parse_rows, (qs, ks, vs, os_))
        lse_exp = np.array([float(x) for x in ls.split(";")])
        S, D = q.shape
        T = k.shape[0]
        o, lse = orc.attention(q.astype(np.float32).reshape(1, S, 1, D), k.astype(np.float32).reshape(1, T, 1, D),
                               v.astype(np.float32).reshape(1, T, 1, -1), B=1, Hq=1, Hkv=1, S=S, T=T, D=D,
                               causal=bool(int(causal)), scale=float(scale))
        np.testing.assert_allclose(o[0, :, 0, :], o_exp, rtol=0, atol=2e-6, err_msg=name)
        np.testing.assert_allclose(lse[0, 0], lse_exp, rtol=0, atol=2e-6, err_msg=name)
        n += 1
    assert n == 4


# ------------------------------------------------------------------ brute force
@pytest.mark.parametrize("kind", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S,T,G", [(1, 1, 1), (3, 5, 2), (5, 3, 1), (8, 8, 2), (4, 7, 3)])
def test_brute_force_prefill(orc, kind, causal, S, T, G):
    Hkv, D, B = 2, 4, 2
    case = gen.prefill_inputs(B, Hkv * G, Hkv, S, T, D, kind=kind, seed=100 + S * 7 + T)
    o, lse = orc.prefill(case, causal=causal)
    Q, K, V = (brute.decode_elems(case[n]) for n in "qkv")
    if kind == "fp8":  # e4m3 bytes times their per-head scales
        Q = Q * case["q_scale"].astype(np.float64)[None, None, :, None]
        K = K * case["k_scale"].astype(np.float64)[None, None, :, None]
        V = V * case["v_scale"].astype(np.float64)[None, None, :, None]
    ob, lb = brute.attention(Q, K, V, causal=causal, scale=case["scale"])
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[fin], lb[fin], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8", "int4"])
@pytest.mark.parametrize("paged", [True, False])
def test_brute_force_decode(orc, kv, paged):
    lens = np.array([0, 5, 16, 37], dtype=np.int32)
    D = 64 if kv == "int4" else 8  # int4 groups span 32 elements
    case = gen.decode_inputs(4, 4, 2, D, lens, kv=kv, page_size=8, paged=paged, spare=3, seed=7)
    o, lse = orc.decode(case)
    K, V, L = brute.dense_kv_from_cache(case)
    Q = brute.decode_elems(case["q"]).reshape(4, 1, 4, D)
    ob, lb = brute.attention(Q, K, V, causal=False, scale=case["scale"], lens=L)
    np.testing.assert_allclose(o, ob[:, 0], rtol=1e-12, atol=1e-12)
    assert np.all(np.isneginf(lse[0])) and np.all(o[0] == 0)
    np.testing.assert_allclose(lse[1:], lb[1:, :, 0], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8", "int4"])
@pytest.mark.parametrize("paged", [True, False])
def test_brute_force_multi_token_decode(orc, kv, paged):
    """n_q = 3 query tokens per sequence, bottom-right causal against each
    sequence's own length; lengths 0 and 2 (< n_q) leave rows with no key."""
    lens = np.array([0, 2, 5, 16, 37], dtype=np.int32)
    case = gen.decode_inputs(5, 4, 2, 32 if kv == "int4" else 8, lens, kv=kv, page_size=8, paged=paged, spare=3,
                             seed=9, n_q=3)
    o, lse = orc.decode(case)
    K, V, L = brute.dense_kv_from_cache(case)
    Q = brute.decode_elems(case["q"])
    ob, lb = brute.attention(Q, K, V, causal=True, scale=case["scale"], lens=L)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-12)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lb))
    assert np.all(np.isneginf(lse[0])) and np.all(np.isneginf(lse[1, :, 0]))  # no key: T=0, and 2 - 3 + 0 < 0
    assert np.all(np.isfinite(lse[1, :, 1:])) and np.all(o[1, 0] == 0)
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[fin], lb[fin], rtol=1e-12, atol=1e-12)


def test_int4_codes_decode_to_twos_complement_nibbles(orc):
    """A zero query and zero keys weigh every key alike, so O is the mean of the
    values.  With V's bytes covering all 256 (low, high) nibble pairs and unit
    scales, each output element is the mean of 4-bit two's-complement codes
    written out here from the definition: nibble n -> n if n < 8 else n - 16."""
    D, T = 64, 256
    nib_value = {n: (n if n < 8 else n - 16) for n in range(16)}
    vbytes = np.zeros((1, 1, T, D // 2), dtype=np.uint8)
    for t in range(T):
        vbytes[0, 0, t, :] = (t + np.arange(D // 2)) % 256  # token t, byte i: (t + i) mod 256
    expect = np.zeros(D)
    for i in range(D // 2):
        vals = [(t + i) % 256 for t in range(T)]
        expect[2 * i] = np.mean([nib_value[b & 15] for b in vals])
        expect[2 * i + 1] = np.mean([nib_value[b >> 4] for b in vals])
    kbytes = np.zeros_like(vbytes)
    ones = np.ones((1, 1, T, D // 32), dtype=np.float32)
    q = np.zeros((1, 1, 1, D), dtype=np.uint16)
    o, lse = orc.attention(q, kbytes, vbytes, B=1, Hq=1, Hkv=1, S=1, T=0, D=D, causal=False, scale=0.125, layout=1,
                           k_scale=ones, v_scale=ones, page_size=T, kv_lens=np.array([T]), kv_kind="int4")
    np.testing.assert_allclose(o[0, 0, 0], expect, rtol=0, atol=1e-12)
    assert abs(lse[0, 0, 0] - np.log(T)) < 1e-12  # T equal scores of 0
    # a group's scale multiplies exactly its 32 elements
    sc = np.ones((1, 1, T, D // 32), dtype=np.float32)
    sc[..., 1] = 2.0
    o2, _ = orc.attention(q, kbytes, vbytes, B=1, Hq=1, Hkv=1, S=1, T=0, D=D, causal=False, scale=0.125, layout=1,
                          k_scale=ones, v_scale=sc, page_size=T, kv_lens=np.array([T]), kv_kind="int4")
    np.testing.assert_allclose(o2[0, 0, 0], expect * np.repeat([1.0, 2.0], 32), rtol=0, atol=1e-12)


def test_fp8_prefill_inputs_follow_per_head_scales():
    """Each head's largest |value| maps to e4m3's largest finite value (448) and
    every decoded value is within half an e4m3 step of the drawn one."""
    case = gen.prefill_inputs(2, 4, 2, 16, 16, 64, kind="fp8", seed=5)
    x = gen.normal((2, 16, 4, 64), 5, gen.TID_Q, "f32")
    dec = brute.decode_elems(case["q"])
    np.testing.assert_allclose(np.max(np.abs(dec), axis=(0, 1, 3)), 448.0)
    back = dec * case["q_scale"][None, None, :, None]
    # e4m3 has 3 mantissa bits: |error| <= 2^-4 |x| for normal values, and
    # <= 2^-10 * scale in the subnormal range
    bound = np.maximum(np.abs(x) * 2.0 ** -4, case["q_scale"][None, None, :, None] * 2.0 ** -10)
    assert np.all(np.abs(back - x) <= bound * (1 + 1e-9))


def test_int4_quantizer_roundtrip():
    x = gen.normal((3, 5, 128), 11, gen.TID_K, "f32")
    x[0, 0, :32] = 0.0  # an all-zero group
    packed, s = gen.quantize_int4(x)
    assert packed.shape == (3, 5, 64) and s.shape == (3, 5, 4)
    vals = brute.int4_values(packed, s)
    err = np.abs(vals - x.astype(np.float64))
    assert np.all(err <= np.repeat(s, 32, axis=-1) / 2 + 1e-6)
    nib = np.concatenate([packed & 15, packed >> 4], axis=-1)
    assert not np.any(nib == 8)  # codes stay in [-7, 7]
    assert np.all(vals[0, 0, :32] == 0) and s[0, 0, 0] == 1.0


def test_multi_token_row_equals_single_token_on_shorter_cache(orc):
    """Query token s of n_q is single-token decode of that query against the
    first T - (n_q - 1 - s) keys of the same cache."""
    lens = np.array([9, 30, 64], dtype=np.int32)
    n_q = 4
    case = gen.decode_inputs(3, 4, 1, 8, lens, kv="int8", page_size=16, paged=True, spare=2, seed=21, n_q=n_q)
    o, lse = orc.decode(case)
    for s in range(n_q):
        one = dict(case, q=case["q"][:, s].copy(), n_q=None, lengths=lens - (n_q - 1 - s))
        o1, l1 = orc.decode(one)
        np.testing.assert_array_equal(o[:, s], o1)
        np.testing.assert_array_equal(lse[:, :, s], l1)


# ------------------------------------------------------------------ closed forms
def test_zero_query_gives_mean_of_visible_values(orc):
    rng = np.random.default_rng(5)
    S, T, D = 6, 9, 8
    q = np.zeros((1, S, 2, D), np.float32)
    k, v = _f32((1, T, 1, D), rng), _f32((1, T, 1, D), rng)
    o, lse = orc.attention(q, k, v, B=1, Hq=2, Hkv=1, S=S, T=T, D=D, causal=True, scale=0.3)
    for i in range(S):
        n = i + T - S + 1
        np.testing.assert_allclose(o[0, i, 1], v[0, :n, 0].astype(np.float64).mean(0), atol=1e-13)
        assert abs(lse[0, 1, i] - math.log(n)) < 1e-13


def test_causal_first_row_and_single_key(orc):
    rng = np.random.default_rng(6)
    S = T = 5
    D = 16
    q, k, v = _f32((1, S, 1, D), rng), _f32((1, T, 1, D), rng), _f32((1, T, 1, D), rng)
    o, lse = orc.attention(q, k, v, B=1, Hq=1, Hkv=1, S=S, T=T, D=D, causal=True, scale=0.25)
    np.testing.assert_array_equal(o[0, 0, 0], v[0, 0, 0].astype(np.float64))
    s00 = 0.25 * float(np.dot(q[0, 0, 0].astype(np.float64), k[0, 0, 0].astype(np.float64)))
    assert abs(lse[0, 0, 0] - s00) < 1e-13
    o1, _ = orc.attention(q, k[:, :1], v[:, :1], B=1, Hq=1, Hkv=1, S=S, T=1, D=D, causal=False, scale=0.25)
    np.testing.assert_array_equal(o1[0, :, 0], np.broadcast_to(v[0, 0, 0].astype(np.float64), (S, D)))


def test_constant_values_and_dominant_key(orc):
    rng = np.random.default_rng(8)
    S, T, D = 3, 50, 8
    q, k = _f32((1, S, 1, D), rng), _f32((1, T, 1, D), rng)
    v = np.full((1, T, 1, D), 1.75, np.float32)
    o, _ = orc.attention(q, k, v, B=1, Hq=1, Hkv=1, S=S, T=T, D=D, causal=False, scale=0.2)
    np.testing.assert_allclose(o, 1.75, rtol=0, atol=1e-14)
    # one key dominates every other by a margin >= 40 in score
    q = np.zeros((1, S, 1, D), np.float32)
    q[..., 0] = 10.0
    k = (rng.standard_normal((1, T, 1, D)) * 0.1).astype(np.float32)
    k[0, 17, 0, 0] = 10.0
    v = _f32((1, T, 1, D), rng)
    o, _ = orc.attention(q, k, v, B=1, Hq=1, Hkv=1, S=S, T=T, D=D, causal=False, scale=1.0)
    err = np.abs(o[0, :, 0] - v[0, 17, 0].astype(np.float64)).max()
    assert err <= math.exp(-40) * T * np.abs(v).max()


def test_fully_masked_rows(orc):
    rng = np.random.default_rng(9)
    S, T, D = 6, 2, 4  # causal with S > T: rows 0..3 see no key
    q, k, v = _f32((1, S, 1, D), rng), _f32((1, T, 1, D), rng), _f32((1, T, 1, D), rng)
    o, lse = orc.attention(q, k, v, B=1, Hq=1, Hkv=1, S=S, T=T, D=D, causal=True, scale=0.5)
    assert np.all(o[0, :4] == 0) and np.all(np.isneginf(lse[0, 0, :4]))
    assert np.all(np.isfinite(lse[0, 0, 4:]))
    o0, l0 = orc.attention(q, k[:, :0], v[:, :0], B=1, Hq=1, Hkv=1, S=S, T=0, D=D, causal=False, scale=0.5)
    assert np.all(o0 == 0) and np.all(np.isneginf(l0))


# ------------------------------------------------------------------ invariants
def test_noncausal_key_permutation_invariance(orc):
    case = gen.prefill_inputs(2, 4, 2, 7, 33, 16, kind="f32", seed=11)
    o, lse = orc.prefill(case, causal=False)
    perm = np.random.default_rng(0).permutation(33)
    c2 = dict(case, k=case["k"][:, perm].copy(), v=case["v"][:, perm].copy())
    o2, lse2 = orc.prefill(c2, causal=False)
    np.testing.assert_allclose(o2, o, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13, atol=1e-13)


def test_linear_in_values(orc):
    case = gen.prefill_inputs(1, 2, 1, 9, 9, 8, kind="f32", seed=12)
    v2 = gen.normal((1, 9, 1, 8), 99, 0, "f32")
    o1, _ = orc.prefill(case)
    o2, _ = orc.prefill(dict(case, v=v2))
    o3, _ = orc.prefill(dict(case, v=(case["v"].astype(np.float64) + 2 * v2.astype(np.float64)).astype(np.float32)))
    vsum = case["v"].astype(np.float64) + 2 * v2.astype(np.float64)
    # the float32 rounding of v1 + 2 v2 is the only difference
    assert np.abs(vsum.astype(np.float32) - vsum).max() < 1e-6
    np.testing.assert_allclose(o3, o1 + 2 * o2, atol=1e-6)


def test_gqa_equals_mha_with_repeated_kv(orc):
    G = 3
    case = gen.prefill_inputs(2, 2 * G, 2, 6, 10, 8, kind="bf16", seed=13)
    o, lse = orc.prefill(case)
    k_rep = np.repeat(case["k"], G, axis=2)
    v_rep = np.repeat(case["v"], G, axis=2)
    o2, lse2 = orc.prefill(dict(case, k=k_rep, v=v_rep, Hkv=2 * G))
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


def test_decode_equals_last_causal_prefill_row(orc):
    S = T = 12
    case = gen.prefill_inputs(2, 4, 2, S, T, 8, kind="bf16", seed=14)
    o, lse = orc.prefill(case, causal=True)
    od, lsed = orc.attention(case["q"][:, -1:].copy(), case["k"], case["v"], B=2, Hq=4, Hkv=2, S=1, T=T, D=8,
                             causal=True, scale=case["scale"])
    np.testing.assert_array_equal(od[:, 0], o[:, -1])
    np.testing.assert_array_equal(lsed[:, :, 0], lse[:, :, -1])


@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8"])
def test_paged_equals_contiguous(orc, kv):
    lens = np.array([20, 3, 31], dtype=np.int32)
    paged = gen.decode_inputs(3, 4, 2, 8, lens, kv=kv, page_size=8, paged=True, spare=2, seed=21)
    # rebuild the same token values as a contiguous [B, Hkv, Tmax, D] cache
    tmax = 32
    ps = 8
    def to_contig(a, tail):
        out = np.zeros((3, 2, tmax) + tail, dtype=a.dtype)
        for b in range(3):
            for t in range(int(lens[b])):
                out[b, :, t] = a[paged["page_table"][b, t // ps], :, t % ps]
        return out
    contig = dict(paged, paged=False, page_table=None, page_size=tmax, k=to_contig(paged["k"], (8,)),
                  v=to_contig(paged["v"], (8,)))
    if kv == "int8":
        contig["k_scale"] = to_contig(paged["k_scale"], ())
        contig["v_scale"] = to_contig(paged["v_scale"], ())
    o1, l1 = orc.decode(paged)
    o2, l2 = orc.decode(contig)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_block_split_merged_by_lse_equals_unsplit(orc):
    case = gen.prefill_inputs(1, 4, 2, 5, 40, 16, kind="f32", seed=15)
    o, lse = orc.prefill(case, causal=False)
    cuts = [0, 7, 8, 23, 40]
    parts_o, parts_l = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        po, pl = orc.prefill(dict(case, k=case["k"][:, a:b].copy(), v=case["v"][:, a:b].copy(), T=b - a),
                             causal=False)
        parts_o.append(po.reshape(-1, 16))  # rows ordered (b, s, h)
        parts_l.append(pl.transpose(0, 2, 1).reshape(-1))
    mo, ml = orc.merge(np.stack(parts_o), np.stack(parts_l))
    np.testing.assert_allclose(mo, o.reshape(-1, 16), rtol=0, atol=1e-12)
    np.testing.assert_allclose(ml, lse.transpose(0, 2, 1).reshape(-1), rtol=0, atol=1e-12)


def test_merge_identities(orc):
    rng = np.random.default_rng(16)
    op = rng.standard_normal((1, 5, 8))
    lp = rng.standard_normal((1, 5))
    mo, ml = orc.merge(op, lp)
    np.testing.assert_array_equal(mo, op[0])
    np.testing.assert_array_equal(ml, lp[0])
    op2 = np.concatenate([op, rng.standard_normal((1, 5, 8))])
    lp2 = np.concatenate([lp, np.full((1, 5), -np.inf)])
    mo, ml = orc.merge(op2, lp2)
    np.testing.assert_array_equal(mo, op[0])
    np.testing.assert_array_equal(ml, lp[0])
    mo, ml = orc.merge(np.zeros((3, 2, 4)), np.full((3, 2), -np.inf))
    assert np.all(mo == 0) and np.all(np.isneginf(ml))
    # two equal-weight partials average
    mo, ml = orc.merge(np.stack([np.ones((1, 2)), 3 * np.ones((1, 2))]), np.zeros((2, 1)))
    np.testing.assert_allclose(mo, 2.0)
    assert abs(ml[0] - math.log(2)) < 1e-15


def test_sampled_rows_match_full(orc):
    case = gen.prefill_inputs(1, 4, 2, 30, 30, 8, kind="bf16", seed=17)
    o, lse = orc.prefill(case)
    rows = gen.sample_rows(30, 6, 3)
    assert rows[0] == 0 and rows[-1] == 29 and len(set(rows)) == 6
    os_, ls = orc.prefill(case, rows=rows)
    np.testing.assert_array_equal(os_[0], o[0, rows])
    np.testing.assert_array_equal(ls[0], lse[0][:, rows])
