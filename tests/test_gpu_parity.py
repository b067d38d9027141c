"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Bars: fp32 inputs -> max relative error 1e-4 (|g-r| / max(|r|, 1e-2)); bf16 /
fp8 / int8-KV inputs -> max absolute error 2e-2, plus the internal guards
normwise error <= 1e-2 and lse error <= 2e-2 (outputs of long-T N(0,1) data are
small, so the absolute bar alone would be weak).  Both sides read the identical
stored bytes produced by attn_inputs."""
import math

import numpy as np
import pytest
import torch

import attn_inputs as gen
import exact_long_context_tiled_amd as attn
from util import lse_err, max_abs_err, max_rel_err, normwise_err, to_dev

pytestmark = pytest.mark.gpu

F32_TOL = 1e-4
LP_TOL = 2e-2
NORM_TOL = 1e-2


def say(*a):
    print(*a, flush=True)


def check_lp(o, lse, ro, rlse, what):
    ea, en, el = max_abs_err(o, ro), normwise_err(o, ro), lse_err(lse, rlse)
    say(f"{what}: max_abs={ea:.3e} normwise={en:.3e} lse={el:.3e}")
    assert np.all(np.isfinite(o)), what
    assert ea <= LP_TOL, what
    assert en <= NORM_TOL, what
    assert el <= LP_TOL, what


def check_f32(o, lse, ro, rlse, what):
    er = max_rel_err(o, ro)
    fin = np.isfinite(rlse)
    assert np.array_equal(np.isneginf(lse), np.isneginf(rlse)), what
    el = float(np.max(np.abs(lse[fin] - rlse[fin]) / np.maximum(1.0, np.abs(rlse[fin])))) if fin.any() else 0.0
    say(f"{what}: max_rel={er:.3e} lse_rel={el:.3e}")
    assert er <= F32_TOL and el <= F32_TOL, what


def gpu_prefill(case, causal=True):
    q, k, v = (to_dev(case[n]) for n in "qkv")
    o, lse = attn.prefill(q, k, v, causal=causal, scale=case["scale"])
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


# ------------------------------------------------------------------ prefill
def test_prefill_tiny_gqa_causal_f32():
    """B=1 Hq=4 Hkv=2 S=T=256 D=64, fp32, scale 1/8, causal: exact to fp32 rounding."""
    w = gen.WORKLOADS["tiny_gqa_causal_f32"]
    case = gen.prefill_inputs(w["B"], w["Hq"], w["Hkv"], w["S"], w["T"], w["D"], kind="f32", seed=0x5EED + 1)
    assert case["scale"] == 1 / 8
    o, lse = gpu_prefill(case)
    import oracle
    ro, rl = oracle.prefill(case)
    check_f32(o, lse, ro, rl, "tiny f32")


@pytest.mark.parametrize("B,Hq,Hkv,S,T,D,causal", [
    (2, 6, 3, 77, 133, 128, True), (1, 4, 4, 200, 200, 64, False), (1, 2, 1, 300, 40, 64, True),
    (1, 5, 5, 1, 97, 128, True), (2, 10, 2, 77, 133, 64, True)])
def test_prefill_f32_shapes(B, Hq, Hkv, S, T, D, causal):
    case = gen.prefill_inputs(B, Hq, Hkv, S, T, D, kind="f32", seed=3 + S + T)
    o, lse = gpu_prefill(case, causal)
    import oracle
    ro, rl = oracle.prefill(case, causal=causal)
    check_f32(o, lse, ro, rl, f"f32 {B,Hq,Hkv,S,T,D,causal}")


# The fp32 launches above are small: their row tiles would leave compute units
# idle, so they run on the key-split kernel.  These shapes make at least 512
# row tiles (two per compute unit of a 256-CU device) and run the row-tile
# kernel; every 8th query row is compared with the oracle.
@pytest.mark.parametrize("B,Hq,Hkv,S,T,D,causal", [
    (2, 16, 8, 4096, 256, 64, False),   # 8192 packed rows per KV head / 256 = 32 tiles x 16
    (2, 32, 8, 1024, 1024, 128, True),  # 4096 packed rows per KV head / 128 = 32 tiles x 16
    (2, 32, 8, 1031, 700, 128, True)])  # dead leading rows, ragged tiles
def test_prefill_f32_row_tiles(B, Hq, Hkv, S, T, D, causal):
    case = gen.prefill_inputs(B, Hq, Hkv, S, T, D, kind="f32", seed=11 + S + T)
    o, lse = gpu_prefill(case, causal)
    import oracle
    rows = np.arange(0, S, 8)
    if rows[-1] != S - 1:
        rows = np.append(rows, S - 1)
    ro, rl = oracle.prefill(case, causal=causal, rows=rows)
    check_f32(o[:, rows], lse[:, :, rows], ro, rl, f"f32 row tiles {B,Hq,Hkv,S,T,D,causal}")
    assert np.all(np.isfinite(o))


BF16_SHAPES = [
    (1, 4, 2, 256, 256, 64, True),     # several tiles, D=64
    (2, 10, 2, 300, 300, 128, True),   # G = 5, ragged tails
    (1, 8, 8, 130, 70, 128, False),    # MHA, non-causal, T < S
    (2, 40, 8, 200, 333, 128, True),   # LLaMa-13B heads, S != T (bottom-right)
    (1, 4, 1, 129, 1000, 64, True),    # G = 4, long keys
    (1, 2, 2, 1, 555, 128, True),      # one query row
    (1, 6, 2, 40, 90, 128, True),      # S < one tile
    (1, 3, 1, 150, 20, 128, True),     # S > T: leading rows fully masked
]


@pytest.mark.parametrize("B,Hq,Hkv,S,T,D,causal", BF16_SHAPES)
def test_prefill_bf16_shapes(B, Hq, Hkv, S, T, D, causal):
    case = gen.prefill_inputs(B, Hq, Hkv, S, T, D, kind="bf16", seed=11 + S * 3 + T)
    o, lse = gpu_prefill(case, causal)
    import oracle
    ro, rl = oracle.prefill(case, causal=causal)
    if causal and S > T:
        dead = S - T
        assert np.all(o[:, :dead] == 0) and np.all(np.isneginf(lse[:, :, :dead]))
    check_lp(o, lse, ro, rl, f"bf16 {B,Hq,Hkv,S,T,D,causal}")


def gpu_prefill_fp8(case, causal=True):
    q, k, v = (to_dev(case[n], "fp8") for n in "qkv")
    qs, ks, vs = (to_dev(case[n + "_scale"]) for n in "qkv")
    o, lse = attn.prefill_fp8(q, k, v, qs, ks, vs, causal=causal, scale=case["scale"])
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("B,Hq,Hkv,S,T,D,causal", BF16_SHAPES)
def test_prefill_fp8_shapes(B, Hq, Hkv, S, T, D, causal):
    """e4m3 Q/K/V with per-head scales == oracle on the same bytes and scales."""
    import oracle
    case = gen.prefill_inputs(B, Hq, Hkv, S, T, D, kind="fp8", seed=13 + S * 3 + T)
    say(f"fp8 prefill {B,Hq,Hkv,S,T,D,causal}")
    o, lse = gpu_prefill_fp8(case, causal)
    ro, rl = oracle.prefill(case, causal=causal)
    if causal and S > T:
        dead = S - T
        assert np.all(o[:, :dead] == 0) and np.all(np.isneginf(lse[:, :, :dead]))
    check_lp(o, lse, ro, rl, f"fp8 {B,Hq,Hkv,S,T,D,causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_prefill_fp8_rising_scores(causal):
    """e4m3 scores rising by ~37 log2 units from one 64-key tile to the next
    (query rows all ones, key j = e4m3(0.05 j) in every dim, unit scales): every
    tile takes the fp8 kernel's recompute-and-rebase path."""
    import oracle
    case = gen.prefill_inputs(1, 2, 1, 300, 300, 64, kind="fp8", seed=9)
    q = np.full_like(case["q"], gen.encode_e4m3fn(np.array([1.0]))[0])
    kf = (0.05 * np.arange(300))[None, :, None, None] * np.ones((1, 300, 1, 64))
    c = dict(case, q=q, k=gen.encode_e4m3fn(kf), q_scale=np.ones_like(case["q_scale"]),
             k_scale=np.ones_like(case["k_scale"]))
    o, lse = gpu_prefill_fp8(c, causal)
    ro, rl = oracle.prefill(c, causal=causal)
    check_lp(o, lse, ro, rl, f"fp8 rising scores causal={causal}")


def rows_in_every_tile(S, G, seed, tile_rows=128):
    """Query positions hitting every tile of `tile_rows` packed rows r = pos * G + g
    (one random packed row per tile, mapped to its position), plus 0 and S - 1."""
    rng = np.random.default_rng(seed)
    n_tiles = (S * G + tile_rows - 1) // tile_rows
    pos = {0, S - 1}
    for t in range(n_tiles):
        r = min(t * tile_rows + int(rng.integers(tile_rows)), S * G - 1)
        pos.add(r // G)
    return np.array(sorted(pos), dtype=np.int64)


@pytest.mark.timeout(600)
def test_prefill_fp8_llama13b_rows_in_every_tile():
    """B=4 Hq=40 Hkv=8 S=T=4096 D=128 causal, e4m3 operands: one query position in
    every 128-packed-row work tile (all heads, all sequences) vs the oracle."""
    import oracle
    w = gen.WORKLOADS["llama13b_gqa_causal_bf16"]
    G = w["Hq"] // w["Hkv"]
    case = gen.prefill_inputs(w["B"], w["Hq"], w["Hkv"], w["S"], w["T"], w["D"], kind="fp8", seed=0x5EED + 8)
    o, lse = gpu_prefill_fp8(case, True)
    rows = rows_in_every_tile(w["S"], G, 0x5EED + 8)
    assert len({(p * G) // 128 for p in rows} | {(p * G + G - 1) // 128 for p in rows}) >= (w["S"] * G) // 128
    ro, rl = oracle.prefill(case, causal=True, rows=rows)
    check_lp(o[:, rows], lse[:, :, rows], ro, rl, f"fp8 llama13b {len(rows)} rows (every tile)")


def test_prefill_fp8_empty_keys_and_errors():
    case = gen.prefill_inputs(1, 4, 2, 10, 0, 128, kind="fp8", seed=5)
    o, lse = gpu_prefill_fp8(case, True)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    q = to_dev(case["q"], "fp8")
    qs = to_dev(case["q_scale"])
    with pytest.raises(attn.AttnError) as e:
        attn.prefill_fp8(q, q, q, qs, qs, qs, causal=True, scale=-1.0)
    assert e.value.status == 1


def test_prefill_empty_keys():
    case = gen.prefill_inputs(1, 4, 2, 10, 0, 128, kind="bf16", seed=5)
    o, lse = gpu_prefill(case, True)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_prefill_peaked_and_needle_variants():
    """Diagnostic inputs with O(1) outputs: Q scaled by 4 (peaked softmax) and
    planted 'needle' keys equal to a query row (one dominant key per row)."""
    import oracle
    case = gen.prefill_inputs(1, 8, 2, 333, 333, 128, kind="bf16", seed=77)
    q4 = case["q"].copy()
    # multiply bf16 values by 4 exactly: add 2 to the exponent field of non-zero finite values
    exp = (q4 >> 7) & 0xFF
    ok = (exp > 0) & (exp < 250)
    q4[ok] = q4[ok] + (2 << 7)
    c4 = dict(case, q=q4)
    o, lse = gpu_prefill(c4)
    ro, rl = oracle.prefill(c4)
    check_lp(o, lse, ro, rl, "peaked q*4")
    assert np.abs(ro).max() > 0.5
    # needles: key j := query row j of head 0 of its group, scaled up (a dominant diagonal)
    k = case["k"].copy()
    for j in range(0, 333, 7):
        k[0, j, :, :] = q4[0, j, ::4, :]
    cn = dict(case, q=q4, k=k)
    o, lse = gpu_prefill(cn)
    ro, rl = oracle.prefill(cn)
    check_lp(o, lse, ro, rl, "needles")


@pytest.mark.parametrize("causal", [False, True])
def test_prefill_rising_scores(causal):
    """Scores that rise by ~37 log2 units from one 64-key tile to the next
    (every query row all ones, key j = 0.05 j in every dim): each tile's weights
    against the reference set by the tile before would pass 2^32, so every
    tile takes the kernel's recompute-and-rebase path."""
    import oracle
    case = gen.prefill_inputs(1, 2, 1, 300, 300, 64, kind="bf16", seed=9)
    q = np.full_like(case["q"], 0x3F80)  # bf16 1.0
    kf = (0.05 * np.arange(300, dtype=np.float32))[None, :, None, None] * np.ones((1, 300, 1, 64), np.float32)
    k = (kf.view(np.uint32) >> 16).astype(np.uint16)  # truncation to bf16 (the oracle sees the same bits)
    c = dict(case, q=q, k=k)
    o, lse = gpu_prefill(c, causal)
    ro, rl = oracle.prefill(c, causal=causal)
    check_lp(o, lse, ro, rl, f"rising scores causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_prefill_f32_rising_and_falling_scores(causal):
    """fp32 key-split kernel: scores that rise along the keys by 1.28 per
    64-key tile (each wave's running max moves on every tile) to 4, then fall
    to -4, so the waves' maxima differ and causal rows leave some waves with
    no key.  (Scores stay small: an fp32 score of size s carries a rounding
    error of ~s * 2^-24, which moves the output by about as much, and the
    fp32 bar is 1e-4 of max(|O|, 0.01).)"""
    import oracle
    case = gen.prefill_inputs(1, 4, 2, 300, 300, 64, kind="f32", seed=13)
    q = np.ones_like(case["q"])
    ramp = np.concatenate([0.0025 * np.arange(200), 0.5 - 0.01 * np.arange(100)]).astype(np.float32)
    k = ramp[None, :, None, None] * np.ones((1, 300, 2, 64), np.float32)
    c = dict(case, q=q, k=k)
    o, lse = gpu_prefill(c, causal)
    ro, rl = oracle.prefill(c, causal=causal)
    check_f32(o, lse, ro, rl, f"f32 rising/falling scores causal={causal}")


def test_prefill_f32_empty_keys():
    case = gen.prefill_inputs(1, 4, 2, 10, 0, 64, kind="f32", seed=5)
    o, lse = gpu_prefill(case, True)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_prefill_llama13b_full_size_every_row():
    """B=4 Hq=40 Hkv=8 S=T=4096 D=128 bf16 causal, in the launch configuration the
    benchmark times: every output row (all 4096 positions x 40 heads x 4 sequences)
    vs the fp64 oracle, which runs in a worker thread meanwhile."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    w = gen.WORKLOADS["llama13b_gqa_causal_bf16"]
    case = gen.prefill_inputs(w["B"], w["Hq"], w["Hkv"], w["S"], w["T"], w["D"], kind="bf16", seed=0x5EED + 2)
    with ThreadPoolExecutor(max_workers=1) as ex:
        fut = ex.submit(oracle.prefill, case)
        o, lse = gpu_prefill(case)
        say(f"llama13b: device run done; oracle on {oracle.threads()} threads")
        ro, rl = fut.result()
    check_lp(o, lse, ro, rl, "llama13b every row")
    # causal S == T: every row sees key 0, so every lse is finite
    assert np.all(np.isfinite(lse))


def test_prefill_deterministic():
    case = gen.prefill_inputs(2, 10, 2, 300, 300, 128, kind="bf16", seed=9)
    o1, l1 = gpu_prefill(case)
    o2, l2 = gpu_prefill(case)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_gqa_equals_mha_with_repeated_kv_on_gpu():
    case = gen.prefill_inputs(1, 8, 2, 150, 150, 128, kind="bf16", seed=19)
    o1, l1 = gpu_prefill(case)
    rep = dict(case, k=np.repeat(case["k"], 4, axis=2), v=np.repeat(case["v"], 4, axis=2), Hkv=8)
    o2, l2 = gpu_prefill(rep)
    assert max_abs_err(o1, o2) <= 1e-6 and lse_err(l1, l2) <= 1e-6


# ------------------------------------------------------------------ decode
def gpu_decode(case, num_splits=0):
    q = to_dev(case["q"])
    kind = case["kv"]
    k = to_dev(case["k"], kind)
    v = to_dev(case["v"], kind)
    ks = to_dev(case["k_scale"]) if case.get("k_scale") is not None else None
    vs = to_dev(case["v_scale"]) if case.get("v_scale") is not None else None
    pt = to_dev(case["page_table"]) if case["paged"] else None
    lens = to_dev(case["lengths"].astype(np.int32))
    maxlen = int(case["lengths"].max()) if len(case["lengths"]) else 0
    fn = attn.decode_multi if case.get("n_q") is not None else attn.decode_splitkv
    o, lse = fn(q, k, v, lens, maxlen, page_table=pt, k_scale=ks, v_scale=vs,
                kv_dtype=kind if kind in ("fp8", "int4") else None, scale=case["scale"], num_splits=num_splits)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


def test_decode_paged_splitkv_bf16_full():
    """B=8 Hq=32 Hkv=8 D=128, bf16 paged cache (512-token pages, random table), T_b ~ U[1024, 32768]."""
    import oracle
    w = gen.WORKLOADS["paged_splitkv_decode_bf16"]
    seed = 0x5EED + 3
    lens = gen.ragged_lengths(w["B"], w["lo"], w["hi"], seed)
    case = gen.decode_inputs(w["B"], w["Hq"], w["Hkv"], w["D"], lens, kv="bf16", page_size=512, seed=seed)
    o, lse = gpu_decode(case)
    ro, rl = oracle.decode(case)
    check_lp(o, lse, ro, rl, f"paged bf16 decode lens={lens.tolist()}")


@pytest.mark.parametrize("kv", ["int8", "fp8", "int4"])
@pytest.mark.parametrize("T", [4096, 65536])
def test_decode_quantised_full(kv, T):
    """B=4 Hq=32 Hkv=8 D=128, contiguous int8 (per-token-per-head scales), fp8 e4m3 (per-head
    scales) or int4 (packed nibbles, per-32-element-group scales)."""
    import oracle
    w = gen.WORKLOADS["quant_decode"]
    lens = np.full(w["B"], T, dtype=np.int32)
    case = gen.decode_inputs(w["B"], w["Hq"], w["Hkv"], w["D"], lens, kv=kv, paged=False,
                             seed=0x5EED + 4 + (T == 65536))
    o, lse = gpu_decode(case)
    ro, rl = oracle.decode(case)
    check_lp(o, lse, ro, rl, f"{kv} decode T={T}")


@pytest.fixture(params=["mfma", "valu"])
def decode_path(request):
    """Both split kernels: matrix cores (the default for bf16 / e4m3 / int8) and vector ALUs."""
    attn.decode_set_tuning(path="auto" if request.param == "mfma" else "valu")
    yield request.param
    attn.decode_set_tuning()


@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8", "int4"])
@pytest.mark.parametrize("paged,page_size", [(True, 16), (True, 512), (False, 0)])
@pytest.mark.parametrize("G,D", [(1, 128), (4, 64), (5, 128), (8, 128), (3, 128), (7, 64)])
def test_decode_ragged_edge_cases(kv, paged, page_size, G, D, decode_path):
    import oracle
    Hkv = 2
    lens = np.array([0, 1, 15, 16, 17, 513, 2000], dtype=np.int32)
    case = gen.decode_inputs(len(lens), G * Hkv, Hkv, D, lens, kv=kv, page_size=page_size or 512, paged=paged,
                             spare=3, seed=100 + G + D + page_size)
    ro, rl = oracle.decode(case)
    for ns in (0, 1, 3, 1000):
        say(f"decode {decode_path} {kv} paged={paged} ps={page_size} G={G} D={D} splits={ns}")
        o, lse = gpu_decode(case, num_splits=ns)
        assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
        check_lp(o, lse, ro, rl, f"{kv} paged={paged} ps={page_size} G={G} D={D} splits={ns}")


@pytest.mark.parametrize("kv", ["bf16", "int8", "int4"])
@pytest.mark.parametrize("n_q", [1, 3])
@pytest.mark.parametrize("piece_bytes", [0, 1, 4096, 1 << 20, 1 << 26])
def test_decode_piece_charge_in_split(kv, n_q, piece_bytes):
    """The matrix-core split charges each non-empty segment piece_bytes worth of
    slots before its groups: from no charge to charges far longer than the sequences (capped),
    so that work units holding only charged slots, segments whose first group lies in a later
    unit than their charge, and every remainder of the three-stage block pipeline occur.
    Output == oracle for each charge and several unit counts."""
    import oracle
    attn.decode_set_tuning(piece_bytes=piece_bytes)
    try:
        _piece_charge_case(kv, n_q, piece_bytes, oracle)
    finally:
        attn.decode_set_tuning()


def _piece_charge_case(kv, n_q, piece_bytes, oracle):
    lens = np.array([0, 1, 31, 33, 129, 640, 641, 1000, 2049, 5000], dtype=np.int32)
    Hkv, G, D = 2, 4, 128
    case = gen.decode_inputs(len(lens), G * Hkv, Hkv, D, lens, kv=kv, page_size=64, paged=True, spare=2,
                             seed=500 + n_q, n_q=n_q if n_q > 1 else None)
    ro, rl = oracle.decode(case)
    for ns in (0, 2, 7, 64):
        say(f"piece charge {piece_bytes} {kv} n_q={n_q} units={ns}")
        o, lse = gpu_decode(case, num_splits=ns)
        assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
        check_lp(o, lse, ro, rl, f"piece charge {piece_bytes} {kv} n_q={n_q} units={ns}")


@pytest.mark.parametrize("kv", ["bf16", "int8"])
def test_decode_page_entries_outside_the_cache(kv, decode_path):
    """Page-table entries outside [0, num_pages) are not dereferenced: the
    sequences holding them come back NaN (every head), the others are exact."""
    import oracle
    lens = np.array([700, 1500, 300, 900], dtype=np.int32)
    case = gen.decode_inputs(4, 8, 2, 128, lens, kv=kv, page_size=16, spare=2, seed=123)
    num_pages = case["k"].shape[0]
    pt = case["page_table"].copy()
    pt[1, 5] = num_pages + 3
    pt[2, 0] = -1
    pt[3, 56] = 2**31 - 1  # the last page of sequence 3 (tokens 896..899)
    bad = dict(case, page_table=pt)
    ro, rl = oracle.decode(case)
    for ns in (0, 1, 5, 1000):
        say(f"bad page entries {decode_path} {kv} units={ns}")
        o, lse = gpu_decode(bad, num_splits=ns)
        assert np.all(np.isnan(o[1:])) and np.all(np.isnan(lse[1:]))
        check_lp(o[:1], lse[:1], ro[:1], rl[:1], f"bad page entries: clean sequence, units={ns}")


def test_decode_many_sequences_mixed_lengths():
    """B=300 sequences (more than one length per thread of the on-chip prefix sum), with empty,
    tiny and long ones mixed, over 1, 7, automatic and more work units than token groups."""
    import oracle
    rng = np.random.default_rng(7)
    lens = rng.choice(np.array([0, 1, 5, 16, 33, 700, 3000], np.int32), size=300)
    case = gen.decode_inputs(300, 8, 2, 128, lens, kv="bf16", page_size=16, paged=True, spare=3, seed=77)
    ro, rl = oracle.decode(case)
    for ns in (1, 7, 0, 20000):
        o, lse = gpu_decode(case, num_splits=ns)
        assert np.all(o[lens == 0] == 0) and np.all(np.isneginf(lse[lens == 0]))
        check_lp(o, lse, ro, rl, f"B=300 mixed lengths units={ns}")


@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8", "int4"])
@pytest.mark.parametrize("G,n_q,D", [(4, 2, 128), (4, 4, 128), (1, 8, 128), (2, 3, 64), (5, 2, 128), (8, 3, 128),
                                     (1, 13, 64), (4, 5, 128), (1, 17, 64)])
def test_decode_multi_token_edge_cases(kv, G, n_q, D, decode_path):
    """Multi-token decode == oracle: lengths shorter than n_q (rows that see no
    key), pieces ending inside the causal tail, 16-token pages and a
    contiguous cache, over several work-unit counts."""
    import oracle
    Hkv = 2
    lens = np.array([0, 1, 2, 3, 15, 16, 17, 100, 513, 2000], dtype=np.int32)
    for paged in (True, False):
        case = gen.decode_inputs(len(lens), G * Hkv, Hkv, D, lens, kv=kv, page_size=16, paged=paged, spare=3,
                                 seed=300 + G * 10 + n_q, n_q=n_q)
        ro, rl = oracle.decode(case)
        for ns in (0, 1, 5, 1000):
            say(f"multi-token {decode_path} {kv} G={G} n_q={n_q} D={D} paged={paged} units={ns}")
            o, lse = gpu_decode(case, num_splits=ns)
            assert o.shape == ro.shape and lse.shape == rl.shape
            assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
            check_lp(o, lse, ro, rl, f"multi-token {kv} G={G} n_q={n_q} paged={paged} units={ns}")


@pytest.mark.parametrize("kv", ["int8", "int4"])
def test_decode_scales_at_unaligned_addresses(kv, decode_path):
    """int8 / int4 scale arrays that start 4 bytes past a 16-byte boundary (copied in 4-byte pieces)."""
    import oracle
    lens = np.array([5, 40, 700], dtype=np.int32)
    case = gen.decode_inputs(3, 8, 2, 128, lens, kv=kv, page_size=16, seed=91)
    ro, rl = oracle.decode(case)
    q = to_dev(case["q"])
    k, v = to_dev(case["k"]), to_dev(case["v"])
    pt = to_dev(case["page_table"])
    lens_d = to_dev(lens)

    def shifted(a):
        t = torch.empty(a.size + 1, dtype=torch.float32, device="cuda")
        t[1:] = torch.from_numpy(a.reshape(-1)).cuda()
        return t[1:].view(a.shape)

    ks, vs = shifted(case["k_scale"]), shifted(case["v_scale"])
    assert ks.data_ptr() % 16 == 4
    o, lse = attn.decode_splitkv(q, k, v, lens_d, int(lens.max()), page_table=pt, k_scale=ks, v_scale=vs,
                                 kv_dtype="int4" if kv == "int4" else None, scale=case["scale"])
    torch.cuda.synchronize()
    check_lp(o.cpu().numpy(), lse.cpu().numpy(), ro, rl, f"{kv} unaligned scales {decode_path}")


def test_decode_multi_one_token_is_splitkv():
    """n_q = 1 through the multi-token entry point is the single-token call, bit for bit."""
    lens = np.array([0, 7, 300, 4000], dtype=np.int32)
    case = gen.decode_inputs(4, 32, 8, 128, lens, kv="int8", page_size=512, seed=31)
    o1, l1 = gpu_decode(case)
    case_m = dict(case, q=case["q"].reshape(4, 1, 32, 128), n_q=1)
    om, lm = gpu_decode(case_m)
    assert np.array_equal(om[:, 0], o1) and np.array_equal(lm[:, :, 0], l1, equal_nan=True)


@pytest.mark.parametrize("kv", ["bf16", "int8"])
def test_decode_multi_token_full(kv):
    """B=8 Hq=32 Hkv=8 D=128, n_q=4 verified tokens per sequence, paged 512-token cache,
    T_b ~ U[1024, 32768]: every output vs the oracle."""
    import oracle
    w = gen.WORKLOADS["multi_token_decode"]
    seed = 0x5EED + 6
    lens = gen.ragged_lengths(w["B"], w["lo"], w["hi"], seed)
    case = gen.decode_inputs(w["B"], w["Hq"], w["Hkv"], w["D"], lens, kv=kv, page_size=w["page_size"], seed=seed,
                             n_q=w["n_q"])
    o, lse = gpu_decode(case)
    ro, rl = oracle.decode(case)
    check_lp(o, lse, ro, rl, f"multi-token {kv} n_q={w['n_q']} lens={lens.tolist()}")


def test_decode_fp8_every_finite_code(decode_path):
    """A cache holding every finite e4m3fn byte: the hardware decode must be OCP e4m3fn."""
    import oracle
    B, Hq, Hkv, D = 1, 1, 1, 128
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    T = 64
    k = np.resize(codes, T * D).reshape(1, 1, T, D).astype(np.uint8)
    v = np.resize(codes[::-1], T * D).reshape(1, 1, T, D).astype(np.uint8)
    q = gen.f32_to_bf16_bits(np.full((B, Hq, D), 0.01, np.float32))
    case = {"q": q, "k": k, "v": v, "k_scale": np.array([0.02], np.float32), "v_scale": np.array([0.5], np.float32),
            "B": B, "Hq": Hq, "Hkv": Hkv, "D": D, "lengths": np.array([T], np.int32), "kv": "fp8",
            "page_table": None, "page_size": T, "paged": False, "scale": 1 / math.sqrt(D)}
    o, lse = gpu_decode(case)
    ro, rl = oracle.decode(case)
    # values reach +-448*0.5: compare relative to the output scale.  A wrong
    # e4m3 decode errs by O(1).  The matrix-core path carries the softmax
    # weights as a bf16 pair (hi + lo), the vector-ALU path in fp32, so both
    # stay far inside the low-precision bar on these O(100) outputs too.
    say(f"fp8 every code {decode_path}: normwise={normwise_err(o, ro):.2e} max_abs={max_abs_err(o, ro):.2e}")
    assert normwise_err(o, ro) <= 1e-3 and lse_err(lse, rl) <= 1e-3
    assert max_abs_err(o, ro) <= LP_TOL


def test_decode_equals_last_prefill_row():
    """GPU cross-check: decode of the last query == last row of causal prefill (contiguous bf16)."""
    S = T = 700
    case = gen.prefill_inputs(2, 8, 2, S, T, 128, kind="bf16", seed=31)
    o, lse = gpu_prefill(case)
    kc = np.ascontiguousarray(case["k"].transpose(0, 2, 1, 3))  # [B, Hkv, T, D]
    vc = np.ascontiguousarray(case["v"].transpose(0, 2, 1, 3))
    dcase = {"q": case["q"][:, -1].copy(), "k": kc, "v": vc, "k_scale": None, "v_scale": None, "B": 2, "Hq": 8,
             "Hkv": 2, "D": 128, "lengths": np.array([T, T], np.int32), "kv": "bf16", "page_table": None,
             "page_size": T, "paged": False, "scale": case["scale"]}
    od, ld = gpu_decode(dcase)
    # decode sums fp32 weights; prefill sums the bf16-rounded weights its P.V product uses
    assert max_abs_err(od, o[:, -1]) <= 5e-3 and lse_err(ld, lse[:, :, -1]) <= 1e-3


# ------------------------------------------------------------------ merge
@pytest.mark.parametrize("n,R,D", [(1, 5, 64), (7, 300, 128), (3, 33, 17), (0, 4, 8), (5, 40, 129), (4, 37, 200),
                                   (6, 20, 255), (3, 50, 256), (9, 11, 384), (5, 7, 1024), (300, 6, 128),
                                   (600, 5, 200), (300, 4, 1024), (600, 3, 8)])
def test_merge_partials(n, R, D):
    """Every column layout of the merge kernel (D <= 128: several column groups;
    128 < D < 256: idle threads; D >= 256: several columns per thread) and more
    partials than one 256-wide weight chunk, with empty (-inf) partials."""
    import oracle
    rng = np.random.default_rng(n * 1000 + R + D)
    op = rng.standard_normal((n, R, D)).astype(np.float32)
    lp = (rng.standard_normal((n, R)) * 5).astype(np.float32)
    if n >= 3:
        lp[1, ::3] = -np.inf      # empty partials
        op[1, ::3] = np.nan       # never read
        lp[:, 0] = -np.inf        # a fully empty row
    if n > 256:
        lp[257:, 1] = -np.inf     # a row whose later weight chunks are empty
        lp[:256, 2] = -np.inf     # a row whose first weight chunk is empty
        op[:256, 2] = np.nan
    o, lse = attn.merge_partials(torch.from_numpy(op).cuda(), torch.from_numpy(lp).cuda())
    torch.cuda.synchronize()
    ro, rl = oracle.merge(np.nan_to_num(op, nan=0.0), lp)
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    # fp32 weights and an fp32 sum over n partials: besides 1e-5 relative, allow
    # the recursive-summation bound (n + 3) u sum_c w_c |O_c| / sum_c w_c (u = 2^-24)
    if n:
        lpd = lp.astype(np.float64)
        mx = np.max(lpd, axis=0)
        w = np.where(np.isneginf(lpd), 0.0, np.exp(lpd - np.where(np.isneginf(mx), 0.0, mx)))
        den = np.maximum(w.sum(axis=0), 1e-300)
        mag = np.einsum("nr,nrd->rd", w, np.abs(np.nan_to_num(op, nan=0.0)).astype(np.float64)) / den[:, None]
    else:
        mag = np.zeros_like(ro)
    bound = 1e-5 * np.maximum(np.abs(ro), 1e-2) + (n + 3) * 2.0**-24 * mag
    err = np.abs(o.astype(np.float64) - ro)
    say(f"merge n={n} R={R} D={D}: max_rel={max_rel_err(o, ro):.2e} worst err/bound={float(np.max(err / bound)):.3f}")
    assert np.all(err <= bound)
    assert lse_err(lse, rl) <= 1e-5


# ------------------------------------------------------------------ streaming
def _pinned(a: np.ndarray):
    t = torch.empty(a.shape, dtype={np.dtype(np.uint16): torch.int16, np.dtype(np.float32): torch.float32}[a.dtype],
                    pin_memory=True)
    t.numpy()[...] = a.view(np.int16) if a.dtype == np.uint16 else a
    return t.view(torch.bfloat16) if a.dtype == np.uint16 else t


@pytest.mark.parametrize("kind", ["bf16", "f32"])
def test_stream_budgeted_small(kind):
    """Streaming under small budgets == oracle, == unbudgeted device run, stable across budgets."""
    import oracle
    B, Hq, Hkv, S, T, D = 2, 8, 2, 1000, 1000, 128
    case = gen.prefill_inputs(B, Hq, Hkv, S, T, D, kind=kind, seed=41)
    qh, kh, vh = (_pinned(case[n]) for n in "qkv")
    o_dev, l_dev = gpu_prefill(case)
    ro, rl = oracle.prefill(case)
    outs = []
    for bq, bk in ((256, 128), (384, 200), (1000, 1000), (0, 0)):
        budget = 1 << 30 if bq == 0 else 64 << 20
        o, lse, rep = attn.stream_budgeted(qh, kh, vh, causal=True, scale=case["scale"], budget=budget,
                                           block_q=bq, block_k=bk)
        o, lse = o.numpy(), lse.numpy()
        say(f"stream {kind} bq={bq} bk={bk}: {rep}")
        assert rep["peak_device_bytes"] <= budget
        if kind == "f32":
            check_f32(o, lse, ro, rl, f"stream f32 {bq}x{bk}")
        else:
            check_lp(o, lse, ro, rl, f"stream bf16 {bq}x{bk}")
        # f32: merge order only; bf16: P is rounded to bf16 against each key block's own max
        tol = 1e-5 if kind == "f32" else 5e-3
        assert max_abs_err(o, o_dev) <= tol and lse_err(lse, l_dev) <= (1e-4 if kind == "f32" else 1e-3)
        outs.append(o)
    o_again, _, _ = attn.stream_budgeted(qh, kh, vh, causal=True, scale=case["scale"], budget=64 << 20,
                                         block_q=256, block_k=128)
    assert np.array_equal(o_again.numpy(), outs[0])


@pytest.mark.parametrize("kind,S,T", [("bf16", 500, 700), ("f32", 500, 700), ("bf16", 700, 500)])
def test_stream_budgeted_d64(kind, S, T):
    """D = 64 streaming (G = 4, S != T, blocks that do not divide the sequence;
    S > T leaves the first S - T query rows with no key) == the unbudgeted
    device run and the oracle."""
    import oracle
    B, Hq, Hkv, D = 2, 8, 2, 64
    case = gen.prefill_inputs(B, Hq, Hkv, S, T, D, kind=kind, seed=53)
    qh, kh, vh = (_pinned(case[n]) for n in "qkv")
    o_dev, l_dev = gpu_prefill(case)
    ro, rl = oracle.prefill(case)
    o, lse, rep = attn.stream_budgeted(qh, kh, vh, causal=True, scale=case["scale"], budget=64 << 20,
                                       block_q=192, block_k=160)
    o, lse = o.numpy(), lse.numpy()
    say(f"stream {kind} D=64 S={S} T={T}: {rep}")
    if S > T:
        assert np.all(o[:, :S - T] == 0) and np.all(np.isneginf(lse[:, :, :S - T]))
    if kind == "f32":
        check_f32(o, lse, ro, rl, "stream f32 D=64")
    else:
        check_lp(o, lse, ro, rl, "stream bf16 D=64")
    tol = 1e-5 if kind == "f32" else 5e-3
    assert max_abs_err(o, o_dev) <= tol and lse_err(lse, l_dev) <= (1e-4 if kind == "f32" else 1e-3)


def test_stream_f32_large_blocks():
    """fp32 streaming whose sub-tasks are large enough for the row-tile kernel
    (2048 x 4 packed rows per KV head: 64 tiles x 8 heads), so the accumulate
    mode of that kernel is checked: == the unbudgeted device run, == the oracle
    on sampled rows."""
    import oracle
    B, Hq, Hkv, S, T, D = 1, 32, 8, 4096, 4096, 128
    case = gen.prefill_inputs(B, Hq, Hkv, S, T, D, kind="f32", seed=47)
    qh, kh, vh = (_pinned(case[n]) for n in "qkv")
    o_dev, l_dev = gpu_prefill(case)
    o, lse, rep = attn.stream_budgeted(qh, kh, vh, causal=True, scale=case["scale"], budget=1 << 30,
                                       block_q=2048, block_k=1024)
    o, lse = o.numpy(), lse.numpy()
    say(f"stream f32 2048x1024: {rep}")
    assert max_abs_err(o, o_dev) <= 1e-5 and lse_err(lse, l_dev) <= 1e-4
    rows = np.concatenate([np.arange(0, S, 64), [1023, 1024, 2047, 2048, S - 1]])
    ro, rl = oracle.prefill(case, rows=rows)
    check_f32(o[:, rows], lse[:, :, rows], ro, rl, "stream f32 large blocks")


def test_stream_rejects_pageable_host_memory():
    case = gen.prefill_inputs(1, 4, 2, 64, 64, 64, kind="bf16", seed=3)
    q = torch.from_numpy(case["q"].view(np.int16)).view(torch.bfloat16)  # pageable
    k = _pinned(case["k"])
    v = _pinned(case["v"])
    with pytest.raises(attn.AttnError) as e:
        attn.stream_budgeted(q, k, v, causal=True, budget=1 << 30)
    assert e.value.status == 1 and "pinned" in str(e.value)


def test_stream_budget_too_small_fails_before_allocating():
    case = gen.prefill_inputs(1, 4, 2, 64, 64, 64, kind="bf16", seed=3)
    qh, kh, vh = (_pinned(case[n]) for n in "qkv")
    free0 = torch.cuda.mem_get_info()[0]
    with pytest.raises(attn.AttnError) as e:
        attn.stream_budgeted(qh, kh, vh, causal=True, budget=4096)
    assert e.value.status == 3
    assert torch.cuda.mem_get_info()[0] == free0


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("plan", ["rectangular", "cyclic_quorum"])
def test_stream_cqsa_million_token_causal(plan):
    """B=1 Hq=32 Hkv=8 S=T=2^20 D=128 bf16 causal from pinned host memory under a 4 GB
    device budget, with either plan: checked against the unbudgeted on-device run on
    every output and against the fp64 oracle on 64 seeded query rows x all heads."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    w = gen.WORKLOADS["stream_cqsa_causal_1m"]
    B, Hq, Hkv, S, T, D = w["B"], w["Hq"], w["Hkv"], w["S"], w["T"], w["D"]
    seed = 0x5EED + 5
    hq = torch.empty((B, S, Hq, D), dtype=torch.int16, pin_memory=True)
    hk = torch.empty((B, T, Hkv, D), dtype=torch.int16, pin_memory=True)
    hv = torch.empty((B, T, Hkv, D), dtype=torch.int16, pin_memory=True)
    qn = gen.normal(hq.shape, seed, gen.TID_Q, "bf16", out=hq.numpy().view(np.uint16))
    kn = gen.normal(hk.shape, seed, gen.TID_K, "bf16", out=hk.numpy().view(np.uint16))
    vn = gen.normal(hv.shape, seed, gen.TID_V, "bf16", out=hv.numpy().view(np.uint16))
    say("stream 1M: inputs generated")
    rows = gen.sample_rows(S, 64, seed)
    scale = 1.0 / math.sqrt(D)
    with ThreadPoolExecutor(max_workers=1) as ex:
        fut = ex.submit(oracle.attention, qn, kn, vn, B=B, Hq=Hq, Hkv=Hkv, S=S, T=T, D=D, causal=True,
                        scale=scale, rows=rows)
        if plan == "rectangular":
            o_h, lse_h, rep = attn.stream_budgeted(hq.view(torch.bfloat16), hk.view(torch.bfloat16),
                                                   hv.view(torch.bfloat16), causal=True, scale=scale,
                                                   budget=w["budget"])
            assert rep["d2h_bytes"] == S * Hq * D * 4 + S * Hq * 4
        else:
            o_h, lse_h, info, rep = attn.stream_cqs(hq.view(torch.bfloat16), hk.view(torch.bfloat16),
                                                    hv.view(torch.bfloat16), causal=True, scale=scale,
                                                    budget=w["budget"])
            assert info["pairs"] == info["n_blocks"] * (info["n_blocks"] + 1) // 2
        say(f"stream 1M {plan}: {rep}")
        assert rep["peak_device_bytes"] <= w["budget"]
        # the unbudgeted run, all on the device
        od, ld = attn.prefill(hq.view(torch.bfloat16).cuda(), hk.view(torch.bfloat16).cuda(),
                              hv.view(torch.bfloat16).cuda(), causal=True, scale=scale)
        torch.cuda.synchronize()
        say("stream 1M: device run done")
        worst_o = worst_l = 0.0
        step = 1 << 16
        for s0 in range(0, S, step):
            a_ = o_h[:, s0:s0 + step].cuda()
            worst_o = max(worst_o, float((a_ - od[:, s0:s0 + step]).abs().max()))
        ld_h = lse_h.cuda()
        worst_l = float((ld_h - ld).abs().max())
        del od
        say(f"stream 1M vs device: max_abs={worst_o:.3e} lse={worst_l:.3e}")
        assert worst_o <= 5e-3 and worst_l <= 1e-3
        assert bool(torch.isfinite(ld_h).all())
        ro, rl = fut.result()
    o_s = o_h.numpy()[:, rows]
    l_s = lse_h.numpy()[:, :, rows]
    check_lp(o_s, l_s, ro, rl, "stream 1M sampled rows")


# ------------------------------------------------------------------ cyclic-quorum streaming
@pytest.mark.parametrize("kind,causal,S,T,n", [("bf16", True, 1000, 1000, 7), ("f32", True, 1000, 1000, 13),
                                               ("bf16", False, 700, 900, 13), ("bf16", True, 900, 500, 7),
                                               ("bf16", True, 500, 900, 31), ("f32", False, 333, 333, 3)])
def test_stream_cqs_small(kind, causal, S, T, n):
    """Cyclic-quorum streaming == oracle and == the unbudgeted device run;
    repeatable bit for bit; without lse_host the output is unchanged."""
    import oracle
    B, Hq, Hkv, D = 2, 8, 2, 128
    case = gen.prefill_inputs(B, Hq, Hkv, S, T, D, kind=kind, seed=43 + n)
    qh, kh, vh = (_pinned(case[c]) for c in "qkv")
    o_dev, l_dev = gpu_prefill(case, causal=causal)
    ro, rl = oracle.prefill(case, causal=causal)
    say(f"stream_cqs {kind} causal={causal} S={S} T={T} N={n}")
    o, lse, info, rep = attn.stream_cqs(qh, kh, vh, causal=causal, scale=case["scale"], budget=1 << 30, n_blocks=n)
    say(f"  info={ {k: v for k, v in info.items() if k != 'base'} } report={rep}")
    assert info["n_blocks"] == n and rep["peak_device_bytes"] <= 1 << 30
    o, lse = o.numpy().copy(), lse.numpy().copy()
    if kind == "f32":
        check_f32(o, lse, ro, rl, f"stream_cqs f32 N={n}")
    else:
        check_lp(o, lse, ro, rl, f"stream_cqs bf16 N={n}")
    tol = 1e-5 if kind == "f32" else 5e-3
    assert max_abs_err(o, o_dev) <= tol and lse_err(lse, l_dev) <= (1e-4 if kind == "f32" else 1e-3)
    o2, lse2, _, _ = attn.stream_cqs(qh, kh, vh, causal=causal, scale=case["scale"], budget=1 << 30, n_blocks=n)
    assert np.array_equal(o2.numpy(), o) and np.array_equal(lse2.numpy(), lse)
    o3, none, _, _ = attn.stream_cqs(qh, kh, vh, causal=causal, scale=case["scale"], budget=1 << 30, n_blocks=n,
                                     return_lse=False)
    assert none is None and np.array_equal(o3.numpy(), o)


def test_stream_cqs_budget_picks_quorums_and_matches_rectangular():
    """Under a budget that forces N > 1 the automatic plan fits, and its output
    equals the rectangular streaming plan's within bf16 merge rounding."""
    B, Hq, Hkv, S, T, D = 1, 8, 2, 3000, 3000, 128
    case = gen.prefill_inputs(B, Hq, Hkv, S, T, D, kind="bf16", seed=77)
    qh, kh, vh = (_pinned(case[c]) for c in "qkv")
    budget = 24 << 20
    o, lse, info, rep = attn.stream_cqs(qh, kh, vh, causal=True, scale=case["scale"], budget=budget)
    say(f"stream_cqs auto: N={info['n_blocks']} k={info['quorum_size']} {rep}")
    assert info["n_blocks"] > 1 and rep["peak_device_bytes"] <= budget
    o_r, l_r, rep_r = attn.stream_budgeted(qh, kh, vh, causal=True, scale=case["scale"], budget=budget)
    assert max_abs_err(o.numpy(), o_r.numpy()) <= 5e-3 and lse_err(lse.numpy(), l_r.numpy()) <= 1e-3
    assert rep["h2d_bytes"] > rep_r["h2d_bytes"]


def test_stream_cqs_empty_keys_and_errors():
    case = gen.prefill_inputs(1, 4, 2, 64, 64, 64, kind="bf16", seed=5)
    qh, kh, vh = (_pinned(case[c]) for c in "qkv")
    empty = torch.empty((1, 0, 2, 64), dtype=torch.bfloat16, pin_memory=True)
    o, lse, info, _ = attn.stream_cqs(qh, empty, empty, causal=True, budget=1 << 30, n_blocks=7)
    assert np.all(o.numpy() == 0) and np.all(np.isneginf(lse.numpy()))
    with pytest.raises(attn.AttnError) as e:
        attn.stream_cqs(qh, kh, vh, causal=True, budget=1 << 30, n_blocks=5)
    assert e.value.status == 2
    q_pageable = torch.from_numpy(case["q"].view(np.int16)).view(torch.bfloat16)
    with pytest.raises(attn.AttnError) as e:
        attn.stream_cqs(q_pageable, kh, vh, causal=True, budget=1 << 30)
    assert e.value.status == 1
    free0 = torch.cuda.mem_get_info()[0]
    with pytest.raises(attn.AttnError) as e:
        attn.stream_cqs(qh, kh, vh, causal=True, budget=4096)
    assert e.value.status == 3 and torch.cuda.mem_get_info()[0] == free0


# ------------------------------------------------------------------ graph replay
@pytest.mark.parametrize("kv", ["bf16", "int8"])
def test_decode_graph_replay_matches_eager(kv):
    """Split-KV decode captured in a HIP graph and replayed several times, with eager
    work and synchronisations between the replays: every replay equals the eager call
    bit for bit (the fused merge's arrival counters are cleared by each call, so a
    replay with the same per-call tag starts from zero)."""
    lens = np.array([700, 1500, 33, 4000], dtype=np.int32)
    case = gen.decode_inputs(4, 32, 8, 128, lens, kv=kv, page_size=512, seed=71)
    q = to_dev(case["q"])
    k, v = to_dev(case["k"], kv), to_dev(case["v"], kv)
    ks = to_dev(case["k_scale"]) if case.get("k_scale") is not None else None
    vs = to_dev(case["v_scale"]) if case.get("v_scale") is not None else None
    pt = to_dev(case["page_table"])
    lens_d = to_dev(lens)
    maxlen = int(lens.max())
    ws = torch.empty(attn.decode_workspace_size(4, 32, 8, 128, maxlen), dtype=torch.uint8, device="cuda")
    o = torch.empty((4, 32, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((4, 32), dtype=torch.float32, device="cuda")

    def call():
        attn.decode_splitkv(q, k, v, lens_d, maxlen, page_table=pt, k_scale=ks, v_scale=vs, scale=case["scale"],
                            workspace=ws, out=o, lse=lse)

    call()
    torch.cuda.synchronize()
    ref_o, ref_l = o.clone(), lse.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # warm the side stream (LDS limits are raised outside the capture)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(4):
        o.zero_()
        lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        say(f"graph replay {rep} {kv}")
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_l), rep
        call()  # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o)
