"""The allocation-free decode entry point (attn_decode_splitkv_noalloc, static
device scratch) against attn_decode_splitkv with a caller workspace: the same
kernels, so the outputs must agree bit for bit, on two calls in a row (the
second smaller, over the scratch the first one left behind)."""
import ctypes
import math

import numpy as np
import pytest
import torch

import attn_inputs as gen
import exact_long_context_tiled_amd as attn
from util import lse_err, max_abs_err, normwise_err, to_dev

pytestmark = pytest.mark.gpu


def _noalloc(case):
    """attn_decode_splitkv_noalloc through the C ABI; returns host (o, lse)."""
    L = attn.lib()
    q = to_dev(case["q"])
    kind = case["kv"]
    k, v = to_dev(case["k"], kind), to_dev(case["v"], kind)
    ks = to_dev(case["k_scale"]) if case.get("k_scale") is not None else None
    vs = to_dev(case["v_scale"]) if case.get("v_scale") is not None else None
    pt = to_dev(case["page_table"]) if case["paged"] else None
    lens = to_dev(case["lengths"].astype(np.int32))
    B, Hq, D = case["B"], case["Hq"], case["D"]
    o = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    kdt = {"bf16": 1, "fp8": 2, "int8": 3, "int4": 4}[kind]
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = L.attn_decode_splitkv_noalloc(kdt, P(q), P(k), P(v), P(ks), P(vs), P(pt),
                                       pt.shape[1] if pt is not None else 0, k.shape[2], k.shape[0], P(lens),
                                       int(case["lengths"].max()), B, Hq, case["Hkv"], D, case["scale"], 0, P(o),
                                       P(lse), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, attn.last_error()
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


def _with_workspace(case):
    kind = case["kv"]
    o, lse = attn.decode_splitkv(
        to_dev(case["q"]), to_dev(case["k"], kind), to_dev(case["v"], kind),
        to_dev(case["lengths"].astype(np.int32)), int(case["lengths"].max()),
        page_table=to_dev(case["page_table"]) if case["paged"] else None,
        k_scale=to_dev(case["k_scale"]) if case.get("k_scale") is not None else None,
        v_scale=to_dev(case["v_scale"]) if case.get("v_scale") is not None else None,
        kv_dtype=kind if kind in ("fp8", "int4") else None, scale=case["scale"])
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("kv", ["bf16", "int8"])
def test_noalloc_decode_matches_workspace_decode_twice(kv):
    import oracle
    # first call: the paged split-KV workload shape (B=8 Hq=32 Hkv=8 D=128, 512-token
    # pages, ragged lengths); second call: a smaller batch over the same scratch
    big = gen.decode_inputs(8, 32, 8, 128, gen.ragged_lengths(8, 1024, 32768, 0x5EED + 3), kv=kv, page_size=512,
                            seed=0x5EED + 3)
    small = gen.decode_inputs(3, 8, 2, 128, np.array([0, 700, 1500], np.int32), kv=kv, page_size=16, seed=17)
    for case, what in ((big, "big"), (small, "small")):
        print(f"noalloc {kv} {what}: lens={case['lengths'].tolist()}", flush=True)
        o1, l1 = _noalloc(case)
        o2, l2 = _with_workspace(case)
        assert np.array_equal(o1, o2), (what, max_abs_err(o1, o2))
        assert np.array_equal(l1, l2), what
        ro, rl = oracle.decode(case)
        ea, en, el = max_abs_err(o1, ro), normwise_err(o1, ro), lse_err(l1, rl)
        print(f"noalloc {kv} {what}: max_abs={ea:.3e} normwise={en:.3e} lse={el:.3e}", flush=True)
        assert ea <= 2e-2 and en <= 1e-2 and el <= 2e-2
