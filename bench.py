#!/usr/bin/env python3
"""Throughput of the exact-attention hot path on one MI355X.

Headline (``value``): causal GQA prefill in TFLOP/s on the LLaMa-13B-shaped
workload (B=4, Hq=40, Hkv=8, S=T=4096, D=128, bf16 in, fp32 out), counting
only unmasked (query, key) pairs at 4*D flop each.  Beside it, in the same run:
  * ``decode``: split-KV decode over the paged bf16 cache (B=8, Hq=32, Hkv=8,
    D=128, 512-token pages, ragged lengths U[1024, 32768]) in GB/s of KV bytes
    of valid tokens (+ q, o, lse), with the cache copies rotated so each
    timed launch streams from HBM rather than from the 256 MB last-level cache;
  * ``prefill_fp8``: the same prefill with e4m3 Q/K/V and per-head scales;
  * ``decode_quant``: the same decode over contiguous int8, OCP e4m3fn and
    int4 caches (B=4, Hq=32, Hkv=8, D=128, T=65536) in GB/s of cache bytes;
  * ``decode_multi``: multi-token decode (n_q=4 verified tokens per sequence)
    over paged bf16 and int8 caches of the decode workload's shape, in GB/s;
  * ``roofline`` / ``decode.roofline``: achieved vs MI355X peak, timed with HIP
    events on the stream the kernels are launched on;
  * ``cpu_baseline``: the fp64 oracle on a bounded sample of query rows of the
    same prefill workload, on this host's cores.
  * ``prefill_f32``: the tiny fp32 causal GQA prefill (B=1, Hq=4, Hkv=2,
    S=T=256, D=64) against the fp32 vector peak, for information;
  * ``stream``: the budgeted streaming prefill (B=1, Hq=32, Hkv=8, S=T=2^20,
    D=128, bf16, 4 GB device budget) from pinned host memory: kernel-only and
    end-to-end TFLOP/s, host-link GB/s, the planned peak device bytes beside
    the free-memory drop seen while it runs, and a budget sweep showing that
    device memory follows the block size, not the sequence length
    (``--no-stream`` skips it);
  * ``cpu_baseline``: the fp64 oracle on this host's cores, on a bounded sample
    of the prefill workload (``value``) and on the small configurations in
    full, with all threads and with one.
``--stream-cqs`` also runs the streaming workload with the cyclic-quorum plan
and compares the two outputs (host-link heavy: minutes).

Prints ONE JSON line.  Inputs are seeded synthetic N(0,1) data.

Each leg times ``--steps`` launches (default 50) after ``--warmup`` untimed
ones (default 50).  After the GPU has been idle, the first few dozen
back-to-back prefill launches run while its clock controller settles (on one
box: 710 us, then up to 970 us, back to a steady 686-694 us from about the
50th launch on, held over 400 launches), and each leg's host-side input
preparation idles the GPU again.  So before a leg's warmup its call runs
untimed for ``--settle-seconds`` (default 0.3 s) of GPU time; with that the
figures are sustained rates whatever ``--warmup`` is.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s (prefill) + decode KV GB/s, as fraction of MI355X peak"
PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 flop/clk (dense, published 2.5 PF)
PEAK_FP8_TFLOPS = 5033.2  # dense fp8 matrix-core peak (published 5.0 PF)
PEAK_HBM_GBS = 8000.0
PEAK_FP32_TFLOPS = 157.3  # fp32 vector (published)
CSRC = os.path.join(ROOT, "exact_long_context_tiled_amd", "csrc")
DECODE_SOURCES = ("decode.hip", "decode_mfma.hip", "decode_common.h")
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest(*names):
    """sha256 of the kernel sources a measurement belongs to."""
    import hashlib

    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(profile, *sources):
    """HBM bytes per launch recorded from PMC counters in a committed profile,
    or None if the profile is missing or the kernel source changed since."""
    path = os.path.join(PROFILES, profile)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_sha256") != source_digest(*sources):
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def causal_pairs(S, T):
    """Number of (query, key) pairs visible under bottom-right causal masking."""
    tot = 0
    for i in range(S):
        tot += max(0, min(T, i + T - S + 1))
    return tot


SETTLE_S = 0.3  # set from --settle-seconds


def timed(fn, steps, warmup, stream):
    """Mean ms per call of fn over `steps` calls on `stream`, bracketed by
    synchronisations, after `warmup` untimed calls.  Before those, fn runs
    untimed for about SETTLE_S seconds of GPU time: the host-side input
    preparation of a leg leaves the GPU idle, and the clock ramp that follows
    an idle GPU would otherwise fall into the timed calls."""
    import torch

    spent = 0.0
    while spent < SETTLE_S:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(20):
            fn(-1)
        e1.record(stream)
        torch.cuda.synchronize()
        spent += e0.elapsed_time(e1) * 1e-3
    for _ in range(warmup):
        fn(-1)
    torch.cuda.synchronize()
    # a short spin kernel right before the timed calls: in a kernel trace its
    # name marks where each leg's timed dispatches start (it runs before t0)
    torch.cuda._sleep(100)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(steps):
        fn(i)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def timed_graph(fn, calls, steps, stream):
    """Mean ms per call of fn(0 .. calls-1) captured once in a HIP graph and
    replayed until at least `steps` calls have run (after SETTLE_S seconds and
    two untimed replays)."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for i in range(calls):
            fn(i)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            fn(i)
    reps = max(1, -(-steps // calls))
    spent = 0.0
    while spent < SETTLE_S:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        spent += e0.elapsed_time(e1) * 1e-3
    g.replay()
    g.replay()
    torch.cuda.synchronize()
    torch.cuda._sleep(100)  # trace marker, as in timed()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(reps):
        g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / (reps * calls)


def bf16_dev(a):
    import numpy as np
    import torch

    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def bench_prefill(args):
    import torch

    import attn_inputs as gen
    import exact_long_context_tiled_amd as attn

    w = gen.WORKLOADS["llama13b_gqa_causal_bf16"]
    case = gen.prefill_inputs(w["B"], w["Hq"], w["Hkv"], w["S"], w["T"], w["D"], kind="bf16", seed=0x5EED + 2)
    q, k, v = bf16_dev(case["q"]), bf16_dev(case["k"]), bf16_dev(case["v"])
    o = torch.empty((w["B"], w["S"], w["Hq"], w["D"]), dtype=torch.float32, device="cuda")
    lse = torch.empty((w["B"], w["Hq"], w["S"]), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(_):
        attn.prefill(q, k, v, causal=True, scale=case["scale"], out=o, lse=lse)

    ms = timed(step, args.steps, args.warmup, stream)
    flops = 4.0 * w["D"] * w["B"] * w["Hq"] * causal_pairs(w["S"], w["T"])
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"prefill: {ms:.4f} ms/launch, {tflops:.1f} TFLOP/s ({flops:.4e} flop)")
    return case, w, ms, flops, tflops


def bench_prefill_f32(args):
    """The tiny fp32 causal GQA prefill (B=1, Hq=4, Hkv=2, S=T=256, D=64):
    throughput against the fp32 vector peak, for information (its bar is
    parity at 1e-4 relative)."""
    import torch

    import attn_inputs as gen
    import exact_long_context_tiled_amd as attn

    w = gen.WORKLOADS["tiny_gqa_causal_f32"]
    case = gen.prefill_inputs(w["B"], w["Hq"], w["Hkv"], w["S"], w["T"], w["D"], kind="f32", seed=0x5EED + 1)
    q, k, v = (torch.from_numpy(case[n]).cuda() for n in "qkv")
    o = torch.empty((w["B"], w["S"], w["Hq"], w["D"]), dtype=torch.float32, device="cuda")
    lse = torch.empty((w["B"], w["Hq"], w["S"]), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(_):
        attn.prefill(q, k, v, causal=True, scale=case["scale"], out=o, lse=lse)

    ms = timed(step, max(args.steps, 200), max(args.warmup, 50), stream)
    flops = 4.0 * w["D"] * w["B"] * w["Hq"] * causal_pairs(w["S"], w["T"])
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"prefill fp32 tiny: {ms * 1e3:.2f} us/launch, {tflops:.3f} TFLOP/s")
    return {"workload": "tiny_gqa_causal_f32", "value": round(tflops, 4), "unit": "TFLOP/s",
            "us_per_launch": round(ms * 1e3, 3), "flop_per_launch": flops,
            "roofline": {"bound": "alu", "achieved": round(tflops, 4), "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / PEAK_FP32_TFLOPS, 5), "traffic": None,
                         "note": "128 work-groups of 8 packed rows, keys split over each one's 4 waves: "
                                 "information only, bound by launch and latency"}}


def bench_prefill_fp8(args):
    """The LLaMa-13B-shaped causal prefill with e4m3 Q/K/V and per-head scales
    (codes drawn on the device).  Q.K^T runs on fp8 matrix cores and P.V on
    bf16 ones, so the roofline peak is the blend of the two for equal flops."""
    import torch

    import attn_inputs as gen
    import exact_long_context_tiled_amd as attn

    w = gen.WORKLOADS["llama13b_gqa_causal_bf16"]
    B, Hq, Hkv, S, T, D = w["B"], w["Hq"], w["Hkv"], w["S"], w["T"], w["D"]
    g = torch.Generator(device="cuda")
    g.manual_seed(0x5EED + 8)
    q = torch.randn((B, S, Hq, D), generator=g, device="cuda").mul_(64).to(torch.float8_e4m3fn)
    k = torch.randn((B, T, Hkv, D), generator=g, device="cuda").mul_(64).to(torch.float8_e4m3fn)
    v = torch.randn((B, T, Hkv, D), generator=g, device="cuda").mul_(64).to(torch.float8_e4m3fn)
    qs = torch.full((Hq,), 1 / 64, device="cuda")
    ks = torch.full((Hkv,), 1 / 64, device="cuda")
    vs = torch.full((Hkv,), 1 / 64, device="cuda")
    o = torch.empty((B, S, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(_):
        attn.prefill_fp8(q, k, v, qs, ks, vs, causal=True, scale=1 / math.sqrt(D), out=o, lse=lse)

    ms = timed(step, args.steps, args.warmup, stream)
    flops = 4.0 * D * B * Hq * causal_pairs(S, T)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
    log(f"prefill fp8: {ms:.4f} ms/launch, {tflops:.1f} TFLOP/s")
    return {"workload": "llama13b_gqa_causal_fp8", "value": round(tflops, 2), "unit": "TFLOP/s",
            "ms_per_launch": round(ms, 5), "dtype": "e4m3 Q.K^T, bf16 P.V",
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": round(peak, 1), "unit": "TFLOP/s",
                         "frac": round(tflops / peak, 4),
                         "traffic": recorded_traffic("prefill_fp8_llama13b_pmc_traffic.md", "prefill_fp8.hip"),
                         "peak_note": "half the flops at the fp8 peak (5.0 PF), half at the bf16 peak (2.5 PF)"}}


def bench_decode(args):
    import numpy as np
    import torch

    import attn_inputs as gen
    import exact_long_context_tiled_amd as attn

    w = gen.WORKLOADS["paged_splitkv_decode_bf16"]
    seed = 0x5EED + 3
    lens = gen.ragged_lengths(w["B"], w["lo"], w["hi"], seed)
    case = gen.decode_inputs(w["B"], w["Hq"], w["Hkv"], w["D"], lens, kv="bf16", page_size=w["page_size"], seed=seed)
    q = bf16_dev(case["q"])
    kc, vc = bf16_dev(case["k"]), bf16_dev(case["v"])
    pt = torch.from_numpy(case["page_table"]).cuda()
    lens_d = torch.from_numpy(lens.astype(np.int32)).cuda()
    maxlen = int(lens.max())
    valid_tokens = int(lens.sum())
    kv_bytes = valid_tokens * w["Hkv"] * w["D"] * 2 * 2
    io_bytes = w["B"] * w["Hq"] * w["D"] * (2 + 4) + w["B"] * w["Hq"] * 4
    nbytes = kv_bytes + io_bytes
    cache_bytes = kc.numel() * 2 * 2
    copies = max(2, math.ceil((1 << 30) / cache_bytes))
    caches = [(kc, vc)] + [(kc.clone(), vc.clone()) for _ in range(copies - 1)]
    ws = torch.empty(attn.decode_workspace_size(w["B"], w["Hq"], w["Hkv"], w["D"], maxlen), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty((w["B"], w["Hq"], w["D"]), dtype=torch.float32, device="cuda")
    lse = torch.empty((w["B"], w["Hq"]), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        kk, vv = caches[i % copies]
        attn.decode_splitkv(q, kk, vv, lens_d, maxlen, page_table=pt, scale=case["scale"], workspace=ws, out=o,
                            lse=lse)

    steps = max(args.steps, copies * 4)
    ms = timed(step, steps, max(args.warmup, copies), stream)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"decode: {ms * 1e3:.2f} us/call, {gbs:.1f} GB/s ({nbytes / 1e6:.1f} MB, {copies} cache copies)")
    return {"workload": "paged_splitkv_decode_bf16", "value": round(gbs, 2), "unit": "GB/s", "us_per_call":
            round(ms * 1e3, 3), "bytes": nbytes, "valid_tokens": valid_tokens, "lengths": lens.tolist(),
            "cache_copies": copies, "steps": steps,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": recorded_traffic("decode_paged_bf16_pmc_traffic.md", *DECODE_SOURCES)}}


def bench_decode_quant(args):
    """Quantised-cache decode (B=4, Hq=32, Hkv=8, D=128, every sequence of
    length T for T = 4096 and 65536, contiguous cache): int8 codes with
    per-(token, KV head) scales, OCP e4m3fn codes with per-KV-head scales, and
    packed int4 codes with one scale per 32-element group.  The codes are
    seeded synthetic draws made on the device (parity on the same shapes is the
    GPU test suite's job); GB/s counts the cache bytes (codes + int8 / int4
    scales).  The caches rotate through >= 1 GiB of copies, so each timed
    launch streams from HBM (at T = 4096 one copy is 34 MB, well inside the
    256 MB last-level cache)."""
    import torch

    import attn_inputs as gen
    import exact_long_context_tiled_amd as attn

    w = gen.WORKLOADS["quant_decode"]
    B, Hq, Hkv, D = w["B"], w["Hq"], w["Hkv"], w["D"]
    g = torch.Generator(device="cuda")
    g.manual_seed(0x5EED + 4)
    q = torch.randn((B, Hq, D), generator=g, device="cuda").to(torch.bfloat16)
    o = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    by_t = {}
    for T in sorted(w["T"]):
        lens = torch.full((B,), T, dtype=torch.int32, device="cuda")
        ws = torch.empty(attn.decode_workspace_size(B, Hq, Hkv, D, T), dtype=torch.uint8, device="cuda")
        res = {}
        for kv in ("int8", "fp8", "int4"):
            shape = (B, Hkv, T, D // 2 if kv == "int4" else D)
            code_bytes = B * Hkv * T * shape[-1] * 2
            copies = max(2, math.ceil((1 << 30) / code_bytes))
            caches = []
            for _ in range(copies):
                if kv == "int4":
                    k = torch.randint(0, 256, shape, generator=g, dtype=torch.uint8, device="cuda")
                    v = torch.randint(0, 256, shape, generator=g, dtype=torch.uint8, device="cuda")
                    ks = torch.rand((B, Hkv, T, D // 32), generator=g, device="cuda") * 0.02 + 0.005
                    vs = torch.rand((B, Hkv, T, D // 32), generator=g, device="cuda") * 0.02 + 0.005
                elif kv == "int8":
                    k = torch.randint(-127, 128, shape, generator=g, dtype=torch.int8, device="cuda")
                    v = torch.randint(-127, 128, shape, generator=g, dtype=torch.int8, device="cuda")
                    ks = torch.rand((B, Hkv, T), generator=g, device="cuda") * 0.02 + 0.005
                    vs = torch.rand((B, Hkv, T), generator=g, device="cuda") * 0.02 + 0.005
                else:
                    k = torch.randn(shape, generator=g, device="cuda").to(torch.float8_e4m3fn)
                    v = torch.randn(shape, generator=g, device="cuda").to(torch.float8_e4m3fn)
                    ks = torch.full((Hkv,), 0.25, device="cuda")
                    vs = torch.full((Hkv,), 0.25, device="cuda")
                caches.append((k, v, ks, vs))

            def step(i, caches=caches, copies=copies, kv=kv, lens=lens, T=T, ws=ws):
                k, v, ks, vs = caches[i % copies]
                attn.decode_splitkv(q, k, v, lens, T, k_scale=ks, v_scale=vs, workspace=ws, out=o, lse=lse,
                                    kv_dtype="int4" if kv == "int4" else None)

            steps = max(args.steps, copies * 4)
            ms = timed(step, steps, max(args.warmup, copies), stream)
            scale_bytes = {"int8": B * Hkv * T * 4 * 2, "int4": B * Hkv * T * (D // 32) * 4 * 2}.get(kv, 0)
            nbytes = code_bytes + scale_bytes
            ms_eager = ms
            if T < 65536:
                # a ~20 us call is as long as the host's launch path: time it
                # as a HIP graph of one call per cache copy, replayed
                ms = timed_graph(step, copies, steps, stream)
            gbs = nbytes / (ms * 1e-3) / 1e9
            log(f"decode {kv} T={T}: {ms * 1e3:.2f} us/call, {gbs:.1f} GB/s ({nbytes / 1e6:.1f} MB, {copies} copies)"
                + (f"; launched one by one from Python: {ms_eager * 1e3:.2f} us/call" if ms != ms_eager else ""))
            prof = f"decode_{kv}_contig_pmc_traffic.md" if T == 65536 else f"decode_{kv}_contig_t4096_pmc_traffic.md"
            res[kv] = {"value": round(gbs, 2), "unit": "GB/s", "us_per_call": round(ms * 1e3, 3), "bytes": nbytes,
                       "cache_copies": copies, "steps": steps,
                       "timing": "hip graph of one call per cache copy, replayed" if ms != ms_eager else "eager",
                       "us_per_call_eager": round(ms_eager * 1e3, 3),
                       "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                    "frac": round(gbs / PEAK_HBM_GBS, 4),
                                    "traffic": recorded_traffic(prof, *DECODE_SOURCES)}}
            del caches
        by_t[T] = res
    return {"workload": "quant_decode", "B": B, "Hq": Hq, "Hkv": Hkv, "D": D, "T": 65536, "kv": by_t[65536],
            "T4096": {"T": 4096, "kv": by_t[4096]}}


def bench_decode_multi(args):
    """Multi-token decode (B=8, Hq=32, Hkv=8, D=128, n_q=4 verified tokens per
    sequence, 512-token pages, T_b ~ U[1024, 32768]) over bf16 and int8 paged
    caches drawn on the device; GB/s counts each valid K/V byte (and int8
    scale) once plus q/o/lse.  Beside it, single-token decode of the last
    query token on the same cache."""
    import numpy as np
    import torch

    import attn_inputs as gen
    import exact_long_context_tiled_amd as attn

    w = gen.WORKLOADS["multi_token_decode"]
    B, Hq, Hkv, D, n_q, ps = w["B"], w["Hq"], w["Hkv"], w["D"], w["n_q"], w["page_size"]
    seed = 0x5EED + 6
    lens = gen.ragged_lengths(B, w["lo"], w["hi"], seed)
    table, P = gen.page_table(lens, ps, 8, seed)
    pt = torch.from_numpy(np.ascontiguousarray(table, dtype=np.int32)).cuda()
    lens_d = torch.from_numpy(lens.astype(np.int32)).cuda()
    maxlen = int(lens.max())
    valid = int(lens.sum())
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    q = torch.randn((B, n_q, Hq, D), generator=g, device="cuda").to(torch.bfloat16)
    q1 = q[:, -1].contiguous()
    ws = torch.empty(attn.decode_multi_workspace_size(B, n_q, Hq, Hkv, D, maxlen), dtype=torch.uint8,
                     device="cuda")
    ws1 = torch.empty(attn.decode_workspace_size(B, Hq, Hkv, D, maxlen), dtype=torch.uint8, device="cuda")
    o = torch.empty((B, n_q, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, n_q), dtype=torch.float32, device="cuda")
    o1 = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    l1 = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    shape = (P, Hkv, ps, D)
    res = {}
    for kv in ("bf16", "int8"):
        eb = 2 if kv == "bf16" else 1
        cache_bytes = P * Hkv * ps * D * eb * 2
        copies = max(2, math.ceil((1 << 30) / cache_bytes))
        caches = []
        for _ in range(copies):
            if kv == "bf16":
                k = torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16)
                v = torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16)
                ks = vs = None
            else:
                k = torch.randint(-127, 128, shape, generator=g, dtype=torch.int8, device="cuda")
                v = torch.randint(-127, 128, shape, generator=g, dtype=torch.int8, device="cuda")
                ks = torch.rand((P, Hkv, ps), generator=g, device="cuda") * 0.02 + 0.005
                vs = torch.rand((P, Hkv, ps), generator=g, device="cuda") * 0.02 + 0.005
            caches.append((k, v, ks, vs))

        def step(i, caches=caches, copies=copies):
            k, v, ks, vs = caches[i % copies]
            attn.decode_multi(q, k, v, lens_d, maxlen, page_table=pt, k_scale=ks, v_scale=vs, workspace=ws, out=o,
                              lse=lse)

        def step1(i, caches=caches, copies=copies):
            k, v, ks, vs = caches[i % copies]
            attn.decode_splitkv(q1, k, v, lens_d, maxlen, page_table=pt, k_scale=ks, v_scale=vs, workspace=ws1,
                                out=o1, lse=l1)

        steps = max(args.steps, copies * 4)
        ms = timed(step, steps, max(args.warmup, copies), stream)
        ms1 = timed(step1, steps, max(args.warmup, copies), stream)
        kv_bytes = valid * Hkv * D * eb * 2 + (valid * Hkv * 4 * 2 if kv == "int8" else 0)
        nbytes = kv_bytes + B * n_q * Hq * (D * (2 + 4) + 4)
        gbs = nbytes / (ms * 1e-3) / 1e9
        log(f"decode multi-token {kv} n_q={n_q}: {ms * 1e3:.2f} us/call, {gbs:.1f} GB/s "
            f"(single-token on the same cache: {ms1 * 1e3:.2f} us)")
        res[kv] = {"value": round(gbs, 2), "unit": "GB/s", "us_per_call": round(ms * 1e3, 3), "bytes": nbytes,
                   "single_token_us_per_call": round(ms1 * 1e3, 3), "cache_copies": copies, "steps": steps,
                   "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": round(gbs / PEAK_HBM_GBS, 4),
                                "traffic": recorded_traffic(f"decode_multi_{kv}_pmc_traffic.md", *DECODE_SOURCES)}}
        del caches
    return {"workload": "multi_token_decode", "B": B, "n_q": n_q, "Hq": Hq, "Hkv": Hkv, "D": D,
            "page_size": ps, "lengths": lens.tolist(), "kv": res}


def cpu_baseline(case, w, target_s):
    """The fp64 oracle on this host: a bounded sample of query rows of the
    headline prefill (``value``, in the metric's TFLOP/s), and the small
    configurations in full -- the tiny fp32 prefill, the paged split-KV decode
    and the quantised decodes -- with all threads and (where it takes seconds)
    with one.  A reported baseline, not a target."""
    import numpy as np

    import attn_inputs as gen
    import oracle

    S, T = w["S"], w["T"]
    n_all = oracle.threads()

    def run(n):
        rows = gen.sample_rows(S, n, 0x5EED + 7)
        t0 = time.perf_counter()
        oracle.prefill(case, rows=rows)
        dt = time.perf_counter() - t0
        pairs = sum(min(T, int(i) + T - S + 1) for i in rows)
        return dt, 4.0 * w["D"] * w["B"] * w["Hq"] * pairs, rows

    dt, fl, rows = run(4)
    n = int(max(4, min(512, 4 * target_s / max(dt, 1e-3))))
    dt, fl, rows = run(n)
    out = {"value": round(fl / dt / 1e12, 8), "unit": "TFLOP/s", "cores": n_all, "kind": "oracle",
           "seconds": round(dt, 2),
           "sample": f"{len(rows)} seeded query rows (incl. 0 and S-1) x all {w['Hq']} heads x B={w['B']} of the "
                     f"same prefill workload, fp64 naive softmax, {fl:.3e} flop",
           "host": {"os_cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)),
                    "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS"), "oracle_threads": n_all}}

    def timed_full(fn, flop, one_thread):
        res = {}
        for th in ((n_all, 1) if one_thread else (n_all,)):
            oracle.set_threads(th)
            t0 = time.perf_counter()
            fn()
            dt = time.perf_counter() - t0
            res[f"threads_{th}"] = {"seconds": round(dt, 3), "gflops": round(flop / dt / 1e9, 3)}
        oracle.set_threads(n_all)
        return dict(res, flop=flop)

    full = {}
    t = gen.WORKLOADS["tiny_gqa_causal_f32"]
    c1 = gen.prefill_inputs(t["B"], t["Hq"], t["Hkv"], t["S"], t["T"], t["D"], kind="f32", seed=0x5EED + 1)
    full["tiny_gqa_causal_f32"] = timed_full(lambda: oracle.prefill(c1),
                                             4.0 * t["D"] * t["B"] * t["Hq"] * causal_pairs(t["S"], t["T"]), True)
    d = gen.WORKLOADS["paged_splitkv_decode_bf16"]
    lens = gen.ragged_lengths(d["B"], d["lo"], d["hi"], 0x5EED + 3)
    c3 = gen.decode_inputs(d["B"], d["Hq"], d["Hkv"], d["D"], lens, kv="bf16", page_size=d["page_size"],
                           seed=0x5EED + 3)
    full["paged_splitkv_decode_bf16"] = timed_full(lambda: oracle.decode(c3),
                                                   4.0 * d["D"] * d["Hq"] * float(lens.sum()), True)
    del c3
    q4 = gen.WORKLOADS["quant_decode"]
    for T4 in q4["T"]:
        for kv in ("int8", "fp8"):
            l4 = np.full(q4["B"], T4, dtype=np.int32)
            c4 = gen.decode_inputs(q4["B"], q4["Hq"], q4["Hkv"], q4["D"], l4, kv=kv, paged=False,
                                   seed=0x5EED + 4 + (T4 == 65536))
            full[f"quant_decode_{kv}_T{T4}"] = timed_full(lambda: oracle.decode(c4),
                                                          4.0 * q4["D"] * q4["Hq"] * q4["B"] * T4, T4 == 4096)
            del c4
    out["full_configs"] = full
    log("cpu baseline: " + ", ".join(f"{k} {v[f'threads_{n_all}']['seconds']} s" for k, v in full.items()))
    return out


class FreeMemoryLow:
    """Lowest free device memory (hipMemGetInfo) seen by a polling thread while
    the block runs: the drop from the free memory before it is what a
    synchronous call held on the device at its peak."""

    def __enter__(self):
        import threading

        import torch

        self._torch = torch
        self.before = torch.cuda.mem_get_info()[0]
        self.low = self.before
        self._stop = threading.Event()

        def poll():
            while not self._stop.is_set():
                self.low = min(self.low, torch.cuda.mem_get_info()[0])
                self._stop.wait(0.0005)

        self._t = threading.Thread(target=poll, daemon=True)
        self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._t.join()
        self.low = min(self.low, self._torch.cuda.mem_get_info()[0])
        self.drop = self.before - self.low
        return False


def bench_stream(args):
    """Budgeted streaming prefill (Stream-CQSA summary, Methodology 2-4):
    B=1, Hq=32, Hkv=8, S=T=2^20, D=128 bf16 causal from pinned host memory
    under a 4e9-byte device budget, plus a budget sweep.  Inputs are N(0,1)
    bf16 drawn on the device and copied to pinned host memory (this leg
    measures throughput and memory; the million-token parity test runs the
    seeded host draws against the oracle)."""
    import torch

    import attn_inputs as gen
    import exact_long_context_tiled_amd as attn

    w = gen.WORKLOADS["stream_cqsa_causal_1m"]
    B, Hq, Hkv, S, T, D = w["B"], w["Hq"], w["Hkv"], w["S"], w["T"], w["D"]
    scale = 1 / math.sqrt(D)
    t0 = time.perf_counter()
    hq = torch.empty((B, S, Hq, D), dtype=torch.bfloat16, pin_memory=True)
    hk = torch.empty((B, T, Hkv, D), dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty((B, T, Hkv, D), dtype=torch.bfloat16, pin_memory=True)
    ho = torch.empty((B, S, Hq, D), dtype=torch.float32, pin_memory=True)
    hl = torch.empty((B, Hq, S), dtype=torch.float32, pin_memory=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(0x5EED + 5)
    step = 1 << 16
    for h in (hq, hk, hv):
        for s0 in range(0, h.shape[1], step):
            h[:, s0:s0 + step].copy_(torch.randn(h[:, s0:s0 + step].shape, generator=g, device="cuda")
                                     .to(torch.bfloat16))
    torch.cuda.synchronize()
    log(f"stream: {(hq.numel() + hk.numel() + hv.numel()) * 2 / 2**30:.1f} GiB of inputs in pinned memory "
        f"({time.perf_counter() - t0:.1f} s)")

    def flops_of(n):
        return 4.0 * D * B * Hq * (n * (n + 1) // 2)

    def run(n, budget, lse=True):
        with FreeMemoryLow() as mem:
            o, _, rep = attn.stream_budgeted(hq[:, :n], hk[:, :n], hv[:, :n], causal=True, scale=scale,
                                             budget=budget, o_host=ho[:, :n], lse_host=hl if lse else None,
                                             return_lse=lse)
        fl = flops_of(n)
        res = {"S": n, "budget_bytes": budget, "report": rep,
               "planned_peak_device_bytes": rep["peak_device_bytes"], "measured_free_memory_drop": mem.drop,
               "tflops_end_to_end": round(fl / rep["wall_s"] / 1e12, 2),
               "tflops_kernels": round(fl / rep["kernel_s"] / 1e12, 2),
               "h2d_gbs": round(rep["h2d_bytes"] / rep["wall_s"] / 1e9, 2),
               "d2h_gbs": round(rep["d2h_bytes"] / rep["wall_s"] / 1e9, 2)}
        log(f"stream S={n} budget={budget / 1e9:.1f} GB: {rep['wall_s']:.2f} s wall ({res['tflops_end_to_end']} "
            f"TFLOP/s), kernels {rep['kernel_s']:.2f} s ({res['tflops_kernels']} TFLOP/s), blocks "
            f"{rep['block_q']}x{rep['block_k']}, planned peak {rep['peak_device_bytes'] / 1e9:.3f} GB, "
            f"free memory drop {mem.drop / 1e9:.3f} GB")
        return res

    out = {"workload": "stream_cqsa_causal_1m", "budget_bytes": w["budget"], "data": "N(0,1) bf16 drawn on the "
           "device, pinned host memory", "flop": flops_of(S)}
    full = run(S, w["budget"])
    out.update({k: v for k, v in full.items() if k not in ("S", "budget_bytes")})
    out["tflops"] = full["tflops_end_to_end"]
    # device bytes follow the block size, not the length (Stream-CQSA summary,
    # "Results & findings"): the planner's choice for S = 2^20 under each
    # budget, and measured runs at S = 2^18 and 2^19
    sweep = []
    for budget in (1e9, 2e9, 4e9, 8e9):
        _, rep = attn.stream_plan("bf16", B, Hq, Hkv, S, T, D, causal=True, budget=int(budget), with_tasks=False)
        sweep.append({"S": S, "budget_bytes": int(budget), "planned_only": True, "block_q": rep["block_q"],
                      "block_k": rep["block_k"], "tasks": rep["tasks"],
                      "planned_peak_device_bytes": rep["peak_device_bytes"], "h2d_bytes": rep["h2d_bytes"]})
    for n, budget in ((1 << 18, int(5e8)), (1 << 18, int(1e9)), (1 << 18, int(2e9)), (1 << 19, int(1e9))):
        r = run(n, budget, lse=False)
        sweep.append({"S": n, "budget_bytes": budget, "planned_only": False, "block_q": r["report"]["block_q"],
                      "block_k": r["report"]["block_k"], "tasks": r["report"]["tasks"],
                      "planned_peak_device_bytes": r["planned_peak_device_bytes"],
                      "measured_free_memory_drop": r["measured_free_memory_drop"],
                      "tflops_end_to_end": r["tflops_end_to_end"]})
    out["budget_sweep"] = sweep
    if args.stream_cqs:
        o_c, _, info, rep = attn.stream_cqs(hq, hk, hv, causal=True, scale=scale, budget=w["budget"])
        log(f"stream (cyclic quorums): N={info['n_blocks']} k={info['quorum_size']} {rep}")
        out["cqs"] = {"report": rep, "tflops_end_to_end": round(flops_of(S) / rep["wall_s"] / 1e12, 2),
                      "tflops_kernels": round(flops_of(S) / rep["kernel_s"] / 1e12, 2),
                      "host_link_gbs": round((rep["h2d_bytes"] + rep["d2h_bytes"]) / rep["wall_s"] / 1e9, 2),
                      "n_blocks": info["n_blocks"], "quorum_size": info["quorum_size"], "pairs": info["pairs"]}
        full_o = attn.stream_budgeted(hq, hk, hv, causal=True, scale=scale, budget=w["budget"], return_lse=False)[0]
        diff = max(float((full_o[:, s0:s0 + step] - o_c[:, s0:s0 + step]).abs().max()) for s0 in range(0, S, step))
        out["cqs"]["max_abs_diff_vs_rectangular"] = diff
        log(f"stream: cyclic-quorum vs rectangular output max |diff| = {diff:.3e}")
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--legs", default="fp8,f32,decode,quant,multi,stream,cpu",
                    help="comma list of the legs to run beside the headline prefill: "
                         "fp8, f32, decode, quant, multi, stream, cpu (default: all)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-stream", action="store_true", help="skip the 2^20-token budgeted streaming workload")
    ap.add_argument("--stream-cqs", action="store_true",
                    help="also run that workload with the cyclic-quorum plan (host-link heavy: minutes)")
    ap.add_argument("--settle-seconds", type=float, default=0.3,
                    help="GPU seconds of untimed calls before each leg's warmup (out of the idle clock ramp)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device-to-device copy three times (PMC byte-counter reference)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (sharding is a design note only); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    torch.cuda.set_device(0)
    global SETTLE_S
    SETTLE_S = args.settle_seconds
    case, w, ms, flops, tflops = bench_prefill(args)
    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded iid N(0,1), bf16)",
        "config": {"workload": "llama13b_gqa_causal_bf16", "B": w["B"], "Hq": w["Hq"], "Hkv": w["Hkv"],
                   "S": w["S"], "T": w["T"], "D": w["D"], "causal": True, "flop_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic("prefill_llama13b_pmc_traffic.md", "prefill_bf16.hip")},
    }
    out["clock_settle_s_per_leg"] = args.settle_seconds
    legs = set(args.legs.split(","))
    if args.no_decode:
        legs -= {"decode", "quant", "multi"}
    if args.no_stream:
        legs.discard("stream")
    if args.no_cpu_baseline:
        legs.discard("cpu")
    if "fp8" in legs:
        out["prefill_fp8"] = bench_prefill_fp8(args)
    if "f32" in legs:
        out["prefill_f32"] = bench_prefill_f32(args)
    if "decode" in legs:
        out["decode"] = bench_decode(args)
    if "quant" in legs:
        out["decode_quant"] = bench_decode_quant(args)
    if "multi" in legs:
        out["decode_multi"] = bench_decode_multi(args)
    if "stream" in legs:
        out["stream"] = bench_stream(args)
    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = src.numel() * 4
    if "cpu" in legs:
        out["cpu_baseline"] = cpu_baseline(case, w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
