#!/usr/bin/env python3
"""Throughput of the attention hot path on one MI355X.

Default workload: the Llama-3-8B-shaped causal GQA prefill (B=1, T=8192,
h_q=32, h_kv=8, d_h=128, bf16 in / fp32 accumulate / bf16 out, scale
1/sqrt(128)) -- ``value`` is its throughput in TFLOP/s, counting only the
visible (query, key) pairs, 4*d_h FLOP per pair (Q.K and P.V).  The same run
also measures the two decode forms on their workloads -- 70B-shaped GQA
decode (B=64, 64/8 heads, cached lengths uniform in [4096, 32768]) and
DeepSeek-V3-shaped MLA absorbed decode (B=32, 128 heads, 16384 tokens of
576 values) -- in KV-cache GB/s, counting only cache rows inside each
sequence plus q and o -- the two sliding-window prefills (B=4, T=4096,
32 query heads, window 1024, with 32 and with 1 K/V head) in TFLOP/s, the
backward (dQ, dK, dV) of the Llama-3-8B prefill in TFLOP/s, counting
10*d_h FLOP per visible pair (five products), and the 70B decode on a paged
cache (pages of 64 positions in a random order) in GB/s.

The tiny fp32 parity configuration (B=1, T=64, 4/2 heads, d_h=16) is timed
too, in microseconds: it is one kernel launch.

Inputs are seeded synthetic N(0,1) tensors (workloads.py), resident in HBM
before timing.  W untimed warm-up steps, then exactly K timed steps between
two device synchronisations; HIP events recorded on the stream the kernels
run on bracket every call, giving the mean (``ms``, ``ms_per_step``) and the
median (``median_ms``) per call.  The JSON line also names the library file
that was timed and its hash.  One JSON line is printed.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--only prefill|swa-mha|swa-mqa|backward|decode|decode-fp8|rope|
                            decode-paged|mla|tiny-fp32|copy]

``--only copy`` times a plain 1 GiB device copy instead: it is the
calibration run for rocprofv3's HBM byte counters, not an attention bench.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
# rocprofv3 FETCH_SIZE/WRITE_SIZE summaries (KiB per dispatch), scaled by the
# same counters read on a plain copy kernel of known size; None until taken
# for the current kernel.
PREFILL_TRAFFIC_BYTES = 211314853   # prefill_bf16_d128 kernel <1,2,4>: FETCH_SIZE x 2.000 + WRITE_SIZE x 1.000 KiB


def prefill_visible_pairs(T: int, causal: bool, window: int) -> int:
    """Number of (query, key) pairs the mask leaves visible in one head."""
    if not causal:
        return T * T
    if window <= 0 or window >= T:
        return T * (T + 1) // 2
    w = window
    return w * (w + 1) // 2 + (T - w) * w


def prefill_flops(shape) -> int:
    return 4 * shape.B * shape.h_q * shape.d_h * prefill_visible_pairs(shape.T, shape.causal,
                                                                        shape.window)


LAST_MEDIAN_MS = {}


SPIN_UP_S = 0.25


def _spin_up(torch, fn):
    """Keeps the GPU busy with `fn` for SPIN_UP_S seconds, untimed, so that the
    timed calls run at the device's steady clocks: from idle the MI355X takes
    far longer than a few calls to raise them (five warm-up calls of the
    Llama-3-8B prefill measured 0.596 ms per call, against 0.521 ms after
    200 warm-up calls, on the same box)."""
    t_end = time.perf_counter() + SPIN_UP_S
    while time.perf_counter() < t_end:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()


def _events_time(torch, fn, steps, warmup, stream, key=None):
    """Mean milliseconds per call over `steps` back-to-back calls (HIP events
    on `stream` around each call), after the spin-up and `warmup` untimed
    calls; the median of the per-call durations is kept in
    LAST_MEDIAN_MS[key]."""
    _spin_up(torch, fn)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    n = len(per_call)
    median = (per_call[n // 2] if n % 2 else 0.5 * (per_call[n // 2 - 1] + per_call[n // 2]))
    if key is not None:
        LAST_MEDIAN_MS[key] = median
    return ev[0].elapsed_time(ev[steps]) / steps, wall


def bench_prefill(torch, ta, W, shape, steps, warmup):
    q, k, v = W.prefill_inputs(shape, seed=0, device="cuda", gen_device="cuda")
    o = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    fn = lambda: ta.attn_prefill(q, k, v, causal=shape.causal, window=shape.window,
                                 scale=shape.scale, o=o)
    ms, wall = _events_time(torch, fn, steps, warmup, stream, key=shape.name)
    flops = prefill_flops(shape)
    tflops = flops / (ms * 1e-3) / 1e12
    del q, k, v, o
    return {"ms": ms, "wall_s": wall, "flops": flops, "tflops": tflops,
            "frac_bf16_peak": tflops / BF16_PEAK_TFLOPS}


def backward_flops(shape) -> int:
    """Five products per visible pair and head (S recomputed, dP, dV, dK, dQ), 2 d_h each;
    the scores and dP that the dQ pass recomputes are not credited."""
    return 10 * shape.B * shape.h_q * shape.d_h * prefill_visible_pairs(shape.T, shape.causal,
                                                                         shape.window)


def bench_backward(torch, ta, W, shape, steps, warmup):
    q, k, v = W.prefill_inputs(shape, seed=0, device="cuda", gen_device="cuda")
    g = torch.Generator(device="cuda").manual_seed(1)
    do = torch.randn(q.shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    o, lse = ta.attn_prefill(q, k, v, causal=shape.causal, window=shape.window, scale=shape.scale,
                             return_lse=True)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(ta.attn_prefill_backward_workspace_size(shape.B, shape.T, shape.h_q),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    fn = lambda: ta.attn_prefill_backward(q, k, v, o, do, lse, causal=shape.causal,
                                          window=shape.window, scale=shape.scale, dq=dq, dk=dk,
                                          dv=dv, workspace=ws)
    ms, wall = _events_time(torch, fn, steps, warmup, stream, key="backward")
    flops = backward_flops(shape)
    tflops = flops / (ms * 1e-3) / 1e12
    del q, k, v, do, o, lse, dq, dk, dv, ws
    return {"ms": ms, "wall_s": wall, "flops": flops, "tflops": tflops,
            "frac_bf16_peak": tflops / BF16_PEAK_TFLOPS}


def bench_decode(torch, ta, W, steps, warmup):
    s = W.GQA70B_DECODE
    q, kc, vc, lens = W.decode_inputs(s, seed=0, device="cuda", gen_device="cuda")
    lens_d = lens.cuda()
    o = torch.empty_like(q)
    ws = torch.empty(ta.attn_decode_workspace_size(s.B, s.S_max, s.h_q, s.h_kv, s.d_h),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    fn = lambda: ta.attn_decode(q, kc, vc, lens_d, scale=s.scale, o=o, workspace=ws)
    ms, wall = _events_time(torch, fn, steps, warmup, stream, key="decode")
    total_len = int(lens.sum())
    cache_bytes = total_len * 2 * s.h_kv * s.d_h * 2
    io_bytes = 2 * s.B * s.h_q * s.d_h * 2
    gbs = (cache_bytes + io_bytes) / (ms * 1e-3) / 1e9
    del q, kc, vc, o, ws
    return {"ms": ms, "wall_s": wall, "bytes": cache_bytes + io_bytes, "sum_len": total_len,
            "gbs": gbs, "frac_hbm_peak": gbs / HBM_PEAK_GBS}


def bench_decode_paged(torch, ta, W, steps, warmup, page_size=64):
    """The 70B decode with its cache in pages of `page_size` positions, in a
    seeded random page order (the same bytes as the contiguous decode)."""
    s = W.GQA70B_DECODE
    q, kc, vc, lens = W.decode_inputs(s, seed=0, device="cuda", gen_device="cuda")
    kp, table = W.paged_layout(kc, page_size, seed=9, fill=0.0)
    del kc
    vp = torch.empty_like(kp)
    vp[table.view(-1).long()] = vc.view(s.B, s.h_kv, s.S_max // page_size, page_size, s.d_h).permute(
        0, 2, 1, 3, 4).reshape(-1, s.h_kv, page_size, s.d_h)
    del vc
    lens_d = lens.to("cuda")
    o = torch.empty_like(q)
    ws = torch.empty(ta.attn_decode_workspace_size(s.B, s.S_max, s.h_q, s.h_kv, s.d_h),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    fn = lambda: ta.attn_decode_paged(q, kp, vp, lens_d, table, scale=s.scale, o=o, workspace=ws)
    ms, wall = _events_time(torch, fn, steps, warmup, stream, key="decode_paged")
    total_len = int(lens.sum())
    nbytes = total_len * 2 * s.h_kv * s.d_h * 2 + 2 * s.B * s.h_q * s.d_h * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    del q, kp, vp, o, ws
    return {"ms": ms, "wall_s": wall, "bytes": nbytes, "gbs": gbs, "page_size": page_size,
            "frac_hbm_peak": gbs / HBM_PEAK_GBS}


def bench_decode_fp8(torch, ta, W, steps, warmup):
    """The 70B decode against the same cache quantised to FP8 (E4M3, one scale
    per 32 positions of a head): half the cache bytes."""
    s = W.GQA70B_DECODE
    q, kc, vc, lens = W.decode_inputs(s, seed=0, device="cuda", gen_device="cuda")
    k8, ks = ta.attn_quantize_kv_fp8(kc)
    del kc
    v8, vs = ta.attn_quantize_kv_fp8(vc)
    del vc
    lens_d = lens.to("cuda")
    o = torch.empty_like(q)
    ws = torch.empty(ta.attn_decode_workspace_size(s.B, s.S_max, s.h_q, s.h_kv, s.d_h),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    fn = lambda: ta.attn_decode_fp8(q, k8, v8, ks, vs, lens_d, scale=s.scale, o=o, workspace=ws)
    ms, wall = _events_time(torch, fn, steps, warmup, stream, key="decode_fp8")
    total_len = int(lens.sum())
    tiles = int(((lens + 31) // 32).sum())
    nbytes = (total_len * 2 * s.h_kv * s.d_h + tiles * 2 * s.h_kv * 4 +
              2 * s.B * s.h_q * s.d_h * 2)
    gbs = nbytes / (ms * 1e-3) / 1e9
    del q, k8, v8, ks, vs, o, ws
    return {"ms": ms, "wall_s": wall, "bytes": nbytes, "gbs": gbs,
            "frac_hbm_peak": gbs / HBM_PEAK_GBS}


def bench_rope(torch, ta, W, steps, warmup):
    """RoPE of the Llama-3-8B prefill's q and k in place (base 5e5): every
    value read and written once."""
    s = W.LLAMA3_8B_PREFILL
    q, k, v = W.prefill_inputs(s, seed=0, device="cuda", gen_device="cuda")
    del v
    stream = torch.cuda.current_stream()
    ms, wall = _events_time(torch, lambda: ta.attn_rope_qk(q, k, base=5e5), steps, warmup, stream, key="rope")
    nbytes = 2 * (q.numel() + k.numel()) * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    del q, k
    return {"ms": ms, "wall_s": wall, "bytes": nbytes, "gbs": gbs, "frac_hbm_peak": gbs / HBM_PEAK_GBS}


def bench_copy(torch, steps, warmup, nbytes=1 << 30):
    """A plain device-to-device copy of known size (reads and writes nbytes
    each).  Not part of the attention path: its HBM counter readings give the
    scale factor between rocprofv3's FETCH_SIZE/WRITE_SIZE and bytes."""
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    ms, wall = _events_time(torch, lambda: dst.copy_(src), steps, warmup, stream, key="copy")
    gbs = 2 * nbytes / (ms * 1e-3) / 1e9
    del src, dst
    return {"ms": ms, "wall_s": wall, "bytes": 2 * nbytes, "gbs": gbs,
            "frac_hbm_peak": gbs / HBM_PEAK_GBS}


def bench_mla(torch, ta, W, steps, warmup, copies=3):
    s = W.DSV3_MLA_DECODE
    sets = [W.mla_inputs(s, seed=i, device="cuda", gen_device="cuda") for i in range(copies)]
    sets = [(q, c, lens.cuda()) for q, c, lens in sets]
    o = torch.empty((s.B, s.H, s.d_c), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(ta.mla_decode_workspace_size(s.B, s.S_max, s.H, s.d_c, s.d_r),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    it = [0]

    def fn():
        q, c, lens = sets[it[0] % copies]     # rotate caches: the timed bytes come from HBM
        it[0] += 1
        ta.mla_decode(q, c, lens, scale=s.scale, o=o, workspace=ws)

    ms, wall = _events_time(torch, fn, steps, warmup, stream, key="mla")
    total = int(sum(int(l.sum()) for _, _, l in sets[:1]))
    cache_bytes = total * (s.d_c + s.d_r) * 2
    io_bytes = s.B * s.H * (s.d_c + s.d_r) * 2 + s.B * s.H * s.d_c * 2
    gbs = (cache_bytes + io_bytes) / (ms * 1e-3) / 1e9
    flops = 2 * s.H * total * (s.d_c + s.d_r + s.d_c)
    del sets, o, ws
    return {"ms": ms, "wall_s": wall, "bytes": cache_bytes + io_bytes, "gbs": gbs,
            "frac_hbm_peak": gbs / HBM_PEAK_GBS,
            "tflops": flops / (ms * 1e-3) / 1e12, "cache_copies_rotated": copies}


def bench_mla_fp8(torch, ta, W, steps, warmup, copies=3):
    """The DeepSeek-V3-shaped MLA decode with FP8 attention: each of the
    rotated bf16 caches quantised to E4M3 (one scale per 32 tokens) by the
    library's quantiser before timing; the query is quantised inside the
    call.  Bytes: codes + scales + q + o."""
    s = W.DSV3_MLA_DECODE
    dk = s.d_c + s.d_r
    sets = []
    for i in range(copies):
        q, c, lens = W.mla_inputs(s, seed=i, device="cuda", gen_device="cuda")
        codes, scales = ta.attn_quantize_kv_fp8(c.view(s.B, 1, s.S_max, dk))
        del c
        sets.append((q, codes.view(s.B, s.S_max, dk), scales.view(s.B, -1), lens.cuda()))
    o = torch.empty((s.B, s.H, s.d_c), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(ta.mla_decode_fp8_workspace_size(s.B, s.S_max, s.H, s.d_c, s.d_r),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    it = [0]

    def fn():
        q, codes, scales, lens = sets[it[0] % copies]
        it[0] += 1
        ta.mla_decode_fp8(q, codes, scales, lens, scale=s.scale, o=o, workspace=ws)

    ms, wall = _events_time(torch, fn, steps, warmup, stream, key="mla_fp8")
    lens0 = sets[0][3]
    total = int(lens0.sum())
    n_scales = int(((lens0 + 31) // 32).sum())
    nbytes = total * dk + n_scales * 4 + s.B * s.H * dk * 2 + s.B * s.H * s.d_c * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    flops = 2 * s.H * total * (s.d_c + s.d_r + s.d_c)
    del sets, o, ws
    return {"ms": ms, "wall_s": wall, "bytes": nbytes, "gbs": gbs,
            "frac_hbm_peak": gbs / HBM_PEAK_GBS, "tflops": flops / (ms * 1e-3) / 1e12,
            "cache_copies_rotated": copies}


FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 (E4M3) MFMA, TFLOP/s


def bench_prefill_fp8(torch, ta, W, shape, steps, warmup):
    """The Llama-3-8B-shaped causal prefill with FP8 attention: q, k and v
    quantised to E4M3 (one scale per 32 positions of a head) by the
    library's quantiser before timing."""
    q, k, v = W.prefill_inputs(shape, seed=0, device="cuda", gen_device="cuda")
    (q8, qs), (k8, ks), (v8, vs) = (ta.attn_quantize_kv_fp8(x) for x in (q, k, v))
    del q, k, v
    o = torch.empty(q8.shape, dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    fn = lambda: ta.attn_prefill_fp8(q8, k8, v8, qs, ks, vs, causal=shape.causal,
                                     window=shape.window, scale=shape.scale, o=o)
    ms, wall = _events_time(torch, fn, steps, warmup, stream, key="prefill_fp8")
    flops = prefill_flops(shape)
    tflops = flops / (ms * 1e-3) / 1e12
    del q8, k8, v8, qs, ks, vs, o
    return {"ms": ms, "wall_s": wall, "flops": flops, "tflops": tflops,
            "frac_fp8_peak": tflops / FP8_PEAK_TFLOPS}


def bench_tiny_fp32(torch, ta, W, steps, warmup):
    """The tiny fp32 causal GQA prefill (B=1, T=64, 4/2 heads, d_h=16): a
    parity case whose time is one kernel launch; reported in microseconds."""
    s = W.TINY_FP32
    q, k, v = W.prefill_inputs(s, seed=0, device="cuda")
    o = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    fn = lambda: ta.attn_prefill(q, k, v, causal=True, scale=s.scale, o=o)
    ms, wall = _events_time(torch, fn, max(steps, 20), warmup, stream, key="tiny_fp32")
    return {"ms": ms, "wall_s": wall, "flops": prefill_flops(s)}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline_prefill(W, shape, budget_s=20.0):
    """The fp64 oracle on a bounded sample of the prefill workload: all heads
    of a growing set of query rows until the budget is used.  `value` counts
    the visible (query, key) pairs, 4 d_h FLOP each, like the GPU figure; the
    oracle as written scores every key of a row before masking, so it also
    does 2 d_h FLOP per masked pair (`flops_as_written`)."""
    import numpy as np
    import oracle
    oracle.build(force=False)
    q, k, v = W.prefill_inputs(shape, seed=0, device="cpu")
    qn, kn, vn = (t.float().numpy() for t in (q, k, v))
    n_rows = 8
    elapsed, rows = 0.0, None
    while True:
        rows = np.linspace(0, shape.T - 1, n_rows).astype(np.int32)
        t0 = time.perf_counter()
        oracle.prefill(qn, kn, vn, causal=shape.causal, window=shape.window, scale=shape.scale,
                       rows=rows)
        elapsed = time.perf_counter() - t0
        if elapsed >= budget_s / 4 or n_rows >= shape.T:
            break
        n_rows = min(shape.T, n_rows * 2)
    vis = 0
    for r in rows.tolist():
        lo = max(0, r - shape.window + 1) if shape.window else 0
        hi = r + 1 if shape.causal else shape.T
        vis += hi - lo
    per_pair = shape.B * shape.h_q * shape.d_h
    flops = 4 * per_pair * vis
    as_written = 2 * per_pair * (len(rows) * shape.T + vis)
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(),
            "kind": "oracle", "cpu_model": _cpu_model(),
            "host_cpus_available": len(os.sched_getaffinity(0)),
            "wall_s": round(elapsed, 2), "flops_visible_pairs": flops,
            "flops_as_written": as_written,
            "value_as_written": as_written / elapsed / 1e12,
            "sample": f"{len(rows)} evenly spaced query rows x all {shape.h_q} heads of "
                      f"the workload ({elapsed:.1f} s, fp64, full score rows materialised)"}


def _library_info(ta):
    import hashlib
    path = os.path.abspath(ta.LIB_PATH)
    with open(path, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    return {"path": os.path.relpath(path, os.path.dirname(os.path.abspath(__file__))),
            "sha256_16": digest[:16]}


BENCHES = ("prefill", "swa-mha", "swa-mqa", "backward", "prefill-fp8", "decode", "decode-fp8",
           "rope", "decode-paged", "mla", "mla-fp8", "tiny-fp32", "copy")


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None, choices=BENCHES)
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the attention path here runs on a single MI355X)", file=sys.stderr)
        return 2

    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import torch
    import transformer_attention_amd as ta
    import workloads as W
    ta.load_library()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)

    only = args.only
    shape = W.LLAMA3_8B_PREFILL
    steps, warmup = args.steps, args.warmup
    runs = {
        "prefill": lambda: bench_prefill(torch, ta, W, shape, steps, warmup),
        "swa-mha": lambda: bench_prefill(torch, ta, W, W.SWA_MHA, steps, warmup),
        "swa-mqa": lambda: bench_prefill(torch, ta, W, W.SWA_MQA, steps, warmup),
        "backward": lambda: bench_backward(torch, ta, W, shape, steps, warmup),
        "prefill-fp8": lambda: bench_prefill_fp8(torch, ta, W, shape, steps, warmup),
        "decode": lambda: bench_decode(torch, ta, W, steps, warmup),
        "decode-fp8": lambda: bench_decode_fp8(torch, ta, W, steps, warmup),
        "rope": lambda: bench_rope(torch, ta, W, steps, warmup),
        "decode-paged": lambda: bench_decode_paged(torch, ta, W, steps, warmup),
        "mla": lambda: bench_mla(torch, ta, W, steps, warmup),
        "mla-fp8": lambda: bench_mla_fp8(torch, ta, W, steps, warmup),
        "tiny-fp32": lambda: bench_tiny_fp32(torch, ta, W, steps, warmup),
        "copy": lambda: bench_copy(torch, steps, warmup),
    }
    median_key = {"prefill": shape.name, "swa-mha": W.SWA_MHA.name, "swa-mqa": W.SWA_MQA.name}
    selected = [only] if only else [b for b in BENCHES if b != "copy"]
    out = {}
    for name in selected:
        r = runs[name]()
        r["median_ms"] = LAST_MEDIAN_MS[median_key.get(name, name.replace("-", "_"))]
        out[name] = r
        rate = (f"{r['tflops']:.1f} TFLOP/s" if "tflops" in r and "gbs" not in r else
                f"{r['gbs']:.0f} GB/s" if "gbs" in r else "")
        print(f"[bench] {name} {r['ms']:.4f} ms (median {r['median_ms']:.4f}) {rate}",
              file=sys.stderr, flush=True)

    line = {
        "metric": "GQA prefill TFLOP/s + decode KV-cache GB/s, as % of MI355X peak, d_h=128",
        "n_gpus": 1, "steps": steps, "warmup": warmup,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic N(0,1), seeded",
        "timing": f"HIP events on the library's stream around each call; ms = mean of the timed "
                  f"calls, median_ms = their median; each workload first keeps the GPU busy with the "
                  f"same call for {SPIN_UP_S} s (untimed, so that the clocks are at their steady "
                  f"state), then runs the warm-up calls, then the timed ones",
        "library": _library_info(ta),
    }
    first = selected[0]
    r = out[first]
    if first == "prefill":
        line.update({
            "value": round(r["tflops"], 2), "unit": "TFLOP/s", "ms_per_step": round(r["ms"], 4),
            "median_ms": round(r["median_ms"], 4),
            "config": {"workload": "Llama-3-8B-shaped causal GQA prefill", "B": shape.B,
                       "seq_len": shape.T, "h_q": shape.h_q, "h_kv": shape.h_kv,
                       "d_h": shape.d_h, "causal": True, "flops_counted": r["flops"]},
            "roofline": {"bound": "mfma", "achieved": round(r["tflops"], 2),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(r["frac_bf16_peak"], 4),
                         "traffic": PREFILL_TRAFFIC_BYTES},
        })
    elif "gbs" in r:
        line.update({"value": round(r["gbs"], 1), "unit": "GB/s", "ms_per_step": round(r["ms"], 4),
                     "median_ms": round(r["median_ms"], 4), "config": {"workload": first},
                     "roofline": {"bound": "hbm", "achieved": round(r["gbs"], 1),
                                  "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(r["frac_hbm_peak"], 4), "traffic": None}})
    elif "frac_bf16_peak" in r:
        line.update({"value": round(r["tflops"], 2), "unit": "TFLOP/s",
                     "ms_per_step": round(r["ms"], 4), "median_ms": round(r["median_ms"], 4),
                     "config": {"workload": first},
                     "roofline": {"bound": "mfma", "achieved": round(r["tflops"], 2),
                                  "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                  "frac": round(r["frac_bf16_peak"], 4), "traffic": None}})
    else:
        line.update({"value": round(r["ms"] * 1e3, 2), "unit": "us", "higher_is_better": False,
                     "ms_per_step": round(r["ms"], 4), "median_ms": round(r["median_ms"], 4),
                     "config": {"workload": first}})

    def sub(key, workload, **extra):
        d = out[key]
        o = {"workload": workload, "ms": round(d["ms"], 4), "median_ms": round(d["median_ms"], 4)}
        if "gbs" in d:
            o.update({"GB_s": round(d["gbs"], 1), "frac_hbm_peak": round(d["frac_hbm_peak"], 4),
                      "bytes": d["bytes"]})
        elif "frac_bf16_peak" in d:
            o.update({"TFLOP_s": round(d["tflops"], 2),
                      "frac_bf16_peak": round(d["frac_bf16_peak"], 4), "flops": d["flops"]})
        elif "tflops" in d:
            o.update({"TFLOP_s": round(d["tflops"], 2), "flops": d["flops"]})
        o.update(extra)
        line[key.replace("-", "_")] = o

    names = {
        "swa-mha": "sliding-window MHA prefill, B=4, T=4096, 32/32 heads, W=1024",
        "swa-mqa": "sliding-window MQA prefill, B=4, T=4096, 32/1 heads, W=1024",
        "backward": "Llama-3-8B-shaped causal GQA prefill backward (dQ, dK, dV)",
        "prefill-fp8": "Llama-3-8B-shaped causal GQA prefill with FP8 attention (E4M3 q, k, v "
                       "with one scale per 32 positions of a head, p quantised in the kernel, "
                       "FP8 MFMA); lower precision, not the bf16 workload",
        "decode": "70B-shaped GQA decode, B=64, 64/8 heads, S_max=32768",
        "decode-fp8": "70B-shaped GQA decode, cache in FP8 E4M3 (one scale per 32 positions of "
                      "a head)",
        "rope": "RoPE of the Llama-3-8B prefill's q and k in place (32/8 heads, T=8192, base 5e5)",
        "decode-paged": "70B-shaped GQA decode, cache in pages of 64 positions (random page "
                        "order)",
        "mla": "DeepSeek-V3-shaped MLA absorbed decode, B=32, 128 heads, S=16384",
        "mla-fp8": "DeepSeek-V3-shaped MLA absorbed decode with FP8 attention (E4M3 cache with "
                   "one scale per 32 tokens, q and p quantised in the call, FP8 MFMA); lower "
                   "precision, not the bf16 workload",
    }
    for key in out:
        if key == first or key == "copy":
            continue
        if key == "tiny-fp32":
            d = out[key]
            line["tiny_fp32"] = {"workload": "tiny causal GQA prefill, fp32, B=1, T=64, 4/2 heads, "
                                             "d_h=16 (one launch; parity case); per call, "
                                             "including the binding's host-side launch overhead",
                                 "us": round(d["ms"] * 1e3, 2),
                                 "median_us": round(d["median_ms"] * 1e3, 2),
                                 "flops": d["flops"]}
            continue
        extra = {}
        if key == "decode":
            extra["sum_len"] = out[key]["sum_len"]
        if key == "decode-fp8" and "decode" in out:
            extra["speedup_vs_bf16_cache"] = round(out["decode"]["ms"] / out[key]["ms"], 3)
        if key in ("mla", "mla-fp8"):
            extra.update({"TFLOP_s": round(out[key]["tflops"], 2),
                          "cache_copies_rotated": out[key]["cache_copies_rotated"]})
        if key == "prefill-fp8":
            extra.update({"dtype": "fp8 e4m3 operands, fp32 accumulate",
                          "frac_fp8_peak": round(out[key]["frac_fp8_peak"], 4)})
            if "prefill" in out:
                extra["speedup_vs_bf16"] = round(out["prefill"]["ms"] / out[key]["ms"], 3)
        if key == "mla-fp8":
            extra["dtype"] = "fp8 e4m3 operands, fp32 accumulate"
            if "mla" in out:
                extra["speedup_vs_bf16"] = round(out["mla"]["ms"] / out[key]["ms"], 3)
        sub(key, names[key], **extra)
    if not args.no_cpu_baseline and first == "prefill":
        line["cpu_baseline"] = cpu_baseline_prefill(W, shape)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
