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

Inputs are seeded synthetic N(0,1) tensors (workloads.py), resident in HBM
before timing.  W untimed warm-up steps, then exactly K timed steps between
two device synchronisations; kernel durations come from HIP events recorded
on the stream the kernels run on.  One JSON line is printed.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--only prefill|backward|decode|decode-paged|decode-fp8|rope|mla|swa-mha|
                            swa-mqa|copy]

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
PREFILL_TRAFFIC_BYTES = 212685895   # prefill_bf16_d128 kernel <1,2,4>: FETCH_SIZE x 2.000 + WRITE_SIZE x 1.000 KiB


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


def _events_time(torch, fn, steps, warmup, stream):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


def bench_prefill(torch, ta, W, shape, steps, warmup):
    q, k, v = W.prefill_inputs(shape, seed=0, device="cuda", gen_device="cuda")
    o = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    fn = lambda: ta.attn_prefill(q, k, v, causal=shape.causal, window=shape.window,
                                 scale=shape.scale, o=o)
    ms, wall = _events_time(torch, fn, steps, warmup, stream)
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
    ms, wall = _events_time(torch, fn, steps, warmup, stream)
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
    ms, wall = _events_time(torch, fn, steps, warmup, stream)
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
    ms, wall = _events_time(torch, fn, steps, warmup, stream)
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
    ms, wall = _events_time(torch, fn, steps, warmup, stream)
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
    ms, wall = _events_time(torch, lambda: ta.attn_rope_qk(q, k, base=5e5), steps, warmup, stream)
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
    ms, wall = _events_time(torch, lambda: dst.copy_(src), steps, warmup, stream)
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

    ms, wall = _events_time(torch, fn, steps, warmup, stream)
    total = int(sum(int(l.sum()) for _, _, l in sets[:1]))
    cache_bytes = total * (s.d_c + s.d_r) * 2
    io_bytes = s.B * s.H * (s.d_c + s.d_r) * 2 + s.B * s.H * s.d_c * 2
    gbs = (cache_bytes + io_bytes) / (ms * 1e-3) / 1e9
    flops = 2 * s.H * total * (s.d_c + s.d_r + s.d_c)
    del sets, o, ws
    return {"ms": ms, "wall_s": wall, "bytes": cache_bytes + io_bytes, "gbs": gbs,
            "frac_hbm_peak": gbs / HBM_PEAK_GBS,
            "tflops": flops / (ms * 1e-3) / 1e12, "cache_copies_rotated": copies}


def cpu_baseline_prefill(W, shape, budget_s=20.0):
    """The fp64 oracle on a bounded sample of the prefill workload: all heads
    of a growing set of query rows until the budget is used."""
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
    flops = 4 * shape.B * shape.h_q * shape.d_h * vis
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"{len(rows)} evenly spaced query rows x all {shape.h_q} heads of "
                      f"the workload ({elapsed:.1f} s, fp64, full score rows materialised)"}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None,
                    choices=["prefill", "backward", "decode", "decode-paged", "decode-fp8", "rope", "mla",
                             "swa-mha",
                             "swa-mqa", "copy"])
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
    out = {}
    if only in (None, "prefill"):
        out["prefill"] = bench_prefill(torch, ta, W, shape, args.steps, args.warmup)
        print(f"[bench] prefill {out['prefill']['ms']:.3f} ms "
              f"{out['prefill']['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
    if only in (None, "swa-mha"):
        out["swa_mha"] = bench_prefill(torch, ta, W, W.SWA_MHA, args.steps, args.warmup)
    if only in (None, "swa-mqa"):
        out["swa_mqa"] = bench_prefill(torch, ta, W, W.SWA_MQA, args.steps, args.warmup)
    if only in (None, "backward"):
        out["backward"] = bench_backward(torch, ta, W, shape, args.steps, args.warmup)
        print(f"[bench] backward {out['backward']['ms']:.3f} ms "
              f"{out['backward']['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
    if only == "copy":
        out["copy"] = bench_copy(torch, args.steps, args.warmup)
    if only in (None, "decode"):
        out["decode"] = bench_decode(torch, ta, W, args.steps, args.warmup)
        print(f"[bench] decode {out['decode']['ms']:.3f} ms {out['decode']['gbs']:.0f} GB/s",
              file=sys.stderr, flush=True)
    if only in (None, "decode-fp8"):
        out["decode_fp8"] = bench_decode_fp8(torch, ta, W, args.steps, args.warmup)
        print(f"[bench] decode (fp8 cache) {out['decode_fp8']['ms']:.3f} ms "
              f"{out['decode_fp8']['gbs']:.0f} GB/s", file=sys.stderr, flush=True)
    if only in (None, "rope"):
        out["rope"] = bench_rope(torch, ta, W, args.steps, args.warmup)
        print(f"[bench] rope (q and k) {out['rope']['ms']:.3f} ms {out['rope']['gbs']:.0f} GB/s",
              file=sys.stderr, flush=True)
    if only in (None, "decode-paged"):
        out["decode_paged"] = bench_decode_paged(torch, ta, W, args.steps, args.warmup)
        print(f"[bench] decode (paged) {out['decode_paged']['ms']:.3f} ms "
              f"{out['decode_paged']['gbs']:.0f} GB/s", file=sys.stderr, flush=True)
    if only in (None, "mla"):
        out["mla"] = bench_mla(torch, ta, W, args.steps, args.warmup)
        print(f"[bench] mla {out['mla']['ms']:.3f} ms {out['mla']['gbs']:.0f} GB/s",
              file=sys.stderr, flush=True)

    line = {
        "metric": "GQA prefill TFLOP/s + decode KV-cache GB/s, as % of MI355X peak, d_h=128",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic N(0,1), seeded",
    }
    if "prefill" in out:
        p = out["prefill"]
        line.update({
            "value": round(p["tflops"], 2), "unit": "TFLOP/s", "ms_per_step": round(p["ms"], 4),
            "config": {"workload": "Llama-3-8B-shaped causal GQA prefill", "B": shape.B,
                       "seq_len": shape.T, "h_q": shape.h_q, "h_kv": shape.h_kv,
                       "d_h": shape.d_h, "causal": True, "flops_counted": p["flops"]},
            "roofline": {"bound": "mfma", "achieved": round(p["tflops"], 2),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(p["frac_bf16_peak"], 4),
                         "traffic": PREFILL_TRAFFIC_BYTES},
        })
    else:
        key = next(iter(out))
        r = out[key]
        if "gbs" in r:
            line.update({"value": round(r["gbs"], 1), "unit": "GB/s", "ms_per_step": round(r["ms"], 4),
                         "config": {"workload": key},
                         "roofline": {"bound": "hbm", "achieved": round(r["gbs"], 1),
                                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": round(r["frac_hbm_peak"], 4), "traffic": None}})
        else:
            line.update({"value": round(r["tflops"], 2), "unit": "TFLOP/s",
                         "ms_per_step": round(r["ms"], 4), "config": {"workload": key},
                         "roofline": {"bound": "mfma", "achieved": round(r["tflops"], 2),
                                      "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                      "frac": round(r["frac_bf16_peak"], 4), "traffic": None}})
    if "decode" in out:
        d = out["decode"]
        line["decode"] = {"workload": "70B-shaped GQA decode, B=64, 64/8 heads, S_max=32768",
                          "ms": round(d["ms"], 4), "GB_s": round(d["gbs"], 1),
                          "frac_hbm_peak": round(d["frac_hbm_peak"], 4), "bytes": d["bytes"],
                          "sum_len": d["sum_len"]}
    for key, shp, name in (("swa_mha", W.SWA_MHA, "sliding-window MHA prefill, B=4, T=4096, 32/32 heads, W=1024"),
                           ("swa_mqa", W.SWA_MQA, "sliding-window MQA prefill, B=4, T=4096, 32/1 heads, W=1024")):
        if key in out and key != next(iter(out)):
            r = out[key]
            line[key] = {"workload": name, "ms": round(r["ms"], 4), "TFLOP_s": round(r["tflops"], 2),
                         "frac_bf16_peak": round(r["frac_bf16_peak"], 4), "flops": r["flops"]}
    if "decode_paged" in out and next(iter(out)) != "decode_paged":
        d = out["decode_paged"]
        line["decode_paged"] = {"workload": "70B-shaped GQA decode, cache in pages of "
                                            f"{d['page_size']} positions (random page order)",
                                "ms": round(d["ms"], 4), "GB_s": round(d["gbs"], 1),
                                "frac_hbm_peak": round(d["frac_hbm_peak"], 4), "bytes": d["bytes"]}
    if "decode_fp8" in out and next(iter(out)) != "decode_fp8":
        d = out["decode_fp8"]
        line["decode_fp8"] = {"workload": "70B-shaped GQA decode, cache in FP8 E4M3 (one scale per "
                                          "32 positions of a head)",
                              "ms": round(d["ms"], 4), "GB_s": round(d["gbs"], 1),
                              "frac_hbm_peak": round(d["frac_hbm_peak"], 4), "bytes": d["bytes"]}
        if "decode" in out:
            line["decode_fp8"]["speedup_vs_bf16_cache"] = round(out["decode"]["ms"] / d["ms"], 3)
    if "rope" in out and next(iter(out)) != "rope":
        d = out["rope"]
        line["rope"] = {"workload": "RoPE of the Llama-3-8B prefill's q and k in place (32/8 heads, "
                                    "T=8192, base 5e5)",
                        "ms": round(d["ms"], 4), "GB_s": round(d["gbs"], 1),
                        "frac_hbm_peak": round(d["frac_hbm_peak"], 4), "bytes": d["bytes"]}
    if "backward" in out and next(iter(out)) != "backward":
        r = out["backward"]
        line["backward"] = {"workload": "Llama-3-8B-shaped causal GQA prefill backward (dQ, dK, dV)",
                            "ms": round(r["ms"], 4), "TFLOP_s": round(r["tflops"], 2),
                            "frac_bf16_peak": round(r["frac_bf16_peak"], 4), "flops": r["flops"]}
    if "mla" in out:
        m = out["mla"]
        line["mla"] = {"workload": "DeepSeek-V3-shaped MLA absorbed decode, B=32, 128 heads, S=16384",
                       "ms": round(m["ms"], 4), "GB_s": round(m["gbs"], 1),
                       "frac_hbm_peak": round(m["frac_hbm_peak"], 4), "bytes": m["bytes"],
                       "TFLOP_s": round(m["tflops"], 2),
                       "cache_copies_rotated": m["cache_copies_rotated"]}
    if not args.no_cpu_baseline and "prefill" in out:
        line["cpu_baseline"] = cpu_baseline_prefill(W, shape)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
