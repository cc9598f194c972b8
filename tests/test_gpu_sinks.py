"""GPU parity of the attention-sink logit: one extra softmax-denominator term
per query head, with no value row, on every entry point that takes `sinks`
(bf16 and fp32 prefill, the prefill backward with the sinks' gradient, the
contiguous and paged GQA and MLA decodes).

Against the fp64 oracle with the same sinks, to the usual bars.  A sink of
-1e30 must reproduce the sink-free result bit for bit (its term underflows to
0 before it reaches the sum), and a row with no visible key gets O = 0 and
L = the sink.  The sinks' gradient sums exp(s - L_i) D_i over every row of a
head, with terms of both signs, so its bar is relative to the sum of the
terms' magnitudes (computed from oracle values): 1e-2 of it, plus 1e-4."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from parity import (F32_MAX_ABS, LSE_BF16_ABS, LSE_F32_ABS, assert_bf16_close,
                    assert_f32_close, assert_lse_close, np32)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ta():
    import transformer_attention_amd as m
    m.load_library()
    return m


def _sinks(n, seed, device="cuda"):
    g = torch.Generator().manual_seed(seed)
    s = 2.0 * torch.randn(n, generator=g)
    s[0] = 6.0           # a sink that outweighs most rows
    if n > 1:
        s[1] = -30.0     # one that is negligible
    return s.to(device)


PREFILL_CASES = [
    # B, T, hq, hkv, causal, window
    (1, 200, 8, 2, True, 0),
    (2, 333, 4, 4, True, 100),
    (1, 130, 8, 1, False, 0),
]


@pytest.mark.parametrize("B,T,hq,hkv,causal,window", PREFILL_CASES)
def test_prefill_bf16_sinks(ta, oracle_mod, B, T, hq, hkv, causal, window):
    g = torch.Generator().manual_seed(300 + T)
    q = torch.randn(B, hq, T, 128, generator=g).to(torch.bfloat16).cuda()
    k = torch.randn(B, hkv, T, 128, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(B, hkv, T, 128, generator=g).to(torch.bfloat16).cuda()
    sinks = _sinks(hq, T)
    scale = 1.0 / math.sqrt(128)
    print(f"[case] prefill bf16 sinks {B},{T},{hq},{hkv},{causal},{window}", flush=True)
    o, lse = ta.attn_prefill(q, k, v, causal=causal, window=window, scale=scale, sinks=sinks,
                             return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle_mod.prefill(np32(q), np32(k), np32(v), causal=causal, window=window,
                                scale=scale, sinks=np32(sinks))
    assert_bf16_close(np32(o), ro, "prefill sinks")
    assert_lse_close(np32(lse), rl, LSE_BF16_ABS, "prefill sinks lse")


def test_prefill_negligible_sink_is_bitwise_sink_free(ta):
    g = torch.Generator().manual_seed(310)
    q = torch.randn(1, 8, 300, 128, generator=g).to(torch.bfloat16).cuda()
    k = torch.randn(1, 2, 300, 128, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(1, 2, 300, 128, generator=g).to(torch.bfloat16).cuda()
    o0, l0 = ta.attn_prefill(q, k, v, return_lse=True)
    o1, l1 = ta.attn_prefill(q, k, v, sinks=torch.full((8,), -1e30, device="cuda"),
                             return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


@pytest.mark.parametrize("d,T,window", [(64, 100, 0), (128, 70, 20), (16, 33, 0)])
def test_prefill_f32_sinks(ta, oracle_mod, d, T, window):
    g = torch.Generator().manual_seed(320 + d)
    B, hq, hkv = 2, 4, 2
    q = torch.randn(B, hq, T, d, generator=g).cuda()
    k = torch.randn(B, hkv, T, d, generator=g).cuda()
    v = torch.randn(B, hkv, T, d, generator=g).cuda()
    sinks = _sinks(hq, d)
    scale = 1.0 / math.sqrt(d)
    print(f"[case] prefill f32 sinks d={d} T={T} w={window}", flush=True)
    o, lse = ta.attn_prefill(q, k, v, causal=True, window=window, scale=scale, sinks=sinks,
                             return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle_mod.prefill(np32(q), np32(k), np32(v), causal=True, window=window,
                                scale=scale, sinks=np32(sinks))
    assert_f32_close(np32(o), ro, "prefill f32 sinks", F32_MAX_ABS)
    assert_lse_close(np32(lse), rl, LSE_F32_ABS, "prefill f32 sinks lse")


@pytest.mark.parametrize("B,T,hq,hkv,window", [(1, 300, 8, 2, 0), (2, 257, 4, 4, 90)])
def test_backward_with_sinks(ta, oracle_mod, B, T, hq, hkv, window):
    g = torch.Generator().manual_seed(330 + T)
    q = torch.randn(B, hq, T, 128, generator=g).to(torch.bfloat16).cuda()
    k = torch.randn(B, hkv, T, 128, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(B, hkv, T, 128, generator=g).to(torch.bfloat16).cuda()
    do = torch.randn(B, hq, T, 128, generator=g).to(torch.bfloat16).cuda()
    sinks = _sinks(hq, 331 + T) * 0.5
    scale = 1.0 / math.sqrt(128)
    print(f"[case] bwd sinks {B},{T},{hq},{hkv},w={window}", flush=True)
    o, lse = ta.attn_prefill(q, k, v, causal=True, window=window, scale=scale, sinks=sinks,
                             return_lse=True)
    dq, dk, dv, ds = ta.attn_prefill_backward(q, k, v, o, do, lse, causal=True, window=window,
                                              scale=scale, sinks=sinks, return_dsinks=True)
    torch.cuda.synchronize()
    sk = np32(sinks)
    rq, rk, rv, rs = oracle_mod.prefill_backward(np32(q), np32(k), np32(v), np32(do), causal=True,
                                                 window=window, scale=scale, sinks=sk,
                                                 return_dsinks=True)
    for got, ref, what in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
        got = np32(got)
        assert np.all(np.isfinite(got)), what
        err = np.abs(got - ref).max()
        rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        print(f"  {what}: max_abs={err:.3e} rel_fro={rel:.3e}", flush=True)
        assert rel <= 1e-2 and err <= 2e-2 * max(1.0, float(np.abs(ref).max())), what
    ro, rl = oracle_mod.prefill(np32(q), np32(k), np32(v), causal=True, window=window,
                                scale=scale, sinks=sk)
    terms = np.exp(sk[None, :, None] - rl) * np.einsum("bhtd,bhtd->bht", ro, np32(do))
    bound = 1e-2 * np.abs(terms).sum(axis=(0, 2)) + 1e-4
    err = np.abs(np32(ds) - rs)
    print(f"  dsinks: err={err.max():.3e} bound_min={bound.min():.3e}", flush=True)
    assert np.all(err <= bound), (np32(ds), rs)
    # the same call twice: same bits
    ds2 = ta.attn_prefill_backward(q, k, v, o, do, lse, causal=True, window=window, scale=scale,
                                   sinks=sinks, return_dsinks=True)[3]
    torch.cuda.synchronize()
    assert torch.equal(ds, ds2)


def _decode_inputs(B, S_max, hq, hkv, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, hq, 1, 128, generator=g).to(torch.bfloat16).cuda()
    kc = torch.randn(B, hkv, S_max, 128, generator=g).to(torch.bfloat16).cuda()
    vc = torch.randn(B, hkv, S_max, 128, generator=g).to(torch.bfloat16).cuda()
    lens = torch.randint(1, S_max + 1, (B,), generator=g, dtype=torch.int32)
    lens[0] = S_max
    lens[-1] = 0                                    # empty sequence: O = 0, L = sink
    return q, kc, vc, lens


@pytest.mark.parametrize("B,S_max,hq,hkv,window,split", [(4, 700, 8, 2, 0, 0),
                                                          (3, 1024, 16, 1, 200, 128)])
def test_decode_sinks(ta, oracle_mod, B, S_max, hq, hkv, window, split):
    q, kc, vc, lens = _decode_inputs(B, S_max, hq, hkv, 340 + S_max)
    sinks = _sinks(hq, 341)
    scale = 1.0 / math.sqrt(128)
    print(f"[case] decode sinks {B},{S_max},{hq},{hkv},w={window},split={split}", flush=True)
    o, lse = ta.attn_decode(q, kc, vc, lens.cuda(), window=window, scale=scale, sinks=sinks,
                            split_tokens=split, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle_mod.decode(np32(q), np32(kc), np32(vc), lens.numpy(), window=window,
                               scale=scale, sinks=np32(sinks))
    assert_bf16_close(np32(o)[:, :, 0], ro, "decode sinks")
    assert_lse_close(np32(lse), rl, LSE_BF16_ABS, "decode sinks lse")
    assert torch.all(o[-1] == 0)
    assert np.allclose(np32(lse)[-1], np32(sinks), rtol=1e-6, atol=1e-6)


def test_paged_decode_sinks_equal_contiguous(ta):
    B, S_max, hq, hkv = 3, 512, 8, 2
    q, kc, vc, lens = _decode_inputs(B, S_max, hq, hkv, 350)
    kp, table = W.paged_layout(kc, 64, seed=3, extra_pages=1)
    vp = torch.zeros_like(kp)
    vp[table.view(-1).long()] = vc.view(B, hkv, S_max // 64, 64, 128).permute(
        0, 2, 1, 3, 4).reshape(-1, hkv, 64, 128)
    sinks = _sinks(hq, 351)
    lens_d = lens.cuda()
    print("[case] paged decode sinks", flush=True)
    o1, l1 = ta.attn_decode_paged(q, kp, vp, lens_d, table, sinks=sinks, return_lse=True)
    o2, l2 = ta.attn_decode(q, kc, vc, lens_d, sinks=sinks, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("B,S_max,H,split", [(3, 640, 128, 0), (2, 1024, 16, 256)])
def test_mla_sinks(ta, oracle_mod, B, S_max, H, split):
    s = W.DSV3_MLA_DECODE
    q, c, lens = W.mla_inputs(s, seed=360 + B, device="cuda", B=B, S_max=S_max, len_lo=1,
                              len_hi=S_max, H=H)
    sinks = _sinks(H, 361)
    lens_d = lens.to("cuda")
    print(f"[case] mla sinks {B},{S_max},{H},split={split}", flush=True)
    o, lse = ta.mla_decode(q, c, lens_d, scale=s.scale, sinks=sinks, split_tokens=split,
                           return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle_mod.mla_decode(np32(q), np32(c), lens.cpu().numpy(), d_c=512, d_r=64,
                                   scale=s.scale, sinks=np32(sinks))
    assert_bf16_close(np32(o), ro, "mla sinks")
    assert_lse_close(np32(lse), rl, LSE_BF16_ABS, "mla sinks lse")
    cp, table = W.paged_layout(c, 64, seed=4, head_axis=False, extra_pages=1)
    o2 = ta.mla_decode_paged(q, cp, lens_d, table, scale=s.scale, sinks=sinks, split_tokens=split)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
