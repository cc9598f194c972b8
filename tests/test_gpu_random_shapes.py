"""GPU parity on seeded random shapes, against the fp64 oracle, through the C ABI.

The hand-picked cases of the other test files cover the shapes each kernel's
decomposition distinguishes; these draw many more from a fixed seed, so that
an edge the hand-picked ones miss (an unusual group size, a length one past a
tile boundary, a window shorter than a tile, a short split) is still met:

* the bf16 prefill: batch 1-3, 1-8 K/V heads with group sizes 1-8 (h_q <= 32),
  lengths at and around 32/64/256-position boundaries or anywhere up to 700,
  causal with or without a window (1 .. T), or bidirectional, optional sink
  logits, two softmax scales;
* the GQA decode: batch 1-6, caches up to 1,500 positions, lengths anywhere in
  [0, S_max] (0, 1 and S_max included), group sizes up to 16, optional window
  and sinks, the library's split or 64 .. 512 positions;
* the MLA decode: batch 1-4, caches up to 1,200 tokens, 16-256 heads,
  lengths including 0 and 1, default or short splits;
* the prefill backward: batch 1-2, lengths up to 400, group sizes 1-4, causal
  with or without a window, or bidirectional;
* the FP8 prefill: the prefill's shape space at lengths up to 400, against the
  oracle's FP8 recipe;
* the FP8-cache decode, the paged decode (pages of 32-256 positions, lengths
  at and just past a page) and the FP8 MLA decode in the same way.

The bars are those of the other files (tests/parity.py).
"""
import math

import numpy as np
import pytest
import torch

from tests.parity import (BF16_MAX_ABS, BF16_REL_FRO, LSE_BF16_ABS, assert_bf16_close,
                          assert_fp8_attention_close, assert_lse_close, errors, np32)

pytestmark = pytest.mark.gpu

_R = np.random.RandomState(20261203)
_EDGES = [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]


def _length(hi):
    if _R.rand() < 0.5:
        return int(_R.choice([x for x in _EDGES if x <= hi]))
    return int(_R.randint(1, hi + 1))


def _heads(max_hkv=8, max_g=8, max_hq=32):
    while True:
        hkv = int(_R.choice([1, 2, 3, 4, 8][: [1, 2, 3, 4, 8].index(max_hkv) + 1]))
        g = int(_R.randint(1, max_g + 1))
        if hkv * g <= max_hq:
            return hkv * g, hkv


def _mask(T):
    kind = _R.randint(3)
    if kind == 0:
        return True, 0
    if kind == 1:
        return True, int(_R.randint(1, T + 1))
    return False, 0


def _prefill_cases(n, max_t):
    out = []
    for _ in range(n):
        B = int(_R.randint(1, 4))
        T = _length(max_t)
        hq, hkv = _heads()
        causal, window = _mask(T)
        sinks = bool(_R.rand() < 0.3)
        scale = float(_R.choice([1.0 / math.sqrt(128), 0.15]))
        out.append((B, T, hq, hkv, causal, window, sinks, scale))
    return out


PREFILL = _prefill_cases(40, 700)


@pytest.fixture(scope="module")
def ta():
    import transformer_attention_amd as m
    m.load_library()
    assert torch.cuda.is_available()
    return m


def _bf16(g, *shape):
    return torch.randn(*shape, generator=g).to(torch.bfloat16)


def _sink_logits(g, hq):
    return (torch.rand(hq, generator=g) * 6.0 - 2.0).float()


@pytest.mark.parametrize("B,T,hq,hkv,causal,window,sinks,scale", PREFILL)
def test_prefill_random(ta, oracle_mod, B, T, hq, hkv, causal, window, sinks, scale):
    g = torch.Generator().manual_seed(B * 100003 + T * 101 + hq * 7 + hkv + window)
    q, k, v = _bf16(g, B, hq, T, 128), _bf16(g, B, hkv, T, 128), _bf16(g, B, hkv, T, 128)
    s = _sink_logits(g, hq) if sinks else None
    print(f"[case] prefill {B},{T},{hq},{hkv},{causal},{window},{sinks},{scale:.4f}", flush=True)
    o, lse = ta.attn_prefill(q.cuda(), k.cuda(), v.cuda(), causal=causal, window=window, scale=scale,
                             sinks=None if s is None else s.cuda(), return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle_mod.prefill(np32(q), np32(k), np32(v), causal=causal, window=window, scale=scale,
                                sinks=None if s is None else s.numpy())
    assert_bf16_close(np32(o), ro, "prefill O")
    assert_lse_close(np32(lse), rl, LSE_BF16_ABS, "prefill LSE")


def _decode_cases(n):
    out = []
    for _ in range(n):
        B = int(_R.randint(1, 7))
        S_max = _length(1500)
        hq, hkv = _heads(max_g=16, max_hq=64)
        lens = [int(_R.choice([0, 1, S_max, _R.randint(0, S_max + 1)])) for _ in range(B)]
        window = 0 if _R.rand() < 0.6 else int(_R.randint(1, S_max + 1))
        split = int(_R.choice([0, 0, 64, 128, 256, 512]))
        sinks = bool(_R.rand() < 0.3)
        out.append((B, S_max, hq, hkv, lens, window, split, sinks))
    return out


DECODE = _decode_cases(32)


@pytest.mark.parametrize("B,S_max,hq,hkv,lens,window,split,sinks", DECODE)
def test_decode_random(ta, oracle_mod, B, S_max, hq, hkv, lens, window, split, sinks):
    g = torch.Generator().manual_seed(S_max * 31 + hq * 7 + hkv + B)
    q = _bf16(g, B, hq, 1, 128)
    kc, vc = _bf16(g, B, hkv, S_max, 128), _bf16(g, B, hkv, S_max, 128)
    for b, L in enumerate(lens):                     # positions at or past a length are never read
        kc[b, :, L:] = float("nan")
        vc[b, :, L:] = float("nan")
    s = _sink_logits(g, hq) if sinks else None
    scale = 1.0 / math.sqrt(128)
    print(f"[case] decode {B},{S_max},{hq},{hkv},{lens},{window},{split},{sinks}", flush=True)
    o, lse = ta.attn_decode(q.cuda(), kc.cuda(), vc.cuda(), torch.tensor(lens, dtype=torch.int32).cuda(),
                            window=window, scale=scale, split_tokens=split,
                            sinks=None if s is None else s.cuda(), return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle_mod.decode(np32(q), np32(kc), np32(vc), lens, window=window, scale=scale,
                               sinks=None if s is None else s.numpy())
    assert_bf16_close(np32(o)[:, :, 0], ro, "decode O")
    assert_lse_close(np32(lse), rl, LSE_BF16_ABS, "decode LSE")


def _mla_cases(n):
    out = []
    for _ in range(n):
        B = int(_R.randint(1, 5))
        S_max = _length(1200)
        H = int(_R.choice([16, 32, 48, 64, 128, 256]))
        lens = [int(_R.choice([0, 1, S_max, _R.randint(0, S_max + 1)])) for _ in range(B)]
        split = int(_R.choice([0, 0, 64, 128, 512]))
        out.append((B, S_max, H, lens, split))
    return out


MLA = _mla_cases(16)


@pytest.mark.parametrize("B,S_max,H,lens,split", MLA)
def test_mla_random(ta, oracle_mod, B, S_max, H, lens, split):
    g = torch.Generator().manual_seed(S_max * 13 + H + B)
    q, c = _bf16(g, B, H, 576), _bf16(g, B, S_max, 576)
    for b, L in enumerate(lens):
        c[b, L:] = float("nan")
    scale = 1.0 / math.sqrt(128 + 64)
    print(f"[case] mla {B},{S_max},{H},{lens},{split}", flush=True)
    o, lse = ta.mla_decode(q.cuda(), c.cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), scale=scale,
                           split_tokens=split, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle_mod.mla_decode(np32(q), np32(c), lens, d_c=512, d_r=64, scale=scale)
    assert_bf16_close(np32(o), ro, "mla O")
    assert_lse_close(np32(lse), rl, LSE_BF16_ABS, "mla LSE")


def _backward_cases(n):
    out = []
    for _ in range(n):
        B = int(_R.randint(1, 3))
        T = _length(400)
        hq, hkv = _heads(max_hkv=4, max_g=4, max_hq=16)
        causal, window = _mask(T)
        out.append((B, T, hq, hkv, causal, window))
    return out


BACKWARD = _backward_cases(16)


def _grad_close(got, ref, what):
    got = np32(got)
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    max_abs, rel = errors(got, ref)
    bound = BF16_MAX_ABS * max(1.0, float(np.abs(ref).max()))
    assert rel <= BF16_REL_FRO and max_abs <= bound, f"{what}: max_abs={max_abs:.3e} rel={rel:.3e}"


@pytest.mark.parametrize("B,T,hq,hkv,causal,window", BACKWARD)
def test_backward_random(ta, oracle_mod, B, T, hq, hkv, causal, window):
    g = torch.Generator().manual_seed(T * 17 + hq * 5 + hkv + window)
    q, k, v = _bf16(g, B, hq, T, 128), _bf16(g, B, hkv, T, 128), _bf16(g, B, hkv, T, 128)
    do = _bf16(g, B, hq, T, 128)
    scale = 1.0 / math.sqrt(128)
    print(f"[case] backward {B},{T},{hq},{hkv},{causal},{window}", flush=True)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = ta.attn_prefill(qd, kd, vd, causal=causal, window=window, scale=scale, return_lse=True)
    dq, dk, dv = ta.attn_prefill_backward(qd, kd, vd, o, dod, lse, causal=causal, window=window,
                                          scale=scale)
    torch.cuda.synchronize()
    rq, rk, rv = oracle_mod.prefill_backward(np32(q), np32(k), np32(v), np32(do), causal=causal,
                                             window=window, scale=scale)
    _grad_close(dq, rq, "dq")
    _grad_close(dk, rk, "dk")
    _grad_close(dv, rv, "dv")


FP8 = [c[:6] for c in _prefill_cases(16, 400)]


@pytest.mark.parametrize("B,T,hq,hkv,causal,window", FP8)
def test_prefill_fp8_random(ta, oracle_mod, B, T, hq, hkv, causal, window):
    g = torch.Generator().manual_seed(T * 19 + hq * 3 + hkv + window)
    x = [_bf16(g, B, h, T, 128) for h in (hq, hkv, hkv)]
    (q8, qs), (k8, ks), (v8, vs) = [oracle_mod.quantize_kv_fp8(np32(t)) for t in x]
    scale = 1.0 / math.sqrt(128)
    print(f"[case] prefill fp8 {B},{T},{hq},{hkv},{causal},{window}", flush=True)
    dev = [torch.from_numpy(a).cuda() for a in (q8, k8, v8, qs, ks, vs)]
    o, lse = ta.attn_prefill_fp8(*dev, causal=causal, window=window, scale=scale, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle_mod.prefill_fp8(q8, qs, k8, ks, v8, vs, causal=causal, window=window, scale=scale)
    vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()[v8]
    vmax = float(np.abs(vals * np.repeat(vs, 32, axis=-1)[..., :T, None]).max())
    assert_fp8_attention_close(np32(o), ro, vmax, "prefill fp8 O")
    assert_lse_close(np32(lse), rl, LSE_BF16_ABS, "prefill fp8 LSE")


FP8_DECODE = [c[:7] for c in _decode_cases(16)]


@pytest.mark.parametrize("B,S_max,hq,hkv,lens,window,split", FP8_DECODE)
def test_decode_fp8_random(ta, oracle_mod, B, S_max, hq, hkv, lens, window, split):
    g = torch.Generator().manual_seed(S_max * 37 + hq * 11 + hkv + B)
    q = _bf16(g, B, hq, 1, 128)
    k8, ks = oracle_mod.quantize_kv_fp8(np32(_bf16(g, B, hkv, S_max, 128)))
    v8, vs = oracle_mod.quantize_kv_fp8(np32(_bf16(g, B, hkv, S_max, 128)))
    for b, n in enumerate(lens):                     # never read: positions >= len
        k8[b, :, n:] = 0x7f
        v8[b, :, n:] = 0xff
        ks[b, :, (n + 31) // 32:] = np.nan
        vs[b, :, (n + 31) // 32:] = np.nan
    scale = 1.0 / math.sqrt(128)
    print(f"[case] fp8 decode {B},{S_max},{hq},{hkv},{lens},{window},{split}", flush=True)
    dev = [torch.from_numpy(x).cuda() for x in (k8, v8, ks, vs)]
    o, lse = ta.attn_decode_fp8(q.cuda(), *dev, torch.tensor(lens, dtype=torch.int32).cuda(),
                                window=window, scale=scale, split_tokens=split, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle_mod.decode_fp8(np32(q), k8, v8, ks, vs, np.array(lens, np.int32), window=window,
                                   scale=scale)
    assert_bf16_close(np32(o)[:, :, 0], ro, "fp8 decode O")
    assert_lse_close(np32(lse), rl, LSE_BF16_ABS, "fp8 decode LSE")


def _paged_cases(n):
    out = []
    for _ in range(n):
        B = int(_R.randint(1, 5))
        page = int(_R.choice([32, 64, 96, 128, 256]))
        S_max = page * int(_R.randint(1, 1200 // page + 1))
        hq, hkv = _heads(max_g=16, max_hq=64)
        lens = [int(_R.choice([1, S_max, page, min(S_max, page + 1), _R.randint(1, S_max + 1)]))
                for _ in range(B)]
        window = 0 if _R.rand() < 0.6 else int(_R.randint(1, S_max + 1))
        split = int(_R.choice([0, 0, 64, 128, 256]))
        out.append((B, S_max, hq, hkv, page, lens, window, split))
    return out


PAGED = _paged_cases(12)


@pytest.mark.parametrize("B,S_max,hq,hkv,page,lens,window,split", PAGED)
def test_decode_paged_random(ta, oracle_mod, B, S_max, hq, hkv, page, lens, window, split):
    import workloads as W
    g = torch.Generator().manual_seed(S_max * 41 + hq * 13 + hkv + page)
    q = _bf16(g, B, hq, 1, 128).cuda()
    kc, vc = _bf16(g, B, hkv, S_max, 128), _bf16(g, B, hkv, S_max, 128)
    for b, L in enumerate(lens):
        kc[b, :, L:] = float("nan")
        vc[b, :, L:] = float("nan")
    kp, table = W.paged_layout(kc.cuda(), page, seed=S_max + B, extra_pages=2)
    vp, _ = W.paged_layout(vc.cuda(), page, seed=S_max + B, extra_pages=2)
    lens_t = torch.tensor(lens, dtype=torch.int32)
    scale = 1.0 / math.sqrt(128)
    print(f"[case] paged decode {B},{S_max},{hq},{hkv},ps={page},{lens},{window},{split}", flush=True)
    o, lse = ta.attn_decode_paged(q, kp, vp, lens_t.cuda(), table, window=window, scale=scale,
                                  split_tokens=split, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle_mod.decode_paged(np32(q), np32(kp), np32(vp), table.cpu().numpy(), lens_t.numpy(),
                                     window=window, scale=scale)
    assert_bf16_close(np32(o)[:, :, 0], ro, "paged decode O")
    assert_lse_close(np32(lse), rl, LSE_BF16_ABS, "paged decode LSE")


MLA_FP8 = _mla_cases(8)


@pytest.mark.parametrize("B,S_max,H,lens,split", MLA_FP8)
def test_mla_fp8_random(ta, oracle_mod, B, S_max, H, lens, split):
    g = torch.Generator().manual_seed(S_max * 43 + H + B)
    q = _bf16(g, B, H, 576)
    codes, scales = oracle_mod.quantize_kv_fp8(np32(_bf16(g, B, S_max, 576))[:, None])
    codes, scales = codes[:, 0], scales[:, 0]
    for b, n in enumerate(lens):                     # never read: positions >= len
        codes[b, n:] = 0x7f
        scales[b, (n + 31) // 32:] = np.nan
    lens_np = np.array(lens, np.int32)
    scale = 1.0 / math.sqrt(192.0)
    print(f"[case] mla fp8 {B},{S_max},{H},{lens},{split}", flush=True)
    o, lse = ta.mla_decode_fp8(q.cuda(), torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                               torch.from_numpy(lens_np).cuda(), scale=scale, split_tokens=split,
                               return_lse=True)
    torch.cuda.synchronize()
    eff = split
    if split == 0:                                   # the library's choice (as in mla_decode_fp8)
        eff = (S_max * B * ((H + 127) // 128) + 255) // 256
        eff = min(max(64, (eff + 63) // 64 * 64), (S_max + 63) // 64 * 64)
    ro, rl = oracle_mod.mla_decode_fp8(np32(q), codes, scales, lens_np, d_c=512, d_r=64, scale=scale,
                                       split=eff)
    vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    vmax = max([float(np.abs(vals[codes[b, :n, :512]] * np.repeat(scales[b], 32)[:n, None]).max())
                for b, n in enumerate(lens) if n] + [0.0])
    assert_fp8_attention_close(np32(o), ro, vmax, "mla fp8 O")
    assert_lse_close(np32(lse), rl, LSE_BF16_ABS, "mla fp8 LSE")
