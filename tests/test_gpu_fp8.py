"""GPU parity of the FP8 (E4M3) KV cache: the quantiser bit for bit against
the oracle's, and the contiguous and paged FP8 decodes against the oracle's
decode of the dequantised cache (bf16 bar: the codes widen to bf16 exactly,
so the kernel rounds only the probabilities and the output, as the bf16
decode does).  Codes past each sequence's length are the NaN code and tile
scales past it are NaN, so any read of them would show."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from parity import LSE_BF16_ABS, assert_bf16_close, assert_lse_close, np32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ta():
    import transformer_attention_amd as m
    m.load_library()
    return m


@pytest.mark.parametrize("B,hkv,S,d", [(2, 2, 100, 128), (1, 3, 64, 64), (3, 1, 5, 16),
                                       (2, 1, 70, 576)])
def test_quantiser_bitwise(ta, oracle_mod, B, hkv, S, d):
    g = torch.Generator().manual_seed(400 + S)
    x = torch.randn(B, hkv, S, d, generator=g) * torch.exp(2 * torch.randn(B, hkv, S, 1, generator=g))
    x[0, 0, :min(S, 32)] = 0.0                      # an all-zero tile
    if S > 40:
        x[-1, -1, 40, 3] = 1e4                      # one tile dominated by an outlier
    if S > 64:                                      # non-finite entries: the signed NaN code,
        x[0, -1, 33, 1] = float("nan")              # scale over the finite values only
        x[-1, 0, 64, 0] = -float("inf")
        x[-1, 0, 65, d - 1] = float("inf")
        x[0, 0, 2, 2] = -float("nan")               # inside the all-zero tile
    x = x.to(torch.bfloat16)
    print(f"[case] quantise {B},{hkv},{S},{d}", flush=True)
    codes, scales = ta.attn_quantize_kv_fp8(x.cuda())
    torch.cuda.synchronize()
    rc, rs = oracle_mod.quantize_kv_fp8(np32(x))
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def _fp8_case(oracle_mod, B, S_max, hq, hkv, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, hq, 1, 128, generator=g).to(torch.bfloat16)
    k = torch.randn(B, hkv, S_max, 128, generator=g).to(torch.bfloat16)
    v = torch.randn(B, hkv, S_max, 128, generator=g).to(torch.bfloat16)
    lens = torch.randint(1, S_max + 1, (B,), generator=g, dtype=torch.int32)
    lens[0] = S_max
    k8, ks = oracle_mod.quantize_kv_fp8(np32(k))
    v8, vs = oracle_mod.quantize_kv_fp8(np32(v))
    for b, n in enumerate(lens.tolist()):            # poison what no read may touch
        k8[b, :, n:] = 0x7f
        v8[b, :, n:] = 0xff
        ks[b, :, (n + 31) // 32:] = np.nan
        vs[b, :, (n + 31) // 32:] = np.nan
    return q, k8, v8, ks, vs, lens


CASES = [
    # B, S_max, hq, hkv, window, split
    (3, 700, 16, 2, 0, 0),
    (2, 1000, 8, 8, 0, 256),
    (2, 900, 32, 1, 0, 64),
    (4, 2048, 16, 2, 100, 0),
    (2, 333, 4, 2, 45, 128),
]


@pytest.mark.parametrize("B,S_max,hq,hkv,window,split", CASES)
def test_decode_fp8(ta, oracle_mod, B, S_max, hq, hkv, window, split):
    q, k8, v8, ks, vs, lens = _fp8_case(oracle_mod, B, S_max, hq, hkv, 410 + S_max + hq)
    scale = 1.0 / math.sqrt(128)
    print(f"[case] fp8 decode {B},{S_max},{hq},{hkv},w={window},split={split}", flush=True)
    dev = [torch.from_numpy(x).cuda() for x in (k8, v8, ks, vs)]
    o, lse = ta.attn_decode_fp8(q.cuda(), *dev, lens.cuda(), window=window, scale=scale,
                                split_tokens=split, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle_mod.decode_fp8(np32(q), k8, v8, ks, vs, lens.numpy(), window=window,
                                   scale=scale)
    assert_bf16_close(np32(o)[:, :, 0], ro, "fp8 decode")
    assert_lse_close(np32(lse), rl, LSE_BF16_ABS, "fp8 decode lse")


def test_decode_fp8_with_sinks_and_empty_sequence(ta, oracle_mod):
    q, k8, v8, ks, vs, lens = _fp8_case(oracle_mod, 3, 300, 8, 2, 430)
    lens[2] = 0
    sinks = torch.tensor([0.5, -1.0, 2.0, 0.0, 1.0, -3.0, 0.25, 4.0])
    dev = [torch.from_numpy(x).cuda() for x in (k8, v8, ks, vs)]
    o, lse = ta.attn_decode_fp8(q.cuda(), *dev, lens.cuda(), sinks=sinks.cuda(), return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle_mod.decode_fp8(np32(q), k8, v8, ks, vs, lens.numpy(), scale=1 / math.sqrt(128),
                                   sinks=sinks.numpy())
    assert_bf16_close(np32(o)[:, :, 0], ro, "fp8 decode sinks")
    assert_lse_close(np32(lse), rl, LSE_BF16_ABS, "fp8 decode sinks lse")
    assert torch.all(o[2] == 0)


@pytest.mark.parametrize("page_size,window", [(32, 0), (128, 0), (64, 100)])
def test_paged_fp8_equals_contiguous(ta, oracle_mod, page_size, window):
    """Both FP8 kernels start tiles on 32-key boundaries, so the paged result
    equals the contiguous one bit for bit, with a window too."""
    B, S_max, hq, hkv = 3, 512, 16, 2
    q, k8, v8, ks, vs, lens = _fp8_case(oracle_mod, B, S_max, hq, hkv, 440 + page_size)
    kc = torch.from_numpy(k8)
    vc = torch.from_numpy(v8)
    kp, table = W.paged_layout(kc.cuda(), page_size, seed=11, extra_pages=2, fill=0)
    vp = torch.zeros_like(kp)
    nb = S_max // page_size
    perm = table.view(-1).long()
    vp[perm] = vc.cuda().view(B, hkv, nb, page_size, 128).permute(0, 2, 1, 3, 4).reshape(-1, hkv, page_size, 128)
    spp = page_size // 32
    ksp = torch.zeros(kp.shape[0], hkv, spp)
    vsp = torch.zeros(kp.shape[0], hkv, spp)
    ksp[perm.cpu()] = torch.from_numpy(ks).view(B, hkv, nb, spp).permute(0, 2, 1, 3).reshape(-1, hkv, spp)
    vsp[perm.cpu()] = torch.from_numpy(vs).view(B, hkv, nb, spp).permute(0, 2, 1, 3).reshape(-1, hkv, spp)
    lens_d = lens.cuda()
    print(f"[case] paged fp8 ps={page_size} w={window}", flush=True)
    o1, l1 = ta.attn_decode_paged_fp8(q.cuda(), kp, vp, ksp.cuda(), vsp.cuda(), lens_d, table,
                                      window=window, return_lse=True)
    dev = [torch.from_numpy(x).cuda() for x in (k8, v8, ks, vs)]
    o2, l2 = ta.attn_decode_fp8(q.cuda(), *dev, lens_d, window=window, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    ro, rl = oracle_mod.decode_paged_fp8(np32(q), kp.cpu().numpy(), vp.cpu().numpy(), ksp.numpy(),
                                         vsp.numpy(), table.cpu().numpy(), lens.numpy(),
                                         window=window, scale=1 / math.sqrt(128))
    assert_bf16_close(np32(o1)[:, :, 0], ro, "paged fp8")


def test_full_size_fp8_decode(ta, oracle_mod):
    """70B-shaped decode (B=64, 64/8 heads, S_max=32768) on a synthetic FP8
    cache, sampled sequences against the oracle."""
    s = W.GQA70B_DECODE
    g = torch.Generator().manual_seed(450)
    q = torch.randn(s.B, s.h_q, 1, s.d_h, generator=g).to(torch.bfloat16).cuda()
    lens = W.seq_lengths(s.B, s.len_lo, s.len_hi, seed=0)
    shape = (s.B, s.h_kv, s.S_max, s.d_h)
    k8, ks = W.random_fp8_cache(shape, seed=1, device="cuda")
    v8, vs = W.random_fp8_cache(shape, seed=2, device="cuda")
    print("[case] full-size fp8 decode", flush=True)
    o = ta.attn_decode_fp8(q, k8, v8, ks, vs, lens.cuda(), scale=s.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    for b in (0, 29, 63):
        n = int(lens[b])
        nt = (n + 31) // 32
        ro, _ = oracle_mod.decode_fp8(np32(q[b:b + 1]), k8[b:b + 1, :, :n].cpu().numpy(),
                                      v8[b:b + 1, :, :n].cpu().numpy(),
                                      ks[b:b + 1, :, :nt].cpu().numpy(),
                                      vs[b:b + 1, :, :nt].cpu().numpy(), lens[b:b + 1].numpy(),
                                      scale=s.scale)
        assert_bf16_close(np32(o[b:b + 1])[:, :, 0], ro, f"fp8 seq {b}")


def test_full_size_quantiser_sampled_tiles(ta, oracle_mod):
    """The 70B workload's bf16 K cache (64 x 8 heads x 32768 positions x 128)
    through the GPU quantiser; sampled 32-position tiles against the oracle's
    quantiser, bit for bit."""
    s = W.GQA70B_DECODE
    _, kc, _, _ = W.decode_inputs(s, seed=0, device="cuda", gen_device="cuda")
    print("[case] full-size quantiser", flush=True)
    codes, scales = ta.attn_quantize_kv_fp8(kc)
    torch.cuda.synchronize()
    for b, g, t in ((0, 0, 0), (17, 3, 511), (63, 7, 1023), (40, 5, 777)):
        x = np32(kc[b:b + 1, g:g + 1, 32 * t:32 * t + 32])
        rc, rs = oracle_mod.quantize_kv_fp8(x)
        assert np.array_equal(codes[b:b + 1, g:g + 1, 32 * t:32 * t + 32].cpu().numpy(), rc)
        assert scales[b, g, t].item() == float(rs[0, 0, 0])
