"""GPU parity of the paged-cache decodes (attn_decode_paged, mla_decode_paged).

Pages are a seeded random permutation of a contiguous cache; unused pages
and cache rows at or past each sequence's length hold NaN, so any read of
them would show.  The paged result must match the fp64 oracle on the
gathered cache (bf16 bar), and, where the tiling is the same (no window),
the contiguous GPU decode bit for bit."""
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


def _poison_tail(cache, lens, head_axis):
    c = cache.clone()
    for b, n in enumerate(lens.tolist()):
        if head_axis:
            c[b, :, n:] = float("nan")
        else:
            c[b, n:] = float("nan")
    return c


CASES = [
    # B, S_max, hq, hkv, page_size, window, split
    (4, 512, 8, 2, 32, 0, 0),
    (3, 1024, 16, 4, 64, 0, 256),
    (2, 768, 64, 8, 128, 0, 0),
    (3, 1024, 8, 1, 64, 300, 0),
    (2, 256, 4, 4, 32, 45, 64),
]


@pytest.mark.parametrize("B,S_max,hq,hkv,page_size,window,split", CASES)
def test_paged_decode(ta, oracle_mod, B, S_max, hq, hkv, page_size, window, split):
    g = torch.Generator().manual_seed(B * 1000 + S_max + hq)
    q = torch.randn(B, hq, 1, 128, generator=g).to(torch.bfloat16).cuda()
    kc = torch.randn(B, hkv, S_max, 128, generator=g).to(torch.bfloat16).cuda()
    vc = torch.randn(B, hkv, S_max, 128, generator=g).to(torch.bfloat16).cuda()
    lens = torch.randint(1, S_max + 1, (B,), generator=g, dtype=torch.int32)
    lens[0] = S_max
    if B > 2:
        lens[2] = min(S_max, page_size + 1)        # just past one page
    kc = _poison_tail(kc, lens, True)
    vc = _poison_tail(vc, lens, True)
    kp, table = W.paged_layout(kc, page_size, seed=7, extra_pages=3)
    vp = torch.full_like(kp, float("nan"))
    vp[table.view(-1).long()] = vc.view(B, hkv, S_max // page_size, page_size, 128).permute(
        0, 2, 1, 3, 4).reshape(-1, hkv, page_size, 128)
    lens_d = lens.cuda()
    scale = 1.0 / math.sqrt(128)
    print(f"[case] paged decode {B},{S_max},{hq},{hkv},ps={page_size},w={window},split={split}", flush=True)
    o, lse = ta.attn_decode_paged(q, kp, vp, lens_d, table, window=window, scale=scale,
                                  split_tokens=split, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle_mod.decode_paged(np32(q), np32(kp), np32(vp), table.cpu().numpy(),
                                     lens.numpy(), window=window, scale=scale)
    assert_bf16_close(np32(o)[:, :, 0], ro, "paged decode")
    assert_lse_close(np32(lse), rl, LSE_BF16_ABS, "paged decode lse")
    if window == 0:
        o2 = ta.attn_decode(q, kc, vc, lens_d, scale=scale, split_tokens=split)
        torch.cuda.synchronize()
        assert torch.equal(o, o2)


@pytest.mark.parametrize("B,S_max,H,page_size,split", [(3, 512, 128, 32, 0), (2, 1024, 64, 128, 256)])
def test_paged_mla(ta, oracle_mod, B, S_max, H, page_size, split):
    s = W.DSV3_MLA_DECODE
    q, c, lens = W.mla_inputs(s, seed=B + S_max, device="cuda", B=B, S_max=S_max, len_lo=1,
                              len_hi=S_max, H=H)
    c = _poison_tail(c, lens, False)
    cp, table = W.paged_layout(c, page_size, seed=8, head_axis=False, extra_pages=2)
    lens_d = lens.to("cuda")
    print(f"[case] paged mla {B},{S_max},{H},ps={page_size},split={split}", flush=True)
    o, lse = ta.mla_decode_paged(q, cp, lens_d, table, scale=s.scale, split_tokens=split,
                                 return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle_mod.mla_decode_paged(np32(q), np32(cp), table.cpu().numpy(), lens.cpu().numpy(),
                                         d_c=512, d_r=64, scale=s.scale)
    assert_bf16_close(np32(o), ro, "paged mla")
    assert_lse_close(np32(lse), rl, LSE_BF16_ABS, "paged mla lse")
    o2 = ta.mla_decode(q, c, lens_d, scale=s.scale, split_tokens=split)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)


def test_full_size_paged_decode_equals_contiguous(ta, oracle_mod):
    """70B-shaped decode at full size in pages of 64 positions: bit-identical to
    the contiguous decode, and sampled sequences against the oracle."""
    s = W.GQA70B_DECODE
    q, kc, vc, lens = W.decode_inputs(s, seed=0, device="cuda", gen_device="cuda")
    kp, table = W.paged_layout(kc, 64, seed=9, fill=0.0)
    vp = torch.empty_like(kp)
    vp[table.view(-1).long()] = vc.view(s.B, s.h_kv, s.S_max // 64, 64, 128).permute(
        0, 2, 1, 3, 4).reshape(-1, s.h_kv, 64, 128)
    lens_d = lens.to("cuda")
    print("[case] full-size paged decode", flush=True)
    o = ta.attn_decode_paged(q, kp, vp, lens_d, table, scale=s.scale)
    o2 = ta.attn_decode(q, kc, vc, lens_d, scale=s.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    lens_h = lens.cpu()
    for b in (0, 17, 63):
        n = int(lens_h[b])
        ro, _ = oracle_mod.decode(np32(q[b:b + 1]), np32(kc[b:b + 1, :, :n]), np32(vc[b:b + 1, :, :n]),
                                  lens_h[b:b + 1].numpy(), scale=s.scale)
        assert_bf16_close(np32(o[b:b + 1])[:, :, 0], ro, f"paged seq {b}")
