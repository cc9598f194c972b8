"""GPU parity of attn_decode (GQA split-KV decode + log-sum-exp merge) against
the fp64 oracle, through the C ABI."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from tests.parity import np32, assert_bf16_close, assert_lse_close, LSE_BF16_ABS, errors

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ta():
    import transformer_attention_amd as ta
    ta.load_library()
    return ta


def _inputs(B, S_max, hq, hkv, lens, seed, poison=True):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, hq, 1, 128, generator=g).to(torch.bfloat16)
    kc = torch.randn(B, hkv, S_max, 128, generator=g).to(torch.bfloat16)
    vc = torch.randn(B, hkv, S_max, 128, generator=g).to(torch.bfloat16)
    if poison:
        # cache slots past each sequence's length are never read
        for b, L in enumerate(lens):
            kc[b, :, L:] = float("nan")
            vc[b, :, L:] = float("nan")
    lens_t = torch.tensor(lens, dtype=torch.int32)
    return q.cuda(), kc.cuda(), vc.cuda(), lens_t.cuda()


CASES = [
    # B, S_max, hq, hkv, lens, window, split
    (3, 700, 16, 2, [700, 1, 333], 0, 0),
    (3, 700, 16, 2, [700, 1, 333], 0, 64),
    (3, 700, 16, 2, [700, 1, 333], 0, 128),
    (2, 1000, 8, 8, [999, 513], 0, 256),         # MHA decode
    (2, 900, 32, 1, [900, 77], 0, 0),            # MQA: 32 heads over one K/V head
    (2, 640, 24, 2, [640, 300], 0, 64),          # G = 12
    (4, 2048, 16, 2, [2048, 1500, 64, 65], 100, 0),   # sliding window
    (2, 333, 4, 2, [0, 200], 0, 0),              # a zero-length sequence
]


@pytest.mark.parametrize("B,S_max,hq,hkv,lens,window,split", CASES)
def test_decode_cases(ta, oracle_mod, B, S_max, hq, hkv, lens, window, split):
    print(f"[case] decode {B},{S_max},{hq},{hkv},{lens},{window},{split}", flush=True)
    q, kc, vc, lens_t = _inputs(B, S_max, hq, hkv, lens, seed=S_max + hq)
    scale = 1.0 / math.sqrt(128)
    o, lse = ta.attn_decode(q, kc, vc, lens_t, window=window, scale=scale, split_tokens=split,
                            return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle_mod.decode(np32(q), np32(kc), np32(vc), lens, window=window, scale=scale)
    assert_bf16_close(np32(o)[:, :, 0], ro, "decode O")
    assert_lse_close(np32(lse), rl, LSE_BF16_ABS, "decode LSE")
    for b, L in enumerate(lens):
        if L == 0:
            assert torch.all(o[b] == 0)
            assert torch.all(torch.isneginf(lse[b]))


def test_split_count_changes_only_rounding(ta):
    q, kc, vc, lens_t = _inputs(2, 4096, 16, 2, [4096, 2500], seed=3)
    outs = [ta.attn_decode(q, kc, vc, lens_t, split_tokens=s).float() for s in (64, 256, 1024, 0)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert (o - outs[0]).abs().max().item() < 1e-2


def test_decode_equals_last_prefill_row(ta):
    """Decode of the token at position L-1 equals row L-1 of causal prefill
    ('Attention deep dive', section 5): two independent kernels."""
    g = torch.Generator().manual_seed(4)
    B, hq, hkv, T = 1, 16, 2, 777
    q = torch.randn(B, hq, T, 128, generator=g).to(torch.bfloat16).cuda()
    k = torch.randn(B, hkv, T, 128, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(B, hkv, T, 128, generator=g).to(torch.bfloat16).cuda()
    op = ta.attn_prefill(q, k, v, causal=True)
    qd = q[:, :, T - 1:T].contiguous()
    od = ta.attn_decode(qd, k, v, torch.tensor([T], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    max_abs, rel = errors(np32(od), np32(op[:, :, T - 1:T]))
    assert max_abs < 2e-2 and rel < 1e-2


def test_deterministic(ta):
    q, kc, vc, lens_t = _inputs(2, 3000, 16, 2, [3000, 1234], seed=5, poison=False)
    a = ta.attn_decode(q, kc, vc, lens_t)
    b = ta.attn_decode(q, kc, vc, lens_t)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_full_size_sampled_sequences(ta, oracle_mod):
    """70B-shaped decode at full size (B=64, S_max=32768, 64/8 heads), checked
    on a sample of sequences (every head) against the oracle."""
    s = W.GQA70B_DECODE
    q, kc, vc, lens = W.decode_inputs(s, seed=0, device="cuda", gen_device="cuda")
    print(f"[case] full decode {tuple(kc.shape)} sum(len)={int(lens.sum())}", flush=True)
    lens_d = lens.cuda()
    o, lse = ta.attn_decode(q, kc, vc, lens_d, scale=s.scale, return_lse=True)
    torch.cuda.synchronize()
    lens_h = lens.tolist()
    order = sorted(range(s.B), key=lambda b: lens_h[b])
    sample = sorted({order[0], order[-1], order[s.B // 2], 0, s.B - 1})
    for b in sample:
        L = lens_h[b]
        ro, rl = oracle_mod.decode(np32(q[b:b + 1]), np32(kc[b:b + 1, :, :L]), np32(vc[b:b + 1, :, :L]),
                                   [L], scale=s.scale)
        assert_bf16_close(np32(o[b:b + 1])[:, :, 0], ro, f"full decode b={b} L={L}")
        assert_lse_close(np32(lse[b:b + 1]), rl, LSE_BF16_ABS, f"full decode lse b={b}")
    assert torch.isfinite(o).all()
