"""GPU parity of attn_prefill against the fp64 oracle (through the C ABI)."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from tests.parity import (np32, assert_bf16_close, assert_f32_close, assert_lse_close,
                          LSE_BF16_ABS, LSE_F32_ABS)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ta():
    import transformer_attention_amd as ta
    ta.load_library()
    assert torch.cuda.is_available()
    return ta


def _run(ta, q, k, v, causal, window, scale):
    o, lse = ta.attn_prefill(q, k, v, causal=causal, window=window, scale=scale, return_lse=True)
    torch.cuda.synchronize()
    return o, lse


def _oracle(oracle_mod, q, k, v, causal, window, scale, rows=None):
    return oracle_mod.prefill(np32(q), np32(k), np32(v), causal=causal, window=window,
                              scale=scale, rows=rows)


def test_tiny_fp32_workload(ta, oracle_mod):
    """B=1, T=64, h_q=4, h_kv=2, d_h=16, fp32, seed 0: max-abs 1e-5."""
    s = W.TINY_FP32
    q, k, v = W.prefill_inputs(s, seed=0, device="cuda")
    print(f"[case] tiny fp32 {tuple(q.shape)}", flush=True)
    o, lse = _run(ta, q, k, v, True, 0, s.scale)
    ro, rl = _oracle(oracle_mod, q, k, v, True, 0, s.scale)
    assert_f32_close(np32(o), ro, "tiny fp32 O")
    assert_lse_close(np32(lse), rl, LSE_F32_ABS, "tiny fp32 LSE")


F32_CASES = [
    # B, T, hq, hkv, d, causal, window
    (2, 100, 4, 1, 32, True, 0),
    (1, 130, 2, 2, 64, True, 17),
    (1, 77, 4, 2, 128, False, 0),
    (3, 1, 2, 1, 16, True, 0),
    # d <= 32: each row's keys split over four waves, then merged
    (1, 300, 4, 2, 16, True, 50),    # several 128-key tiles, window
    (2, 200, 2, 1, 32, False, 0),    # several 64-key tiles, bidirectional
    (1, 129, 2, 2, 16, True, 0),     # one key past the first tile
]


@pytest.mark.parametrize("B,T,hq,hkv,d,causal,window", F32_CASES)
def test_fp32_cases(ta, oracle_mod, B, T, hq, hkv, d, causal, window):
    g = torch.Generator().manual_seed(T + d)
    q = torch.randn(B, hq, T, d, generator=g).cuda()
    k = torch.randn(B, hkv, T, d, generator=g).cuda()
    v = torch.randn(B, hkv, T, d, generator=g).cuda()
    scale = 1.0 / math.sqrt(d)
    print(f"[case] fp32 {B},{T},{hq},{hkv},{d},{causal},{window}", flush=True)
    o, lse = _run(ta, q, k, v, causal, window, scale)
    ro, rl = _oracle(oracle_mod, q, k, v, causal, window, scale)
    assert_f32_close(np32(o), ro, "fp32 O")
    assert_lse_close(np32(lse), rl, LSE_F32_ABS, "fp32 LSE")


BF16_CASES = [
    # B, T, hq, hkv, causal, window   (d = 128)
    (1, 64, 4, 4, True, 0),          # one tile, MHA
    (1, 300, 8, 2, True, 0),         # several tiles + ragged tail, GQA G=4
    (2, 513, 8, 8, True, 100),       # MHA with window, tail of one row
    (1, 517, 8, 1, True, 100),       # MQA (G=8) with window
    (1, 333, 6, 3, True, 0),         # G=2
    (1, 200, 4, 2, False, 0),        # bidirectional
    (2, 1, 4, 1, True, 0),           # T = 1
    (1, 700, 32, 1, True, 64),       # G=32: several workgroups per K/V head
    (1, 257, 3, 1, True, 0),         # G=3: one head per workgroup
]


@pytest.mark.parametrize("B,T,hq,hkv,causal,window", BF16_CASES)
def test_bf16_cases(ta, oracle_mod, B, T, hq, hkv, causal, window):
    g = torch.Generator().manual_seed(1000 + T)
    q = torch.randn(B, hq, T, 128, generator=g).to(torch.bfloat16).cuda()
    k = torch.randn(B, hkv, T, 128, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(B, hkv, T, 128, generator=g).to(torch.bfloat16).cuda()
    scale = 1.0 / math.sqrt(128)
    print(f"[case] bf16 {B},{T},{hq},{hkv},{causal},{window}", flush=True)
    o, lse = _run(ta, q, k, v, causal, window, scale)
    ro, rl = _oracle(oracle_mod, q, k, v, causal, window, scale)
    assert_bf16_close(np32(o), ro, "bf16 O")
    assert_lse_close(np32(lse), rl, LSE_BF16_ABS, "bf16 LSE")


def _sample_rows(T, window, step=512):
    rows = {0, 1, 63, 64, 65, 127, 128, 255, 256, T // 2, T - 2, T - 1}
    rows |= set(range(0, T, step))
    if window:
        rows |= {window - 1, window, window + 1, 2 * window + 7}
    return sorted(r for r in rows if 0 <= r < T)


@pytest.mark.parametrize("shape", [W.LLAMA3_8B_PREFILL, W.SWA_MHA, W.SWA_MQA],
                         ids=["llama3-8b", "swa-mha", "swa-mqa"])
def test_full_size_sampled_rows(ta, oracle_mod, shape):
    """Full workload sizes, in the launch configuration the benchmark times;
    every head of every batch entry on sampled query rows."""
    q, k, v = W.prefill_inputs(shape, seed=0, device="cuda", gen_device="cuda")
    print(f"[case] full {shape.name} {tuple(q.shape)} hkv={shape.h_kv}", flush=True)
    o, lse = _run(ta, q, k, v, shape.causal, shape.window, shape.scale)
    rows = _sample_rows(shape.T, shape.window)
    ro, rl = _oracle(oracle_mod, q, k, v, shape.causal, shape.window, shape.scale, rows=rows)
    assert_bf16_close(np32(o[:, :, rows]), ro, shape.name)
    assert_lse_close(np32(lse[:, :, rows]), rl, LSE_BF16_ABS, shape.name)
    assert torch.isfinite(o).all()


def test_gqa_equals_mha_on_repeated_kv_bitwise(ta):
    """GQA through the kernel equals MHA on repeat_interleave'd K/V bit for bit
    ('Attention Engineering', section 6, verification (1))."""
    g = torch.Generator().manual_seed(5)
    B, T, hq, hkv = 1, 400, 8, 2
    q = torch.randn(B, hq, T, 128, generator=g).to(torch.bfloat16).cuda()
    k = torch.randn(B, hkv, T, 128, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(B, hkv, T, 128, generator=g).to(torch.bfloat16).cuda()
    o1 = ta.attn_prefill(q, k, v, causal=True)
    kr = k.repeat_interleave(hq // hkv, dim=1).contiguous()
    vr = v.repeat_interleave(hq // hkv, dim=1).contiguous()
    # MHA on the repeated tensors, one head at a time (same per-head kernel path)
    o2 = torch.empty_like(o1)
    for h in range(hq):
        o2[:, h:h + 1] = ta.attn_prefill(q[:, h:h + 1].contiguous(), kr[:, h:h + 1].contiguous(),
                                         vr[:, h:h + 1].contiguous(), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_deterministic(ta):
    g = torch.Generator().manual_seed(6)
    q = torch.randn(1, 8, 1000, 128, generator=g).to(torch.bfloat16).cuda()
    k = torch.randn(1, 2, 1000, 128, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(1, 2, 1000, 128, generator=g).to(torch.bfloat16).cuda()
    a = ta.attn_prefill(q, k, v, causal=True, window=300)
    b = ta.attn_prefill(q, k, v, causal=True, window=300)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_constant_values_give_constant_output(ta):
    """V = 1 everywhere: every output entry is 1 (weights sum to 1)."""
    g = torch.Generator().manual_seed(7)
    q = torch.randn(2, 4, 300, 128, generator=g).to(torch.bfloat16).cuda()
    k = torch.randn(2, 2, 300, 128, generator=g).to(torch.bfloat16).cuda()
    v = torch.ones(2, 2, 300, 128, dtype=torch.bfloat16, device="cuda")
    o = ta.attn_prefill(q, k, v, causal=True, window=50)
    torch.cuda.synchronize()
    assert (o.float() - 1).abs().max().item() <= 2 ** -7


def test_weights_are_a_causal_distribution(ta):
    """V = I (T <= d) makes the output row the weight row: rows sum to 1, zero
    above the diagonal and outside the window."""
    T = 100
    g = torch.Generator().manual_seed(8)
    q = torch.randn(1, 2, T, 128, generator=g).to(torch.bfloat16).cuda()
    k = torch.randn(1, 1, T, 128, generator=g).to(torch.bfloat16).cuda()
    v = torch.zeros(1, 1, T, 128, dtype=torch.bfloat16)
    v[0, 0, :, :T] = torch.eye(T)
    v = v.cuda()
    P = ta.attn_prefill(q, k, v, causal=True, window=30).float().cpu()[0, :, :, :T]
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    hidden = (j > i) | (i - j >= 30)
    assert torch.all(P[:, hidden] == 0)
    assert (P.sum(-1) - 1).abs().max().item() < 2e-2


def test_large_logits_stay_finite(ta, oracle_mod):
    """Scores far above 88 ('Attention Engineering', section 5, failure mode 1)."""
    g = torch.Generator().manual_seed(9)
    q = (torch.randn(1, 4, 200, 128, generator=g) * 30).to(torch.bfloat16).cuda()
    k = (torch.randn(1, 2, 200, 128, generator=g) * 30).to(torch.bfloat16).cuda()
    v = torch.randn(1, 2, 200, 128, generator=g).to(torch.bfloat16).cuda()
    o = ta.attn_prefill(q, k, v, causal=True)
    torch.cuda.synchronize()
    ro, _ = _oracle(oracle_mod, q, k, v, True, 0, 1 / math.sqrt(128))
    assert torch.isfinite(o).all()
    # near one-hot rows: compare with the bf16 bar
    assert_bf16_close(np32(o), ro, "large logits")


@pytest.mark.parametrize("slope", [10.0, -10.0])
def test_scores_rising_or_falling_along_the_keys(ta, oracle_mod, slope):
    """Score of key j grows (or falls) by about 40 log2 units per 64-key tile,
    so with a rising slope every tile's probabilities overflow the current
    reference max and the running max moves on every tile; with a falling
    slope every later tile underflows against the first one."""
    g = torch.Generator().manual_seed(11)
    B, T, hq, hkv = 1, 700, 4, 2
    q = torch.randn(B, hq, T, 128, generator=g)
    k = torch.randn(B, hkv, T, 128, generator=g)
    v = torch.randn(B, hkv, T, 128, generator=g)
    q[..., 0] = slope
    k[..., 0] = 0.5 * torch.arange(T, dtype=torch.float32)
    q, k, v = (x.to(torch.bfloat16).cuda() for x in (q, k, v))
    scale = 1.0 / math.sqrt(128)
    for window in (0, 200):
        print(f"[case] slope {slope} window {window}", flush=True)
        o, lse = _run(ta, q, k, v, True, window, scale)
        ro, rl = _oracle(oracle_mod, q, k, v, True, window, scale)
        assert torch.isfinite(o).all()
        assert_bf16_close(np32(o), ro, f"slope {slope} window {window}")
        assert_lse_close(np32(lse), rl, LSE_BF16_ABS, f"slope {slope} window {window}")


def test_finite_values_at_masked_positions_do_not_leak(ta):
    """Huge finite K/V at future positions leave the output bit-identical."""
    g = torch.Generator().manual_seed(10)
    T = 256
    q = torch.randn(1, 4, T, 128, generator=g).to(torch.bfloat16).cuda()
    k = torch.randn(1, 2, T, 128, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(1, 2, T, 128, generator=g).to(torch.bfloat16).cuda()
    o = ta.attn_prefill(q, k, v, causal=True)
    cut = 150
    kp, vp = k.clone(), v.clone()
    kp[:, :, cut:] = 1e30
    vp[:, :, cut:] = -1e30
    o2 = ta.attn_prefill(q, kp, vp, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o[:, :, :cut], o2[:, :, :cut])
