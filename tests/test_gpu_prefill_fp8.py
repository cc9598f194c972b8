"""GPU parity of attn_prefill_fp8 (prefill with FP8 attention) against the
oracle's FP8 prefill, through the C ABI.

q, k and v are quantised on the host by the oracle's quantiser (one scale
per 32 positions of a head), so both sides read the same codes.  The
oracle follows the kernel's recipe step by step; the two differ by fp32
against fp64, the output's bf16 rounding, and the FP8 matrix instruction's
accumulation error, which can round a weight to the neighbouring E4M3 code:
the bar is the FP8 attention bar of tests/parity.py.  Cases: one tile,
several tiles with a ragged tail, GQA / MHA / MQA, windows, bidirectional,
T = 1, sink logits, a head long enough to run past the kernel's table of
per-key-block constants, and the Llama-3-8B shape at full size on a
synthetic FP8 input (sampled rows of every head, the benchmark's launch
configuration).
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from tests.parity import LSE_BF16_ABS, assert_fp8_attention_close, assert_lse_close, np32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ta():
    import transformer_attention_amd as m
    m.load_library()
    assert torch.cuda.is_available()
    return m


def _vmax(v8, vs):
    vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()[v8]
    return float(np.abs(vals * np.repeat(vs, 32, axis=-1)[..., :v8.shape[2], None]).max())


def _quantised(oracle_mod, B, T, hq, hkv, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, hq, T, 128, generator=g).to(torch.bfloat16)
    k = torch.randn(B, hkv, T, 128, generator=g).to(torch.bfloat16)
    v = torch.randn(B, hkv, T, 128, generator=g).to(torch.bfloat16)
    return [oracle_mod.quantize_kv_fp8(np32(x)) for x in (q, k, v)]


def _run(ta, qkv, **kw):
    (q8, qs), (k8, ks), (v8, vs) = qkv
    dev = [torch.from_numpy(x).cuda() for x in (q8, k8, v8, qs, ks, vs)]
    o, lse = ta.attn_prefill_fp8(*dev, return_lse=True, **kw)
    torch.cuda.synchronize()
    return o, lse


CASES = [
    # B, T, hq, hkv, causal, window
    (1, 64, 4, 4, True, 0),
    (1, 300, 8, 2, True, 0),
    (2, 513, 8, 8, True, 100),
    (1, 517, 8, 1, True, 100),
    (1, 333, 6, 3, True, 0),
    (1, 200, 4, 2, False, 0),
    (2, 1, 4, 1, True, 0),
    (1, 700, 32, 1, True, 64),
    (1, 257, 3, 1, True, 0),
]


@pytest.mark.parametrize("B,T,hq,hkv,causal,window", CASES)
def test_prefill_fp8_cases(ta, oracle_mod, B, T, hq, hkv, causal, window):
    qkv = _quantised(oracle_mod, B, T, hq, hkv, seed=900 + T + hq)
    scale = 1.0 / math.sqrt(128)
    print(f"[case] prefill fp8 {B},{T},{hq},{hkv},{causal},{window}", flush=True)
    o, lse = _run(ta, qkv, causal=causal, window=window, scale=scale)
    (q8, qs), (k8, ks), (v8, vs) = qkv
    ro, rl = oracle_mod.prefill_fp8(q8, qs, k8, ks, v8, vs, causal=causal, window=window,
                                    scale=scale)
    assert_fp8_attention_close(np32(o), ro, _vmax(v8, vs), "prefill fp8 O")
    assert_lse_close(np32(lse), rl, LSE_BF16_ABS, "prefill fp8 LSE")


def test_prefill_fp8_sinks(ta, oracle_mod):
    qkv = _quantised(oracle_mod, 1, 300, 8, 2, seed=950)
    sinks = torch.linspace(-2.0, 3.0, 8)
    o, lse = _run(ta, qkv, causal=True, window=0, scale=0.09, sinks=sinks.cuda())
    (q8, qs), (k8, ks), (v8, vs) = qkv
    ro, rl = oracle_mod.prefill_fp8(q8, qs, k8, ks, v8, vs, causal=True, scale=0.09,
                                    sinks=sinks.numpy())
    assert_fp8_attention_close(np32(o), ro, _vmax(v8, vs), "prefill fp8 sinks O")
    assert_lse_close(np32(lse), rl, LSE_BF16_ABS, "prefill fp8 sinks LSE")


def test_prefill_fp8_deterministic(ta, oracle_mod):
    qkv = _quantised(oracle_mod, 1, 1000, 8, 2, seed=951)
    a, _ = _run(ta, qkv, causal=True, window=300)
    b, _ = _run(ta, qkv, causal=True, window=300)
    assert torch.equal(a, b)


def test_full_size_llama3_sampled_rows(ta, oracle_mod):
    """The Llama-3-8B shape (B=1, T=8192, 32/8 heads) on synthetic FP8 q, k, v
    (random codes, power-of-two scales), every head on sampled rows."""
    s = W.LLAMA3_8B_PREFILL
    q8, qs = W.random_fp8_cache((s.B, s.h_q, s.T, s.d_h), seed=960, device="cuda")
    k8, ks = W.random_fp8_cache((s.B, s.h_kv, s.T, s.d_h), seed=961, device="cuda")
    v8, vs = W.random_fp8_cache((s.B, s.h_kv, s.T, s.d_h), seed=962, device="cuda")
    print("[case] full-size prefill fp8", flush=True)
    o, lse = ta.attn_prefill_fp8(q8, k8, v8, qs, ks, vs, causal=True, scale=s.scale,
                                 return_lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    rows = sorted(set(range(0, s.T, 97)) | {0, 1, 63, 64, 255, 256, s.T - 2, s.T - 1})
    h = [x.cpu().numpy() for x in (q8, qs, k8, ks, v8, vs)]
    ro, rl = oracle_mod.prefill_fp8(h[0], h[1], h[2], h[3], h[4], h[5], causal=True,
                                    scale=s.scale, rows=rows)
    assert_fp8_attention_close(np32(o[:, :, rows]), ro, _vmax(h[4], h[5]), "full prefill fp8")
    assert_lse_close(np32(lse[:, :, rows]), rl, LSE_BF16_ABS, "full prefill fp8 LSE")


def test_long_head_past_the_block_table(ta, oracle_mod):
    """One causal head of T = 64 x 2051 + 8 positions: the last workgroup's
    tiles (up to 2,052) run past the kernel's table of per-key-block constants
    (4,096 blocks of 32 keys), which it fills once per workgroup, so its last
    tiles take the constants per tile; the workgroup before it ends exactly at
    the table's last entry.  Rows on both sides of those boundaries, a ragged
    tail, and early rows."""
    T = 64 * 2051 + 8
    qkv = _quantised(oracle_mod, 1, T, 1, 1, seed=970)
    scale = 1.0 / math.sqrt(128)
    print(f"[case] prefill fp8 long head T={T}", flush=True)
    o, lse = _run(ta, qkv, causal=True, window=0, scale=scale)
    rows = [0, 5, 70000, 130815, 130816, 131000, 131071, 131072, 131100, 131200, T - 2, T - 1]
    (q8, qs), (k8, ks), (v8, vs) = qkv
    ro, rl = oracle_mod.prefill_fp8(q8, qs, k8, ks, v8, vs, causal=True, scale=scale, rows=rows)
    assert_fp8_attention_close(np32(o[:, :, rows]), ro, _vmax(v8, vs), "long head fp8 O")
    assert_lse_close(np32(lse[:, :, rows]), rl, LSE_BF16_ABS, "long head fp8 LSE")
