"""GPU parity of mla_decode_fp8 (MLA decode with FP8 attention) against the
oracle's FP8 MLA decode, through the C ABI.

The oracle follows the same recipe step by step (query quantised per head,
E4M3 cache with 32-token scales, weights quantised against each chunk's
running reference in 64-token tiles, unquantised denominator).  The two
differ by fp32 against fp64 arithmetic, the output's bf16 rounding, and the
FP8 matrix instruction's own accumulation error (about 2^-15 of the sum of
the term magnitudes, measured), which can round a weight to the
neighbouring E4M3 code: the bar is the bf16 one with the elementwise bound
widened to one E4M3 step of the values, max(2e-2, max|v| / 8)
(tests/parity.py).  Cases span several chunks and tiles, ragged lengths,
an empty sequence, sink logits, head counts that leave part of a workgroup
idle, and cache positions past each length poisoned with NaN codes and NaN
scales.  The full-size test runs the DeepSeek-V3-shaped workload (B=32, 128
heads, 16384 tokens) on a synthetic FP8 cache in the launch configuration
the benchmark times and checks every sequence.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from tests.parity import LSE_BF16_ABS, assert_fp8_attention_close, assert_lse_close, np32

pytestmark = pytest.mark.gpu

DC, DR = 512, 64


@pytest.fixture(scope="module")
def ta():
    import transformer_attention_amd as m
    m.load_library()
    assert torch.cuda.is_available()
    return m


def _vmax(codes, scales, lens):
    """Largest dequantised value magnitude in the visible cache (the values
    are the first 512 entries of each row)."""
    v = 0.0
    for b, n in enumerate(lens):
        if n:
            vals = _e4m3_values()[codes[b, :n, :DC]] * np.repeat(scales[b], 32)[:n, None]
            v = max(v, float(np.abs(vals).max()))
    return v


_TABLE = []


def _e4m3_values():
    """The value of each of the 256 E4M3 codes (torch's float8_e4m3fn)."""
    if not _TABLE:
        _TABLE.append(torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy())
    return _TABLE[0]


def _case(oracle_mod, B, S_max, H, lens, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, DC + DR, generator=g).to(torch.bfloat16)
    c = (torch.randn(B, S_max, DC + DR, generator=g) *
         torch.exp(0.5 * torch.randn(B, S_max, 1, generator=g))).to(torch.bfloat16)
    codes, scales = oracle_mod.quantize_kv_fp8(np32(c)[:, None])
    codes, scales = codes[:, 0], scales[:, 0]
    for b, n in enumerate(lens):                     # never read: positions >= len
        codes[b, n:] = 0x7f
        scales[b, (n + 31) // 32:] = np.nan
    return q, codes, scales, np.array(lens, np.int32)


def _default_split(B, S_max, H):
    """The split mla_decode chooses with split_tokens = 0 (about one
    workgroup per compute unit for full-length sequences)."""
    split = (S_max * B * ((H + 127) // 128) + 255) // 256
    split = max(64, (split + 63) // 64 * 64)
    return min(split, (S_max + 63) // 64 * 64)


CASES = [
    # B, S_max, H, lens, split
    (2, 256, 128, [256, 200], 64),
    (3, 700, 128, [700, 1, 383], 128),
    (2, 1024, 32, [1024, 640], 256),
    (1, 2048, 16, [2048], 0),
    (4, 513, 128, [513, 0, 64, 65], 192),
    (1, 300, 200, [300], 128),
]


@pytest.mark.parametrize("B,S_max,H,lens,split", CASES)
def test_mla_fp8_cases(ta, oracle_mod, B, S_max, H, lens, split):
    q, codes, scales, lens_np = _case(oracle_mod, B, S_max, H, lens, seed=700 + S_max + H)
    scale = 1.0 / math.sqrt(192.0)
    print(f"[case] mla fp8 B={B} S_max={S_max} H={H} lens={lens} split={split}", flush=True)
    o, lse = ta.mla_decode_fp8(q.cuda(), torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                               torch.from_numpy(lens_np).cuda(), scale=scale, split_tokens=split,
                               return_lse=True)
    torch.cuda.synchronize()
    eff = split
    if split == 0:                                   # the library's choice, same workspace
        eff = _default_split(B, S_max, H)
        assert (ta.mla_decode_fp8_workspace_size(B, S_max, H, DC, DR, 0) ==
                ta.mla_decode_fp8_workspace_size(B, S_max, H, DC, DR, eff))
    ro, rl = oracle_mod.mla_decode_fp8(np32(q), codes, scales, lens_np, d_c=DC, d_r=DR, scale=scale,
                                       split=eff)
    assert_fp8_attention_close(np32(o), ro, _vmax(codes, scales, lens), "mla fp8 O")
    assert_lse_close(np32(lse), rl, LSE_BF16_ABS, "mla fp8 LSE")
    for b, n in enumerate(lens):
        if n == 0:
            assert torch.all(o[b] == 0) and torch.all(torch.isneginf(lse[b]))


def test_mla_fp8_sinks(ta, oracle_mod):
    B, S_max, H = 2, 400, 128
    q, codes, scales, lens = _case(oracle_mod, B, S_max, H, [400, 0], seed=711)
    sinks = torch.linspace(-3.0, 4.0, H)
    o, lse = ta.mla_decode_fp8(q.cuda(), torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                               torch.from_numpy(lens).cuda(), scale=0.07, split_tokens=128,
                               sinks=sinks.cuda(), return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle_mod.mla_decode_fp8(np32(q), codes, scales, lens, d_c=DC, d_r=DR, scale=0.07,
                                       split=128, sinks=sinks.numpy())
    assert_fp8_attention_close(np32(o), ro, _vmax(codes, scales, lens), "mla fp8 sinks O")
    assert_lse_close(np32(lse), rl, LSE_BF16_ABS, "mla fp8 sinks LSE")


def test_mla_fp8_deterministic(ta, oracle_mod):
    B, S_max, H = 2, 2048, 128
    q, codes, scales, lens = _case(oracle_mod, B, S_max, H, [2048, 1500], seed=712)
    args = (q.cuda(), torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
            torch.from_numpy(lens).cuda())
    a = ta.mla_decode_fp8(*args, scale=0.07, split_tokens=256)
    b = ta.mla_decode_fp8(*args, scale=0.07, split_tokens=256)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_full_size_every_sequence(ta, oracle_mod):
    """DeepSeek-V3-shaped MLA decode (B=32, 128 heads, 16384 tokens of 576
    values) on a synthetic FP8 cache, in the benchmark's launch
    configuration (default split); every sequence against the oracle."""
    s = W.DSV3_MLA_DECODE
    g = torch.Generator().manual_seed(720)
    q = torch.randn(s.B, s.H, s.d_c + s.d_r, generator=g).to(torch.bfloat16)
    codes, scales = W.random_fp8_cache((s.B, 1, s.S_max, s.d_c + s.d_r), seed=721, device="cuda")
    codes, scales = codes[:, 0].contiguous(), scales[:, 0].contiguous()
    lens = torch.full((s.B,), s.S_max, dtype=torch.int32)
    split = _default_split(s.B, s.S_max, s.H)        # the library's choice: 2048
    assert (ta.mla_decode_fp8_workspace_size(s.B, s.S_max, s.H, s.d_c, s.d_r, 0) ==
            ta.mla_decode_fp8_workspace_size(s.B, s.S_max, s.H, s.d_c, s.d_r, split))
    print("[case] full-size mla fp8", flush=True)
    o, lse = ta.mla_decode_fp8(q.cuda(), codes, scales, lens.cuda(), scale=s.scale, return_lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    c_h, sc_h = codes.cpu().numpy(), scales.cpu().numpy()
    for b0 in range(0, s.B, 8):
        ro, rl = oracle_mod.mla_decode_fp8(np32(q[b0:b0 + 8]), c_h[b0:b0 + 8], sc_h[b0:b0 + 8],
                                           lens[b0:b0 + 8].numpy(), d_c=s.d_c, d_r=s.d_r,
                                           scale=s.scale, split=split)
        vm = _vmax(c_h[b0:b0 + 8], sc_h[b0:b0 + 8], lens[b0:b0 + 8].tolist())
        assert_fp8_attention_close(np32(o[b0:b0 + 8]), ro, vm, f"full mla fp8 b={b0}..{b0 + 7}")
        assert_lse_close(np32(lse[b0:b0 + 8]), rl, LSE_BF16_ABS, f"full mla fp8 lse b={b0}")
        print(f"  sequences {b0}..{b0 + 7} ok", flush=True)
