"""GPU parity of mla_decode (absorbed-latent MLA decode) against the fp64
oracle, through the C ABI."""
import math

import pytest
import torch

import workloads as W
from tests.parity import np32, assert_bf16_close, assert_lse_close, LSE_BF16_ABS

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(128 + 64)


@pytest.fixture(scope="module")
def ta():
    import transformer_attention_amd as ta
    ta.load_library()
    return ta


def _inputs(B, S_max, H, lens, seed, poison=True):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, 576, generator=g).to(torch.bfloat16)
    c = torch.randn(B, S_max, 576, generator=g).to(torch.bfloat16)
    if poison:
        for b, L in enumerate(lens):
            c[b, L:] = float("nan")
    return q.cuda(), c.cuda(), torch.tensor(lens, dtype=torch.int32).cuda()


CASES = [
    # B, S_max, H, lens, split
    (2, 300, 128, [300, 37], 0),
    (2, 300, 128, [300, 37], 64),
    (1, 1000, 16, [999], 128),       # one active wave
    (3, 513, 48, [513, 1, 0], 0),    # partial head chunk, length 1 and 0
    (1, 700, 256, [700], 256),       # two head chunks
]


@pytest.mark.parametrize("B,S_max,H,lens,split", CASES)
def test_mla_cases(ta, oracle_mod, B, S_max, H, lens, split):
    print(f"[case] mla {B},{S_max},{H},{lens},{split}", flush=True)
    q, c, lens_t = _inputs(B, S_max, H, lens, seed=S_max + H)
    o, lse = ta.mla_decode(q, c, lens_t, scale=SCALE, split_tokens=split, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle_mod.mla_decode(np32(q), np32(c), lens, d_c=512, d_r=64, scale=SCALE)
    assert_bf16_close(np32(o), ro, "mla O")
    assert_lse_close(np32(lse), rl, LSE_BF16_ABS, "mla LSE")
    for b, L in enumerate(lens):
        if L == 0:
            assert torch.all(o[b] == 0)


def test_split_count_changes_only_rounding(ta):
    q, c, lens_t = _inputs(2, 2048, 128, [2048, 999], seed=3, poison=False)
    outs = [ta.mla_decode(q, c, lens_t, scale=SCALE, split_tokens=s).float() for s in (64, 512, 0)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert (o - outs[0]).abs().max().item() < 1e-2


def test_deterministic(ta):
    q, c, lens_t = _inputs(2, 1500, 128, [1500, 1100], seed=4, poison=False)
    a = ta.mla_decode(q, c, lens_t, scale=SCALE)
    b = ta.mla_decode(q, c, lens_t, scale=SCALE)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_full_size_sampled_sequences(ta, oracle_mod):
    """DeepSeek-V3-shaped MLA decode at full size (B=32, 128 heads, 16384
    tokens), all heads of sampled sequences against the oracle."""
    s = W.DSV3_MLA_DECODE
    q, c, lens = W.mla_inputs(s, seed=0, device="cuda", gen_device="cuda")
    print(f"[case] full mla {tuple(c.shape)}", flush=True)
    o, lse = ta.mla_decode(q, c, lens.cuda(), scale=s.scale, return_lse=True)
    torch.cuda.synchronize()
    for b in (0, 17, s.B - 1):
        L = int(lens[b])
        ro, rl = oracle_mod.mla_decode(np32(q[b:b + 1]), np32(c[b:b + 1, :L]), [L], d_c=512,
                                       d_r=64, scale=s.scale)
        assert_bf16_close(np32(o[b:b + 1]), ro, f"full mla b={b}")
        assert_lse_close(np32(lse[b:b + 1]), rl, LSE_BF16_ABS, f"full mla lse b={b}")
    assert torch.isfinite(o).all()
