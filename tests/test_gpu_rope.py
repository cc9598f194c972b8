"""GPU parity of attn_rope_qk (rotary position embedding of q and k, in
place) against the fp64 oracle: fp32 max-abs 1e-5, bf16 the usual bar on
the rotated values (rounded to bf16 once).  Dimensions outside the rotated
range and position 0 must come back bit for bit."""
import numpy as np
import pytest
import torch

import workloads as W
from parity import assert_bf16_close, assert_f32_close, np32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ta():
    import transformer_attention_amd as m
    m.load_library()
    return m


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
# Odd head counts (11 / 3) and a 132-wide row, besides the two head sizes.
@pytest.mark.parametrize("B,T,hq,hk,d,base", [(2, 300, 8, 2, 128, 5e5), (1, 77, 4, 4, 64, 1e4),
                                             (1, 50, 11, 3, 64, 1e4), (1, 33, 3, 1, 132, 1e4)])
def test_rope_prefill_shapes(ta, oracle_mod, dtype, B, T, hq, hk, d, base):
    g = torch.Generator().manual_seed(500 + T)
    q = torch.randn(B, hq, T, d, generator=g).to(dtype)
    k = torch.randn(B, hk, T, d, generator=g).to(dtype)
    print(f"[case] rope {dtype} {B},{T},{hq},{hk},{d}", flush=True)
    qg, kg = q.cuda(), k.cuda()
    ta.attn_rope_qk(qg, kg, base=base)
    torch.cuda.synchronize()
    rq = oracle_mod.rope(np32(q), base=base)
    rk = oracle_mod.rope(np32(k), base=base)
    check = assert_f32_close if dtype == torch.float32 else assert_bf16_close
    check(np32(qg), rq, "rope q")
    check(np32(kg), rk, "rope k")


def test_rope_decode_positions_far_out(ta, oracle_mod):
    """One new token per sequence at positions up to 2^17 (fp32)."""
    g = torch.Generator().manual_seed(510)
    B, hq, hk, d = 16, 8, 2, 128
    q = torch.randn(B, hq, 1, d, generator=g)
    k = torch.randn(B, hk, 1, d, generator=g)
    pos = torch.randint(0, 1 << 17, (B, 1), generator=g, dtype=torch.int32)
    pos[0, 0] = (1 << 17) - 1
    qg, kg = q.cuda(), k.cuda()
    ta.attn_rope_qk(qg, kg, base=5e5, positions=pos.cuda())
    torch.cuda.synchronize()
    assert_f32_close(np32(qg), oracle_mod.rope(np32(q), positions=pos.numpy(), base=5e5), "rope q far")
    assert_f32_close(np32(kg), oracle_mod.rope(np32(k), positions=pos.numpy(), base=5e5), "rope k far")


def test_rope_mla_tail_and_untouched_dims(ta, oracle_mod):
    """MLA: only the 64-d RoPE tail of the 576-wide query rows and of the
    shared key row is rotated."""
    g = torch.Generator().manual_seed(520)
    B, H, T = 3, 16, 5
    q = torch.randn(B, H, T, 576, generator=g).to(torch.bfloat16)
    k = torch.randn(B, 1, T, 576, generator=g).to(torch.bfloat16)
    pos = torch.randint(0, 20000, (B, T), generator=g, dtype=torch.int32)
    qg, kg = q.cuda(), k.cuda()
    ta.attn_rope_qk(qg, kg, base=1e4, positions=pos.cuda(), rope_offset=512, rope_dim=64)
    torch.cuda.synchronize()
    assert torch.equal(qg[..., :512].cpu(), q[..., :512])
    assert torch.equal(kg[..., :512].cpu(), k[..., :512])
    rq = oracle_mod.rope(np32(q), positions=pos.numpy(), base=1e4, rope_offset=512, rope_dim=64)
    rk = oracle_mod.rope(np32(k), positions=pos.numpy(), base=1e4, rope_offset=512, rope_dim=64)
    assert_bf16_close(np32(qg)[..., 512:], rq[..., 512:], "mla q tail")
    assert_bf16_close(np32(kg)[..., 512:], rk[..., 512:], "mla k tail")


def test_rope_position_zero_is_identity(ta):
    g = torch.Generator().manual_seed(530)
    q = torch.randn(2, 4, 3, 128, generator=g).to(torch.bfloat16).cuda()
    q0 = q.clone()
    ta.attn_rope_qk(q, None, base=1e4, positions=torch.zeros(2, 3, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(q, q0)


def test_rope_full_size_llama3(ta, oracle_mod):
    """The Llama-3-8B prefill's q and k (T = 8192, 32/8 heads, base 5e5), rows
    sampled against the oracle."""
    s = W.LLAMA3_8B_PREFILL
    q, k, _ = W.prefill_inputs(s, seed=0, device="cuda", gen_device="cuda")
    q0, k0 = q.clone(), k.clone()
    print("[case] rope full size", flush=True)
    ta.attn_rope_qk(q, k, base=5e5)
    torch.cuda.synchronize()
    for t in (0, 1, 4095, 8191):
        pos = np.array([[t]], dtype=np.int32)
        rq = oracle_mod.rope(np32(q0[:, :, t:t + 1]), positions=pos, base=5e5)
        rk = oracle_mod.rope(np32(k0[:, :, t:t + 1]), positions=pos, base=5e5)
        assert_bf16_close(np32(q[:, :, t:t + 1]), rq, f"q row {t}")
        assert_bf16_close(np32(k[:, :, t:t + 1]), rk, f"k row {t}")
