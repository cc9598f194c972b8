"""attn_decode_noalloc (the decode with its workspace in the library's static
device array) against attn_decode, through the C ABI.

Two calls in a row, the second with a smaller problem, so the second runs
on whatever the first left in the shared array; then the full 70B-shaped
workload.  Each result must equal attn_decode's bit for bit (same kernels,
same split) and meet the bf16 bar against the oracle.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests.parity import LSE_BF16_ABS, assert_bf16_close, assert_lse_close, np32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ta():
    import transformer_attention_amd as m
    m.load_library()
    assert torch.cuda.is_available()
    return m


def _case(B, S_max, hq, hkv, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, hq, 1, 128, generator=g).to(torch.bfloat16)
    k = torch.randn(B, hkv, S_max, 128, generator=g).to(torch.bfloat16)
    v = torch.randn(B, hkv, S_max, 128, generator=g).to(torch.bfloat16)
    lens = torch.randint(1, S_max + 1, (B,), generator=g, dtype=torch.int32)
    lens[0] = S_max
    for b, n in enumerate(lens.tolist()):          # never read: positions >= len
        k[b, :, n:] = float("nan")
        v[b, :, n:] = float("nan")
    return q.cuda(), k.cuda(), v.cuda(), lens


@pytest.mark.parametrize("order", ["large-then-small"])
def test_two_calls_in_a_row_match_attn_decode(ta, oracle_mod, order):
    cases = [(8, 4096, 32, 4, 0, 501), (3, 1000, 16, 2, 300, 502)]
    sinks = None
    for i, (B, S_max, hq, hkv, window, seed) in enumerate(cases):
        q, k, v, lens = _case(B, S_max, hq, hkv, seed)
        if i == 1:
            sinks = torch.linspace(-2.0, 1.0, hq, device="cuda")
        print(f"[case] noalloc call {i}: B={B} S_max={S_max} {hq}/{hkv} window={window}", flush=True)
        o_na = torch.empty_like(q)
        l_na = torch.empty((B, hq), dtype=torch.float32, device="cuda")
        ta.attn_decode_noalloc(q, k, v, lens.cuda(), window=window, sinks=sinks, o=o_na, lse=l_na)
        o_ws, l_ws = ta.attn_decode(q, k, v, lens.cuda(), window=window, sinks=sinks,
                                    return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws)
        ro, rl = oracle_mod.decode(np32(q), np32(k), np32(v), lens.numpy(), window=window,
                                   scale=1 / np.sqrt(128),
                                   sinks=None if sinks is None else np32(sinks))
        assert_bf16_close(np32(o_na)[:, :, 0], ro, f"noalloc call {i}")
        assert_lse_close(np32(l_na), rl, LSE_BF16_ABS, f"noalloc call {i} lse")


def test_full_size_70b_decode_matches_attn_decode(ta):
    s = W.GQA70B_DECODE
    q, kc, vc, lens = W.decode_inputs(s, seed=0, device="cuda", gen_device="cuda")
    need = ta.attn_decode_workspace_size(s.B, s.S_max, s.h_q, s.h_kv, s.d_h)
    assert 0 < need <= ta.DECODE_NOALLOC_SCRATCH_BYTES
    print(f"[case] noalloc full size, workspace {need} bytes", flush=True)
    lens_d = lens.cuda()
    o1 = ta.attn_decode_noalloc(q, kc, vc, lens_d, scale=s.scale)
    o2 = ta.attn_decode(q, kc, vc, lens_d, scale=s.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_too_large_problem_is_refused_before_launch(ta):
    q = torch.zeros(64, 64, 1, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(64, 8, 256, 128, dtype=torch.bfloat16, device="cuda")
    lens = torch.full((64,), 256, dtype=torch.int32, device="cuda")
    # split 64 over a 256-position cache: 64 x 64 heads x 4 splits x 128 x 4 B fits;
    # the same call on a cache 8192 positions long with split 64 does not
    big = torch.zeros(64, 8, 8192, 128, dtype=torch.bfloat16, device="cuda")
    lens_big = torch.full((64,), 8192, dtype=torch.int32, device="cuda")
    assert ta.attn_decode_workspace_size(64, 8192, 64, 8, 128, 64) > ta.DECODE_NOALLOC_SCRATCH_BYTES
    o = torch.full_like(q, 7.0)
    with pytest.raises(ta.AttnError) as exc:
        ta.attn_decode_noalloc(q, big, big, lens_big, split_tokens=64, o=o)
    assert exc.value.status == ta.ATTN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(o == 7.0)                       # nothing was launched
    ta.attn_decode_noalloc(q, k, k, lens, split_tokens=64, o=o)
    torch.cuda.synchronize()
    assert torch.all(o == 0.0)
