"""GPU parity of attn_prefill_backward (dQ, dK, dV) against the fp64 oracle.

The GPU forward supplies o and lse (as a training step would); the oracle
recomputes everything from q, k, v and dout.  Bar: relative Frobenius error
<= 1e-2 and max-abs error <= 2e-2 x max(1, max |reference|): the gradients
are rounded to bf16 on output, whose error grows with their magnitude (the
K/V gradients sum over every query row and every query head of a group).
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from parity import BF16_MAX_ABS, BF16_REL_FRO, errors, np32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ta():
    import transformer_attention_amd as m
    m.load_library()
    return m


def _check(got, ref, what):
    got = np32(got)
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    max_abs, rel = errors(got, ref)
    bound = BF16_MAX_ABS * max(1.0, float(np.abs(ref).max()))
    print(f"  {what}: max_abs={max_abs:.3e} (bound {bound:.3e}) rel_fro={rel:.3e}", flush=True)
    assert rel <= BF16_REL_FRO and max_abs <= bound, f"{what}: max_abs={max_abs:.3e} rel={rel:.3e}"


def _inputs(B, T, hq, hkv, seed, device="cuda"):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, hq, T, 128, generator=g).to(torch.bfloat16)
    k = torch.randn(B, hkv, T, 128, generator=g).to(torch.bfloat16)
    v = torch.randn(B, hkv, T, 128, generator=g).to(torch.bfloat16)
    do = torch.randn(B, hq, T, 128, generator=g).to(torch.bfloat16)
    return q.to(device), k.to(device), v.to(device), do.to(device)


def _run(ta, q, k, v, do, causal, window, scale):
    o, lse = ta.attn_prefill(q, k, v, causal=causal, window=window, scale=scale, return_lse=True)
    dq, dk, dv = ta.attn_prefill_backward(q, k, v, o, do, lse, causal=causal, window=window,
                                          scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


CASES = [
    # B, T, hq, hkv, causal, window
    (1, 64, 4, 4, True, 0),          # one tile, MHA
    (1, 300, 8, 2, True, 0),         # several tiles + ragged tail, G = 4
    (2, 257, 4, 4, True, 100),       # MHA with window, ragged
    (1, 333, 8, 1, True, 50),        # MQA (G = 8) with window
    (1, 200, 4, 2, False, 0),        # bidirectional
    (2, 1, 4, 1, True, 0),           # T = 1
    (1, 520, 6, 3, True, 0),         # G = 2, several key blocks
]


@pytest.mark.parametrize("B,T,hq,hkv,causal,window", CASES)
def test_backward_cases(ta, oracle_mod, B, T, hq, hkv, causal, window):
    q, k, v, do = _inputs(B, T, hq, hkv, 2000 + T)
    scale = 1.0 / math.sqrt(128)
    print(f"[case] bwd {B},{T},{hq},{hkv},{causal},{window}", flush=True)
    dq, dk, dv = _run(ta, q, k, v, do, causal, window, scale)
    rq, rk, rv = oracle_mod.prefill_backward(np32(q), np32(k), np32(v), np32(do), causal=causal,
                                             window=window, scale=scale)
    _check(dq, rq, "dq")
    _check(dk, rk, "dk")
    _check(dv, rv, "dv")


def test_backward_is_deterministic(ta):
    q, k, v, do = _inputs(1, 400, 8, 2, 77)
    a = _run(ta, q, k, v, do, True, 0, 0.0883883)
    b = _run(ta, q, k, v, do, True, 0, 0.0883883)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_gqa_gradients_equal_mha_on_repeated_kv_summed(ta):
    """GQA backward through the kernels equals MHA on repeat_interleave'd K/V
    with the K/V gradients summed over the repeats (to bf16 output rounding:
    the group sum happens in fp32 inside the GQA kernel, after the bf16
    rounding in the MHA run)."""
    B, T, hq, hkv = 1, 260, 8, 2
    G = hq // hkv
    q, k, v, do = _inputs(B, T, hq, hkv, 78)
    dq1, dk1, dv1 = _run(ta, q, k, v, do, True, 0, 0.0883883)
    kr = k.repeat_interleave(G, dim=1).contiguous()
    vr = v.repeat_interleave(G, dim=1).contiguous()
    dq2, dk2, dv2 = _run(ta, q, kr, vr, do, True, 0, 0.0883883)
    assert torch.equal(dq1, dq2)
    dk2s = dk2.float().view(B, hkv, G, T, 128).sum(2)
    dv2s = dv2.float().view(B, hkv, G, T, 128).sum(2)
    assert (dk1.float() - dk2s).abs().max().item() <= 2e-2 * max(1.0, dk2s.abs().max().item())
    assert (dv1.float() - dv2s).abs().max().item() <= 2e-2 * max(1.0, dv2s.abs().max().item())


def test_future_keys_do_not_touch_earlier_gradients(ta):
    """Causal: changing K/V at positions >= cut leaves dQ of rows < cut and the
    whole backward's dK/dV of positions < cut unchanged bit for bit, except
    through rows >= cut, whose dO is zeroed here."""
    B, T, hq, hkv = 1, 256, 4, 2
    q, k, v, do = _inputs(B, T, hq, hkv, 79)
    cut = 150
    do[:, :, cut:] = 0
    a = _run(ta, q, k, v, do, True, 0, 0.0883883)
    kp, vp = k.clone(), v.clone()
    kp[:, :, cut:] = 3.0
    vp[:, :, cut:] = -3.0
    b = _run(ta, q, kp, vp, do, True, 0, 0.0883883)
    assert torch.equal(a[0][:, :, :cut], b[0][:, :, :cut])
    assert torch.equal(a[1][:, :, :cut], b[1][:, :, :cut])
    assert torch.equal(a[2][:, :, :cut], b[2][:, :, :cut])


@pytest.mark.parametrize("shape", [W.LLAMA3_8B_PREFILL, W.SWA_MHA], ids=["llama3-8b", "swa-mha"])
def test_full_size_one_group(ta, oracle_mod, shape):
    """Full workload size through the kernels (every head); the oracle checks
    the first K/V group of batch entry 0 (its query heads, keys and values)."""
    q, k, v = W.prefill_inputs(shape, seed=0, device="cuda", gen_device="cuda")
    g = torch.Generator(device="cuda").manual_seed(1)
    do = torch.randn(q.shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    print(f"[case] bwd full {shape.name} {tuple(q.shape)} hkv={shape.h_kv}", flush=True)
    dq, dk, dv = _run(ta, q, k, v, do, shape.causal, shape.window, shape.scale)
    G = shape.h_q // shape.h_kv
    rq, rk, rv = oracle_mod.prefill_backward(np32(q[:1, :G]), np32(k[:1, :1]), np32(v[:1, :1]),
                                             np32(do[:1, :G]), causal=shape.causal,
                                             window=shape.window, scale=shape.scale)
    _check(dq[:1, :G], rq, "dq")
    _check(dk[:1, :1], rk, "dk")
    _check(dv[:1, :1], rv, "dv")
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()
