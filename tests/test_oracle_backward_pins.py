"""Pins for the oracle's prefill backward (CPU only).

The pages keep the per-row log-sum-exp of the forward for the backward pass
and have it recompute the scores ("Attention Engineering: From MHA to GQA,
MLA & FlashAttention", section 4; "Attention, Worked Out by Hand (Part 2)",
section 2); the gradient itself is the derivative of the forward.  So the
oracle's gradients are pinned to things other than its own formula:
  * central finite differences of an independent pure-Python forward;
  * torch autograd through fp64 SDPA (a library routine the oracle does not
    use);
  * closed forms: uniform weights (K = 0) give dV_j = sum over the rows that
    see j of dO_i / n_i; constant values give dQ = dK = 0;
  * invariants: the softmax gradient of a row sums to zero, so the key
    gradients of one K/V head sum to zero; GQA gradients equal MHA gradients
    on repeat_interleaved K/V summed over the repeats.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F


def _rng(seed):
    return np.random.default_rng(seed)


def _dyadic(rng, shape, den=16, lim=3):
    """Values k/den with |k| <= lim*den: exact in float32, so a +-eps step
    with eps a power of two is exact too."""
    return (rng.integers(-lim * den, lim * den + 1, size=shape) / den).astype(np.float32)


def _visible(i, j, causal, window):
    return (not causal or j <= i) and (window <= 0 or i - j < window)


def _forward_py(q, k, v, causal, window, scale):
    """The forward written out with Python loops and math.exp (float64)."""
    B, hq, T, d = q.shape
    G = hq // k.shape[1]
    o = np.zeros((B, hq, T, d))
    for b in range(B):
        for h in range(hq):
            g = h // G
            for i in range(T):
                vis = [j for j in range(T) if _visible(i, j, causal, window)]
                sc = [scale * sum(float(q[b, h, i, e]) * float(k[b, g, j, e]) for e in range(d))
                      for j in vis]
                m = max(sc)
                w = [math.exp(x - m) for x in sc]
                z = sum(w)
                for e in range(d):
                    o[b, h, i, e] = sum(wj * float(v[b, g, j, e]) for wj, j in zip(w, vis)) / z
    return o


def _loss_py(q, k, v, dout, causal, window, scale):
    return float(np.sum(_forward_py(q, k, v, causal, window, scale) * dout))


@pytest.mark.parametrize("B,T,hq,hkv,d,causal,window", [
    (1, 6, 2, 1, 3, True, 0),      # GQA, causal
    (1, 5, 2, 2, 2, True, 2),      # MHA, window
    (1, 4, 1, 1, 3, False, 0),     # bidirectional
])
def test_backward_matches_finite_differences(oracle_mod, B, T, hq, hkv, d, causal, window):
    rng = _rng(40 + T)
    q = _dyadic(rng, (B, hq, T, d))
    k = _dyadic(rng, (B, hkv, T, d))
    v = _dyadic(rng, (B, hkv, T, d))
    dout = _dyadic(rng, (B, hq, T, d))
    scale = 0.5
    dq, dk, dv = oracle_mod.prefill_backward(q, k, v, dout, causal=causal, window=window, scale=scale)
    eps = 2.0 ** -12
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros(x.shape)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            args_p[name], args_m[name] = xp, xm
            num[idx] = (_loss_py(args_p["q"], args_p["k"], args_p["v"], dout, causal, window, scale) -
                        _loss_py(args_m["q"], args_m["k"], args_m["v"], dout, causal, window, scale)) / (2 * eps)
        # central difference error is O(eps^2 * f''') ~ 1e-7 here
        assert np.abs(num - g).max() < 2e-5, name


@pytest.mark.parametrize("B,T,hq,hkv,d,causal,window", [
    (2, 33, 8, 2, 16, True, 0),
    (1, 40, 4, 1, 8, True, 7),
    (1, 31, 2, 2, 8, False, 0),
    (1, 70, 4, 4, 32, True, 0),
])
def test_backward_matches_torch_autograd_fp64(oracle_mod, B, T, hq, hkv, d, causal, window):
    rng = _rng(50 + T)
    q = rng.standard_normal((B, hq, T, d)).astype(np.float32)
    k = rng.standard_normal((B, hkv, T, d)).astype(np.float32)
    v = rng.standard_normal((B, hkv, T, d)).astype(np.float32)
    dout = rng.standard_normal((B, hq, T, d)).astype(np.float32)
    scale = 1.0 / math.sqrt(d)
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    mask = np.ones((T, T), dtype=bool)
    if causal:
        mask &= j <= i
    if window > 0:
        mask &= (i - j) < window
    qt, kt, vt = (torch.from_numpy(x.astype(np.float64)).requires_grad_(True) for x in (q, k, v))
    out = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask), scale=scale,
                                         enable_gqa=hq != hkv)
    out.backward(torch.from_numpy(dout.astype(np.float64)))
    dq, dk, dv = oracle_mod.prefill_backward(q, k, v, dout, causal=causal, window=window, scale=scale)
    for name, a, b in (("dq", dq, qt.grad), ("dk", dk, kt.grad), ("dv", dv, vt.grad)):
        assert np.abs(a - b.numpy()).max() < 1e-10, name


def test_uniform_weights_closed_form(oracle_mod):
    """K = 0 makes every visible weight 1/n_i, so dV_j = sum_{i sees j} dO_i / n_i
    and dQ = 0."""
    rng = _rng(60)
    B, T, hq, hkv, d, W = 1, 20, 4, 2, 8, 5
    q = rng.standard_normal((B, hq, T, d)).astype(np.float32)
    k = np.zeros((B, hkv, T, d), dtype=np.float32)
    v = rng.standard_normal((B, hkv, T, d)).astype(np.float32)
    dout = rng.standard_normal((B, hq, T, d)).astype(np.float32)
    dq, dk, dv = oracle_mod.prefill_backward(q, k, v, dout, causal=True, window=W, scale=0.3)
    G = hq // hkv
    ref = np.zeros((B, hkv, T, d))
    for g in range(hkv):
        for h in range(g * G, (g + 1) * G):
            for i in range(T):
                vis = [j for j in range(T) if _visible(i, j, True, W)]
                for j in vis:
                    ref[0, g, j] += dout[0, h, i].astype(np.float64) / len(vis)
    assert np.abs(dv - ref).max() < 1e-12
    assert np.abs(dq).max() == 0.0


def test_constant_values_give_zero_query_and_key_gradients(oracle_mod):
    """V_j = c for every key: O_i = c whatever the weights, so dQ = dK = 0,
    and dV_j is the weight-sum of dO."""
    rng = _rng(61)
    B, T, hq, hkv, d = 1, 24, 4, 1, 8
    q = rng.standard_normal((B, hq, T, d)).astype(np.float32)
    k = rng.standard_normal((B, hkv, T, d)).astype(np.float32)
    c = rng.standard_normal(d).astype(np.float32)
    v = np.broadcast_to(c, (B, hkv, T, d)).copy()
    dout = rng.standard_normal((B, hq, T, d)).astype(np.float32)
    dq, dk, dv = oracle_mod.prefill_backward(q, k, v, dout, causal=True, window=0, scale=0.35)
    assert np.abs(dq).max() < 1e-12
    assert np.abs(dk).max() < 1e-12


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 9), (False, 0)])
def test_key_gradients_of_a_head_sum_to_zero(oracle_mod, causal, window):
    """sum_j dS_ij = 0 for every row, so sum_j dK_j = scale sum_i q_i sum_j dS_ij = 0."""
    rng = _rng(62)
    B, T, hq, hkv, d = 2, 37, 6, 2, 8
    q = rng.standard_normal((B, hq, T, d)).astype(np.float32)
    k = rng.standard_normal((B, hkv, T, d)).astype(np.float32)
    v = rng.standard_normal((B, hkv, T, d)).astype(np.float32)
    dout = rng.standard_normal((B, hq, T, d)).astype(np.float32)
    _, dk, _ = oracle_mod.prefill_backward(q, k, v, dout, causal=causal, window=window, scale=0.4)
    assert np.abs(dk.sum(axis=2)).max() < 1e-11


def test_gqa_gradients_equal_mha_on_repeated_kv_summed(oracle_mod):
    rng = _rng(63)
    B, T, hq, hkv, d = 1, 30, 8, 2, 8
    G = hq // hkv
    q = rng.standard_normal((B, hq, T, d)).astype(np.float32)
    k = rng.standard_normal((B, hkv, T, d)).astype(np.float32)
    v = rng.standard_normal((B, hkv, T, d)).astype(np.float32)
    dout = rng.standard_normal((B, hq, T, d)).astype(np.float32)
    dq, dk, dv = oracle_mod.prefill_backward(q, k, v, dout, causal=True, window=0, scale=0.3)
    kr = np.repeat(k, G, axis=1)
    vr = np.repeat(v, G, axis=1)
    dq2, dk2, dv2 = oracle_mod.prefill_backward(q, kr, vr, dout, causal=True, window=0, scale=0.3)
    assert np.abs(dq - dq2).max() < 1e-13
    assert np.abs(dk - dk2.reshape(B, hkv, G, T, d).sum(axis=2)).max() < 1e-12
    assert np.abs(dv - dv2.reshape(B, hkv, G, T, d).sum(axis=2)).max() < 1e-12
