"""Pins for the oracle's attention-sink logit (CPU only).

A sink logit s adds exp(s) to every row's softmax denominator and carries no
value ("Attention Engineering: From MHA to GQA, MLA & FlashAttention",
section 5, failure mode 2).  So, against the same row without a sink:
  O_sink = O / (1 + exp(s - L)),  L_sink = logaddexp(L, s),
a closed form in the no-sink oracle's outputs; a very negative sink changes
nothing; a row with no visible key gets O = 0 and L = s.  The gradients
with a sink, the sink's own included, are pinned by torch autograd through
an fp64 softmax that carries the extra column, and the sink's gradient also
by central differences of the (closed-form pinned) forward."""
import numpy as np
import pytest
import torch


def _rng(seed):
    return np.random.default_rng(seed)


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 7), (False, 0)])
def test_prefill_sink_closed_form(oracle_mod, causal, window):
    rng = _rng(100 + window)
    B, T, hq, hkv, d = 2, 37, 4, 2, 8
    q = rng.standard_normal((B, hq, T, d)).astype(np.float32)
    k = rng.standard_normal((B, hkv, T, d)).astype(np.float32)
    v = rng.standard_normal((B, hkv, T, d)).astype(np.float32)
    sinks = np.array([-1.0, 0.5, 2.0, 4.0], dtype=np.float32)
    o0, l0 = oracle_mod.prefill(q, k, v, causal=causal, window=window, scale=0.3)
    o1, l1 = oracle_mod.prefill(q, k, v, causal=causal, window=window, scale=0.3, sinks=sinks)
    s = sinks.astype(np.float64)[None, :, None]
    assert np.abs(o1 - o0 / (1.0 + np.exp(s - l0))[..., None]).max() < 1e-13
    assert np.abs(l1 - np.logaddexp(l0, s)).max() < 1e-13
    o2, l2 = oracle_mod.prefill(q, k, v, causal=causal, window=window, scale=0.3,
                                sinks=np.full(hq, -1e30, np.float32))
    assert np.array_equal(o2, o0) and np.array_equal(l2, l0)


def test_decode_sink_closed_form_and_empty_row(oracle_mod):
    rng = _rng(110)
    B, hq, hkv, S, d = 3, 8, 2, 50, 16
    q = rng.standard_normal((B, hq, d)).astype(np.float32)
    kc = rng.standard_normal((B, hkv, S, d)).astype(np.float32)
    vc = rng.standard_normal((B, hkv, S, d)).astype(np.float32)
    lens = np.array([50, 13, 0], dtype=np.int32)
    sinks = rng.standard_normal(hq).astype(np.float32)
    o0, l0 = oracle_mod.decode(q, kc, vc, lens, scale=0.25)
    o1, l1 = oracle_mod.decode(q, kc, vc, lens, scale=0.25, sinks=sinks)
    s = sinks.astype(np.float64)[None, :]
    fin = np.isfinite(l0)
    ref_o = np.where(fin[..., None], o0 / (1.0 + np.exp(s - np.where(fin, l0, 0)))[..., None], 0.0)
    assert np.abs(o1 - ref_o).max() < 1e-13
    assert np.abs(l1[fin] - np.logaddexp(l0, s)[fin]).max() < 1e-13
    assert np.all(o1[2] == 0) and np.array_equal(l1[2], sinks.astype(np.float64))


def test_mla_sink_closed_form(oracle_mod):
    rng = _rng(120)
    B, H, S, dc, dr = 2, 4, 40, 48, 16
    q = rng.standard_normal((B, H, dc + dr)).astype(np.float32)
    c = rng.standard_normal((B, S, dc + dr)).astype(np.float32)
    lens = np.array([40, 9], dtype=np.int32)
    sinks = np.array([0.0, 1.0, -2.0, 3.0], dtype=np.float32)
    o0, l0 = oracle_mod.mla_decode(q, c, lens, d_c=dc, d_r=dr, scale=0.2)
    o1, l1 = oracle_mod.mla_decode(q, c, lens, d_c=dc, d_r=dr, scale=0.2, sinks=sinks)
    s = sinks.astype(np.float64)[None, :]
    assert np.abs(o1 - o0 / (1.0 + np.exp(s - l0))[..., None]).max() < 1e-13
    assert np.abs(l1 - np.logaddexp(l0, s)).max() < 1e-13


def test_backward_with_sink_matches_autograd(oracle_mod):
    rng = _rng(130)
    B, T, hq, hkv, d = 1, 23, 4, 2, 8
    G = hq // hkv
    q = rng.standard_normal((B, hq, T, d)).astype(np.float32)
    k = rng.standard_normal((B, hkv, T, d)).astype(np.float32)
    v = rng.standard_normal((B, hkv, T, d)).astype(np.float32)
    do = rng.standard_normal((B, hq, T, d)).astype(np.float32)
    sinks = np.array([0.3, -1.0, 2.0, 0.0], dtype=np.float32)
    scale = 0.35
    qt, kt, vt = (torch.from_numpy(x.astype(np.float64)).requires_grad_(True) for x in (q, k, v))
    st = torch.from_numpy(sinks.astype(np.float64)).requires_grad_(True)
    kr = kt.repeat_interleave(G, dim=1)
    vr = vt.repeat_interleave(G, dim=1)
    s = scale * qt @ kr.transpose(-1, -2)
    mask = torch.tril(torch.ones(T, T, dtype=torch.bool))
    s = s.masked_fill(~mask, float("-inf"))
    sk = st.view(1, hq, 1, 1).expand(B, hq, T, 1)
    w = torch.softmax(torch.cat([s, sk], dim=-1), dim=-1)[..., :T]
    out = w @ vr
    out.backward(torch.from_numpy(do.astype(np.float64)))
    dq, dk, dv, ds = oracle_mod.prefill_backward(q, k, v, do, causal=True, scale=scale,
                                                 sinks=sinks, return_dsinks=True)
    for name, a, b in (("dq", dq, qt.grad), ("dk", dk, kt.grad), ("dv", dv, vt.grad),
                       ("dsinks", ds, st.grad)):
        assert np.abs(a - b.numpy()).max() < 1e-10, name


def test_sink_gradient_matches_finite_differences(oracle_mod):
    """d loss / d sink_h by central differences of the oracle's own forward
    (loss = sum o * dout) -- the forward is pinned by the closed form above,
    the gradient is a separate code path."""
    rng = _rng(131)
    B, T, hq, hkv, d = 2, 11, 3, 1, 4
    q = rng.standard_normal((B, hq, T, d)).astype(np.float32)
    k = rng.standard_normal((B, hkv, T, d)).astype(np.float32)
    v = rng.standard_normal((B, hkv, T, d)).astype(np.float32)
    do = rng.standard_normal((B, hq, T, d)).astype(np.float32)
    sinks = np.array([0.5, -0.25, 1.5], dtype=np.float32)
    scale = 0.4
    *_, ds = oracle_mod.prefill_backward(q, k, v, do, causal=True, window=5, scale=scale,
                                         sinks=sinks, return_dsinks=True)
    eps = 2.0 ** -10
    for h in range(hq):
        sp, sm = sinks.copy(), sinks.copy()
        sp[h] += eps
        sm[h] -= eps
        op, _ = oracle_mod.prefill(q, k, v, causal=True, window=5, scale=scale, sinks=sp)
        om, _ = oracle_mod.prefill(q, k, v, causal=True, window=5, scale=scale, sinks=sm)
        num = (np.sum(op * do) - np.sum(om * do)) / (2 * eps)
        assert abs(num - ds[h]) < 1e-6, h
