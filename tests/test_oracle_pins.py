"""Pins for the CPU oracle: checks against what the pages and the mathematics
fix, independent of the oracle's own code (CPU only).

Each pin names the passage (page title and section) it follows.  Library
routines used as independent checks: torch's scaled_dot_product_attention in
float64 on the CPU (math path) and numpy / scipy.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _randn(rng, *shape):
    return rng.standard_normal(shape).astype(np.float32)


def _window_mask(T, causal, window):
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    m = np.ones((T, T), dtype=bool)
    if causal:
        m &= j <= i
    if window > 0:
        m &= (i - j) < window
    return m


def _sdpa64(q, k, v, mask, scale):
    """torch SDPA in float64 on the CPU, GQA through enable_gqa."""
    qt = torch.from_numpy(np.asarray(q, dtype=np.float64))
    kt = torch.from_numpy(np.asarray(k, dtype=np.float64))
    vt = torch.from_numpy(np.asarray(v, dtype=np.float64))
    mt = torch.from_numpy(mask)
    out = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mt, scale=scale,
                                         enable_gqa=qt.shape[1] != kt.shape[1])
    return out.numpy()


# --- library routine: SDPA in fp64 ------------------------------------------------

PREFILL_CASES = [
    # B, T, hq, hkv, d, causal, window
    (1, 64, 4, 2, 16, True, 0),     # the tiny fp32 workload's shape
    (2, 33, 8, 2, 4, True, 0),      # ragged T
    (1, 40, 4, 4, 8, True, 0),      # MHA
    (2, 37, 6, 1, 8, True, 0),      # MQA
    (1, 50, 4, 2, 16, True, 7),     # sliding window
    (2, 29, 4, 1, 8, True, 1),      # window of one: only the diagonal
    (1, 31, 2, 2, 8, False, 0),     # non-causal
    (1, 1, 2, 1, 1, True, 0),       # single token, d = 1
]


@pytest.mark.parametrize("B,T,hq,hkv,d,causal,window", PREFILL_CASES)
def test_prefill_matches_sdpa_fp64(oracle_mod, B, T, hq, hkv, d, causal, window):
    """'Attention Engineering', section 2 (GQA formulation) and 'Attention deep
    dive', section 6 (window mask) against torch SDPA in float64."""
    rng = _rng(B * 1000 + T)
    q, k, v = _randn(rng, B, hq, T, d), _randn(rng, B, hkv, T, d), _randn(rng, B, hkv, T, d)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle_mod.prefill(q, k, v, causal=causal, window=window, scale=scale)
    ref = _sdpa64(q, k, v, _window_mask(T, causal, window), scale)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("B,T,hq,hkv,d,causal,window", PREFILL_CASES[:5])
def test_lse_normalises_independent_scores(oracle_mod, B, T, hq, hkv, d, causal, window):
    """LSE is the natural-log partition function ('Attention Engineering',
    section 4 epilogue): sum_j exp(s_ij - LSE_i) over visible j equals 1,
    with the scores recomputed here by torch.matmul in float64."""
    rng = _rng(7 + T)
    q, k, v = _randn(rng, B, hq, T, d), _randn(rng, B, hkv, T, d), _randn(rng, B, hkv, T, d)
    scale = 0.37
    _, lse = oracle_mod.prefill(q, k, v, causal=causal, window=window, scale=scale)
    kk = np.repeat(k.astype(np.float64), hq // hkv, axis=1)
    s = (q.astype(np.float64) @ np.swapaxes(kk, -1, -2)) * scale
    mask = _window_mask(T, causal, window)
    z = np.where(mask, np.exp(s - lse[..., None]), 0.0).sum(-1)
    np.testing.assert_allclose(z, 1.0, rtol=0, atol=1e-12)


def _brute_force_prefill(q, k, v, causal, window, scale):
    """The definition written out with Python loops and math.exp, one score
    at a time (no numpy reductions): for each row, the visible keys' scores,
    their max, the exponentials, their sum, and the weighted value sum."""
    B, hq, T, d = q.shape
    G = hq // k.shape[1]
    o = [[[[0.0] * d for _ in range(T)] for _ in range(hq)] for _ in range(B)]
    lse = [[[0.0] * T for _ in range(hq)] for _ in range(B)]
    for b in range(B):
        for h in range(hq):
            g = h // G
            for i in range(T):
                vis = [j for j in range(T)
                       if (not causal or j <= i) and (window <= 0 or i - j < window)]
                sc = []
                for j in vis:
                    acc = 0.0
                    for e in range(d):
                        acc += float(q[b, h, i, e]) * float(k[b, g, j, e])
                    sc.append(acc * scale)
                m = max(sc)
                w = [math.exp(x - m) for x in sc]
                z = sum(w)
                for e in range(d):
                    o[b][h][i][e] = sum(wj * float(v[b, g, j, e]) for wj, j in zip(w, vis)) / z
                lse[b][h][i] = m + math.log(z)
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("B,T,hq,hkv,d,causal,window", [
    (1, 9, 4, 2, 3, True, 0), (2, 7, 2, 1, 4, True, 3), (1, 6, 3, 3, 2, False, 0), (1, 5, 4, 1, 1, True, 1)])
def test_prefill_matches_python_brute_force(oracle_mod, B, T, hq, hkv, d, causal, window):
    """Brute force on tiny inputs: the oracle agrees with the definition of
    'Attention Engineering', section 2 (GQA formulation; head h reads K/V
    group h // G) evaluated with scalar Python loops."""
    rng = _rng(11 * T + d)
    q, k, v = _randn(rng, B, hq, T, d), _randn(rng, B, hkv, T, d), _randn(rng, B, hkv, T, d)
    scale = 0.7
    o, lse = oracle_mod.prefill(q, k, v, causal=causal, window=window, scale=scale)
    ro, rl = _brute_force_prefill(q, k, v, causal, window, scale)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-13)


def test_prefill_subset_rows_match_full(oracle_mod):
    rng = _rng(3)
    q, k, v = _randn(rng, 2, 4, 45, 8), _randn(rng, 2, 2, 45, 8), _randn(rng, 2, 2, 45, 8)
    o, lse = oracle_mod.prefill(q, k, v, causal=True, window=9, scale=0.3)
    rows = [44, 0, 17, 8, 9]
    o2, lse2 = oracle_mod.prefill(q, k, v, causal=True, window=9, scale=0.3, rows=rows)
    np.testing.assert_array_equal(o2, o[:, :, rows])
    np.testing.assert_array_equal(lse2, lse[:, :, rows])


# --- the pages' worked online-softmax trace ----------------------------------------

def test_worked_online_softmax_trace(oracle_mod):
    """'Attention, Worked Out by Hand (Part 2)', section 2 (tile trace) and
    'Check it yourself' (weights 0.145, 0.133, 0.609, 0.114)."""
    g = json.load(open(os.path.join(GOLDEN, "online_softmax_trace.json")))
    tol = g["print_tolerance"]
    s = np.array(g["scores"])
    d, T = 4, 4
    # q_3 = e0 and k_j = 2 s_j e0 with scale 1/2 give the printed score row.
    q = np.zeros((1, 1, T, d), np.float32)
    q[0, 0, :, 0] = 1.0
    k = np.zeros((1, 1, T, d), np.float32)
    k[0, 0, :, 0] = 2.0 * s
    # V = I recovers the weights of row 3 (the 'on' row sees all four keys).
    v = np.eye(T, d, dtype=np.float32)[None, None]
    o, lse = oracle_mod.prefill(q, k, v, causal=True, scale=0.5)
    np.testing.assert_allclose(o[0, 0, 3], g["weights"], atol=tol)
    # Final state m = 1.200, l = 1.6430  ->  LSE = m + ln l.
    np.testing.assert_allclose(lse[0, 0, 3], g["tile1"]["m"] + math.log(g["tile1"]["l"]), atol=tol)
    # After tile 0 (keys 'the', 'cat'): m = -0.238, l = 1.9197; row 1 sees exactly those.
    np.testing.assert_allclose(lse[0, 0, 1], g["tile0"]["m"] + math.log(g["tile0"]["l"]), atol=tol)

    # Mixing step with value rows reconstructed from the printed accumulators.
    acc0 = np.array(g["tile0"]["acc"])
    acc1 = np.array(g["tile1"]["acc"])
    V = np.zeros((T, d))
    V[0] = acc0                                  # V[the] + 0.9197 V[cat] = acc0, V[cat] = 0
    V[2] = acc1 - g["tile1"]["rescale"] * acc0   # acc1 = 0.2376 acc0 + V[sat] + 0.1869 V[on], V[on] = 0
    o, _ = oracle_mod.prefill(q, k, V[None, None].astype(np.float32), causal=True, scale=0.5)
    np.testing.assert_allclose(o[0, 0, 3], g["out"], atol=tol)


def test_worked_trace_merge_of_two_tiles(oracle_mod):
    """Merging the two tiles' states with the log-sum-exp algebra gives the
    page's final state (m = 1.200, l = 1.6430)."""
    g = json.load(open(os.path.join(GOLDEN, "online_softmax_trace.json")))
    t0, t1 = g["tile0"], g["tile1"]
    l1_alone = sum(t1["p"])                      # tile 1 relative to its own max
    L0 = t0["m"] + math.log(t0["l"])
    L1 = t1["m"] + math.log(l1_alone)
    acc0 = np.array(t0["acc"]) / t0["l"]
    parts = np.stack([acc0, acc0 * 0])           # second part's output is irrelevant here
    _, L = oracle_mod.merge_partials(parts, [L0, L1])
    assert abs(L - (t1["m"] + math.log(t1["l"]))) < g["print_tolerance"]


# --- closed forms and invariants ------------------------------------------------

def test_identical_keys_give_mean_of_visible_values(oracle_mod):
    """All keys equal -> uniform weights over the visible set: causal row i is
    mean(V_0..V_i), windowed row i the mean of the last W values."""
    rng = _rng(11)
    T, d, W = 23, 8, 5
    q = _randn(rng, 1, 2, T, d)
    k = np.broadcast_to(_randn(rng, 1, 1, 1, d), (1, 1, T, d)).copy()
    v = _randn(rng, 1, 1, T, d).astype(np.float64)
    o, _ = oracle_mod.prefill(q, k, v, causal=True, scale=0.7)
    for i in range(T):
        np.testing.assert_allclose(o[0, :, i], np.broadcast_to(v[0, 0, :i + 1].mean(0), (2, d)), atol=1e-13)
    o, _ = oracle_mod.prefill(q, k, v, causal=True, window=W, scale=0.7)
    for i in range(T):
        np.testing.assert_allclose(o[0, :, i], np.broadcast_to(v[0, 0, max(0, i - W + 1):i + 1].mean(0), (2, d)), atol=1e-13)


def test_scale_zero_gives_mean(oracle_mod):
    rng = _rng(12)
    T, d = 17, 4
    q, k, v = _randn(rng, 1, 1, T, d), _randn(rng, 1, 1, T, d), _randn(rng, 1, 1, T, d)
    o, lse = oracle_mod.prefill(q, k, v, causal=True, scale=0.0)
    for i in range(T):
        np.testing.assert_allclose(o[0, 0, i], v[0, 0, :i + 1].astype(np.float64).mean(0), atol=1e-13)
        assert abs(lse[0, 0, i] - math.log(i + 1)) < 1e-13


def test_causal_row0_attends_only_to_itself(oracle_mod):
    """'Attention, Worked Out by Hand (Part 2)': the first token attends 100% to itself."""
    rng = _rng(13)
    q, k, v = _randn(rng, 2, 4, 9, 8), _randn(rng, 2, 2, 9, 8), _randn(rng, 2, 2, 9, 8)
    o, _ = oracle_mod.prefill(q, k, v, causal=True, scale=0.35)
    np.testing.assert_array_equal(o[:, :, 0], np.repeat(v[:, :, 0], 2, axis=1).astype(np.float64))


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 6), (False, 0)])
def test_weights_rows_sum_to_one_and_respect_mask(oracle_mod, causal, window):
    """With V = I the output row is the weight row: it sums to 1 and is zero
    wherever the mask hides a key (causal: j > i; window: i - j >= W)."""
    rng = _rng(14)
    T = 16
    q, k = _randn(rng, 1, 3, T, T), _randn(rng, 1, 3, T, T)
    v = np.broadcast_to(np.eye(T, dtype=np.float32), (1, 3, T, T)).copy()
    P, _ = oracle_mod.prefill(q, k, v, causal=causal, window=window, scale=0.5)
    np.testing.assert_allclose(P.sum(-1), 1.0, atol=1e-14)
    mask = _window_mask(T, causal, window)
    assert np.all(P[..., ~mask] == 0.0)
    assert np.all(P[..., mask] > 0.0)


def test_gqa_equals_mha_on_repeat_interleaved_kv(oracle_mod):
    """'Attention Engineering', section 6 verification (1) and '2.4 ...',
    repeat_kv: GQA equals MHA on K/V repeated G times along the head axis
    (repeat_interleave order: query head j reads group j // G)."""
    rng = _rng(15)
    B, T, hq, hkv, d = 2, 21, 8, 2, 8
    q, k, v = _randn(rng, B, hq, T, d), _randn(rng, B, hkv, T, d), _randn(rng, B, hkv, T, d)
    o, lse = oracle_mod.prefill(q, k, v, causal=True, scale=0.3)
    kr, vr = np.repeat(k, hq // hkv, axis=1), np.repeat(v, hq // hkv, axis=1)
    o2, lse2 = oracle_mod.prefill(q, kr, vr, causal=True, scale=0.3)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)
    # and a tiled (j % n_kv) mapping would differ
    kt, vt = np.tile(k, (1, hq // hkv, 1, 1)), np.tile(v, (1, hq // hkv, 1, 1))
    o3, _ = oracle_mod.prefill(q, kt, vt, causal=True, scale=0.3)
    assert np.abs(o3 - o).max() > 1e-3


def test_masked_positions_never_read(oracle_mod):
    """Non-finite K/V at future and out-of-window positions leave the output
    bit-identical (mask = select)."""
    rng = _rng(16)
    T, W = 20, 4
    q, k, v = _randn(rng, 1, 2, T, 8), _randn(rng, 1, 1, T, 8), _randn(rng, 1, 1, T, 8)
    o, lse = oracle_mod.prefill(q, k, v, causal=True, window=W, scale=0.3)
    i = 10
    kp, vp = k.copy(), v.copy()
    kp[0, 0, i + 1:] = np.nan
    vp[0, 0, i + 1:] = np.inf
    kp[0, 0, :i - W + 1] = 1e30
    vp[0, 0, :i - W + 1] = np.nan
    o2, lse2 = oracle_mod.prefill(q, kp, vp, causal=True, window=W, scale=0.3, rows=[i])
    np.testing.assert_array_equal(o2[:, :, 0], o[:, :, i])
    np.testing.assert_array_equal(lse2[:, :, 0], lse[:, :, i])


def test_large_logits_closed_form(oracle_mod):
    """Logits far above 88 ('Attention Engineering', section 5, failure mode 1):
    two keys with scores 1000 and 990 give weights 1/(1+e^-10), e^-10/(1+e^-10)."""
    q = np.zeros((1, 1, 2, 2), np.float32)
    q[0, 0, 1] = [1.0, 0.0]
    k = np.zeros((1, 1, 2, 2), np.float32)
    k[0, 0, :, 0] = [1000.0, 990.0]
    v = np.eye(2, dtype=np.float32)[None, None]
    o, lse = oracle_mod.prefill(q, k, v, causal=True, scale=1.0)
    w1 = 1.0 / (1.0 + math.exp(-10.0))
    w2 = math.exp(-10.0) / (1.0 + math.exp(-10.0))
    np.testing.assert_allclose(o[0, 0, 1], [w1, w2], rtol=1e-13)
    np.testing.assert_allclose(lse[0, 0, 1], 1000.0 + math.log1p(math.exp(-10.0)), rtol=1e-15)


# --- decode ---------------------------------------------------------------------

def test_decode_equals_last_prefill_row(oracle_mod):
    """'Attention deep dive', section 5: the new query attends to all cached
    keys (cached + new); that is row len-1 of causal prefill."""
    rng = _rng(17)
    B, hq, hkv, d, S = 3, 8, 2, 16, 40
    lens = [40, 1, 23]
    q_full, k, v = _randn(rng, B, hq, S, d), _randn(rng, B, hkv, S, d), _randn(rng, B, hkv, S, d)
    kc, vc = k.copy(), v.copy()
    qd = np.zeros((B, hq, d), np.float32)
    for b, L in enumerate(lens):
        qd[b] = q_full[b, :, L - 1]
        kc[b, :, L:] = np.nan          # cache slots past the length are never read
        vc[b, :, L:] = np.nan
    od, lsed = oracle_mod.decode(qd, kc, vc, lens, scale=0.25)
    for b, L in enumerate(lens):
        op, lsep = oracle_mod.prefill(q_full[b:b + 1, :, :L], k[b:b + 1, :, :L], v[b:b + 1, :, :L],
                                      causal=True, scale=0.25, rows=[L - 1])
        np.testing.assert_allclose(od[b], op[0, :, 0], atol=1e-14)
        np.testing.assert_allclose(lsed[b], lsep[0, :, 0], atol=1e-14)


@pytest.mark.parametrize("window", [0, 5])
def test_decode_matches_sdpa_fp64(oracle_mod, window):
    rng = _rng(18 + window)
    B, hq, hkv, d, S = 4, 8, 2, 8, 30
    lens = [30, 7, 1, 16]
    q, kc, vc = _randn(rng, B, hq, d), _randn(rng, B, hkv, S, d), _randn(rng, B, hkv, S, d)
    o, _ = oracle_mod.decode(q, kc, vc, lens, window=window, scale=0.4)
    for b, L in enumerate(lens):
        mask = np.ones((1, L), bool)
        if window:
            mask[0, : max(0, L - window)] = False
        ref = _sdpa64(q[b:b + 1, :, None], kc[b:b + 1, :, :L], vc[b:b + 1, :, :L], mask, 0.4)
        np.testing.assert_allclose(o[b], ref[0, :, 0], atol=1e-12)


def test_decode_zero_length_is_zero(oracle_mod):
    rng = _rng(19)
    q, kc, vc = _randn(rng, 2, 2, 4), _randn(rng, 2, 1, 5, 4), _randn(rng, 2, 1, 5, 4)
    o, lse = oracle_mod.decode(q, kc, vc, [0, 5], scale=0.5)
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(o[1]))


def test_split_merge_equals_unsplit(oracle_mod):
    """Split-KV: partial results over disjoint key ranges, merged with the
    log-sum-exp algebra, equal the unsplit result."""
    rng = _rng(20)
    hq, hkv, d, S = 4, 1, 16, 97
    q, kc, vc = _randn(rng, 1, hq, d), _randn(rng, 1, hkv, S, d), _randn(rng, 1, hkv, S, d)
    o, lse = oracle_mod.decode(q, kc, vc, [S], scale=0.25)
    for bounds in ([0, 97], [0, 40, 97], [0, 1, 2, 50, 96, 97], [0, 32, 64, 96, 97]):
        parts_o, parts_l = [], []
        for a, b in zip(bounds[:-1], bounds[1:]):
            # a range [a, b) is the decode of a cache that holds only those keys
            po, pl = oracle_mod.decode(q, kc[:, :, a:b], vc[:, :, a:b], [b - a], scale=0.25)
            parts_o.append(po[0])
            parts_l.append(pl[0])
        parts_o, parts_l = np.stack(parts_o), np.stack(parts_l)
        for h in range(hq):
            om, lm = oracle_mod.merge_partials(parts_o[:, h], parts_l[:, h])
            np.testing.assert_allclose(om, o[0, h], atol=1e-14)
            assert abs(lm - lse[0, h]) < 1e-13
    # an empty part (L = -inf) drops out
    om, lm = oracle_mod.merge_partials(np.stack([o[0, 0], np.full(d, 7.0)]), [lse[0, 0], -np.inf])
    np.testing.assert_allclose(om, o[0, 0], atol=1e-15)


# --- MLA ------------------------------------------------------------------------

def _dyadic(rng, shape, den=8, lim=4):
    return (rng.integers(-lim, lim + 1, size=shape) / den).astype(np.float64)


@pytest.mark.parametrize("H,d_c,d_h,d_r,S", [(8, 48, 32, 16, 64), (4, 512, 128, 64, 48)])
def test_mla_absorbed_equals_unabsorbed(oracle_mod, H, d_c, d_h, d_r, S):
    """'Attention Engineering', section 3 (associative weight absorption and
    the complete MLA score) and section 6 verification (2): attention over
    the absorbed query and the latent cache, followed by W_UV, equals
    standard attention with per-head keys W_UK c, values W_UV c and the
    decoupled RoPE key, scale 1/sqrt(d_h + d_R).  Dyadic inputs keep the
    absorbed query exact in float32."""
    rng = _rng(21 + H)
    w_uk = _dyadic(rng, (H, d_h, d_c))
    w_uv = _dyadic(rng, (H, d_h, d_c))
    c = _dyadic(rng, (S, d_c))
    k_r = _dyadic(rng, (S, d_r))
    q_c = _dyadic(rng, (H, d_h))
    q_r = _dyadic(rng, (H, d_r))
    scale = 1.0 / math.sqrt(d_h + d_r)
    # unabsorbed: per-head content keys/values, SDPA in float64
    k_c = np.einsum("hcd,sd->hsc", w_uk, c)                      # [H,S,d_h]
    v_c = np.einsum("hcd,sd->hsc", w_uv, c)
    k_full = np.concatenate([k_c, np.broadcast_to(k_r, (H, S, d_r))], -1)
    q_full = np.concatenate([q_c, q_r], -1)[:, None]             # [H,1,d_h+d_r]
    ref = _sdpa64(q_full[None], k_full[None], v_c[None], np.ones((1, S), bool), scale)[0, :, 0]
    # absorbed: the oracle over [q~ ; q_R] and [c ; k_R], then W_UV
    q_abs = np.einsum("hcd,hc->hd", w_uk, q_c)                   # W_UK^T q_C  [H,d_c]
    qm = np.concatenate([q_abs, q_r], -1)[None].astype(np.float32)
    assert np.array_equal(qm.astype(np.float64)[0], np.concatenate([q_abs, q_r], -1))
    cache = np.concatenate([c, k_r], -1)[None].astype(np.float32)
    lat, _ = oracle_mod.mla_decode(qm, cache, [S], d_c=d_c, d_r=d_r, scale=scale)
    out = np.einsum("hcd,hd->hc", w_uv, lat[0])
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-11 * max(1.0, np.abs(ref).max()))


def test_mla_matches_sdpa_with_value_alias(oracle_mod):
    """The latent cache row is both key (576 wide) and value (its first 512)."""
    rng = _rng(22)
    B, H, d_c, d_r, S = 2, 4, 32, 8, 19
    q, cache = _randn(rng, B, H, d_c + d_r), _randn(rng, B, S, d_c + d_r)
    lens = [19, 6]
    scale = 1.0 / math.sqrt(24)
    o, lse = oracle_mod.mla_decode(q, cache, lens, d_c=d_c, d_r=d_r, scale=scale)
    for b, L in enumerate(lens):
        kk = cache[b:b + 1, None, :L]
        vv = cache[b:b + 1, None, :L, :d_c]
        ref = _sdpa64(q[b:b + 1, :, None], kk, vv, np.ones((1, L), bool), scale)
        np.testing.assert_allclose(o[b], ref[0, :, 0], atol=1e-12)


# --- the KV-cache byte formula ------------------------------------------------------

def test_kv_cache_byte_formula_against_printed_sizes(oracle_mod):
    """'Attention Engineering', section 0 (M_KV = 2 B S L n_kv d_h b) and the
    sizes printed on the pages (cited per case in the fixture)."""
    cases = json.load(open(os.path.join(GOLDEN, "kv_cache_sizes.json")))["cases"]
    gib = 1024 ** 3
    for c in cases:
        if c["kind"] == "kv":
            n = oracle_mod.kv_cache_bytes(c["B"], c["S"], c["L"], c["n_kv"], c["d_h"], c["b_bytes"])
            if "expect_bytes" in c:
                assert n == c["expect_bytes"], c
            if "expect_gib" in c:
                assert n / gib == pytest.approx(c["expect_gib"], abs=1e-9), c
            if "printed_gb" in c:
                assert n / 1e9 == pytest.approx(c["printed_gb"], abs=c.get("gb_tolerance", 0.05)), c
            if "expect_kib" in c:
                assert n / 1024 == pytest.approx(c["expect_kib"]), c
                m = oracle_mod.kv_cache_bytes(c["B"], c["S"], c["L"], c["mha_n_kv"], c["d_h"], c["b_bytes"])
                assert m / 1024 == pytest.approx(c["expect_mha_kib"]), c
        elif c["kind"] == "mla":
            n = oracle_mod.mla_cache_bytes(c["B"], c["S"], c["L"], c["d_c"], c["d_r"], c["b_bytes"])
            assert n / gib == pytest.approx(c["expect_gib"], abs=1e-9), c
            assert n / 1e9 == pytest.approx(c["printed_gb"], abs=0.05), c
            mha = oracle_mod.kv_cache_bytes(c["B"], c["S"], c["L"], 64, 128, 2)
            gqa = oracle_mod.kv_cache_bytes(c["B"], c["S"], c["L"], 8, 128, 2)
            assert mha / n == pytest.approx(c["ratio_vs_mha"], abs=0.05)
            assert gqa / n == pytest.approx(c["ratio_vs_gqa8"], abs=0.05)
        elif c["kind"] == "kv_elems":
            assert oracle_mod.kv_cache_bytes(1, 1, 1, c["n_kv"], c["d_h"], 1) == c["expect_elems"], c
        elif c["kind"] == "crossover":
            per_head = oracle_mod.kv_cache_bytes(1, 1, 1, 1, c["d_h"], 1)
            mla = oracle_mod.mla_cache_bytes(1, 1, 1, c["d_c"], c["d_r"], 1)
            assert mla / per_head == pytest.approx(c["expect_heads"]), c
