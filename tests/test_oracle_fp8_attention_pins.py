"""Pins for the oracle's FP8 attention on the MLA decode (CPU only).

The recipe is the pages' FP8 attention ("Flash Attention 3 and Multi-Headed
Latent Attention", the FP8 attention section and the FA3FP8BlockProcessor
listing: q, k, v and p quantised to E4M3 per tile with scale amax / 448,
both products on the quantised operands, dequantised by the scales),
applied to the absorbed MLA decode ("Attention Engineering ...", section 3).
It is an approximation, so it is pinned against things it must reduce to
and bounds it must meet, not against a retyped copy of itself:
  * inputs built so that every quantisation is exact (values on the E4M3
    grid under power-of-two tile scales, scores whose log2 differ by
    integers): the FP8 result is then the plain MLA decode of the same
    inputs, over several chunks and compute tiles, tiles with different
    scales, ragged lengths and a sink logit;
  * random inputs: the FP8 result differs from the plain decode of the
    dequantised inputs by at most the E4M3 rounding of the weights (relative
    half-step 2^-4 of a 3-bit mantissa), elementwise;
  * cache positions at or past the length (codes and scales poisoned with
    NaN) are never read; an empty sequence gives 0 and -inf (or the sink).
"""
import math

import numpy as np
import pytest

DC, DR = 512, 64
DK = DC + DR


def _exact_case(rng, B, H, S, lens):
    """q and cache whose FP8 quantisation is exact and whose weights are
    exact E4M3 values after the reference shift."""
    # query: amax 7 * 2^-h at d = 0 (scale amax / 448 = 2^(-h-6) exactly), the
    # score-carrying entry 2^-h at d = 1 (code 64 exactly)
    q = np.zeros((B, H, DK), np.float32)
    for h in range(H):
        q[:, h, 0] = 7.0 * 2.0 ** -h
        q[:, h, 1] = 2.0 ** -h
    nt = (S + 31) // 32
    grid = np.array([v for v in (np.arange(0, 16) / 8.0) * 2.0 ** 0] + [2.0, 3.0, 4.0, 6.0, 8.0],
                    np.float64)
    c = np.zeros((B, S, DK), np.float32)
    for b in range(B):
        for t in range(nt):
            k_t = [6, 5, 7][(b + t) % 3]                       # tile scale 2^(k_t - 6)
            f = 2.0 ** (k_t - 6)
            r0, r1 = 32 * t, min(S, 32 * t + 32)
            vals = rng.choice(grid, size=(r1 - r0, DK)) * rng.choice([-1.0, 1.0], size=(r1 - r0, DK))
            vals[0, 5] = 448.0                                 # the tile's amax -> scale exactly f
            # d = 0 meets the query's amax entry: zero, so it adds nothing;
            # the score-carrying entry d = 1 is 4m, so that the log2 weight
            # 2^-h 4m + (k_t - 6) is an integer for h <= 2
            m = rng.integers(-1, 2, size=r1 - r0)              # -1, 0, 1
            vals[:, 0] = 0.0
            vals[:, 1] = 4.0 * m / f
            c[b, r0:r1] = (vals * f).astype(np.float32)
    return q, c


@pytest.mark.parametrize("split,tile", [(64, 64), (128, 64), (4096, 64), (96, 32)])
def test_exactly_representable_inputs_give_the_plain_mla_decode(oracle_mod, split, tile):
    rng = np.random.default_rng(31)
    B, H, S = 3, 3, 230
    lens = np.array([230, 131, 64], np.int32)
    q, c = _exact_case(rng, B, H, S, lens)
    codes, scales = oracle_mod.quantize_kv_fp8(c[:, None])
    codes, scales = codes[:, 0], scales[:, 0]
    # the construction is exact: dequantised cache == cache, scales powers of two
    assert np.array_equal(oracle_mod.fp8_dequantize(codes[:, None], scales[:, None])[:, 0], c)
    assert set(np.log2(scales).ravel().tolist()) <= {-1.0, 0.0, 1.0}
    sinks = np.array([0.5, -1.0, 2.0], np.float32)
    for sk in (None, sinks):
        o8, l8 = oracle_mod.mla_decode_fp8(q, codes, scales, lens, d_c=DC, d_r=DR, scale=math.log(2.0),
                                           split=split, tile=tile, sinks=sk)
        o, l = oracle_mod.mla_decode(q, c, lens, d_c=DC, d_r=DR, scale=math.log(2.0), sinks=sk)
        assert np.abs(o8 - o).max() <= 1e-12 * max(1.0, np.abs(o).max())
        assert np.abs(l8 - l).max() <= 1e-12 * max(1.0, np.abs(l).max())


def _random_case(rng, B, H, S):
    q = rng.standard_normal((B, H, DK)).astype(np.float32)
    c = (rng.standard_normal((B, S, DK)) * rng.uniform(0.2, 3.0, (B, S, 1))).astype(np.float32)
    return q, c


@pytest.mark.parametrize("split", [64, 256, 8192])
def test_weight_rounding_stays_within_the_e4m3_step(oracle_mod, split):
    """Against the plain decode of the dequantised q and cache, the only
    difference left is the E4M3 rounding of each weight (relative error at
    most 2^-4 for normal values, 2^-10 x 448 absolute below): so every output
    entry is within max|v| / 16 of it, and the log-sum-exp (unquantised
    denominator) agrees to rounding."""
    rng = np.random.default_rng(32)
    B, H, S = 2, 5, 700
    lens = np.array([700, 333], np.int32)
    q, c = _random_case(rng, B, H, S)
    codes, scales = oracle_mod.quantize_kv_fp8(c[:, None])
    codes, scales = codes[:, 0], scales[:, 0]
    q8, qs = oracle_mod.quantize_kv_fp8(q[:, :, None])
    qd = oracle_mod.fp8_dequantize(q8, qs)[:, :, 0]
    cd = oracle_mod.fp8_dequantize(codes[:, None], scales[:, None])[:, 0]
    scale = 1.0 / math.sqrt(192.0)
    o8, l8 = oracle_mod.mla_decode_fp8(q, codes, scales, lens, d_c=DC, d_r=DR, scale=scale,
                                       split=split)
    oq, lq = oracle_mod.mla_decode(qd, cd, lens, d_c=DC, d_r=DR, scale=scale)
    for b in range(B):
        vmax = np.abs(cd[b, :lens[b], :DC]).max()
        assert np.abs(o8[b] - oq[b]).max() <= vmax / 16.0
    # (the plain decode takes the dequantised values rounded to float32)
    assert np.abs(l8 - lq).max() < 1e-5
    # and the weights really are rounded (not the exact product)
    rel = np.linalg.norm(o8 - oq) / np.linalg.norm(oq)
    assert 1e-4 < rel < 5e-2
    # against the unquantised inputs the FP8 result keeps the output's scale
    o, _ = oracle_mod.mla_decode(q, c, lens, d_c=DC, d_r=DR, scale=scale)
    assert np.linalg.norm(o8 - o) / np.linalg.norm(o) < 0.15


def test_positions_past_the_length_are_never_read(oracle_mod):
    rng = np.random.default_rng(33)
    B, H, S = 2, 4, 300
    lens = np.array([100, 257], np.int32)
    q, c = _random_case(rng, B, H, S)
    codes, scales = oracle_mod.quantize_kv_fp8(c[:, None])
    codes, scales = codes[:, 0], scales[:, 0]
    a = oracle_mod.mla_decode_fp8(q, codes, scales, lens, d_c=DC, d_r=DR, scale=0.07, split=128)
    cp, sp = codes.copy(), scales.copy()
    for b, n in enumerate(lens):
        cp[b, n:] = 0x7f
        sp[b, (n + 31) // 32:] = np.nan
    b_ = oracle_mod.mla_decode_fp8(q, cp, sp, lens, d_c=DC, d_r=DR, scale=0.07, split=128)
    assert np.array_equal(a[0], b_[0]) and np.array_equal(a[1], b_[1])


def test_empty_sequence(oracle_mod):
    rng = np.random.default_rng(34)
    q, c = _random_case(rng, 2, 3, 64)
    codes, scales = oracle_mod.quantize_kv_fp8(c[:, None])
    lens = np.array([0, 64], np.int32)
    o, l = oracle_mod.mla_decode_fp8(q, codes[:, 0], scales[:, 0], lens, d_c=DC, d_r=DR,
                                     scale=0.07, split=64)
    assert np.all(o[0] == 0) and np.all(np.isneginf(l[0]))
    sk = np.array([0.25, -3.0, 1.0], np.float32)
    o, l = oracle_mod.mla_decode_fp8(q, codes[:, 0], scales[:, 0], lens, d_c=DC, d_r=DR,
                                     scale=0.07, split=64, sinks=sk)
    assert np.all(o[0] == 0) and np.allclose(l[0], sk)


# ---------------------------------------------------------------- prefill ---

def _tile_exact(rng, rows, d, f, score_col=None, score_vals=None):
    """rows x d values on the E4M3 grid times f (a power of two), with the
    amax 448 f at [0, 5] so the tile's scale is exactly f."""
    grid = np.array(list(np.arange(0, 16) / 8.0) + [2.0, 3.0, 4.0, 6.0, 8.0])
    vals = rng.choice(grid, size=(rows, d)) * rng.choice([-1.0, 1.0], size=(rows, d))
    vals[0, 5] = 448.0
    if score_col is not None:
        vals[:, 0] = 0.0
        vals[:, score_col] = score_vals / f
    return (vals * f).astype(np.float32)


def _exact_prefill_case(rng, B, T, hq, hkv, d):
    # q: per row amax 7 at e = 0 (scale 7 / 448 = 2^-6 exactly), 1 at e = 1,
    # zero elsewhere, so a score is exactly k[1] times the scale
    q = np.zeros((B, hq, T, d), np.float32)
    q[..., 0] = 7.0
    q[..., 1] = 1.0
    k = np.zeros((B, hkv, T, d), np.float32)
    v = np.zeros((B, hkv, T, d), np.float32)
    for b in range(B):
        for g in range(hkv):
            for t in range((T + 31) // 32):
                r0, r1 = 32 * t, min(T, 32 * t + 32)
                fk = 2.0 ** [0, -1, 1][(b + g + t) % 3]
                fv = 2.0 ** [1, 0, -1][(b + 2 * g + t) % 3]
                m = rng.integers(-1, 2, size=r1 - r0) * 4.0          # k . q = 4m: integer log2 weights
                k[b, g, r0:r1] = _tile_exact(rng, r1 - r0, d, fk, score_col=1, score_vals=m)
                v[b, g, r0:r1] = _tile_exact(rng, r1 - r0, d, fv)
    return q, k, v


@pytest.mark.parametrize("causal,window,tile", [(True, 0, 64), (True, 40, 64), (False, 0, 32),
                                                (True, 0, 128)])
def test_prefill_fp8_exact_case_is_the_plain_prefill(oracle_mod, causal, window, tile):
    rng = np.random.default_rng(41)
    B, T, hq, hkv, d = 2, 150, 4, 2, 16
    q, k, v = _exact_prefill_case(rng, B, T, hq, hkv, d)
    q8, qs = oracle_mod.quantize_kv_fp8(q)
    k8, ks = oracle_mod.quantize_kv_fp8(k)
    v8, vs = oracle_mod.quantize_kv_fp8(v)
    for x8, xs, x in ((q8, qs, q), (k8, ks, k), (v8, vs, v)):      # the construction is exact
        assert np.array_equal(oracle_mod.fp8_dequantize(x8, xs), x)
    sinks = np.array([0.3, -2.0, 1.5, 0.0], np.float32)
    for sk in (None, sinks):
        o8, l8 = oracle_mod.prefill_fp8(q8, qs, k8, ks, v8, vs, causal=causal, window=window,
                                        scale=math.log(2.0), tile=tile, sinks=sk)
        o, l = oracle_mod.prefill(q, k, v, causal=causal, window=window, scale=math.log(2.0),
                                  sinks=sk)
        assert np.abs(o8 - o).max() <= 1e-12 * max(1.0, np.abs(o).max())
        assert np.abs(l8 - l).max() <= 1e-12 * max(1.0, np.abs(l).max())


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 70), (False, 0)])
def test_prefill_fp8_weight_rounding_within_the_e4m3_step(oracle_mod, causal, window):
    rng = np.random.default_rng(42)
    B, T, hq, hkv, d = 1, 300, 4, 2, 64
    q = rng.standard_normal((B, hq, T, d)).astype(np.float32)
    k = rng.standard_normal((B, hkv, T, d)).astype(np.float32)
    v = (rng.standard_normal((B, hkv, T, d)) * rng.uniform(0.3, 3, (B, hkv, T, 1))).astype(np.float32)
    q8, qs = oracle_mod.quantize_kv_fp8(q)
    k8, ks = oracle_mod.quantize_kv_fp8(k)
    v8, vs = oracle_mod.quantize_kv_fp8(v)
    qd, kd, vd = (oracle_mod.fp8_dequantize(a, s) for a, s in ((q8, qs), (k8, ks), (v8, vs)))
    scale = 1.0 / math.sqrt(d)
    o8, l8 = oracle_mod.prefill_fp8(q8, qs, k8, ks, v8, vs, causal=causal, window=window,
                                    scale=scale)
    oq, lq = oracle_mod.prefill(qd, kd, vd, causal=causal, window=window, scale=scale)
    assert np.abs(o8 - oq).max() <= np.abs(vd).max() / 16.0
    assert np.abs(l8 - lq).max() < 1e-5
    rel = np.linalg.norm(o8 - oq) / np.linalg.norm(oq)
    assert 1e-4 < rel < 5e-2
    o, _ = oracle_mod.prefill(q, k, v, causal=causal, window=window, scale=scale)
    assert np.linalg.norm(o8 - o) / np.linalg.norm(o) < 0.15


def test_prefill_fp8_masked_keys_are_excluded(oracle_mod):
    rng = np.random.default_rng(43)
    B, T, hq, hkv, d = 1, 130, 2, 1, 32
    q = rng.standard_normal((B, hq, T, d)).astype(np.float32)
    k = rng.standard_normal((B, hkv, T, d)).astype(np.float32)
    v = rng.standard_normal((B, hkv, T, d)).astype(np.float32)
    q8, qs = oracle_mod.quantize_kv_fp8(q)
    k8, ks = oracle_mod.quantize_kv_fp8(k)
    v8, vs = oracle_mod.quantize_kv_fp8(v)
    a = oracle_mod.prefill_fp8(q8, qs, k8, ks, v8, vs, causal=True, window=20, scale=0.2)
    cut = 70
    kp, vp = k8.copy(), v8.copy()
    kp[:, :, cut:] = 0x7f
    vp[:, :, cut:] = 0xff
    b_ = oracle_mod.prefill_fp8(q8, qs, kp, ks, vp, vs, causal=True, window=20, scale=0.2)
    assert np.array_equal(a[0][:, :, :cut], b_[0][:, :, :cut])
    kp, vp = k8.copy(), v8.copy()
    kp[:, :, :30] = 0x7f                             # outside the window of rows >= 49
    vp[:, :, :30] = 0xff
    c_ = oracle_mod.prefill_fp8(q8, qs, kp, ks, vp, vs, causal=True, window=20, scale=0.2)
    assert np.array_equal(a[0][:, :, 49:], c_[0][:, :, 49:])


def test_prefill_fp8_selected_rows_equal_the_full_result(oracle_mod):
    rng = np.random.default_rng(44)
    B, T, hq, hkv, d = 2, 140, 4, 2, 32
    x = [rng.standard_normal((B, h, T, d)).astype(np.float32) for h in (hq, hkv, hkv)]
    (q8, qs), (k8, ks), (v8, vs) = (oracle_mod.quantize_kv_fp8(a) for a in x)
    o, l = oracle_mod.prefill_fp8(q8, qs, k8, ks, v8, vs, causal=True, window=50, scale=0.17)
    rows = [0, 5, 63, 64, 99, 139]
    o2, l2 = oracle_mod.prefill_fp8(q8, qs, k8, ks, v8, vs, causal=True, window=50, scale=0.17,
                                    rows=rows)
    assert np.array_equal(o[:, :, rows], o2) and np.array_equal(l[:, :, rows], l2)
