"""Pins for the oracle's FP8 KV cache (CPU only).

The FP8 type is OCP E4M3 ("e4m3fn"), the type of the pages' per-tile
quantisation ("Flash Attention 3 and Multi-Headed Latent Attention", the FP8
attention section: scale = tile amax / 448, the E4M3 maximum), applied to the
quantised caches the pages name ("Attention deep dive ...", section 5,
production-engine notes).  Pinned against things other than the oracle:
  * the value of every one of the 256 codes against torch.float8_e4m3fn;
  * encoding against torch's float32 -> float8_e4m3fn conversion, on a dense
    grid (normals, subnormals, exact ties) and on random values;
  * hand-worked ties to even;
  * non-finite input: NaN and +-infinity against torch's cast (the NaN code
    with the input's sign), and a tile holding them quantises its finite
    entries exactly as the same tile with zeros in their place;
  * the quantiser against the same recipe written with torch ops (amax / 448,
    division, cast), bit for bit, including a ragged last tile and an
    all-zero tile;
  * the FP8 decode against the (separately pinned) plain decode of the
    dequantised cache, with power-of-two scales so that dequantisation is
    exact in float32.
"""
import numpy as np
import pytest
import torch


def test_every_code_value_matches_torch(oracle_mod):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle_mod.fp8_e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert list(np.where(nan)[0]) == [0x7f, 0xff]
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert oracle_mod.fp8_e4m3_value(0x7e) == 448.0
    assert oracle_mod.fp8_e4m3_value(0x01) == 2.0 ** -9


def test_encode_matches_torch_on_a_dense_grid(oracle_mod):
    vals = []
    for e in range(-11, 9):
        for m in range(256):
            v = np.ldexp(1.0 + m / 256.0, e)
            if v <= 448.0:
                vals += [v, -v]
    vals += [0.0, 2.0 ** -10, 3 * 2.0 ** -11, 440.0, 447.9]
    rng = np.random.default_rng(5)
    vals += list(rng.standard_normal(500) * 40.0)
    v32 = np.array(vals, dtype=np.float32)
    ref = torch.from_numpy(v32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle_mod.fp8_e4m3_encode(x) for x in v32], dtype=np.uint8)
    assert np.array_equal(got, ref)


def test_ties_go_to_the_even_code(oracle_mod):
    # 1.0 = 0x38, 1.125 = 0x39, 1.25 = 0x3a: 1.0625 is halfway -> 0x38 (even);
    # 1.1875 is halfway between 0x39 and 0x3a -> 0x3a
    assert oracle_mod.fp8_e4m3_encode(1.0625) == 0x38
    assert oracle_mod.fp8_e4m3_encode(1.1875) == 0x3a
    assert oracle_mod.fp8_e4m3_encode(-1.1875) == 0xba
    # subnormals: 2^-9 steps; 1.5 * 2^-9 is halfway between codes 1 and 2 -> 2
    assert oracle_mod.fp8_e4m3_encode(1.5 * 2.0 ** -9) == 0x02
    assert oracle_mod.fp8_e4m3_encode(0.5 * 2.0 ** -9) == 0x00
    assert oracle_mod.fp8_e4m3_encode(1000.0) == 0x7e          # saturates at 448


@pytest.mark.parametrize("S", [64, 77, 5])
def test_quantiser_matches_the_recipe_written_in_torch(oracle_mod, S):
    rng = np.random.default_rng(S)
    B, hkv, d = 2, 3, 16
    x = (rng.standard_normal((B, hkv, S, d)) * rng.uniform(0.01, 50, (B, hkv, S, 1))).astype(np.float32)
    x[1, 2, :min(S, 32)] = 0.0                                   # an all-zero tile
    codes, scales = oracle_mod.quantize_kv_fp8(x)
    nt = (S + 31) // 32
    xt = torch.from_numpy(x)
    for t in range(nt):
        blk = xt[:, :, 32 * t:32 * t + 32]
        amax = blk.abs().amax(dim=(2, 3))
        sc = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
        assert torch.equal(torch.from_numpy(scales[:, :, t]), sc)
        ref = (blk / sc[:, :, None, None]).to(torch.float8_e4m3fn).view(torch.uint8)
        assert torch.equal(torch.from_numpy(codes[:, :, 32 * t:32 * t + 32]), ref)
    assert np.all(codes[1, 2, :min(S, 32)] == 0)


def test_fp8_decode_is_the_decode_of_the_dequantised_cache(oracle_mod):
    rng = np.random.default_rng(9)
    B, hq, hkv, S, d = 3, 8, 2, 100, 16
    q = rng.standard_normal((B, hq, d)).astype(np.float32)
    k8 = rng.integers(0, 256, (B, hkv, S, d), dtype=np.uint8)
    v8 = rng.integers(0, 256, (B, hkv, S, d), dtype=np.uint8)
    k8[(k8 & 0x7f) == 0x7f] = 0x3c                             # no NaN codes
    v8[(v8 & 0x7f) == 0x7f] = 0x41
    nt = (S + 31) // 32
    ks = np.ldexp(1.0, rng.integers(-8, -3, (B, hkv, nt))).astype(np.float32)
    vs = np.ldexp(1.0, rng.integers(-6, 0, (B, hkv, nt))).astype(np.float32)
    lens = np.array([100, 33, 0], dtype=np.int32)
    sinks = rng.standard_normal(hq).astype(np.float32)
    kf = oracle_mod.fp8_dequantize(k8, ks)
    vf = oracle_mod.fp8_dequantize(v8, vs)
    assert np.array_equal(kf.astype(np.float32).astype(np.float64), kf)   # exact in f32
    for window, sk in ((0, None), (20, sinks)):
        o1, l1 = oracle_mod.decode_fp8(q, k8, v8, ks, vs, lens, window=window, scale=0.3, sinks=sk)
        o2, l2 = oracle_mod.decode(q, kf, vf, lens, window=window, scale=0.3, sinks=sk)
        assert np.abs(o1 - o2).max() < 1e-13
        fin = np.isfinite(l2)
        assert np.array_equal(np.isfinite(l1), fin) and np.abs(l1[fin] - l2[fin]).max() < 1e-13


def test_paged_fp8_gathers_codes_and_scales(oracle_mod):
    rng = np.random.default_rng(10)
    B, hq, hkv, S, d, ps = 2, 4, 2, 128, 8, 64
    q = rng.standard_normal((B, hq, d)).astype(np.float32)
    x = rng.standard_normal((B, hkv, S, d)).astype(np.float32)
    y = rng.standard_normal((B, hkv, S, d)).astype(np.float32)
    k8, ks = oracle_mod.quantize_kv_fp8(x)
    v8, vs = oracle_mod.quantize_kv_fp8(y)
    nb = S // ps
    perm = rng.permutation(B * nb + 1)[:B * nb]
    table = perm.reshape(B, nb).astype(np.int32)
    kp = np.zeros((B * nb + 1, hkv, ps, d), np.uint8)
    vp = np.zeros_like(kp)
    ksp = np.zeros((B * nb + 1, hkv, ps // 32), np.float32)
    vsp = np.zeros_like(ksp)
    for b in range(B):
        for j in range(nb):
            pg = table[b, j]
            kp[pg] = k8[b, :, j * ps:(j + 1) * ps]
            vp[pg] = v8[b, :, j * ps:(j + 1) * ps]
            ksp[pg] = ks[b, :, j * ps // 32:(j + 1) * ps // 32]
            vsp[pg] = vs[b, :, j * ps // 32:(j + 1) * ps // 32]
    lens = np.array([128, 70], dtype=np.int32)
    o1, l1 = oracle_mod.decode_paged_fp8(q, kp, vp, ksp, vsp, table, lens, scale=0.35)
    o2, l2 = oracle_mod.decode_fp8(q, k8, v8, ks, vs, lens, scale=0.35)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_non_finite_values_encode_as_the_signed_nan_code(oracle_mod):
    """E4M3 has no infinities; torch's float32 -> float8_e4m3fn cast stores
    NaN and +-inf as the NaN code with the input's sign bit."""
    vals = np.array([np.nan, -np.nan, np.inf, -np.inf], dtype=np.float32)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle_mod.fp8_e4m3_encode(x) for x in vals], dtype=np.uint8)
    assert list(ref) == [0x7f, 0xff, 0x7f, 0xff]
    assert np.array_equal(got, ref)


def test_non_finite_entries_leave_their_tile_neighbours_unchanged(oracle_mod):
    """The tile scale is taken over finite values only: putting NaN / +-inf
    into a tile changes the codes of exactly those entries (to the signed
    NaN code) and neither the scale nor any other code."""
    rng = np.random.default_rng(21)
    B, hkv, S, d = 2, 2, 70, 16
    x = (rng.standard_normal((B, hkv, S, d)) * 3).astype(np.float32)
    bad = np.zeros(x.shape, dtype=bool)
    spots = [(0, 0, 3, 5, np.nan), (0, 1, 40, 0, np.inf), (1, 0, 69, 15, -np.inf),
             (1, 1, 31, 7, -np.nan), (1, 1, 0, 0, np.inf)]
    xb = x.copy()
    xz = x.copy()
    for b, h, s_, e, val in spots:
        xb[b, h, s_, e] = val
        xz[b, h, s_, e] = 0.0
        bad[b, h, s_, e] = True
    cb, sb = oracle_mod.quantize_kv_fp8(xb)
    cz, sz = oracle_mod.quantize_kv_fp8(xz)
    assert np.array_equal(sb, sz)
    assert np.array_equal(cb[~bad], cz[~bad])
    want = [0xff if np.signbit(val) else 0x7f for *_, val in spots]
    assert [int(cb[b, h, s_, e]) for b, h, s_, e, _ in spots] == want
    # a tile of nothing but non-finite values gets scale 1
    xa = np.full((1, 1, 32, 8), np.inf, dtype=np.float32)
    ca, sa = oracle_mod.quantize_kv_fp8(xa)
    assert sa[0, 0, 0] == 1.0 and np.all(ca == 0x7f)
