"""Pins for the oracle's rotary position embedding (CPU only).

The pages define RoPE in the complex plane: pair j of a head, z_j = x_{2j} +
i x_{2j+1}, is multiplied by e^{i m theta_j} at position m, theta_j =
base^(-2j/d), and the inner product of a rotated query and key depends only
on their distance ("Attention Engineering: From MHA to GQA, MLA &
FlashAttention", section 1, the complex-plane derivation and the
"RoPE Relative-Distance Invariance Identity").  Pinned against:
  * numpy complex multiplication (the complex form, not the oracle's real
    rotation);
  * the relative-distance identity, over many (m, n);
  * hand values (theta_0 = 1 at any base; position 0 is the identity);
  * per-pair norms, and untouched dimensions outside the rotated range.
"""
import math

import numpy as np
import pytest


@pytest.mark.parametrize("rd,base", [(128, 5e5), (64, 1e4), (16, 1e4)])
def test_rope_is_complex_multiplication(oracle_mod, rd, base):
    rng = np.random.default_rng(rd)
    B, H, T = 2, 3, 17
    x = rng.standard_normal((B, H, T, rd)).astype(np.float32)
    pos = rng.integers(0, 40000, (B, T)).astype(np.int32)
    got = oracle_mod.rope(x, positions=pos, base=base)
    z = x[..., 0::2].astype(np.float64) + 1j * x[..., 1::2].astype(np.float64)
    theta = base ** (-np.arange(0, rd, 2) / rd)
    zr = z * np.exp(1j * pos[:, None, :, None].astype(np.float64) * theta)
    ref = np.stack([zr.real, zr.imag], axis=-1).reshape(x.shape)
    assert np.abs(got - ref).max() < 1e-9


def test_relative_distance_identity(oracle_mod):
    rng = np.random.default_rng(3)
    d = 32
    q = rng.standard_normal((1, 1, 1, d)).astype(np.float32)
    k = rng.standard_normal((1, 1, 1, d)).astype(np.float32)
    pairs = [(5, 2), (100, 97), (3000, 2997), (7, 7), (4000, 4000), (0, 9), (500, 509)]
    dots = {}
    for m, n in pairs:
        rq = oracle_mod.rope(q, positions=np.array([[m]]), base=1e4)
        rk = oracle_mod.rope(k, positions=np.array([[n]]), base=1e4)
        dots.setdefault(m - n, []).append(float(np.sum(rq * rk)))
    for dist, vals in dots.items():
        assert max(vals) - min(vals) < 1e-9, dist
    # and the dot depends on the distance: distances 3 and 0 differ
    assert abs(dots[3][0] - dots[0][0]) > 1e-3


def test_hand_values_and_identity_at_zero(oracle_mod):
    x = np.array([[[[1.0, 0.0, 1.0, 0.0]]]], dtype=np.float32)
    got = oracle_mod.rope(x, positions=np.array([[1]]), base=1e4)[0, 0, 0]
    # theta_0 = 1, theta_1 = 1e4^(-1/2) = 0.01
    assert np.allclose(got, [math.cos(1.0), math.sin(1.0), math.cos(0.01), math.sin(0.01)], atol=1e-15)
    rng = np.random.default_rng(4)
    y = rng.standard_normal((2, 2, 5, 8)).astype(np.float32)
    assert np.array_equal(oracle_mod.rope(y, positions=np.zeros((2, 5), np.int32), base=1e4), y)


def test_norms_and_the_untouched_dimensions(oracle_mod):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 4, 9, 576)).astype(np.float32)
    got = oracle_mod.rope(x, base=1e4, rope_offset=512, rope_dim=64)
    assert np.array_equal(got[..., :512], x[..., :512])
    n0 = x[..., 512::2].astype(np.float64) ** 2 + x[..., 513::2].astype(np.float64) ** 2
    n1 = got[..., 512::2] ** 2 + got[..., 513::2] ** 2
    assert np.abs(n0 - n1).max() < 1e-12
    # default positions are 0..T-1: row t equals an explicit position t
    pos = np.tile(np.arange(9, dtype=np.int32), (2, 1))
    assert np.array_equal(got, oracle_mod.rope(x, positions=pos, base=1e4, rope_offset=512, rope_dim=64))
