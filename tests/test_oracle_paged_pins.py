"""Pins for the oracle's paged-cache helpers (CPU only): a paged cache built
from a contiguous one with a random page permutation gathers back to it
exactly, and the paged decodes equal the contiguous ones on that cache."""
import numpy as np
import pytest


def _scatter(cache, page_size, rng, head_axis, extra_pages=3):
    """Pages in a random order (plus unused pages filled with NaN) and the
    block table that maps every sequence back."""
    if head_axis:
        B, hkv, S, d = cache.shape
    else:
        B, S, d = cache.shape
    nb = S // page_size
    n_pages = B * nb + extra_pages
    perm = rng.permutation(n_pages)[:B * nb]
    shape = (n_pages, hkv, page_size, d) if head_axis else (n_pages, page_size, d)
    pages = np.full(shape, np.nan, dtype=np.float32)
    table = np.zeros((B, nb), dtype=np.int32)
    for b in range(B):
        for j in range(nb):
            pg = int(perm[b * nb + j])
            table[b, j] = pg
            if head_axis:
                pages[pg] = cache[b, :, j * page_size:(j + 1) * page_size]
            else:
                pages[pg] = cache[b, j * page_size:(j + 1) * page_size]
    return pages, table


@pytest.mark.parametrize("page_size", [32, 64])
def test_gather_inverts_a_random_page_layout(oracle_mod, page_size):
    rng = np.random.default_rng(70 + page_size)
    B, hkv, S, d = 3, 2, 256, 8
    cache = rng.standard_normal((B, hkv, S, d)).astype(np.float32)
    lens = np.array([256, 100, 33], dtype=np.int32)
    pages, table = _scatter(cache, page_size, rng, head_axis=True)
    back = oracle_mod.gather_pages(pages, table, lens, head_axis=True)
    for b in range(B):
        assert np.array_equal(back[b, :, :lens[b]], cache[b, :, :lens[b]])
        assert np.all(back[b, :, lens[b]:] == 0)


@pytest.mark.parametrize("window", [0, 40])
def test_paged_decode_equals_contiguous(oracle_mod, window):
    rng = np.random.default_rng(80 + window)
    B, hq, hkv, S, d = 3, 8, 2, 192, 16
    k = rng.standard_normal((B, hkv, S, d)).astype(np.float32)
    v = rng.standard_normal((B, hkv, S, d)).astype(np.float32)
    q = rng.standard_normal((B, hq, d)).astype(np.float32)
    lens = np.array([192, 77, 1], dtype=np.int32)
    kp, table = _scatter(k, 32, rng, head_axis=True)
    # V's pages use K's table (one permutation for both)
    vp = np.full_like(kp, np.nan)
    for b in range(B):
        for j in range(S // 32):
            vp[table[b, j]] = v[b, :, 32 * j:32 * (j + 1)]
    o1, l1 = oracle_mod.decode_paged(q, kp, vp, table, lens, window=window, scale=0.25)
    o2, l2 = oracle_mod.decode(q, k, v, lens, window=window, scale=0.25)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_paged_mla_equals_contiguous(oracle_mod):
    rng = np.random.default_rng(90)
    B, H, S, dc, dr = 2, 4, 128, 48, 16
    c = rng.standard_normal((B, S, dc + dr)).astype(np.float32)
    q = rng.standard_normal((B, H, dc + dr)).astype(np.float32)
    lens = np.array([128, 50], dtype=np.int32)
    pages, table = _scatter(c, 32, rng, head_axis=False)
    o1, l1 = oracle_mod.mla_decode_paged(q, pages, table, lens, d_c=dc, d_r=dr, scale=0.2)
    o2, l2 = oracle_mod.mla_decode(q, c, lens, d_c=dc, d_r=dr, scale=0.2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
