"""CPU oracle for exact scaled-dot-product attention (prefill, decode, MLA decode).

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain reference that the
HIP kernels are checked against.  Only the test suite, the package smoke check
and the benchmark's CPU-baseline leg may import it; the GPU library never does,
and the two share no code.

The arithmetic lives in ``attn_oracle.c`` (fp64, OpenMP over output rows),
compiled with gcc into ``oracle/_build/libattn_oracle.so`` by :func:`build`.
This module only marshals numpy arrays: inputs are widened to float32 (exact
for the bf16 and fp32 inputs the kernels take) and results come back as
float64.

Pages the definitions follow (cited by title and section):
  * "Attention Engineering: From MHA to GQA, MLA & FlashAttention", section 2
    (GQA formulation), section 3 (MLA absorbed score and output), section 4
    (online-softmax state and log-sum-exp, kept for the backward pass),
    section 5 (KV-cache byte formula).
  * "Attention, Worked Out by Hand (Part 2)", section 2 (the backward pass
    recomputes the scores).
  * "Attention deep dive (MHA -> MQA -> GQA -> FlashAttention)", section 5
    (decode against the cache) and section 6 (sliding-window mask).
  * "2.4 Multi-Head Attention, MQA, GQA & MLA", "Implementing the MHA -> GQA
    conversion" (query head j reads KV group j // n_rep).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "libattn_oracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (fp64, no fast-math, OpenMP)."""
    os.makedirs(_BUILD_DIR, exist_ok=True)
    if force or not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    D = ctypes.c_double
    lib.oracle_prefill.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, D, P, I, P]
    lib.oracle_prefill.restype = I
    lib.oracle_prefill_backward.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, D, P, P]
    lib.oracle_prefill_backward.restype = I
    lib.oracle_decode.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, D, P]
    lib.oracle_decode.restype = I
    lib.oracle_mla_decode.argtypes = [P, P, P, P, P, I, I, I, I, I, D, P]
    lib.oracle_mla_decode.restype = I
    lib.oracle_fp8_e4m3_value.argtypes = [I]
    lib.oracle_fp8_e4m3_value.restype = D
    lib.oracle_fp8_e4m3_encode.argtypes = [ctypes.c_float]
    lib.oracle_fp8_e4m3_encode.restype = I
    lib.oracle_quantize_kv_fp8.argtypes = [P, P, P, I, I, I, I]
    lib.oracle_quantize_kv_fp8.restype = I
    lib.oracle_decode_fp8.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, D, P]
    lib.oracle_decode_fp8.restype = I
    lib.oracle_mla_decode_fp8.argtypes = [P, P, P, P, P, P, I, I, I, I, I, D, P, I, I]
    lib.oracle_mla_decode_fp8.restype = I
    lib.oracle_prefill_fp8.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, D, P, I, P, I]
    lib.oracle_prefill_fp8.restype = I
    lib.oracle_rope.argtypes = [P, P, P, I, I, I, I, I, I, D]
    lib.oracle_rope.restype = I
    lib.oracle_merge_partials.argtypes = [P, P, I, I, P, P]
    lib.oracle_merge_partials.restype = None
    lib.oracle_set_threads.argtypes = [I]
    lib.oracle_set_threads.restype = None
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = I
    _lib = lib
    return lib


def _f32(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != np.float32:
        a = a.astype(np.float32)
    return np.ascontiguousarray(a)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _sinks(sinks, hq):
    if sinks is None:
        return None, None
    a = _f32(sinks).reshape(-1)
    assert a.shape == (hq,)
    return a, _ptr(a)


def prefill(q, k, v, *, causal: bool, window: int = 0, scale: float,
            rows=None, sinks=None):
    """Exact attention forward.

    q:[B,hq,T,d]  k,v:[B,hkv,T,d].  ``rows`` optionally lists the query
    positions to evaluate (all T when None); ``sinks`` optionally gives one
    sink logit per query head (an extra softmax-denominator term, in the
    units of the scaled scores).  Returns (o, lse): o:[B,hq,n_rows,d]
    float64, lse:[B,hq,n_rows] float64 (natural log).
    """
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, hq, T, d = q.shape
    hkv = k.shape[1]
    assert k.shape == (B, hkv, T, d) and v.shape == k.shape
    if rows is None:
        rows_arr, n_rows, rows_ptr = None, T, None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
        assert rows_arr.ndim == 1 and (rows_arr.size == 0 or (
            rows_arr.min() >= 0 and rows_arr.max() < T))
        n_rows, rows_ptr = int(rows_arr.size), _ptr(rows_arr)
    o = np.zeros((B, hq, n_rows, d), dtype=np.float64)
    lse = np.zeros((B, hq, n_rows), dtype=np.float64)
    sk, sk_ptr = _sinks(sinks, hq)
    rc = _load().oracle_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                B, T, hq, hkv, d, int(bool(causal)),
                                int(window), float(scale), rows_ptr, n_rows, sk_ptr)
    if rc != 0:
        raise ValueError("oracle_prefill: invalid shape")
    return o, lse


def prefill_backward(q, k, v, dout, *, causal: bool, window: int = 0, scale: float,
                     sinks=None, return_dsinks: bool = False):
    """Gradients of the exact attention forward with respect to q, k, v for
    the output gradient ``dout``.  q, dout:[B,hq,T,d]  k,v:[B,hkv,T,d].
    Returns (dq, dk, dv) float64, shaped like q, k, v; dk and dv sum over the
    query heads of each K/V group.  With ``return_dsinks`` (needs ``sinks``)
    the gradient of the sink logits, [hq] float64, is appended."""
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    B, hq, T, d = q.shape
    hkv = k.shape[1]
    assert k.shape == (B, hkv, T, d) and v.shape == k.shape and dout.shape == q.shape
    dq = np.zeros((B, hq, T, d), dtype=np.float64)
    dk = np.zeros((B, hkv, T, d), dtype=np.float64)
    dv = np.zeros((B, hkv, T, d), dtype=np.float64)
    sk, sk_ptr = _sinks(sinks, hq)
    assert sinks is not None or not return_dsinks
    ds = np.zeros(hq, dtype=np.float64)
    rc = _load().oracle_prefill_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                                         _ptr(dq), _ptr(dk), _ptr(dv), B, T, hq, hkv, d,
                                         int(bool(causal)), int(window), float(scale), sk_ptr,
                                         _ptr(ds) if return_dsinks else None)
    if rc != 0:
        raise ValueError("oracle_prefill_backward: invalid shape")
    return (dq, dk, dv, ds) if return_dsinks else (dq, dk, dv)


def decode(q, k_cache, v_cache, seq_lens, *, window: int = 0, scale: float, sinks=None):
    """Single-token decode.  q:[B,hq,d] (or [B,hq,1,d]),
    caches:[B,hkv,S_max,d], seq_lens:[B].  Returns (o:[B,hq,d], lse:[B,hq])."""
    q = _f32(q)
    if q.ndim == 4:
        q = np.ascontiguousarray(q[:, :, 0, :])
    kc, vc = _f32(k_cache), _f32(v_cache)
    B, hq, d = q.shape
    _, hkv, S_max, _ = kc.shape
    assert kc.shape == (B, hkv, S_max, d) and vc.shape == kc.shape
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    assert lens.shape == (B,)
    o = np.zeros((B, hq, d), dtype=np.float64)
    lse = np.zeros((B, hq), dtype=np.float64)
    sk, sk_ptr = _sinks(sinks, hq)
    rc = _load().oracle_decode(_ptr(q), _ptr(kc), _ptr(vc), _ptr(lens),
                               _ptr(o), _ptr(lse), B, S_max, hq, hkv, d,
                               int(window), float(scale), sk_ptr)
    if rc != 0:
        raise ValueError("oracle_decode: invalid shape")
    return o, lse


def mla_decode(q, cache, seq_lens, *, d_c: int, d_r: int, scale: float, sinks=None):
    """MLA absorbed decode.  q:[B,H,d_c+d_r]  cache:[B,S_max,d_c+d_r].
    Returns (o:[B,H,d_c], lse:[B,H])."""
    q, c = _f32(q), _f32(cache)
    B, H, dk = q.shape
    assert dk == d_c + d_r and c.shape[0] == B and c.shape[2] == dk
    S_max = c.shape[1]
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    assert lens.shape == (B,)
    o = np.zeros((B, H, d_c), dtype=np.float64)
    lse = np.zeros((B, H), dtype=np.float64)
    sk, sk_ptr = _sinks(sinks, H)
    rc = _load().oracle_mla_decode(_ptr(q), _ptr(c), _ptr(lens), _ptr(o),
                                   _ptr(lse), B, S_max, H, d_c, d_r,
                                   float(scale), sk_ptr)
    if rc != 0:
        raise ValueError("oracle_mla_decode: invalid shape")
    return o, lse


def gather_pages(pages, block_table, seq_lens, *, head_axis: bool):
    """Contiguous cache from a paged one: position t of sequence b is row
    t % page_size of page block_table[b, t // page_size].  pages is
    [num_pages, h_kv, page_size, d] (head_axis) or [num_pages, page_size, d];
    returns [B, h_kv, S_max, d] or [B, S_max, d] with S_max = max_blocks *
    page_size; positions at or past seq_lens[b] are left at zero."""
    pages = np.asarray(pages)
    bt = np.asarray(block_table)
    lens = np.asarray(seq_lens)
    B, max_blocks = bt.shape
    ps = pages.shape[2] if head_axis else pages.shape[1]
    S_max = max_blocks * ps
    if head_axis:
        out = np.zeros((B, pages.shape[1], S_max, pages.shape[3]), dtype=pages.dtype)
    else:
        out = np.zeros((B, S_max, pages.shape[2]), dtype=pages.dtype)
    for b in range(B):
        n = int(min(max(int(lens[b]), 0), S_max))
        for t0 in range(0, n, ps):
            pg = int(bt[b, t0 // ps])
            m = min(ps, n - t0)
            if head_axis:
                out[b, :, t0:t0 + m] = pages[pg, :, :m]
            else:
                out[b, t0:t0 + m] = pages[pg, :m]
    return out


def decode_paged(q, k_pages, v_pages, block_table, seq_lens, *, window: int = 0, scale: float):
    """attn decode on a paged cache: the contiguous decode of the gathered cache."""
    kc = gather_pages(_f32(k_pages), block_table, seq_lens, head_axis=True)
    vc = gather_pages(_f32(v_pages), block_table, seq_lens, head_axis=True)
    return decode(q, kc, vc, seq_lens, window=window, scale=scale)


def mla_decode_paged(q, kv_pages, block_table, seq_lens, *, d_c: int, d_r: int, scale: float):
    """MLA decode on a paged cache: the contiguous MLA decode of the gathered cache."""
    c = gather_pages(_f32(kv_pages), block_table, seq_lens, head_axis=False)
    return mla_decode(q, c, seq_lens, d_c=d_c, d_r=d_r, scale=scale)


def fp8_e4m3_value(code: int) -> float:
    """Value of an OCP FP8 E4M3 code (NaN for 0x7f / 0xff)."""
    return float(_load().oracle_fp8_e4m3_value(int(code)))


def fp8_e4m3_encode(v: float) -> int:
    """Nearest E4M3 code to the float32 value v (ties to even, saturating);
    NaN and +-infinity give the NaN code 0x7f / 0xff with v's sign."""
    return int(_load().oracle_fp8_e4m3_encode(float(np.float32(v))))


def fp8_dequantize(codes, scales, *, tile: int = 32) -> np.ndarray:
    """codes:[..., S, d] uint8, scales:[..., ceil(S/tile)] -> float64 values."""
    codes = np.asarray(codes, dtype=np.uint8)
    table = np.array([fp8_e4m3_value(c) for c in range(256)], dtype=np.float64)
    sc = np.repeat(np.asarray(scales, dtype=np.float64), tile, axis=-1)[..., :codes.shape[-2]]
    return table[codes] * sc[..., None]


def quantize_kv_fp8(x):
    """Per-tile FP8 quantisation of a cache x:[B, h_kv, S, d]: 32 positions of
    one head per tile, scale = amax / 448 with amax over the tile's finite
    values; NaN and +-infinity are stored as the NaN code with their sign.
    Returns (codes uint8 like x, scales float32 [B, h_kv, ceil(S/32)])."""
    x = _f32(x)
    B, hkv, S, d = x.shape
    codes = np.zeros(x.shape, dtype=np.uint8)
    scales = np.zeros((B, hkv, (S + 31) // 32), dtype=np.float32)
    rc = _load().oracle_quantize_kv_fp8(_ptr(x), _ptr(codes), _ptr(scales), B, hkv, S, d)
    if rc != 0:
        raise ValueError("oracle_quantize_kv_fp8: invalid shape")
    return codes, scales


def decode_fp8(q, k8, v8, k_scales, v_scales, seq_lens, *, window: int = 0, scale: float,
               sinks=None):
    """Decode against an FP8 cache (codes [B,h_kv,S_max,d], per-tile scales
    [B,h_kv,ceil(S_max/32)]): the plain decode of the dequantised cache."""
    q = _f32(q)
    B, hq = q.shape[0], q.shape[1]
    d = q.shape[-1]
    k8 = np.ascontiguousarray(np.asarray(k8, dtype=np.uint8))
    v8 = np.ascontiguousarray(np.asarray(v8, dtype=np.uint8))
    _, hkv, S_max, d2 = k8.shape
    assert d2 == d and v8.shape == k8.shape
    ks, vs = _f32(k_scales), _f32(v_scales)
    assert ks.shape == (B, hkv, (S_max + 31) // 32) and vs.shape == ks.shape
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    o = np.zeros((B, hq, d), dtype=np.float64)
    lse = np.zeros((B, hq), dtype=np.float64)
    sk, sk_ptr = _sinks(sinks, hq)
    rc = _load().oracle_decode_fp8(_ptr(np.ascontiguousarray(q.reshape(B, hq, d))), _ptr(k8),
                                   _ptr(v8), _ptr(ks), _ptr(vs), _ptr(lens), _ptr(o), _ptr(lse),
                                   B, S_max, hq, hkv, d, int(window), float(scale), sk_ptr)
    if rc != 0:
        raise ValueError("oracle_decode_fp8: invalid shape")
    return o, lse


def mla_decode_fp8(q, codes, scales, seq_lens, *, d_c: int, d_r: int, scale: float,
                   split: int, tile: int = 64, sinks=None):
    """MLA absorbed decode with FP8 attention (the pages' FA3 FP8 recipe):
    the query quantised per head (amax / 448), the cache given as E4M3 codes
    [B, S_max, d_c+d_r] with one scale per 32 tokens [B, ceil(S_max/32)],
    both products on the dequantised codes, the probabilities quantised to
    E4M3 against each chunk's reference (chunks of ``split`` tokens, compute
    tiles of ``tile`` tokens; the reference moves to a tile's max plus 5, in
    log2 units, when the tile exceeds it) with the value scale folded in, the
    denominator from the unquantised probabilities.  Returns (o:[B,H,d_c],
    lse:[B,H])."""
    q = _f32(q)
    B, H, dk = q.shape
    codes = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    assert dk == d_c + d_r and codes.shape[0] == B and codes.shape[2] == dk
    S_max = codes.shape[1]
    sc = _f32(scales).reshape(B, -1)
    assert sc.shape[1] == (S_max + 31) // 32
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    assert lens.shape == (B,)
    o = np.zeros((B, H, d_c), dtype=np.float64)
    lse = np.zeros((B, H), dtype=np.float64)
    sk, sk_ptr = _sinks(sinks, H)
    rc = _load().oracle_mla_decode_fp8(_ptr(q), _ptr(codes), _ptr(sc), _ptr(lens), _ptr(o),
                                       _ptr(lse), B, S_max, H, d_c, d_r, float(scale), sk_ptr,
                                       int(split), int(tile))
    if rc != 0:
        raise ValueError("oracle_mla_decode_fp8: invalid shape")
    return o, lse


def prefill_fp8(q8, q_scales, k8, k_scales, v8, v_scales, *, causal: bool, window: int = 0,
                scale: float, tile: int = 64, sinks=None, rows=None):
    """Prefill with FP8 attention (the pages' FA3 FP8 recipe): q, k, v as
    E4M3 codes [B,h,T,d] with one scale per 32 positions of a head
    [B,h,ceil(T/32)] (the cache quantiser's layout), both products on the
    dequantised codes, each row's probabilities quantised to E4M3 against
    its reference (keys in ``tile``-aligned tiles; the reference moves to a
    tile's max plus 5, log2 units, when the tile exceeds it) with the value
    scale folded in, the denominator from the unquantised probabilities.
    ``rows`` optionally lists the query positions to evaluate.  Returns
    (o:[B,hq,n_rows,d], lse:[B,hq,n_rows])."""
    q8 = np.ascontiguousarray(np.asarray(q8, dtype=np.uint8))
    k8 = np.ascontiguousarray(np.asarray(k8, dtype=np.uint8))
    v8 = np.ascontiguousarray(np.asarray(v8, dtype=np.uint8))
    B, hq, T, d = q8.shape
    hkv = k8.shape[1]
    assert k8.shape == (B, hkv, T, d) and v8.shape == k8.shape
    nt = (T + 31) // 32
    qs, ks, vs = (_f32(x).reshape(-1) for x in (q_scales, k_scales, v_scales))
    assert qs.size == B * hq * nt and ks.size == B * hkv * nt and vs.size == ks.size
    if rows is None:
        rows_arr, n_rows, rows_ptr = None, T, None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
        assert rows_arr.ndim == 1 and (rows_arr.size == 0 or (
            rows_arr.min() >= 0 and rows_arr.max() < T))
        n_rows, rows_ptr = int(rows_arr.size), _ptr(rows_arr)
    o = np.zeros((B, hq, n_rows, d), dtype=np.float64)
    lse = np.zeros((B, hq, n_rows), dtype=np.float64)
    sk, sk_ptr = _sinks(sinks, hq)
    rc = _load().oracle_prefill_fp8(_ptr(q8), _ptr(qs), _ptr(k8), _ptr(ks), _ptr(v8), _ptr(vs),
                                    _ptr(o), _ptr(lse), B, T, hq, hkv, d, int(bool(causal)),
                                    int(window), float(scale), sk_ptr, int(tile), rows_ptr,
                                    n_rows)
    if rc != 0:
        raise ValueError("oracle_prefill_fp8: invalid shape")
    return o, lse


def decode_paged_fp8(q, k8_pages, v8_pages, k_scale_pages, v_scale_pages, block_table, seq_lens,
                     *, window: int = 0, scale: float, sinks=None):
    """FP8 decode on a paged cache: codes [num_pages, h_kv, page_size, d], scales
    [num_pages, h_kv, page_size / 32]; gathered, then decode_fp8."""
    ps = np.asarray(k8_pages).shape[2]
    lens = np.asarray(seq_lens)
    k8 = gather_pages(k8_pages, block_table, lens, head_axis=True)
    v8 = gather_pages(v8_pages, block_table, lens, head_axis=True)
    lens_t = (np.maximum(lens, 0) + 31) // 32
    ks = gather_pages(_f32(k_scale_pages)[..., None], block_table, lens_t, head_axis=True)[..., 0]
    vs = gather_pages(_f32(v_scale_pages)[..., None], block_table, lens_t, head_axis=True)[..., 0]
    assert ks.shape[2] * 32 == k8.shape[2] and ps % 32 == 0
    return decode_fp8(q, k8, v8, ks, vs, lens, window=window, scale=scale, sinks=sinks)


def rope(x, *, positions=None, base: float, rope_offset: int = 0, rope_dim=None):
    """Rotary position embedding of x:[B, H, T, row] (dimensions [rope_offset,
    rope_offset + rope_dim) in interleaved pairs, theta_j = base^(-2j/rope_dim),
    angle = position * theta_j); positions:[B, T] ints, default t.  float64."""
    x = _f32(x)
    B, H, T, row = x.shape
    rd = row - rope_offset if rope_dim is None else rope_dim
    out = np.zeros(x.shape, dtype=np.float64)
    pos = None if positions is None else np.ascontiguousarray(np.asarray(positions, dtype=np.int32))
    if pos is not None:
        assert pos.shape == (B, T)
    rc = _load().oracle_rope(_ptr(x), None if pos is None else _ptr(pos), _ptr(out), B, H, T, row,
                             int(rope_offset), int(rd), float(base))
    if rc != 0:
        raise ValueError("oracle_rope: invalid arguments")
    return out


def merge_partials(parts_o, parts_lse):
    """Merge normalised partial results over disjoint key sets.
    parts_o:[n,dv] parts_lse:[n] -> (o:[dv], lse)."""
    po = np.ascontiguousarray(np.asarray(parts_o, dtype=np.float64))
    pl = np.ascontiguousarray(np.asarray(parts_lse, dtype=np.float64))
    n, dv = po.shape
    assert pl.shape == (n,)
    o = np.zeros(dv, dtype=np.float64)
    lse = np.zeros(1, dtype=np.float64)
    _load().oracle_merge_partials(_ptr(po), _ptr(pl), n, dv, _ptr(o), _ptr(lse))
    return o, float(lse[0])


def kv_cache_bytes(B: int, S: int, L: int, n_kv: int, d_h: int,
                   b_bytes: int) -> int:
    """KV-cache footprint M_KV = 2 * B * S * L * (n_kv * d_h) * b_bytes
    ("Attention Engineering ...", section 0, equation "KV-Cache Memory
    Footprint & Arithmetic Intensity")."""
    return 2 * B * S * L * (n_kv * d_h) * b_bytes


def mla_cache_bytes(B: int, S: int, L: int, d_c: int, d_r: int,
                    b_bytes: int) -> int:
    """MLA cache: d_c + d_R scalars per token per layer ("Attention
    Engineering ...", section 3, text after the complete MLA score)."""
    return B * S * L * (d_c + d_r) * b_bytes
