"""Seeded synthetic workloads for attention (shapes and input generators only).

This module holds no attention arithmetic.  It defines the five workload
shapes and draws their inputs: i.i.d. standard-normal values drawn in fp32
and rounded to bf16 (round-to-nearest-even, torch's ``.to``) where the
workload is bf16, and per-sequence cache lengths drawn uniformly.  Both the
tests and the benchmark take their inputs from here, and so do the CPU oracle
and the HIP path, so a parity check always compares the two on the same bits.

Generation order (one ``torch.Generator`` per call, seeded):
  prefill: Q, then K, then V;
  decode:  lengths (CPU generator), then q, K cache, V cache;
  MLA:     lengths (CPU generator), then q, then the latent cache.
Large tensors can be drawn directly on the GPU with a generator of that
device; small ones are drawn on the CPU and copied.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class PrefillShape:
    name: str
    B: int
    T: int
    h_q: int
    h_kv: int
    d_h: int
    dtype: torch.dtype
    causal: bool = True
    window: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d_h)


@dataclass(frozen=True)
class DecodeShape:
    name: str
    B: int
    S_max: int
    h_q: int
    h_kv: int
    d_h: int
    len_lo: int
    len_hi: int          # inclusive
    window: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d_h)


@dataclass(frozen=True)
class MlaShape:
    name: str
    B: int
    S_max: int
    H: int
    d_c: int
    d_r: int
    d_h_nope: int        # per-head content width whose sum with d_r sets the scale
    len_lo: int
    len_hi: int          # inclusive

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d_h_nope + self.d_r)


# The five workloads the kernels are built and measured for.
TINY_FP32 = PrefillShape("tiny causal GQA prefill fp32", B=1, T=64, h_q=4,
                         h_kv=2, d_h=16, dtype=torch.float32)
LLAMA3_8B_PREFILL = PrefillShape("Llama-3-8B causal GQA prefill", B=1, T=8192,
                                 h_q=32, h_kv=8, d_h=128, dtype=torch.bfloat16)
SWA_MHA = PrefillShape("sliding-window MHA prefill", B=4, T=4096, h_q=32,
                       h_kv=32, d_h=128, dtype=torch.bfloat16, window=1024)
SWA_MQA = PrefillShape("sliding-window MQA prefill", B=4, T=4096, h_q=32,
                       h_kv=1, d_h=128, dtype=torch.bfloat16, window=1024)
GQA70B_DECODE = DecodeShape("70B GQA decode", B=64, S_max=32768, h_q=64,
                            h_kv=8, d_h=128, len_lo=4096, len_hi=32768)
DSV3_MLA_DECODE = MlaShape("DeepSeek-V3 MLA absorbed decode", B=32,
                           S_max=16384, H=128, d_c=512, d_r=64, d_h_nope=128,
                           len_lo=16384, len_hi=16384)

ALL_PREFILL = (TINY_FP32, LLAMA3_8B_PREFILL, SWA_MHA, SWA_MQA)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def randn(shape, dtype, *, generator, device) -> torch.Tensor:
    """Standard-normal fp32 draw, then rounded to ``dtype``."""
    x = torch.randn(shape, generator=generator, device=device,
                    dtype=torch.float32)
    return x if dtype == torch.float32 else x.to(dtype)


def prefill_inputs(shape: PrefillShape, *, seed: int = 0, device="cpu",
                   gen_device=None, B=None, T=None):
    """Q:[B,h_q,T,d]  K,V:[B,h_kv,T,d], drawn in the order Q, K, V.
    ``B``/``T`` override the workload's batch and length (smaller parity
    cases with the same head layout)."""
    B = shape.B if B is None else B
    T = shape.T if T is None else T
    gd = device if gen_device is None else gen_device
    g = _gen(seed, gd)
    q = randn((B, shape.h_q, T, shape.d_h), shape.dtype, generator=g, device=gd)
    k = randn((B, shape.h_kv, T, shape.d_h), shape.dtype, generator=g, device=gd)
    v = randn((B, shape.h_kv, T, shape.d_h), shape.dtype, generator=g, device=gd)
    return q.to(device), k.to(device), v.to(device)


def random_fp8_cache(shape, *, seed: int, device="cpu", tile: int = 32):
    """A synthetic FP8 (E4M3) cache: random one-byte codes of both signs with
    exponent fields 3..10 and any mantissa (so never the NaN code), and one
    random power-of-two scale per `tile` positions, 2^-8 .. 2^-5.  The
    dequantised values then span about 2^-12 .. 2^-1.  shape = [..., S, d];
    generated on `device`; returns (codes uint8, scales float32
    [..., ceil(S / tile)])."""
    g = _gen(seed, device)
    r = torch.randint(0, 256, shape, generator=g, dtype=torch.uint8, device=device)
    codes = (r & 0x87) | ((((r >> 3) & 7) + 3) << 3)
    nt = (shape[-2] + tile - 1) // tile
    e = torch.randint(-8, -4, tuple(shape[:-2]) + (nt,), generator=g, dtype=torch.int32, device=device)
    scales = torch.pow(2.0, e.to(torch.float32))
    return codes, scales


def seq_lengths(B: int, lo: int, hi: int, *, seed: int) -> torch.Tensor:
    """Per-sequence cache lengths, uniform on the integers [lo, hi]."""
    g = _gen(seed, "cpu")
    if lo == hi:
        return torch.full((B,), lo, dtype=torch.int32)
    return torch.randint(lo, hi + 1, (B,), generator=g,
                         dtype=torch.int64).to(torch.int32)


def decode_inputs(shape: DecodeShape, *, seed: int = 0, device="cpu",
                  gen_device=None, B=None, S_max=None, len_lo=None,
                  len_hi=None, dtype=torch.bfloat16):
    """q:[B,h_q,1,d]  K,V caches:[B,h_kv,S_max,d]  lens:int32[B]."""
    B = shape.B if B is None else B
    S_max = shape.S_max if S_max is None else S_max
    lo = shape.len_lo if len_lo is None else len_lo
    hi = shape.len_hi if len_hi is None else len_hi
    lens = seq_lengths(B, lo, hi, seed=seed)
    gd = device if gen_device is None else gen_device
    g = _gen(seed, gd)
    q = randn((B, shape.h_q, 1, shape.d_h), dtype, generator=g, device=gd)
    kc = randn((B, shape.h_kv, S_max, shape.d_h), dtype, generator=g, device=gd)
    vc = randn((B, shape.h_kv, S_max, shape.d_h), dtype, generator=g, device=gd)
    return q.to(device), kc.to(device), vc.to(device), lens.to(device)


def mla_inputs(shape: MlaShape, *, seed: int = 0, device="cpu",
               gen_device=None, B=None, S_max=None, len_lo=None, len_hi=None,
               H=None):
    """q:[B,H,d_c+d_r]  cache:[B,S_max,d_c+d_r]  lens:int32[B]."""
    B = shape.B if B is None else B
    H = shape.H if H is None else H
    S_max = shape.S_max if S_max is None else S_max
    lo = shape.len_lo if len_lo is None else len_lo
    hi = shape.len_hi if len_hi is None else len_hi
    lens = seq_lengths(B, min(lo, S_max), min(hi, S_max), seed=seed)
    gd = device if gen_device is None else gen_device
    g = _gen(seed, gd)
    dk = shape.d_c + shape.d_r
    q = randn((B, H, dk), torch.bfloat16, generator=g, device=gd)
    cache = randn((B, S_max, dk), torch.bfloat16, generator=g, device=gd)
    return q.to(device), cache.to(device), lens.to(device)


def paged_layout(cache: torch.Tensor, page_size: int, *, seed: int = 0, head_axis: bool = True,
                 extra_pages: int = 0, fill=float("nan")):
    """Lay a contiguous cache out in pages of `page_size` positions, in a
    seeded random page order, the way a paged allocator scatters them.

    cache: [B, h_kv, S, d] (head_axis) or [B, S, d], S a multiple of
    page_size.  Returns (pages, block_table): pages [num_pages, h_kv,
    page_size, d] or [num_pages, page_size, d] with num_pages = B * S /
    page_size + extra_pages (the extra pages and nothing else hold `fill`),
    block_table int32 [B, S / page_size] on the cache's device."""
    if head_axis:
        B, hkv, S, d = cache.shape
    else:
        B, S, d = cache.shape
    if S % page_size:
        raise ValueError("S must be a multiple of page_size")
    nb = S // page_size
    n_pages = B * nb + extra_pages
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(n_pages, generator=g)[:B * nb]
    if head_axis:
        blocks = cache.view(B, hkv, nb, page_size, d).permute(0, 2, 1, 3, 4).reshape(B * nb, hkv, page_size, d)
        pages = torch.full((n_pages, hkv, page_size, d), fill, dtype=cache.dtype, device=cache.device)
    else:
        blocks = cache.view(B * nb, page_size, d)
        pages = torch.full((n_pages, page_size, d), fill, dtype=cache.dtype, device=cache.device)
    pages[perm.to(cache.device)] = blocks
    table = perm.view(B, nb).to(torch.int32).to(cache.device)
    return pages, table
