"""Every output of the full-size workloads against the fp64 oracle.

The kernels run once per workload at full size, in the launch configuration
bench.py times (the workloads' seeded inputs, the library's default split,
tiling and workspace); the oracle then recomputes every output row, in
chunks that each finish in seconds:
  * Llama-3-8B causal GQA prefill (B=1, T=8192, 32/8 heads): all 8192 rows of
    every head, one K/V group (4 query heads) per test;
  * sliding-window prefill (B=4, T=4096, 32 query heads, W=1024) with 32 and
    with 1 K/V head: all rows of every head, one batch entry per test;
  * 70B-shaped GQA decode (B=64, 64/8 heads, S_max=32768): all 64 sequences,
    16 per test, on the bf16 cache and on a synthetic FP8 cache; the paged
    layouts (pages of 64 positions in random order) are bit-identical to the
    contiguous results, which the oracle checks in full;
  * DeepSeek-V3-shaped MLA decode (B=32, 128 heads, 16384 tokens): all 32
    sequences, 8 per test; the paged layout bit-identical to the contiguous;
  * the Llama-3-8B prefill backward: dQ, dK and dV of every K/V group, one
    group per test.
Bars: bf16 max-abs 2e-2 and relative Frobenius 1e-2 (backward: max-abs
2e-2 x max(1, max |reference|)); log-sum-exp 2e-2 absolute.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests.parity import (BF16_MAX_ABS, BF16_REL_FRO, LSE_BF16_ABS, assert_bf16_close,
                          assert_lse_close, errors, np32)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ta():
    import transformer_attention_amd as m
    m.load_library()
    assert torch.cuda.is_available()
    return m


@pytest.fixture(scope="module", autouse=True)
def _release_device_buffers():
    """The workloads' device buffers live for this module only."""
    yield
    for st in (_prefill_cache, _decode_state, _fp8_state, _mla_state, _bwd_state):
        st.clear()
    torch.cuda.empty_cache()


def _report(what, got, ref):
    max_abs, rel = errors(got, ref)
    print(f"  {what}: max_abs={max_abs:.3e} rel_fro={rel:.3e}", flush=True)


# ---------------------------------------------------------------- prefill ---

_PREFILL = {"llama3-8b": W.LLAMA3_8B_PREFILL, "swa-mha": W.SWA_MHA, "swa-mqa": W.SWA_MQA}
_prefill_cache = {}


def _prefill_run(ta, name):
    """Inputs and the kernel's outputs of one workload, as host float32."""
    if name not in _prefill_cache:
        _prefill_cache.clear()
        s = _PREFILL[name]
        q, k, v = W.prefill_inputs(s, seed=0, device="cuda", gen_device="cuda")
        print(f"[case] full-size prefill {name} {tuple(q.shape)} hkv={s.h_kv}", flush=True)
        o, lse = ta.attn_prefill(q, k, v, causal=s.causal, window=s.window, scale=s.scale,
                                 return_lse=True)
        torch.cuda.synchronize()
        assert torch.isfinite(o).all()
        _prefill_cache[name] = tuple(np32(t) for t in (q, k, v, o, lse))
        del q, k, v, o, lse
        torch.cuda.empty_cache()
    return _prefill_cache[name]


PREFILL_CHUNKS = ([("llama3-8b", g) for g in range(8)] + [("swa-mha", b) for b in range(4)] +
                  [("swa-mqa", b) for b in range(4)])


@pytest.mark.parametrize("name,chunk", PREFILL_CHUNKS, ids=[f"{n}-{c}" for n, c in PREFILL_CHUNKS])
def test_prefill_every_row(ta, oracle_mod, name, chunk):
    s = _PREFILL[name]
    q, k, v, o, lse = _prefill_run(ta, name)
    G = s.h_q // s.h_kv
    if name == "llama3-8b":                 # one K/V group: its G query heads, all rows
        b, hs, gs = slice(0, 1), slice(chunk * G, (chunk + 1) * G), slice(chunk, chunk + 1)
    else:                                   # one batch entry, every head, all rows
        b, hs, gs = slice(chunk, chunk + 1), slice(None), slice(None)
    print(f"[case] {name} chunk {chunk}: oracle on {q[b, hs].shape}", flush=True)
    ro, rl = oracle_mod.prefill(q[b, hs], k[b, gs], v[b, gs], causal=s.causal, window=s.window,
                                scale=s.scale)
    _report(f"{name} chunk {chunk} O", o[b, hs], ro)
    assert_bf16_close(o[b, hs], ro, f"{name} chunk {chunk}")
    assert_lse_close(lse[b, hs], rl, LSE_BF16_ABS, f"{name} chunk {chunk} LSE")


# ----------------------------------------------------------------- decode ---

_decode_state = {}


def _decode_run(ta):
    if "o" not in _decode_state:
        s = W.GQA70B_DECODE
        q, kc, vc, lens = W.decode_inputs(s, seed=0, device="cuda", gen_device="cuda")
        print(f"[case] full-size decode {tuple(kc.shape)} sum(len)={int(lens.sum())}", flush=True)
        o, lse = ta.attn_decode(q, kc, vc, lens.cuda(), scale=s.scale, return_lse=True)
        torch.cuda.synchronize()
        _decode_state.update(q=q, kc=kc, vc=vc, lens=lens, o=o, lse=lse)
    return _decode_state


@pytest.mark.parametrize("chunk", range(4))
def test_decode_every_sequence(ta, oracle_mod, chunk):
    st = _decode_run(ta)
    s = W.GQA70B_DECODE
    lens = st["lens"].tolist()
    for b in range(16 * chunk, 16 * chunk + 16):
        n = lens[b]
        ro, rl = oracle_mod.decode(np32(st["q"][b:b + 1]), np32(st["kc"][b:b + 1, :, :n]),
                                   np32(st["vc"][b:b + 1, :, :n]), [n], scale=s.scale)
        got = np32(st["o"][b:b + 1])[:, :, 0]
        assert_bf16_close(got, ro, f"decode b={b} len={n}")
        assert_lse_close(np32(st["lse"][b:b + 1]), rl, LSE_BF16_ABS, f"decode lse b={b}")
    print(f"  decode sequences {16 * chunk}..{16 * chunk + 15} ok", flush=True)


def test_paged_decode_is_the_contiguous_decode(ta):
    """Pages of 64 positions in a seeded random order, the bench's paged
    layout: bit-identical to the contiguous result checked above."""
    st = _decode_run(ta)
    s = W.GQA70B_DECODE
    kp, table = W.paged_layout(st["kc"], 64, seed=9, fill=0.0)
    vp = torch.empty_like(kp)
    vp[table.view(-1).long()] = st["vc"].view(s.B, s.h_kv, s.S_max // 64, 64, s.d_h).permute(
        0, 2, 1, 3, 4).reshape(-1, s.h_kv, 64, s.d_h)
    print("[case] full-size paged decode", flush=True)
    o, lse = ta.attn_decode_paged(st["q"], kp, vp, st["lens"].cuda(), table, scale=s.scale,
                                  return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o, st["o"])
    assert torch.equal(lse, st["lse"])


_fp8_state = {}


def _fp8_run(ta):
    if "o" not in _fp8_state:
        s = W.GQA70B_DECODE
        g = torch.Generator().manual_seed(450)
        q = torch.randn(s.B, s.h_q, 1, s.d_h, generator=g).to(torch.bfloat16).cuda()
        lens = W.seq_lengths(s.B, s.len_lo, s.len_hi, seed=0)
        shape = (s.B, s.h_kv, s.S_max, s.d_h)
        k8, ks = W.random_fp8_cache(shape, seed=1, device="cuda")
        v8, vs = W.random_fp8_cache(shape, seed=2, device="cuda")
        print("[case] full-size fp8 decode", flush=True)
        o, lse = ta.attn_decode_fp8(q, k8, v8, ks, vs, lens.cuda(), scale=s.scale,
                                    return_lse=True)
        torch.cuda.synchronize()
        _fp8_state.update(q=q, k8=k8, v8=v8, ks=ks, vs=vs, lens=lens, o=o, lse=lse)
    return _fp8_state


@pytest.mark.parametrize("chunk", range(4))
def test_fp8_decode_every_sequence(ta, oracle_mod, chunk):
    """The 70B decode on a synthetic FP8 cache (random codes, power-of-two
    tile scales), every sequence against the oracle's FP8 decode."""
    st = _fp8_run(ta)
    s = W.GQA70B_DECODE
    lens = st["lens"].tolist()
    for b in range(16 * chunk, 16 * chunk + 16):
        n = lens[b]
        nt = (n + 31) // 32
        ro, rl = oracle_mod.decode_fp8(np32(st["q"][b:b + 1]), st["k8"][b:b + 1, :, :n].cpu().numpy(),
                                       st["v8"][b:b + 1, :, :n].cpu().numpy(),
                                       st["ks"][b:b + 1, :, :nt].cpu().numpy(),
                                       st["vs"][b:b + 1, :, :nt].cpu().numpy(), [n], scale=s.scale)
        assert_bf16_close(np32(st["o"][b:b + 1])[:, :, 0], ro, f"fp8 decode b={b} len={n}")
        assert_lse_close(np32(st["lse"][b:b + 1]), rl, LSE_BF16_ABS, f"fp8 lse b={b}")
    print(f"  fp8 decode sequences {16 * chunk}..{16 * chunk + 15} ok", flush=True)


def test_paged_fp8_decode_is_the_contiguous_fp8_decode(ta):
    st = _fp8_run(ta)
    s = W.GQA70B_DECODE
    ps = 64
    k8p, table = W.paged_layout(st["k8"], ps, seed=9, fill=0)
    perm = table.view(-1).long()
    v8p = torch.empty_like(k8p)
    v8p[perm] = st["v8"].view(s.B, s.h_kv, s.S_max // ps, ps, s.d_h).permute(
        0, 2, 1, 3, 4).reshape(-1, s.h_kv, ps, s.d_h)
    nsp = ps // 32

    def scale_pages(sc):
        out = torch.empty((k8p.shape[0], s.h_kv, nsp), dtype=torch.float32, device="cuda")
        out[perm] = sc.view(s.B, s.h_kv, s.S_max // ps, nsp).permute(0, 2, 1, 3).reshape(
            -1, s.h_kv, nsp)
        return out

    print("[case] full-size paged fp8 decode", flush=True)
    o, lse = ta.attn_decode_paged_fp8(st["q"], k8p, v8p, scale_pages(st["ks"]),
                                      scale_pages(st["vs"]), st["lens"].cuda(), table,
                                      scale=s.scale, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o, st["o"])
    assert torch.equal(lse, st["lse"])


def test_quantiser_one_head_of_every_sequence(ta, oracle_mod):
    """The bench's FP8 cache writer on the 70B workload's bf16 K cache:
    bit-exact with the oracle's quantiser on one K/V head of every sequence
    (rotating over the heads), 268 M values."""
    st = _decode_run(ta)
    s = W.GQA70B_DECODE
    print("[case] full-size quantiser", flush=True)
    codes, scales = ta.attn_quantize_kv_fp8(st["kc"])
    torch.cuda.synchronize()
    for b in range(s.B):
        g = b % s.h_kv
        rc, rs = oracle_mod.quantize_kv_fp8(np32(st["kc"][b:b + 1, g:g + 1]))
        assert np.array_equal(codes[b:b + 1, g:g + 1].cpu().numpy(), rc), f"codes b={b} g={g}"
        assert np.array_equal(scales[b:b + 1, g:g + 1].cpu().numpy(), rs), f"scales b={b} g={g}"
    del codes, scales


# -------------------------------------------------------------------- MLA ---

_mla_state = {}


def _mla_run(ta):
    if "o" not in _mla_state:
        s = W.DSV3_MLA_DECODE
        q, c, lens = W.mla_inputs(s, seed=0, device="cuda", gen_device="cuda")
        print(f"[case] full-size mla {tuple(c.shape)}", flush=True)
        o, lse = ta.mla_decode(q, c, lens.cuda(), scale=s.scale, return_lse=True)
        torch.cuda.synchronize()
        _mla_state.update(q=q, c=c, lens=lens, o=o, lse=lse)
    return _mla_state


@pytest.mark.parametrize("chunk", range(4))
def test_mla_every_sequence(ta, oracle_mod, chunk):
    st = _mla_run(ta)
    s = W.DSV3_MLA_DECODE
    lens = st["lens"].tolist()
    for b in range(8 * chunk, 8 * chunk + 8):
        n = lens[b]
        ro, rl = oracle_mod.mla_decode(np32(st["q"][b:b + 1]), np32(st["c"][b:b + 1, :n]), [n],
                                       d_c=s.d_c, d_r=s.d_r, scale=s.scale)
        assert_bf16_close(np32(st["o"][b:b + 1]), ro, f"mla b={b}")
        assert_lse_close(np32(st["lse"][b:b + 1]), rl, LSE_BF16_ABS, f"mla lse b={b}")
    print(f"  mla sequences {8 * chunk}..{8 * chunk + 7} ok", flush=True)


def test_paged_mla_is_the_contiguous_mla(ta):
    st = _mla_run(ta)
    s = W.DSV3_MLA_DECODE
    pages, table = W.paged_layout(st["c"], 64, seed=11, head_axis=False, fill=0.0)
    print("[case] full-size paged mla", flush=True)
    o, lse = ta.mla_decode_paged(st["q"], pages, st["lens"].cuda(), table, scale=s.scale,
                                 return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o, st["o"])
    assert torch.equal(lse, st["lse"])


# --------------------------------------------------------------- backward ---

_bwd_state = {}


def _bwd_run(ta):
    if "dq" not in _bwd_state:
        s = W.LLAMA3_8B_PREFILL
        q, k, v = W.prefill_inputs(s, seed=0, device="cuda", gen_device="cuda")
        g = torch.Generator(device="cuda").manual_seed(1)
        do = torch.randn(q.shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        print(f"[case] full-size backward {tuple(q.shape)}", flush=True)
        o, lse = ta.attn_prefill(q, k, v, causal=True, scale=s.scale, return_lse=True)
        dq, dk, dv = ta.attn_prefill_backward(q, k, v, o, do, lse, causal=True, scale=s.scale)
        torch.cuda.synchronize()
        _bwd_state.update({n: np32(t) for n, t in
                           (("q", q), ("k", k), ("v", v), ("do", do), ("dq", dq), ("dk", dk),
                            ("dv", dv))})
        del q, k, v, do, o, lse, dq, dk, dv
        torch.cuda.empty_cache()
    return _bwd_state


def _check_grad(got, ref, what):
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    max_abs, rel = errors(got, ref)
    bound = BF16_MAX_ABS * max(1.0, float(np.abs(ref).max()))
    print(f"  {what}: max_abs={max_abs:.3e} (bound {bound:.3e}) rel_fro={rel:.3e}", flush=True)
    assert rel <= BF16_REL_FRO and max_abs <= bound, f"{what}: max_abs={max_abs:.3e} rel={rel:.3e}"


@pytest.mark.parametrize("group", range(8))
def test_backward_every_group(ta, oracle_mod, group):
    st = _bwd_run(ta)
    s = W.LLAMA3_8B_PREFILL
    G = s.h_q // s.h_kv
    hs, gs = slice(group * G, (group + 1) * G), slice(group, group + 1)
    print(f"[case] backward group {group}", flush=True)
    rq, rk, rv = oracle_mod.prefill_backward(st["q"][:, hs], st["k"][:, gs], st["v"][:, gs],
                                             st["do"][:, hs], causal=True, scale=s.scale)
    _check_grad(st["dq"][:, hs], rq, f"dq group {group}")
    _check_grad(st["dk"][:, gs], rk, f"dk group {group}")
    _check_grad(st["dv"][:, gs], rv, f"dv group {group}")
