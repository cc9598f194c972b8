"""The C-ABI library builds, loads and exports what include/*.h declares, and
its host-side validation rejects bad arguments before any launch (CPU only:
no call here reaches the GPU)."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                             text, flags=re.M):
            names.add(m.group(1))
    return names


@pytest.fixture(scope="module")
def lib():
    import transformer_attention_amd as ta
    return ta.load_library()


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("attn_prefill", "attn_prefill_backward", "attn_prefill_backward_workspace_size",
              "attn_decode", "mla_decode", "attn_decode_workspace_size",
              "attn_decode_paged", "attn_decode_paged_workspace_size", "mla_decode_paged",
              "mla_decode_paged_workspace_size", "attn_quantize_kv_fp8", "attn_decode_fp8",
              "attn_decode_paged_fp8", "attn_rope_qk", "attn_decode_noalloc",
              "mla_decode_workspace_size", "attn_status_string", "attn_abi_version"):
        assert n in names, n


def test_library_exports_every_declared_symbol(lib):
    for n in _declared_functions():
        assert hasattr(lib, n), f"symbol {n} declared in include/ but not exported"


def test_status_strings(lib):
    import transformer_attention_amd as ta
    assert ta.status_string(0) == "ok"
    for s in range(1, 5):
        assert ta.status_string(s) not in ("ok", "unknown status")
    assert lib.attn_abi_version() == 2


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def _prefill(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, T=16, hq=4, hkv=2, d=128,
             dtype=1, causal=1, window=0, scale=0.1)
    a.update(kw)
    return lib.attn_prefill(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["T"], a["hq"],
                            a["hkv"], a["d"], a["dtype"], a["causal"], a["window"], a["scale"], None,
                            None)


def test_prefill_validation(lib):
    assert _prefill(lib, q=None) == 1
    assert _prefill(lib, o=None) == 1
    assert _prefill(lib, B=0) == 1
    assert _prefill(lib, T=-1) == 1
    assert _prefill(lib, hq=6, hkv=4) == 1          # h_q must be a multiple of h_kv
    assert _prefill(lib, window=-1) == 1
    assert _prefill(lib, window=8, causal=0) == 1   # window needs causal
    assert _prefill(lib, scale=float("nan")) == 1
    assert _prefill(lib, scale=float("inf")) == 1
    assert _prefill(lib, scale=0.0) == 1
    assert _prefill(lib, scale=-0.5) == 1
    assert _prefill(lib, d=64) == 2                 # bf16 kernel is d = 128
    assert _prefill(lib, dtype=0, d=48) == 2        # fp32 d not instantiated
    assert _prefill(lib, dtype=7) == 2


def test_prefill_backward_validation(lib):
    def bwd(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
                 B=1, T=100, hq=4, hkv=2, d=128, dtype=1, causal=1, window=0, scale=0.1,
                 sinks=None, dsinks=None, ws=FAKE, wsb=1 << 30)
        a.update(kw)
        return lib.attn_prefill_backward(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"],
                                         a["dq"], a["dk"], a["dv"], a["B"], a["T"], a["hq"],
                                         a["hkv"], a["d"], a["dtype"], a["causal"], a["window"],
                                         a["scale"], a["sinks"], a["dsinks"], a["ws"], a["wsb"],
                                         None)
    assert bwd(lse=None) == 1
    assert bwd(dsinks=FAKE) == 1                    # a sink gradient needs the sinks
    assert bwd(dk=None) == 1
    assert bwd(T=0) == 1
    assert bwd(hq=6, hkv=4) == 1
    assert bwd(window=5, causal=0) == 1
    assert bwd(scale=0.0) == 1
    assert bwd(d=64) == 2
    assert bwd(dtype=0) == 2                        # backward is bf16 only
    assert bwd(ws=None) == 3
    need = lib.attn_prefill_backward_workspace_size(1, 100, 4)
    assert need >= 1 * 4 * 128 * 8                  # rows padded to 128, two floats each
    assert bwd(wsb=need - 1) == 3
    assert lib.attn_prefill_backward_workspace_size(0, 100, 4) == 0


def test_decode_validation(lib):
    def dec(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lens=FAKE, B=2, S=64, hq=8, hkv=2, d=128,
                 window=0, scale=0.1, split=0, ws=FAKE, wsb=1 << 30)
        a.update(kw)
        return lib.attn_decode(a["q"], a["k"], a["v"], a["o"], None, a["lens"], a["B"], a["S"],
                               a["hq"], a["hkv"], a["d"], a["window"], a["scale"], None, a["split"],
                               a["ws"], a["wsb"], None)
    assert dec(lens=None) == 1
    assert dec(hq=7) == 1
    assert dec(window=-3) == 1
    assert dec(split=100) == 1                      # not a multiple of 64
    assert dec(d=64) == 2
    assert dec(ws=None) == 3
    need = lib.attn_decode_workspace_size(2, 64, 8, 2, 128, 0)
    assert need > 0
    assert dec(wsb=need - 1) == 3
    assert lib.attn_decode_workspace_size(2, 64, 7, 2, 128, 0) == 0


def test_decode_noalloc_validation(lib):
    """The allocation-free decode: the same argument checks as attn_decode,
    and a problem whose workspace exceeds the static array is refused with
    ATTN_ERR_WORKSPACE before anything is launched."""
    def dec(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lens=FAKE, B=2, S=64, hq=8, hkv=2, d=128,
                 window=0, scale=0.1, split=0)
        a.update(kw)
        return lib.attn_decode_noalloc(a["q"], a["k"], a["v"], a["o"], None, a["lens"], a["B"],
                                       a["S"], a["hq"], a["hkv"], a["d"], a["window"], a["scale"],
                                       None, a["split"], None)
    assert dec(lens=None) == 1
    assert dec(q=None) == 1
    assert dec(hq=7) == 1
    assert dec(window=-3) == 1
    assert dec(split=100) == 1
    assert dec(scale=float("nan")) == 1
    assert dec(d=64) == 2
    limit = 64 << 20
    assert lib.attn_decode_workspace_size(64, 8192, 64, 8, 128, 64) > limit
    assert dec(B=64, S=8192, hq=64, hkv=8, split=64) == 3
    assert dec(B=64, S=8192, hq=64, hkv=8, split=64, d=64) == 2


def test_fp8_validation(lib):
    def quant(**kw):
        a = dict(x=FAKE, c=FAKE, s=FAKE, B=2, hkv=2, S=100, d=128)
        a.update(kw)
        return lib.attn_quantize_kv_fp8(a["x"], a["c"], a["s"], a["B"], a["hkv"], a["S"], a["d"],
                                        None)
    assert quant(x=None) == 1
    assert quant(s=None) == 1
    assert quant(S=0) == 1
    assert quant(d=12) == 2                          # d_h must be a multiple of 8

    def dec(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, ks=FAKE, vs=FAKE, o=FAKE, lens=FAKE, B=2, S=64, hq=8,
                 hkv=2, d=128, window=0, scale=0.1, split=0, ws=FAKE, wsb=1 << 30)
        a.update(kw)
        return lib.attn_decode_fp8(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["o"], None,
                                   a["lens"], a["B"], a["S"], a["hq"], a["hkv"], a["d"],
                                   a["window"], a["scale"], None, a["split"], a["ws"], a["wsb"],
                                   None)
    assert dec(ks=None) == 1
    assert dec(vs=None) == 1
    assert dec(hq=7) == 1
    assert dec(d=64) == 2
    assert dec(ws=None) == 3

    def pdec(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, ks=FAKE, vs=FAKE, o=FAKE, lens=FAKE, bt=FAKE, B=2, mb=8,
                 ps=64, np_=16, hq=8, hkv=2, d=128, window=0, scale=0.1, split=0, ws=FAKE,
                 wsb=1 << 30)
        a.update(kw)
        return lib.attn_decode_paged_fp8(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["o"], None,
                                         a["lens"], a["bt"], a["B"], a["mb"], a["ps"], a["np_"],
                                         a["hq"], a["hkv"], a["d"], a["window"], a["scale"], None,
                                         a["split"], a["ws"], a["wsb"], None)
    assert pdec(ks=None) == 1
    assert pdec(bt=None) == 1
    assert pdec(ps=48) == 2
    assert pdec(ws=None) == 3


def test_rope_validation(lib):
    def rope(**kw):
        a = dict(q=FAKE, k=FAKE, pos=None, B=1, T=8, hq=4, hk=2, rq=128, rk=128, off=0, rd=128,
                 base=1e4, dtype=1)
        a.update(kw)
        return lib.attn_rope_qk(a["q"], a["k"], a["pos"], a["B"], a["T"], a["hq"], a["hk"], a["rq"],
                                a["rk"], a["off"], a["rd"], a["base"], a["dtype"], None)
    assert rope(q=None) == 1
    assert rope(k=None) == 1                         # keys announced but missing
    assert rope(rd=7) == 1                           # odd rotated width
    assert rope(off=64, rd=128) == 1                 # past the row
    assert rope(base=0.0) == 1
    assert rope(base=float("nan")) == 1
    assert rope(dtype=5) == 2


def test_paged_validation(lib):
    def dec(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lens=FAKE, bt=FAKE, B=2, mb=8, ps=64, np_=16,
                 hq=8, hkv=2, d=128, window=0, scale=0.1, split=0, ws=FAKE, wsb=1 << 30)
        a.update(kw)
        return lib.attn_decode_paged(a["q"], a["k"], a["v"], a["o"], None, a["lens"], a["bt"],
                                     a["B"], a["mb"], a["ps"], a["np_"], a["hq"], a["hkv"], a["d"],
                                     a["window"], a["scale"], None, a["split"], a["ws"], a["wsb"],
                                     None)
    assert dec(bt=None) == 1
    assert dec(mb=0) == 1
    assert dec(np_=0) == 1
    assert dec(ps=0) == 1
    assert dec(ps=48) == 2                          # pages are multiples of 32 positions
    assert dec(hq=7) == 1
    assert dec(d=64) == 2
    assert dec(ws=None) == 3
    need = lib.attn_decode_paged_workspace_size(2, 8, 64, 8, 2, 128, 0)
    assert need == lib.attn_decode_workspace_size(2, 512, 8, 2, 128, 0) > 0
    assert dec(wsb=need - 1) == 3

    def mla(**kw):
        a = dict(q=FAKE, c=FAKE, o=FAKE, lens=FAKE, bt=FAKE, B=2, mb=4, ps=64, np_=8, H=128,
                 dc=512, dr=64, scale=0.1, split=0, ws=FAKE, wsb=1 << 30)
        a.update(kw)
        return lib.mla_decode_paged(a["q"], a["c"], a["o"], None, a["lens"], a["bt"], a["B"],
                                    a["mb"], a["ps"], a["np_"], a["H"], a["dc"], a["dr"],
                                    a["scale"], None, a["split"], a["ws"], a["wsb"], None)
    assert mla(bt=None) == 1
    assert mla(ps=100) == 2
    assert mla(dc=256) == 2
    assert mla(ws=None) == 3
    need = lib.mla_decode_paged_workspace_size(2, 4, 64, 128, 512, 64, 0)
    assert need == lib.mla_decode_workspace_size(2, 256, 128, 512, 64, 0) > 0
    assert mla(wsb=need - 1) == 3


def test_mla_validation(lib):
    def mla(**kw):
        a = dict(q=FAKE, c=FAKE, o=FAKE, lens=FAKE, B=2, S=64, H=128, dc=512, dr=64, scale=0.07,
                 split=0, ws=FAKE, wsb=1 << 30)
        a.update(kw)
        return lib.mla_decode(a["q"], a["c"], a["o"], None, a["lens"], a["B"], a["S"], a["H"],
                              a["dc"], a["dr"], a["scale"], None, a["split"], a["ws"], a["wsb"],
                              None)
    assert mla(c=None) == 1
    assert mla(scale=float("nan")) == 1
    assert mla(scale=0.0) == 1
    assert mla(split=32) == 1
    assert mla(dc=256) == 2
    assert mla(H=24) == 2
    assert mla(ws=None) == 3
    need = lib.mla_decode_workspace_size(2, 64, 128, 512, 64, 0)
    assert mla(wsb=need - 1) == 3


def test_workspace_grows_with_splits(lib):
    a = lib.attn_decode_workspace_size(4, 4096, 16, 2, 128, 64)
    b = lib.attn_decode_workspace_size(4, 4096, 16, 2, 128, 1024)
    assert a > b > 0


@pytest.mark.parametrize("lang,compiler", [("c", "gcc"), ("c++", "g++")])
def test_header_compiles_as_c_and_cpp(tmp_path, lang, compiler):
    """include/mi355attn.h is a plain C header (usable from C and C++)."""
    import shutil
    import subprocess
    if shutil.which(compiler) is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"):
        pytest.skip("compiler or HIP headers not available")
    src = tmp_path / "use_header.c"
    src.write_text('#include "mi355attn.h"\nint main(void) { return attn_abi_version() == 2 ? 0 : 1; }\n')
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    r = subprocess.run([compiler, "-fsyntax-only", "-x", lang, "-D__HIP_PLATFORM_AMD__", "-I", inc,
                        "-I", "/opt/rocm/include", str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
