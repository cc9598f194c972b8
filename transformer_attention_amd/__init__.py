"""Python binding of libmi355attn.so (exact GQA/MQA/MHA attention on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/mi355attn.h``.  PyTorch
provides device memory and the current stream; the functions below check
tensor shapes/dtypes/devices, pass raw pointers, and raise
:class:`AttnError` on a non-OK status.  There is no CPU fallback: if the
library is not built, importing the entry points raises.

Entry points (same names as the C ABI):
  attn_prefill(q, k, v, *, causal, window=0, scale=None, o=None, lse=None)
  attn_prefill_backward(q, k, v, o, dout, lse, *, causal, window=0, scale=None,
                        dq=None, dk=None, dv=None, workspace=None)
  attn_decode(q, k_cache, v_cache, seq_lens, *, window=0, scale=None,
              split_tokens=0, o=None, lse=None, workspace=None)
  mla_decode(q, kv_cache, seq_lens, *, d_c=512, d_r=64, scale,
             split_tokens=0, o=None, lse=None, workspace=None)
  attn_decode_paged(q, k_pages, v_pages, seq_lens, block_table, ...)
  mla_decode_paged(q, kv_pages, seq_lens, block_table, ...)
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# MI355ATTN_LIB may point at another build of the same library (e.g. a
# differently tuned one); by default the in-tree build is used.
LIB_PATH = os.environ.get("MI355ATTN_LIB") or os.path.join(_PKG_DIR, "libmi355attn.so")

ATTN_OK = 0
ATTN_ERR_INVALID_ARG = 1
ATTN_ERR_UNSUPPORTED = 2
ATTN_ERR_WORKSPACE = 3
ATTN_ERR_HIP = 4
ATTN_F32 = 0
ATTN_BF16 = 1

EXPORTED_SYMBOLS = (
    "attn_prefill", "attn_prefill_backward", "attn_prefill_backward_workspace_size",
    "attn_decode", "attn_decode_workspace_size",
    "mla_decode", "mla_decode_workspace_size", "attn_decode_paged",
    "attn_decode_paged_workspace_size", "mla_decode_paged", "mla_decode_paged_workspace_size",
    "attn_quantize_kv_fp8", "attn_decode_fp8", "attn_decode_paged_fp8", "attn_rope_qk",
    "attn_decode_noalloc", "mla_decode_fp8", "mla_decode_fp8_workspace_size", "attn_prefill_fp8",
    "attn_status_string",
    "attn_abi_version",
)


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the shared library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m transformer_attention_amd.build`")
    lib = ctypes.CDLL(path)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.attn_prefill.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, I, F, P, P]
    lib.attn_prefill.restype = I
    lib.attn_prefill_backward_workspace_size.argtypes = [I, I, I]
    lib.attn_prefill_backward_workspace_size.restype = Z
    lib.attn_prefill_backward.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F,
                                          P, P, P, Z, P]
    lib.attn_prefill_backward.restype = I
    lib.attn_decode_workspace_size.argtypes = [I, I, I, I, I, I]
    lib.attn_decode_workspace_size.restype = Z
    lib.attn_decode.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, F, P, I, P, Z, P]
    lib.attn_decode.restype = I
    lib.mla_decode_workspace_size.argtypes = [I, I, I, I, I, I]
    lib.mla_decode_workspace_size.restype = Z
    lib.mla_decode.argtypes = [P, P, P, P, P, I, I, I, I, I, F, P, I, P, Z, P]
    lib.mla_decode.restype = I
    lib.attn_decode_paged_workspace_size.argtypes = [I, I, I, I, I, I, I]
    lib.attn_decode_paged_workspace_size.restype = Z
    lib.attn_decode_paged.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, P, I, P, Z,
                                      P]
    lib.attn_decode_paged.restype = I
    lib.mla_decode_paged_workspace_size.argtypes = [I, I, I, I, I, I, I]
    lib.mla_decode_paged_workspace_size.restype = Z
    lib.mla_decode_paged.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, F, P, I, P, Z, P]
    lib.mla_decode_paged.restype = I
    lib.attn_quantize_kv_fp8.argtypes = [P, P, P, I, I, I, I, P]
    lib.attn_quantize_kv_fp8.restype = I
    lib.attn_decode_fp8.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, P, I, P, Z, P]
    lib.attn_decode_fp8.restype = I
    lib.attn_decode_paged_fp8.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, P,
                                          I, P, Z, P]
    lib.attn_decode_paged_fp8.restype = I
    lib.attn_prefill_fp8.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, P, P]
    lib.attn_prefill_fp8.restype = I
    lib.mla_decode_fp8_workspace_size.argtypes = [I, I, I, I, I, I]
    lib.mla_decode_fp8_workspace_size.restype = Z
    lib.mla_decode_fp8.argtypes = [P, P, P, P, P, P, I, I, I, I, I, F, P, I, P, Z, P]
    lib.mla_decode_fp8.restype = I
    lib.attn_decode_noalloc.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, F, P, I, P]
    lib.attn_decode_noalloc.restype = I
    lib.attn_rope_qk.argtypes = [P, P, P, I, I, I, I, I, I, I, I, F, I, P]
    lib.attn_rope_qk.restype = I
    lib.attn_status_string.argtypes = [I]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_abi_version.argtypes = []
    lib.attn_abi_version.restype = I
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().attn_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != ATTN_OK:
        raise AttnError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require(t, name, dtype, device=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_DT = {torch.float32: ATTN_F32, torch.bfloat16: ATTN_BF16}


def _sinks(sinks, h_q, device):
    """Optional sink logits: one fp32 value per query head on the device."""
    if sinks is None:
        return None
    _require(sinks, "sinks", torch.float32, device)
    if sinks.numel() != h_q:
        raise ValueError(f"sinks must hold h_q = {h_q} values")
    return sinks


def _lse_out(lse, B, hq, device, return_lse):
    """The optional [B, h_q] fp32 log-sum-exp output of a decode call: checked
    here because the merge kernel writes all B * h_q entries."""
    if lse is None and return_lse:
        lse = torch.empty((B, hq), dtype=torch.float32, device=device)
    if lse is not None:
        _require(lse, "lse", torch.float32, device)
        if lse.numel() != B * hq:
            raise ValueError(f"lse must hold B * h_q = {B * hq} values, got {lse.numel()}")
    return lse


def attn_prefill(q, k, v, *, causal: bool = True, window: int = 0, scale=None,
                 sinks=None, o=None, lse=None, return_lse: bool = False):
    """q:[B,h_q,T,d]  k,v:[B,h_kv,T,d] (bf16 or fp32, contiguous, same device).
    sinks: optional fp32[h_q] sink logits.  Returns o (and lse:[B,h_q,T] fp32
    when requested)."""
    lib = load_library()
    if q.dtype not in _DT:
        raise ValueError(f"unsupported dtype {q.dtype}")
    _require(q, "q", q.dtype, ndim=4)
    _require(k, "k", q.dtype, q.device, 4)
    _require(v, "v", q.dtype, q.device, 4)
    B, hq, T, d = q.shape
    hkv = k.shape[1]
    if tuple(k.shape) != (B, hkv, T, d) or tuple(v.shape) != (B, hkv, T, d):
        raise ValueError("k/v shape mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty_like(q)
    _require(o, "o", q.dtype, q.device)
    if tuple(o.shape) != tuple(q.shape):
        raise ValueError("o shape mismatch")
    if lse is None and return_lse:
        lse = torch.empty((B, hq, T), dtype=torch.float32, device=q.device)
    if lse is not None:
        _require(lse, "lse", torch.float32, q.device)
        if lse.numel() != B * hq * T:
            raise ValueError("lse shape mismatch")
    sinks = _sinks(sinks, hq, q.device)
    st = lib.attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, T, hq,
                          hkv, d, _DT[q.dtype], int(bool(causal)), int(window),
                          float(scale), _ptr(sinks), _stream(q.device))
    _check(st, "attn_prefill")
    return (o, lse) if (return_lse or lse is not None) else o


def attn_prefill_fp8(q8, k8, v8, q_scales, k_scales, v_scales, *, causal: bool = True,
                     window: int = 0, scale=None, sinks=None, o=None, lse=None,
                     return_lse: bool = False):
    """Prefill with FP8 attention.  q8:[B,h_q,T,128], k8,v8:[B,h_kv,T,128] uint8
    E4M3 codes; scales fp32 [B,h,ceil(T/32)] (attn_quantize_kv_fp8 of q, k, v).
    Returns o:[B,h_q,T,128] bf16 (and lse when requested)."""
    lib = load_library()
    _require(q8, "q8", torch.uint8, ndim=4)
    _require(k8, "k8", torch.uint8, q8.device, 4)
    _require(v8, "v8", torch.uint8, q8.device, 4)
    B, hq, T, d = q8.shape
    hkv = k8.shape[1]
    if tuple(k8.shape) != (B, hkv, T, d) or tuple(v8.shape) != (B, hkv, T, d):
        raise ValueError("k8/v8 shape mismatch")
    nt = (T + 31) // 32
    for t, name, hh in ((q_scales, "q_scales", hq), (k_scales, "k_scales", hkv),
                        (v_scales, "v_scales", hkv)):
        _require(t, name, torch.float32, q8.device)
        if t.numel() != B * hh * nt:
            raise ValueError(f"{name} must hold [B, h, ceil(T/32)] values")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty((B, hq, T, d), dtype=torch.bfloat16, device=q8.device)
    _require(o, "o", torch.bfloat16, q8.device)
    if o.numel() != B * hq * T * d:
        raise ValueError("o shape mismatch")
    if lse is None and return_lse:
        lse = torch.empty((B, hq, T), dtype=torch.float32, device=q8.device)
    if lse is not None:
        _require(lse, "lse", torch.float32, q8.device)
        if lse.numel() != B * hq * T:
            raise ValueError("lse shape mismatch")
    st = lib.attn_prefill_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_scales), _ptr(k_scales),
                              _ptr(v_scales), _ptr(o), _ptr(lse), B, T, hq, hkv, d,
                              int(bool(causal)), int(window), float(scale),
                              _ptr(_sinks(sinks, hq, q8.device)), _stream(q8.device))
    _check(st, "attn_prefill_fp8")
    return (o, lse) if (return_lse or lse is not None) else o


def attn_prefill_backward_workspace_size(B, T, h_q) -> int:
    return int(load_library().attn_prefill_backward_workspace_size(B, T, h_q))


def attn_prefill_backward(q, k, v, o, dout, lse, *, causal: bool = True, window: int = 0,
                          scale=None, sinks=None, return_dsinks: bool = False, dq=None,
                          dk=None, dv=None, dsinks=None, workspace=None):
    """Gradients of attn_prefill.  q, o, dout:[B,h_q,T,128] bf16; k,v:[B,h_kv,T,128]
    bf16; lse:[B,h_q,T] fp32 (the forward's).  Returns (dq, dk, dv), and the
    sink logits' gradient fp32[h_q] as a fourth item with ``return_dsinks``
    (which needs ``sinks``, the forward's)."""
    lib = load_library()
    _require(q, "q", torch.bfloat16, ndim=4)
    for t, name in ((k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _require(t, name, torch.bfloat16, q.device, 4)
    _require(lse, "lse", torch.float32, q.device)
    B, hq, T, d = q.shape
    hkv = k.shape[1]
    if tuple(k.shape) != (B, hkv, T, d) or tuple(v.shape) != (B, hkv, T, d):
        raise ValueError("k/v shape mismatch")
    if tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("o/dout shape mismatch")
    if lse.numel() != B * hq * T:
        raise ValueError("lse shape mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _require(dq, "dq", torch.bfloat16, q.device)
    _require(dk, "dk", torch.bfloat16, q.device)
    _require(dv, "dv", torch.bfloat16, q.device)
    if dq.shape != q.shape or dk.shape != k.shape or dv.shape != v.shape:
        raise ValueError("gradient shape mismatch")
    need = attn_prefill_backward_workspace_size(B, T, hq)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _require(workspace, "workspace", torch.uint8, q.device)
    sinks = _sinks(sinks, hq, q.device)
    if return_dsinks and sinks is None:
        raise ValueError("return_dsinks needs sinks")
    if return_dsinks and dsinks is None:
        dsinks = torch.empty(hq, dtype=torch.float32, device=q.device)
    if dsinks is not None:
        _require(dsinks, "dsinks", torch.float32, q.device)
        if dsinks.numel() != hq:
            raise ValueError("dsinks shape mismatch")
    st = lib.attn_prefill_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                   _ptr(dq), _ptr(dk), _ptr(dv), B, T, hq, hkv, d,
                                   _DT[q.dtype], int(bool(causal)), int(window), float(scale),
                                   _ptr(sinks), _ptr(dsinks), _ptr(workspace),
                                   workspace.numel(), _stream(q.device))
    _check(st, "attn_prefill_backward")
    return (dq, dk, dv, dsinks) if (return_dsinks or dsinks is not None) else (dq, dk, dv)


def attn_decode_workspace_size(B, S_max, h_q, h_kv, d_h, split_tokens=0) -> int:
    return int(load_library().attn_decode_workspace_size(B, S_max, h_q, h_kv, d_h,
                                                         split_tokens))


def attn_decode(q, k_cache, v_cache, seq_lens, *, window: int = 0, scale=None,
                sinks=None, split_tokens: int = 0, o=None, lse=None, workspace=None,
                return_lse: bool = False):
    """q:[B,h_q,d] or [B,h_q,1,d] bf16; caches:[B,h_kv,S_max,d] bf16;
    seq_lens: int32[B] on the device.  Returns o shaped like q."""
    lib = load_library()
    _require(q, "q", torch.bfloat16)
    _require(k_cache, "k_cache", torch.bfloat16, q.device, 4)
    _require(v_cache, "v_cache", torch.bfloat16, q.device, 4)
    _require(seq_lens, "seq_lens", torch.int32, q.device, 1)
    B, hkv, S_max, d = k_cache.shape
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("v_cache shape mismatch")
    hq = q.shape[1]
    if q.numel() != B * hq * d or q.shape[0] != B or q.shape[-1] != d:
        raise ValueError("q shape mismatch")
    if seq_lens.shape[0] != B:
        raise ValueError("seq_lens shape mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty_like(q)
    _require(o, "o", torch.bfloat16, q.device)
    if o.numel() != q.numel():
        raise ValueError("o shape mismatch")
    lse = _lse_out(lse, B, hq, q.device, return_lse)
    need = lib.attn_decode_workspace_size(B, S_max, hq, hkv, d, int(split_tokens))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _require(workspace, "workspace", None, q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    sinks = _sinks(sinks, hq, q.device)
    st = lib.attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse),
                         _ptr(seq_lens), B, S_max, hq, hkv, d, int(window),
                         float(scale), _ptr(sinks), int(split_tokens), _ptr(workspace), ws_bytes,
                         _stream(q.device))
    _check(st, "attn_decode")
    return (o, lse) if (return_lse or lse is not None) else o


# Size of the static device array attn_decode_noalloc works in (bytes).
DECODE_NOALLOC_SCRATCH_BYTES = 64 << 20


def attn_decode_noalloc(q, k_cache, v_cache, seq_lens, *, window: int = 0, scale=None,
                        sinks=None, split_tokens: int = 0, o=None, lse=None,
                        return_lse: bool = False):
    """attn_decode without a workspace: the library's static device array holds
    the partials, so the C call allocates nothing (pass ``o`` and ``lse`` to
    keep this wrapper from allocating them).  Raises AttnError
    (ATTN_ERR_WORKSPACE) when the problem's workspace exceeds
    DECODE_NOALLOC_SCRATCH_BYTES.  Calls overlapping on one GPU race."""
    lib = load_library()
    _require(q, "q", torch.bfloat16)
    _require(k_cache, "k_cache", torch.bfloat16, q.device, 4)
    _require(v_cache, "v_cache", torch.bfloat16, q.device, 4)
    _require(seq_lens, "seq_lens", torch.int32, q.device, 1)
    B, hkv, S_max, d = k_cache.shape
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("v_cache shape mismatch")
    hq = q.shape[1]
    if q.numel() != B * hq * d or q.shape[0] != B or q.shape[-1] != d or seq_lens.shape[0] != B:
        raise ValueError("q / seq_lens shape mismatch")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    o, lse = _decode_out(q, B, hq, o, lse, return_lse)
    st = lib.attn_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse),
                                 _ptr(seq_lens), B, S_max, hq, hkv, d, int(window), float(scale),
                                 _ptr(_sinks(sinks, hq, q.device)), int(split_tokens),
                                 _stream(q.device))
    _check(st, "attn_decode_noalloc")
    return (o, lse) if (return_lse or lse is not None) else o


def mla_decode_workspace_size(B, S_max, h_q, d_c=512, d_r=64, split_tokens=0) -> int:
    return int(load_library().mla_decode_workspace_size(B, S_max, h_q, d_c, d_r,
                                                        split_tokens))


def mla_decode(q, kv_cache, seq_lens, *, d_c: int = 512, d_r: int = 64, scale: float,
               sinks=None, split_tokens: int = 0, o=None, lse=None, workspace=None,
               return_lse: bool = False):
    """q:[B,H,d_c+d_r] bf16; kv_cache:[B,S_max,d_c+d_r] bf16; seq_lens int32[B].
    Returns o:[B,H,d_c] bf16 (the latent context before W_UV)."""
    lib = load_library()
    _require(q, "q", torch.bfloat16, ndim=3)
    _require(kv_cache, "kv_cache", torch.bfloat16, q.device, 3)
    _require(seq_lens, "seq_lens", torch.int32, q.device, 1)
    B, H, dk = q.shape
    if dk != d_c + d_r or kv_cache.shape[0] != B or kv_cache.shape[2] != dk:
        raise ValueError("q / kv_cache shape mismatch")
    S_max = kv_cache.shape[1]
    if o is None:
        o = torch.empty((B, H, d_c), dtype=torch.bfloat16, device=q.device)
    _require(o, "o", torch.bfloat16, q.device)
    if o.numel() != B * H * d_c:
        raise ValueError("o shape mismatch")
    lse = _lse_out(lse, B, H, q.device, return_lse)
    need = lib.mla_decode_workspace_size(B, S_max, H, d_c, d_r, int(split_tokens))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _require(workspace, "workspace", None, q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    sinks = _sinks(sinks, H, q.device)
    st = lib.mla_decode(_ptr(q), _ptr(kv_cache), _ptr(o), _ptr(lse), _ptr(seq_lens),
                        B, S_max, H, d_c, d_r, float(scale), _ptr(sinks), int(split_tokens),
                        _ptr(workspace), ws_bytes, _stream(q.device))
    _check(st, "mla_decode")
    return (o, lse) if (return_lse or lse is not None) else o


def mla_decode_fp8_workspace_size(B, S_max, h_q, d_c=512, d_r=64, split_tokens=0) -> int:
    return int(load_library().mla_decode_fp8_workspace_size(B, S_max, h_q, d_c, d_r,
                                                            split_tokens))


def mla_decode_fp8(q, kv_codes, kv_scales, seq_lens, *, d_c: int = 512, d_r: int = 64,
                   scale: float, sinks=None, split_tokens: int = 0, o=None, lse=None,
                   workspace=None, return_lse: bool = False):
    """MLA decode with FP8 attention.  q:[B,H,d_c+d_r] bf16 (quantised in the
    call); kv_codes:[B,S_max,d_c+d_r] uint8 E4M3; kv_scales:[B,ceil(S_max/32)]
    fp32 (attn_quantize_kv_fp8 of the cache viewed as [B,1,S_max,d_c+d_r]);
    seq_lens int32[B].  Returns o:[B,H,d_c] bf16."""
    lib = load_library()
    _require(q, "q", torch.bfloat16, ndim=3)
    _require(kv_codes, "kv_codes", torch.uint8, q.device, 3)
    _require(kv_scales, "kv_scales", torch.float32, q.device)
    _require(seq_lens, "seq_lens", torch.int32, q.device, 1)
    B, H, dk = q.shape
    if dk != d_c + d_r or kv_codes.shape[0] != B or kv_codes.shape[2] != dk:
        raise ValueError("q / kv_codes shape mismatch")
    S_max = kv_codes.shape[1]
    if kv_scales.numel() != B * ((S_max + 31) // 32):
        raise ValueError("kv_scales must hold [B, ceil(S_max/32)] values")
    if seq_lens.shape[0] != B:
        raise ValueError("seq_lens shape mismatch")
    if o is None:
        o = torch.empty((B, H, d_c), dtype=torch.bfloat16, device=q.device)
    _require(o, "o", torch.bfloat16, q.device)
    if o.numel() != B * H * d_c:
        raise ValueError("o shape mismatch")
    lse = _lse_out(lse, B, H, q.device, return_lse)
    need = lib.mla_decode_fp8_workspace_size(B, S_max, H, d_c, d_r, int(split_tokens))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _require(workspace, "workspace", None, q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.mla_decode_fp8(_ptr(q), _ptr(kv_codes), _ptr(kv_scales), _ptr(o), _ptr(lse),
                            _ptr(seq_lens), B, S_max, H, d_c, d_r, float(scale),
                            _ptr(_sinks(sinks, H, q.device)), int(split_tokens), _ptr(workspace),
                            ws_bytes, _stream(q.device))
    _check(st, "mla_decode_fp8")
    return (o, lse) if (return_lse or lse is not None) else o


def attn_decode_paged(q, k_pages, v_pages, seq_lens, block_table, *, window: int = 0, scale=None,
                      sinks=None, split_tokens: int = 0, o=None, lse=None, workspace=None,
                      return_lse: bool = False):
    """q:[B,h_q,d] or [B,h_q,1,d] bf16; pages:[num_pages,h_kv,page_size,d] bf16;
    block_table: int32[B,max_blocks] and seq_lens: int32[B] on the device."""
    lib = load_library()
    _require(q, "q", torch.bfloat16)
    _require(k_pages, "k_pages", torch.bfloat16, q.device, 4)
    _require(v_pages, "v_pages", torch.bfloat16, q.device, 4)
    _require(seq_lens, "seq_lens", torch.int32, q.device, 1)
    _require(block_table, "block_table", torch.int32, q.device, 2)
    num_pages, hkv, page_size, d = k_pages.shape
    if tuple(v_pages.shape) != tuple(k_pages.shape):
        raise ValueError("v_pages shape mismatch")
    B, max_blocks = block_table.shape
    hq = q.shape[1]
    if q.numel() != B * hq * d or q.shape[0] != B or q.shape[-1] != d:
        raise ValueError("q shape mismatch")
    if seq_lens.shape[0] != B:
        raise ValueError("seq_lens shape mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty_like(q)
    _require(o, "o", torch.bfloat16, q.device)
    if o.numel() != q.numel():
        raise ValueError("o shape mismatch")
    lse = _lse_out(lse, B, hq, q.device, return_lse)
    need = lib.attn_decode_paged_workspace_size(B, max_blocks, page_size, hq, hkv, d,
                                                int(split_tokens))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _require(workspace, "workspace", None, q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.attn_decode_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(o), _ptr(lse),
                               _ptr(seq_lens), _ptr(block_table), B, max_blocks, page_size,
                               num_pages, hq, hkv, d, int(window), float(scale),
                               _ptr(_sinks(sinks, hq, q.device)), int(split_tokens), _ptr(workspace), ws_bytes, _stream(q.device))
    _check(st, "attn_decode_paged")
    return (o, lse) if (return_lse or lse is not None) else o


def mla_decode_paged(q, kv_pages, seq_lens, block_table, *, d_c: int = 512, d_r: int = 64,
                     scale: float, sinks=None, split_tokens: int = 0, o=None, lse=None,
                     workspace=None, return_lse: bool = False):
    """q:[B,H,d_c+d_r] bf16; kv_pages:[num_pages,page_size,d_c+d_r] bf16;
    block_table: int32[B,max_blocks] and seq_lens: int32[B] on the device."""
    lib = load_library()
    _require(q, "q", torch.bfloat16, ndim=3)
    _require(kv_pages, "kv_pages", torch.bfloat16, q.device, 3)
    _require(seq_lens, "seq_lens", torch.int32, q.device, 1)
    _require(block_table, "block_table", torch.int32, q.device, 2)
    B, H, dk = q.shape
    num_pages, page_size, dk2 = kv_pages.shape
    if dk != d_c + d_r or dk2 != dk or block_table.shape[0] != B:
        raise ValueError("q / kv_pages / block_table shape mismatch")
    max_blocks = block_table.shape[1]
    if o is None:
        o = torch.empty((B, H, d_c), dtype=torch.bfloat16, device=q.device)
    _require(o, "o", torch.bfloat16, q.device)
    if o.numel() != B * H * d_c:
        raise ValueError("o shape mismatch")
    lse = _lse_out(lse, B, H, q.device, return_lse)
    need = lib.mla_decode_paged_workspace_size(B, max_blocks, page_size, H, d_c, d_r,
                                               int(split_tokens))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _require(workspace, "workspace", None, q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.mla_decode_paged(_ptr(q), _ptr(kv_pages), _ptr(o), _ptr(lse), _ptr(seq_lens),
                              _ptr(block_table), B, max_blocks, page_size, num_pages, H, d_c,
                              d_r, float(scale), _ptr(_sinks(sinks, H, q.device)),
                              int(split_tokens), _ptr(workspace), ws_bytes,
                              _stream(q.device))
    _check(st, "mla_decode_paged")
    return (o, lse) if (return_lse or lse is not None) else o


def attn_quantize_kv_fp8(x, *, codes=None, scales=None):
    """Per-tile FP8 (E4M3) quantisation of a bf16 cache x:[B,h_kv,S,d] (or pages
    [num_pages,h_kv,page_size,d]): tiles of 32 positions of one head, scale =
    amax / 448.  Returns (codes uint8 like x, scales fp32 [B,h_kv,ceil(S/32)])."""
    lib = load_library()
    _require(x, "x", torch.bfloat16, ndim=4)
    B, hkv, S, d = x.shape
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if codes is None else codes
    nt = (S + 31) // 32
    scales = torch.empty((B, hkv, nt), dtype=torch.float32, device=x.device) if scales is None else scales
    _require(codes, "codes", torch.uint8, x.device)
    _require(scales, "scales", torch.float32, x.device)
    if tuple(codes.shape) != tuple(x.shape) or scales.numel() != B * hkv * nt:
        raise ValueError("codes / scales shape mismatch")
    st = lib.attn_quantize_kv_fp8(_ptr(x), _ptr(codes), _ptr(scales), B, hkv, S, d,
                                  _stream(x.device))
    _check(st, "attn_quantize_kv_fp8")
    return codes, scales


def _decode_out(q, B, hq, o, lse, return_lse):
    o = torch.empty_like(q) if o is None else o
    _require(o, "o", torch.bfloat16, q.device)
    if o.numel() != q.numel():
        raise ValueError("o shape mismatch")
    return o, _lse_out(lse, B, hq, q.device, return_lse)


def attn_decode_fp8(q, k_codes, v_codes, k_scales, v_scales, seq_lens, *, window: int = 0,
                    scale=None, sinks=None, split_tokens: int = 0, o=None, lse=None,
                    workspace=None, return_lse: bool = False):
    """Decode against an FP8 cache: q:[B,h_q,d] or [B,h_q,1,d] bf16; codes:[B,h_kv,S_max,d]
    uint8 (E4M3); scales:[B,h_kv,ceil(S_max/32)] fp32 (attn_quantize_kv_fp8's layout)."""
    lib = load_library()
    _require(q, "q", torch.bfloat16)
    _require(k_codes, "k_codes", torch.uint8, q.device, 4)
    _require(v_codes, "v_codes", torch.uint8, q.device, 4)
    _require(seq_lens, "seq_lens", torch.int32, q.device, 1)
    B, hkv, S_max, d = k_codes.shape
    nt = (S_max + 31) // 32
    for t, name in ((k_scales, "k_scales"), (v_scales, "v_scales")):
        _require(t, name, torch.float32, q.device)
        if t.numel() != B * hkv * nt:
            raise ValueError(f"{name} must hold [B, h_kv, ceil(S_max/32)] values")
    if tuple(v_codes.shape) != tuple(k_codes.shape):
        raise ValueError("v_codes shape mismatch")
    hq = q.shape[1]
    if q.numel() != B * hq * d or q.shape[0] != B or q.shape[-1] != d or seq_lens.shape[0] != B:
        raise ValueError("q / seq_lens shape mismatch")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    o, lse = _decode_out(q, B, hq, o, lse, return_lse)
    need = lib.attn_decode_workspace_size(B, S_max, hq, hkv, d, int(split_tokens))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _require(workspace, "workspace", None, q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.attn_decode_fp8(_ptr(q), _ptr(k_codes), _ptr(v_codes), _ptr(k_scales),
                             _ptr(v_scales), _ptr(o), _ptr(lse), _ptr(seq_lens), B, S_max, hq,
                             hkv, d, int(window), float(scale), _ptr(_sinks(sinks, hq, q.device)),
                             int(split_tokens), _ptr(workspace), ws_bytes, _stream(q.device))
    _check(st, "attn_decode_fp8")
    return (o, lse) if (return_lse or lse is not None) else o


def attn_decode_paged_fp8(q, k_pages, v_pages, k_scales, v_scales, seq_lens, block_table, *,
                          window: int = 0, scale=None, sinks=None, split_tokens: int = 0,
                          o=None, lse=None, workspace=None, return_lse: bool = False):
    """FP8 decode on a paged cache: pages:[num_pages,h_kv,page_size,d] uint8 codes,
    scales:[num_pages,h_kv,page_size/32] fp32; block_table int32[B,max_blocks]."""
    lib = load_library()
    _require(q, "q", torch.bfloat16)
    _require(k_pages, "k_pages", torch.uint8, q.device, 4)
    _require(v_pages, "v_pages", torch.uint8, q.device, 4)
    _require(seq_lens, "seq_lens", torch.int32, q.device, 1)
    _require(block_table, "block_table", torch.int32, q.device, 2)
    num_pages, hkv, page_size, d = k_pages.shape
    if tuple(v_pages.shape) != tuple(k_pages.shape):
        raise ValueError("v_pages shape mismatch")
    for t, name in ((k_scales, "k_scales"), (v_scales, "v_scales")):
        _require(t, name, torch.float32, q.device)
        if t.numel() != num_pages * hkv * (page_size // 32):
            raise ValueError(f"{name} must hold [num_pages, h_kv, page_size/32] values")
    B, max_blocks = block_table.shape
    hq = q.shape[1]
    if q.numel() != B * hq * d or q.shape[0] != B or q.shape[-1] != d or seq_lens.shape[0] != B:
        raise ValueError("q / seq_lens shape mismatch")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    o, lse = _decode_out(q, B, hq, o, lse, return_lse)
    need = lib.attn_decode_paged_workspace_size(B, max_blocks, page_size, hq, hkv, d,
                                                int(split_tokens))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _require(workspace, "workspace", None, q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.attn_decode_paged_fp8(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(k_scales),
                                   _ptr(v_scales), _ptr(o), _ptr(lse), _ptr(seq_lens),
                                   _ptr(block_table), B, max_blocks, page_size, num_pages, hq, hkv,
                                   d, int(window), float(scale), _ptr(_sinks(sinks, hq, q.device)),
                                   int(split_tokens), _ptr(workspace), ws_bytes, _stream(q.device))
    _check(st, "attn_decode_paged_fp8")
    return (o, lse) if (return_lse or lse is not None) else o


def attn_rope_qk(q, k=None, *, base: float, positions=None, rope_offset: int = 0, rope_dim=None):
    """Rotary position embedding, in place: q:[B,h_q,T,row_q] and k:[B,h_k,T,row_k]
    (bf16 or fp32, same dtype); dimensions [rope_offset, rope_offset + rope_dim)
    of every row (default: the rest of the row); positions int32[B,T] on the
    device, default 0..T-1.  Returns (q, k)."""
    lib = load_library()
    if q.dtype not in _DT:
        raise ValueError(f"unsupported dtype {q.dtype}")
    _require(q, "q", q.dtype, ndim=4)
    B, hq, T, row_q = q.shape
    hk, row_k = 0, 0
    if k is not None:
        _require(k, "k", q.dtype, q.device, 4)
        if k.shape[0] != B or k.shape[2] != T:
            raise ValueError("k shape mismatch")
        hk, row_k = k.shape[1], k.shape[3]
    if positions is not None:
        _require(positions, "positions", torch.int32, q.device)
        if positions.numel() != B * T:
            raise ValueError("positions must hold [B, T] values")
    rd = row_q - rope_offset if rope_dim is None else rope_dim
    st = lib.attn_rope_qk(_ptr(q), _ptr(k), _ptr(positions), B, T, hq, hk, row_q, row_k,
                          int(rope_offset), int(rd), float(base), _DT[q.dtype], _stream(q.device))
    _check(st, "attn_rope_qk")
    return q, k

