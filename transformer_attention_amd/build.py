"""Build libmi355attn.so (the HIP kernels + C ABI) for gfx950 with hipcc.

Run as ``python -m transformer_attention_amd.build`` or call :func:`build`.
The library is written next to this file so it travels with the source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(os.path.dirname(PKG_DIR), "include")
LIB_PATH = os.path.join(PKG_DIR, "libmi355attn.so")
SOURCES = ["api.hip", "prefill_bf16.hip", "prefill_bwd_bf16.hip", "prefill_f32.hip",
           "decode_bf16.hip", "mla_decode_bf16.hip", "mla_decode_fp8.hip", "prefill_fp8.hip", "quant_fp8.hip",
           "rope.hip"]
ARCH = "gfx950"

# Packed fp32 VALU forms are disabled for all device code.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False, extra_flags=None) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = [hipcc()] + HIPCC_FLAGS + ["-I", INCLUDE] + list(extra_flags or []) + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
