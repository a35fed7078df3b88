"""Builds libattn.so (the HIP kernels plus the C ABI) in-tree for gfx950.

    python -m dense_attention_amd.build

Cross-compiles without a GPU.  Every HIP translation unit is compiled with
packed-fp32 instruction selection turned off.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn.so")
SOURCES = [os.path.join(CSRC, "attn_api.hip")]
HEADERS = [os.path.join(CSRC, "attn_fwd_kernel.h"), os.path.join(CSRC, "attn_merge_kernel.h"),
           os.path.join(INCLUDE, "attn.h")]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build dense_attention_amd)")


def compile_command(out: str = LIB) -> list:
    return [
        hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        "-I", INCLUDE, "-I", CSRC,
        *SOURCES, "-o", out,
    ]


def build(verbose: bool = False) -> str:
    """Compiles the library (always) and returns its path."""
    tmp = LIB + ".tmp"
    cmd = compile_command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libattn.so")
    if verbose:
        sys.stderr.write(res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
