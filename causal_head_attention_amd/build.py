"""Build ``libattn.so`` in-tree with hipcc for gfx950.

Usage: ``python -m causal_head_attention_amd.build`` (or ``build()``).
Each source compiles to an object under ``_build/`` in parallel, then one
link step writes ``causal_head_attention_amd/libattn.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libattn.so")

SOURCES = [
    os.path.join(CSRC, "attn_api.cpp"),
    os.path.join(CSRC, "kernels", "fwd_tile_bf16.hip"),
    os.path.join(CSRC, "kernels", "fwd_row.hip"),
    os.path.join(CSRC, "kernels", "decode.hip"),
]

ARCH = "gfx950"
# Packed fp32 VALU forms are switched off for every device pass. MFMA
# accumulators are kept in ordinary VGPRs: the softmax rescale touches them
# with vector instructions, and accumulators in AGPRs would be copied in and
# out of the loop.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form=1"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-result",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libattn.so")
    return exe


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc()] + COMMON + DEVICE_FLAGS + lang + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln and ln.strip()]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if msgs:
        print("\n".join(msgs), file=sys.stderr)
    return obj


def build(jobs: int = 4) -> str:
    """Compile every HIP/C++ source for gfx950 and link ``libattn.so``."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
