"""Build ``libattn.so`` in-tree with hipcc for gfx950.

Usage: ``python -m causal_head_attention_amd.build`` (or ``build()``).
Each source compiles to an object under ``_build/`` in parallel, then one
link step writes ``causal_head_attention_amd/libattn.so``.
"""
from __future__ import annotations

import json
import os
import re
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
    os.path.join(CSRC, "kernels", "fwd_prefill.hip"),
    os.path.join(CSRC, "kernels", "fwd_row.hip"),
    os.path.join(CSRC, "kernels", "fwd_f32.hip"),
    os.path.join(CSRC, "kernels", "decode.hip"),
    os.path.join(CSRC, "kernels", "qkv_proj.hip"),
    os.path.join(CSRC, "kernels", "pe.hip"),
    os.path.join(CSRC, "kernels", "softmax.hip"),
]

# The bench's read-only HBM reference: a separate library, not part of the
# attention path or its C ABI.
PROBE_SOURCES = [os.path.join(CSRC, "probe", "read_stream.hip")]
PROBE_LIB = os.path.join(PKG, "libattn_probe.so")

ARCH = "gfx950"
# Packed fp32 VALU forms are switched off for every device pass. MFMA
# accumulators are kept in ordinary VGPRs: the softmax rescale touches them
# with vector instructions, and accumulators in AGPRs would be copied in and
# out of the loop.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form=1"]
# Extra flags per source file (none at present: every kernel keeps IEEE NaN
# semantics; the prefill row maximum uses the NaN-propagating maximum
# instruction instead of relaxing them).
PER_SOURCE_FLAGS: dict = {}
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-result",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libattn.so")
    return exe


RESOURCES = os.path.join(BUILD_DIR, "kernel_resources.json")
_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]|"
                     r"SGPRs Spill|VGPRs Spill|LDS Size \[bytes/block\]):\s+(\S+)")


def _resources(text: str) -> dict:
    """Per-kernel register, scratch, spill and LDS figures from hipcc's
    kernel-resource-usage remarks."""
    out, cur = {}, None
    for m in _REMARK.finditer(text):
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[key.split(" [")[0]] = int(val)
    return out


def _compile(src: str) -> tuple[str, dict]:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    hip = src.endswith(".hip")
    lang = ["-x", "hip", "-Rpass-analysis=kernel-resource-usage"] if hip else []
    extra = PER_SOURCE_FLAGS.get(os.path.basename(src), [])
    cmd = [hipcc()] + COMMON + DEVICE_FLAGS + extra + lang + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    text = r.stdout + r.stderr
    noise = ("'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)",
             "[-Rpass-analysis=kernel-resource-usage]")
    # keep real diagnostics; drop the resource remarks and their source excerpts
    msgs = [ln for ln in text.splitlines() if ln.strip() and not any(n in ln for n in noise)
            and not re.match(r"^\s*(\d+\s*)?[|^]", ln)]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if msgs:
        print("\n".join(msgs), file=sys.stderr)
    return obj, _resources(text)


def build(jobs: int = 4) -> str:
    """Compile every HIP/C++ source for gfx950 and link ``libattn.so`` (and
    the bench's ``libattn_probe.so``)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        done = list(ex.map(_compile, SOURCES + PROBE_SOURCES))
    objs = [o for o, _ in done[:len(SOURCES)]]
    probe_objs = [o for o, _ in done[len(SOURCES):]]
    res = {}
    for _, r in done:
        res.update(r)
    with open(RESOURCES, "w") as f:
        json.dump(res, f, indent=1, sort_keys=True)
    for name, r in res.items():
        if r.get("ScratchSize", 0) or r.get("VGPRs Spill", 0):
            print(f"warning: {name} uses {r.get('ScratchSize')} B/lane of scratch "
                  f"({r.get('VGPRs Spill')} VGPRs spilled)", file=sys.stderr)
    for lib, parts in ((LIB, objs), (PROBE_LIB, probe_objs)):
        tmp = lib + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + parts
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build())
