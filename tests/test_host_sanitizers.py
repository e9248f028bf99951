"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The C ABI's host side (causal_head_attention_amd/csrc/attn_api.cpp with the
planning helpers of plan.h) is built with host-only stand-ins for the GPU
launchers (tests/sanitize/hip_stubs.cpp) and driven through every entry point
with valid, invalid and extreme arguments (tests/sanitize/abi_driver.cpp); the
fp64 oracle (oracle/attn_oracle.c) is built with the same sanitizers and run
on small inputs (tests/sanitize/oracle_driver.c). Any out-of-bounds access,
signed overflow, misaligned access or other undefined behaviour aborts the
driver with a report.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2",
           LSAN_OPTIONS="suppressions=" + os.path.join(HERE, "lsan.supp"))


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return r.returncode, r.stdout + r.stderr


@pytest.fixture(scope="module")
def outdir(tmp_path_factory):
    if not (os.path.exists(CLANGXX) and os.path.exists(CLANG)):
        pytest.skip("the ROCm clang toolchain is needed for the sanitizer builds")
    return str(tmp_path_factory.mktemp("sanitize"))


def test_c_abi_host_code_is_clean_under_asan_and_ubsan(outdir):
    exe = os.path.join(outdir, "abi_driver")
    cmd = [CLANGXX, "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "causal_head_attention_amd", "csrc")] + SAN + [
        os.path.join(ROOT, "causal_head_attention_amd", "csrc", "attn_api.cpp"),
        os.path.join(HERE, "hip_stubs.cpp"), os.path.join(HERE, "abi_driver.cpp"), "-o", exe]
    rc, out = _run(cmd)
    assert rc == 0, out[-4000:]
    rc, out = _run([exe], env=ENV, timeout=300)
    assert rc == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert "0 failures" in out


def test_oracle_is_clean_under_asan_and_ubsan(outdir):
    exe = os.path.join(outdir, "oracle_driver")
    cmd = [CLANG, "-std=c99", "-fopenmp"] + SAN + [os.path.join(ROOT, "oracle", "attn_oracle.c"),
                                                   os.path.join(HERE, "oracle_driver.c"), "-o", exe, "-lm"]
    rc, out = _run(cmd)
    if rc != 0 and "omp" in out.lower():
        # no OpenMP runtime for this clang: build the oracle without it
        cmd = [c for c in cmd if c != "-fopenmp"]
        rc, out = _run(cmd)
    assert rc == 0, out[-4000:]
    rc, out = _run([exe], env=ENV, timeout=300)
    assert rc == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert "0 failures" in out
