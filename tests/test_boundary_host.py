"""Host-side checks of the C ABI (no GPU needed).

Every argument check in attn_api.cpp runs before any HIP call, so invalid
calls can be exercised here with fake device addresses: a rejected call
launches nothing and touches no memory.
"""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import causal_head_attention_amd as attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")
L = attn.lib
A = 0x10000  # fake, 16-byte aligned "device" addresses (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


def test_header_symbols_are_exported():
    names = declared_functions()
    assert {"attn_fwd", "attn_decode", "attn_decode_workspace_bytes", "attn_set_stream",
            "attn_last_error"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"{n} declared in include/attn.h but not exported by libattn.so"


def fwd(q=A, k=A + 0x100000, v=A + 0x200000, o=A + 0x300000, B=1, H=2, S_q=64, S_kv=64, D=128, causal=1,
        dtype=attn.ATTN_BF16):
    return L.attn_fwd(q, k, v, o, B, H, S_q, S_kv, D, causal, dtype)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(B=-1), attn.ATTN_ERR_INVALID_ARG, "negative"),
    (dict(S_kv=-5), attn.ATTN_ERR_INVALID_ARG, "negative"),
    (dict(D=0), attn.ATTN_ERR_INVALID_ARG, "head dim"),
    (dict(D=48), attn.ATTN_ERR_UNSUPPORTED, "D=48"),
    (dict(D=256), attn.ATTN_ERR_UNSUPPORTED, "D=256"),
    (dict(dtype=3), attn.ATTN_ERR_UNSUPPORTED, "dtype"),                 # no such element type
    (dict(dtype=7), attn.ATTN_ERR_UNSUPPORTED, "dtype"),
    (dict(causal=2), attn.ATTN_ERR_INVALID_ARG, "causal"),
    (dict(S_q=65, S_kv=64), attn.ATTN_ERR_INVALID_ARG, "S_q <= S_kv"),
    (dict(S_kv=0), attn.ATTN_ERR_INVALID_ARG, "S_kv == 0"),
    (dict(q=0), attn.ATTN_ERR_INVALID_ARG, "NULL"),
    (dict(o=0), attn.ATTN_ERR_INVALID_ARG, "NULL"),
    (dict(k=A + 0x100008), attn.ATTN_ERR_INVALID_ARG, "aligned"),
    (dict(o=A + 0x10), attn.ATTN_ERR_INVALID_ARG, "overlaps"),          # o inside q
    (dict(o=A + 0x200000 - 0x10), attn.ATTN_ERR_INVALID_ARG, "overlaps"),  # o runs into v
    (dict(B=1 << 30, H=1 << 20, S_q=1 << 10, S_kv=1 << 10), attn.ATTN_ERR_INVALID_ARG, "overflow"),
    (dict(B=1 << 20, H=1 << 12, S_q=1 << 12, S_kv=1 << 12), attn.ATTN_ERR_INVALID_ARG, "launch grid"),
])
def test_fwd_rejections(kw, status, needle):
    assert fwd(**kw) == status
    msg = L.attn_last_error().decode()
    assert needle in msg, msg


def test_fwd_empty_calls_are_ok_and_launch_nothing():
    # B, H or S_q == 0: valid, nothing to compute (NULL pointers allowed)
    for kw in (dict(B=0), dict(H=0), dict(S_q=0)):
        assert fwd(q=0, k=0, v=0, o=0, **kw) == attn.ATTN_OK
    assert L.attn_last_error().decode() == ""


def test_non_causal_allows_more_queries_than_keys_in_validation():
    p = attn.attn_fwd_plan(1, 2, 100, 50, 64, False, attn.ATTN_BF16)
    assert p.kernel == 1 and p.grid == 2 and p.max_tiles == 1   # one block per head: nothing to pair


def test_status_strings():
    assert L.attn_status_string(0) == b"ATTN_OK"
    assert L.attn_status_string(3) == b"ATTN_ERR_WORKSPACE"
    assert L.attn_status_string(99) == b"ATTN_UNKNOWN_STATUS"


def test_stream_is_per_thread_setting():
    import threading
    assert L.attn_set_stream(ctypes.c_void_p(0x1234)) == 0
    assert L.attn_get_stream() == 0x1234
    seen = []
    t = threading.Thread(target=lambda: seen.append(L.attn_get_stream()))
    t.start()
    t.join()
    assert seen == [None]
    L.attn_set_stream(None)


# ---------------------------------------------------------------------------
# Launch plans: the causal triangle folded so every workgroup gets equal work
# ---------------------------------------------------------------------------
def test_plan_bf16_s2048():
    p = attn.attn_fwd_plan(1, 32, 2048, 2048, 128, True, attn.ATTN_BF16)
    assert (p.kernel, p.block_m, p.block_n, p.paired, p.threads) == (1, 128, 64, 1, 512)
    assert p.grid == 32 * 8                 # 16 query blocks per head, paired
    assert p.max_tiles == p.min_tiles == 34  # (2r+2) + (2(15-r)+2) for every r
    # one workgroup per CU: three K/V stages (rows padded / swizzled) and the merge region
    assert p.lds_bytes == 3 * (64 * 272 + 64 * 256) + 4 * 64 * 36 * 4 <= 160 * 1024


def test_plan_bf16_s4096_and_odd_block_counts():
    p = attn.attn_fwd_plan(1, 32, 4096, 4096, 128, True, attn.ATTN_BF16)
    assert p.grid == 32 * 16 and p.max_tiles == p.min_tiles == 66
    p = attn.attn_fwd_plan(2, 3, 1000, 1000, 64, True, attn.ATTN_BF16)   # 8 blocks (last ragged)
    assert p.grid == 2 * 3 * 4 and p.paired == 1
    p = attn.attn_fwd_plan(1, 1, 640, 640, 64, True, attn.ATTN_BF16)     # 5 blocks: middle one alone
    assert p.grid == 3 and (p.max_tiles, p.min_tiles) == (12, 6)


def test_plan_non_causal_and_fp32():
    p = attn.attn_fwd_plan(2, 8, 512, 512, 64, False, attn.ATTN_BF16)
    # no causal rule: blocks 3+0 and 2+1 of each head share a workgroup
    assert p.paired == 1 and p.grid == 2 * 8 * 2 and p.max_tiles == p.min_tiles == 16
    # fp32: the MFMA kernel, one workgroup per 32 queries; block j of a causal
    # head sees j + 1 tiles of 32 keys
    p = attn.attn_fwd_plan(2, 8, 512, 512, 64, True, attn.ATTN_F32)
    assert p.kernel == 3 and p.grid == 2 * 8 * 16 and (p.block_m, p.block_n) == (32, 32)
    assert (p.max_tiles, p.min_tiles) == (16, 1) and p.threads == 512 and p.lds_bytes == (8 * 64 * 35 + 32 * 8) * 4
    p = attn.attn_fwd_plan(1, 2, 100, 300, 32, True, attn.ATTN_F32)     # bottom-right: block 0 sees 232 keys
    assert p.grid == 2 * 4 and (p.max_tiles, p.min_tiles) == (10, 8)
    p = attn.attn_fwd_plan(1, 1, 70, 50, 128, False, attn.ATTN_F32)
    assert p.grid == 3 and p.max_tiles == p.min_tiles == 2


def test_plan_fp32_row_switch(monkeypatch):
    monkeypatch.setenv("ATTN_ALGO", "row")
    p = attn.attn_fwd_plan(2, 8, 512, 512, 64, True, attn.ATTN_F32)
    assert p.kernel == 2 and p.grid == 2 * 8 * 512


def test_plan_env_switch(monkeypatch):
    monkeypatch.setenv("ATTN_ALGO", "row")
    assert attn.attn_fwd_plan(1, 32, 2048, 2048, 128, True, attn.ATTN_BF16).kernel == 2
    monkeypatch.setenv("ATTN_ALGO", "tile")
    assert attn.attn_fwd_plan(1, 32, 2048, 2048, 128, True, attn.ATTN_BF16).kernel == 1


@pytest.mark.parametrize("n", [1, 7, 8, 9, 15, 16, 17, 63, 64, 100, 255, 256, 257, 512, 1000, 4099])
def test_xcd_remap_is_a_bijection_with_contiguous_ranges(n):
    ids = [L.attn_xcd_remap(x, n) for x in range(n)]
    assert sorted(ids) == list(range(n))
    if n >= 16:
        # workgroups on one XCD (x % 8 equal) get one contiguous range of logical ids
        for xcd in range(8):
            mine = sorted(ids[x] for x in range(xcd, n, 8))
            assert mine == list(range(mine[0], mine[0] + len(mine)))
    assert L.attn_xcd_remap(n, n) == -1


# ---------------------------------------------------------------------------
# Decode boundary
# ---------------------------------------------------------------------------
def test_decode_workspace_and_plan():
    # one record per (workgroup, sequence) segment: at most 256 + B - 1, per
    # head: max, sum, two pad floats, D accumulators; then a 64-bit flag each
    assert attn.attn_decode_workspace_bytes(16, 32, 4096, 128) == (256 + 15) * 32 * (132 * 4 + 8)
    assert attn.attn_decode_workspace_bytes(16, 32, 1, 128) == attn.attn_decode_workspace_bytes(16, 32, 4096, 128)
    assert attn.attn_decode_workspace_bytes(0, 32, 4096, 128) == 0
    p = attn.attn_decode_plan(16, 32, 4096, 128, attn.ATTN_BF16)
    assert (p.split_workgroups, p.records, p.threads) == (256, 271, 512)
    assert p.workspace_bytes == attn.attn_decode_workspace_bytes(16, 32, 4096, 128)
    with pytest.raises(attn.AttnError):   # one sequence's cache beyond 32-bit offsets
        attn.attn_decode_plan(1, 32, 1 << 18, 128, attn.ATTN_BF16)


@pytest.mark.parametrize("T", [1, 2, 3, 13, 127, 128, 129, 255, 256, 257, 258, 300, 383, 384, 385, 1000, 24304,
                               65535, 1 << 20, (1 << 31) - 1])
def test_decode_ranges_tile_the_token_space(T):
    G = attn.attn_decode_plan(16, 32, 4096, 128, attn.ATTN_BF16).split_workgroups
    starts = [L.attn_decode_range_start(w, T) for w in range(G + 1)]
    assert starts[0] == 0 and starts[G] == T
    assert all(a <= b for a, b in zip(starts, starts[1:]))
    # the empty ranges come last: a sequence's keys never skip a workgroup
    sizes = [b - a for a, b in zip(starts, starts[1:])]
    n_full = sum(1 for x in sizes if x > 0)
    assert all(x > 0 for x in sizes[:n_full]) and not any(sizes[n_full:])
    probes = {0, T - 1} | {min(T - 1, s) for s in starts} | {max(0, s - 1) for s in starts}
    probes |= set(range(0, T, max(1, T // 509)))
    for t in sorted(probes):
        w = L.attn_decode_range_of(t, T)
        assert 0 <= w < G and starts[w] <= t < starts[w + 1], (t, w)
    assert L.attn_decode_range_start(G + 1, T) == -1 and L.attn_decode_range_start(-1, T) == -1
    assert L.attn_decode_range_of(T, T) == -1 and L.attn_decode_range_of(0, 0) == -1


def test_decode_ranges_favour_even_xcds():
    # 24,304 keys (the 16-sequence decode workload): spans of 190 keys per
    # pair of workgroups, 101 for the even one (53%, rounded up), 89 for the odd
    starts = [L.attn_decode_range_start(w, 24304) for w in range(257)]
    sizes = [b - a for a, b in zip(starts, starts[1:])]
    assert sizes[:4] == [101, 89, 101, 89]
    assert sum(sizes) == 24304 and max(sizes) == 101


@pytest.mark.parametrize("seed", range(12))
def test_decode_record_index_is_unique(seed):
    # segment (w, b) -- workgroup w's part of sequence b -- writes record w + b;
    # for any lengths (zeros included) no two segments share a record, and all
    # fall below the plan's record count
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 300))
    lens = rng.integers(0, (3, 5000, 40)[seed % 3], size=B)
    lens[rng.random(B) < 0.2] = 0
    T = int(lens.sum())
    if T == 0:
        return
    G = 256
    starts = [L.attn_decode_range_start(w, T) for w in range(G + 1)]
    seen = set()
    P = 0
    for b, n in enumerate(lens.tolist()):
        if n:
            w0, w1 = L.attn_decode_range_of(P, T), L.attn_decode_range_of(P + n - 1, T)
            for w in range(w0, w1 + 1):   # every one of them holds keys of b
                assert max(starts[w], P) < min(starts[w + 1], P + n), (w, b)
                assert w + b not in seen
                seen.add(w + b)
        P += n
    assert max(seen) < attn.attn_decode_plan(B, 8, 64, 64, attn.ATTN_BF16).records


def dec(q=A, kc=A + 0x100000, vc=A + 0x200000, sl=A + 0x300000, o=A + 0x310000, B=2, H=2, S_cap=100,
        D=128, dtype=attn.ATTN_BF16, ws=A + 0x400000, wsb=None):
    if wsb is None:
        wsb = attn.attn_decode_workspace_bytes(B, H, S_cap, D)
    return L.attn_decode(q, kc, vc, sl, o, B, H, S_cap, D, dtype, ws, wsb)


@pytest.mark.parametrize("kw,status", [
    (dict(ws=0), attn.ATTN_ERR_WORKSPACE),
    (dict(wsb=16), attn.ATTN_ERR_WORKSPACE),
    (dict(S_cap=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(D=96), attn.ATTN_ERR_UNSUPPORTED),
    (dict(dtype=3), attn.ATTN_ERR_UNSUPPORTED),
    (dict(sl=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(sl=A + 0x300002), attn.ATTN_ERR_INVALID_ARG),
    (dict(o=A + 0x100000), attn.ATTN_ERR_INVALID_ARG),         # o on the K cache
    (dict(ws=A + 0x200000), attn.ATTN_ERR_INVALID_ARG),        # workspace on the V cache
    (dict(q=A + 8), attn.ATTN_ERR_INVALID_ARG),
])
def test_decode_rejections(kw, status):
    assert dec(**kw) == status, L.attn_last_error()


def test_decode_empty_call():
    assert dec(q=0, kc=0, vc=0, sl=0, o=0, ws=0, B=0, wsb=0) == attn.ATTN_OK


# ---------------------------------------------------------------------------
# Q/K/V projection boundary (fake device addresses: every case is rejected
# on the host before any HIP call)
# ---------------------------------------------------------------------------
def qkv(x=A, w=A + 0x1000000, q=A + 0x4000000, k=A + 0x5000000, v=A + 0x6000000, M=100, E=256, H=2, D=64,
        dtype=attn.ATTN_BF16):
    return L.attn_qkv_proj(x, w, q, k, v, M, E, H, D, dtype)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dtype=attn.ATTN_F32), attn.ATTN_ERR_UNSUPPORTED, "dtype"),
    (dict(E=100), attn.ATTN_ERR_UNSUPPORTED, "multiple of 32"),
    (dict(H=1, D=48), attn.ATTN_ERR_UNSUPPORTED, "multiple of 32"),
    (dict(M=-1), attn.ATTN_ERR_INVALID_ARG, "sizes"),
    (dict(E=0), attn.ATTN_ERR_INVALID_ARG, "sizes"),
    (dict(x=0), attn.ATTN_ERR_INVALID_ARG, "NULL"),
    (dict(w=A + 0x1000008), attn.ATTN_ERR_INVALID_ARG, "aligned"),
    (dict(q=A + 0x100), attn.ATTN_ERR_INVALID_ARG, "overlaps an input"),          # q inside x
    (dict(k=A + 0x4000000), attn.ATTN_ERR_INVALID_ARG, "each other"),            # k on q
    (dict(E=1 << 23), attn.ATTN_ERR_UNSUPPORTED, "32-bit"),
    (dict(E=3 << 20), attn.ATTN_ERR_UNSUPPORTED, "32-bit"),   # the 384-row W tile passes 2^31 bytes first
])
def test_qkv_rejections(kw, status, needle):
    assert qkv(**kw) == status, L.attn_last_error()
    assert needle in attn.load().attn_last_error().decode()


def test_qkv_empty_call():
    assert qkv(x=0, w=0, q=0, k=0, v=0, M=0) == attn.ATTN_OK


@pytest.mark.parametrize("args,needle", [
    ((A, 10, 63, 0), "even"),
    ((A, -1, 64, 0), "sizes"),
    ((A, 10, 64, -1), "sizes"),
    ((A, 10, 64, (1 << 31) - 5), "2^31"),
    ((0, 10, 64, 0), "NULL"),
    ((A + 4, 10, 64, 0), "aligned"),
])
def test_pe_rejections(args, needle):
    assert L.attn_sinusoidal_pe(*args) == attn.ATTN_ERR_INVALID_ARG
    assert needle in attn.load().attn_last_error().decode()


@pytest.mark.parametrize("args,needle", [
    ((A, 1 << 30, 2, 0), "S exceeds"),
    ((A, 1, 1 << 26, 0), "d_model exceeds"),
])
def test_pe_grid_limits(args, needle):
    assert L.attn_sinusoidal_pe(*args) == attn.ATTN_ERR_UNSUPPORTED
    assert needle in attn.load().attn_last_error().decode()


def test_pe_empty_call():
    assert L.attn_sinusoidal_pe(0, 0, 64, 0) == attn.ATTN_OK


def sm(s=A, p=A + 0x4000000, B=1, H=2, S_q=64, S_kv=64, scale=0.125, causal=1, dtype=attn.ATTN_BF16):
    return L.attn_masked_softmax(s, p, B, H, S_q, S_kv, scale, causal, dtype)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dtype=3), attn.ATTN_ERR_UNSUPPORTED, "dtype"),
    (dict(S_kv=8200), attn.ATTN_ERR_UNSUPPORTED, "exceeds"),
    (dict(S_kv=4100, dtype=attn.ATTN_F32), attn.ATTN_ERR_UNSUPPORTED, "exceeds"),
    (dict(S_kv=12), attn.ATTN_ERR_UNSUPPORTED, "16-byte"),
    (dict(S_kv=6, dtype=attn.ATTN_F32), attn.ATTN_ERR_UNSUPPORTED, "16-byte"),
    (dict(causal=2), attn.ATTN_ERR_INVALID_ARG, "causal"),
    (dict(scale=float("inf")), attn.ATTN_ERR_INVALID_ARG, "finite"),
    (dict(scale=float("nan")), attn.ATTN_ERR_INVALID_ARG, "finite"),
    (dict(B=-1), attn.ATTN_ERR_INVALID_ARG, "negative"),
    (dict(s=0), attn.ATTN_ERR_INVALID_ARG, "NULL"),
    (dict(p=A + 0x4000008), attn.ATTN_ERR_INVALID_ARG, "aligned"),
    (dict(p=A + 0x100), attn.ATTN_ERR_INVALID_ARG, "overlaps"),       # p inside s, not s itself
    (dict(B=1 << 20, H=64, S_q=4, S_kv=8), attn.ATTN_ERR_UNSUPPORTED, "grid"),
])
def test_masked_softmax_rejections(kw, status, needle):
    assert sm(**kw) == status, L.attn_last_error()
    assert needle in attn.load().attn_last_error().decode()


def test_masked_softmax_empty_calls():
    assert sm(s=0, p=0, B=0) == attn.ATTN_OK
    assert sm(s=0, p=0, S_kv=0) == attn.ATTN_OK


def test_binding_rejects_host_tensors():
    q = torch.zeros(1, 4, 1, 32)
    with pytest.raises(ValueError):
        attn.attn_fwd(q, q, q)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """No fallback: without libattn.so the first call raises ImportError."""
    monkeypatch.setattr(attn, "LIB_PATH", str(tmp_path / "libattn.so"))
    monkeypatch.setattr(attn, "_lib", None)
    with pytest.raises(ImportError):
        attn.load()


def test_kernels_use_no_scratch():
    """Every kernel keeps its state in registers and LDS: a register array
    indexed at run time, or a spill, would move it to scratch memory (a
    several-fold slowdown). The figures come from hipcc's resource report,
    which the build writes next to its objects."""
    import json
    path = os.path.join(ROOT, "_build", "kernel_resources.json")
    if not os.path.exists(path):
        pytest.skip("no build report (build the library first)")
    res = json.load(open(path))
    for kern in ("prefill_kernel", "decode_kernel", "fwd_f32_kernel"):
        assert any(kern in k for k in res), f"report lists {kern}"
    bad = {k: v for k, v in res.items() if v.get("ScratchSize", 0) or v.get("VGPRs Spill", 0)}
    assert not bad, bad


def _bench_module():
    import importlib.util
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(root, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_traffic_record_matches_the_current_build_and_goes_stale(monkeypatch, tmp_path):
    """profiles/traffic.json is keyed by each kernel's build: its code (source
    and the headers it includes, comments left out), the device flags and the
    compiler. The committed record matches this build, and a changed flag, or
    a code change in the source or a header, nulls it."""
    from causal_head_attention_amd import build as B
    bench = _bench_module()
    import json
    doc = json.load(open(bench.TRAFFIC_JSON))
    assert bench.measured_traffic("prefill", bench.PREFILL_SRC) == doc["prefill"]["bytes_per_launch"]
    assert bench.measured_traffic("decode", bench.DECODE_SRC) == doc["decode"]["bytes_per_launch"]
    monkeypatch.setitem(B.PER_SOURCE_FLAGS, "fwd_prefill.hip", ["-fno-honor-nans"])
    assert bench.measured_traffic("prefill", bench.PREFILL_SRC) is None
    monkeypatch.undo()
    src = open(bench.DECODE_SRC, "rb").read()
    # a comment-only edit keeps the fingerprint; a code edit nulls the record
    commented = tmp_path / "decode.hip"
    commented.write_bytes(src.replace(b"\n", b"  // note\n", 3) + b"\n/* a remark */\n")
    assert bench.measured_traffic("decode", str(commented)) == doc["decode"]["bytes_per_launch"]
    edited = tmp_path / "decode_edited.hip"
    edited.write_bytes(src + b"\nnamespace { constexpr int kEdited = 1; }\n")
    assert bench.measured_traffic("decode", str(edited)) is None
    # a code edit of plan.h (tile sizes, the decode split) changes every kernel's fingerprint
    plan = tmp_path / "plan.h"
    text = open(bench.KERNEL_HEADERS[0], "rb").read()
    edited_plan = re.sub(rb"constexpr int kDecodeBatch = (\d+);",
                         lambda m: b"constexpr int kDecodeBatch = %d;" % (int(m.group(1)) + 2), text)
    assert edited_plan != text
    plan.write_bytes(edited_plan)
    headers = [str(plan)] + bench.KERNEL_HEADERS[1:]
    assert bench.build_sha256(bench.DECODE_SRC, headers) != bench.build_sha256(bench.DECODE_SRC)
    assert bench.build_sha256(bench.PREFILL_SRC, headers) != doc["prefill"]["build_sha256"]


def test_clock_probe_arming():
    """attn_set_clock_probe accepts NULL and an 8-byte aligned pointer (nothing
    is written until an attn_fwd runs) and rejects a misaligned one."""
    assert L.attn_set_clock_probe(None) == attn.ATTN_OK
    assert L.attn_set_clock_probe(A + 8) == attn.ATTN_OK
    assert L.attn_set_clock_probe(A + 4) == attn.ATTN_ERR_INVALID_ARG
    assert L.attn_set_clock_probe(None) == attn.ATTN_OK   # disarm: no call below may write through it


def test_perf_log_has_one_record_per_leg(monkeypatch, tmp_path):
    """bench.py --perf-log appends one JSON line per measured leg, keyed by
    workload, kernel, source revision and kernel build, with P50/P95 and the
    fraction of the roofline (the per-version timing table)."""
    import json
    bench = _bench_module()
    monkeypatch.setenv("ATTN_GIT_REV", "0123abcd")
    roof = {"kernel": "prefill_kernel<bf16,128>", "frac": 0.25, "median_launch_us": 56.0, "p95_launch_us": 58.0}
    line = {"value": 613.9, "unit": "TFLOPS", "roofline": roof,
            "config": {"workload": "bf16 causal prefill S=2048 + bf16 decode B=16"},
            "decode": {"value": 5600.0, "roofline": {"frac": 0.7, "median_call_us": 71.0, "p95_call_us": 73.0}},
            "fp16_prefill": {"value": 540.0, "unit": "TFLOPS", "workload": "fp16 causal prefill",
                             "roofline": {"frac": 0.21, "median_launch_us": 64.0}},
            "cpu_baseline": {"value": 0.04, "cores": 16}, "parity": {"prefill_max_abs": 8e-3}}
    path = tmp_path / "perf.jsonl"
    bench.append_perf_log(str(path), line)
    bench.append_perf_log(str(path), line)
    recs = [json.loads(x) for x in path.read_text().splitlines()]
    assert [r["leg"] for r in recs] == ["prefill", "decode", "fp16_prefill"] * 2
    assert all(r["rev"] == "0123abcd" and len(r["build"]["prefill"]) == 16 for r in recs)
    assert recs[0]["median_us"] == 56.0 and recs[0]["p95_us"] == 58.0 and recs[0]["max_abs"] == 8e-3
    assert recs[1]["workload"] == "bf16 decode B=16" and recs[1]["frac"] == 0.7
    assert recs[2]["value"] == 540.0 and recs[2]["median_us"] == 64.0
