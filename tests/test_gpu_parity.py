"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle.

Bars (written here, applied per output tensor):
  fp32 storage : max |gpu - oracle| <= 1e-4
  bf16 storage : max |gpu - oracle| <= 2e-2  AND  ||gpu - oracle||_2 / ||oracle||_2 <= 1e-2
  fp16 storage : max |gpu - oracle| <= 5e-3  AND  ||gpu - oracle||_2 / ||oracle||_2 <= 3e-3
The fp16 bar follows from the arithmetic: the output is rounded to fp16
(half an ulp is at most 2^-9 ~ 2e-3 for |O| < 8) and the probabilities
enter P.V rounded to fp16 (relative 2^-11, at most ~2e-3 on a convex
combination of |V| <= 4), everything else is fp32.
The oracle receives exactly the values the GPU receives (16-bit values
widened to fp64), so input rounding is not counted as error.
"""
import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

FP32_ATOL = 1e-4
BF16_ATOL = 2e-2
BF16_RELL2 = 1e-2
FP16_ATOL = 5e-3
FP16_RELL2 = 3e-3
ALL_DTYPES = [torch.bfloat16, torch.float16, torch.float32]
DTYPE_IDS = ["bf16", "fp16", "fp32"]


def say(msg):
    print(f"[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def attn():
    import causal_head_attention_amd as m
    return m


def check(got: torch.Tensor, ref: np.ndarray, dtype: torch.dtype, what: str = ""):
    g = got.detach().float().cpu().double().numpy()
    assert g.shape == ref.shape, what
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - ref)
    max_abs = float(err.max()) if err.size else 0.0
    if dtype == torch.float32:
        assert max_abs <= FP32_ATOL, f"{what}: max abs err {max_abs:.3e} > {FP32_ATOL}"
        return max_abs, None
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(g - ref) / den) if den > 0 else float(np.linalg.norm(g - ref))
    atol, rell2 = (FP16_ATOL, FP16_RELL2) if dtype == torch.float16 else (BF16_ATOL, BF16_RELL2)
    assert max_abs <= atol, f"{what}: max abs err {max_abs:.3e} > {atol}"
    assert rel <= rell2, f"{what}: rel L2 err {rel:.3e} > {rell2}"
    return max_abs, rel


# ---------------------------------------------------------------------------
# The workloads at their full sizes, in the configuration the benchmark times
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", workloads.PREFILL_CONFIGS, ids=lambda c: c.name)
def test_prefill_workload(attn, cfg):
    say(f"prefill {cfg.name} B={cfg.B} H={cfg.H} S={cfg.S_q} D={cfg.D} {cfg.dtype}")
    q, k, v = workloads.make_prefill(cfg)
    o = attn.attn_fwd(q.cuda(), k.cuda(), v.cuda(), causal=cfg.causal)
    torch.cuda.synchronize()
    ref = oracle.attn_fwd(q, k, v, cfg.causal)
    max_abs, rel = check(o, ref, cfg.dtype, cfg.name)
    say(f"  {cfg.name}: max abs {max_abs:.3e} rel L2 {rel}")


def test_decode_workload(attn):
    cfg = workloads.BF16_DECODE
    say(f"decode {cfg.name} B={cfg.B} H={cfg.H} S_cap={cfg.S_cap} D={cfg.D} (NaN past each length)")
    seqlens, q, kc, vc = workloads.make_decode(cfg, nan_fill=True)
    o = attn.attn_decode(q.cuda(), kc.cuda(), vc.cuda(), seqlens.cuda())
    torch.cuda.synchronize()
    ref = np.zeros((cfg.B, 1, cfg.H, cfg.D))
    for b in range(cfg.B):
        n = int(seqlens[b])
        ref[b:b + 1] = oracle.attn_decode(q[b:b + 1], kc[b:b + 1, :n], vc[b:b + 1, :n],
                                          np.array([n], dtype=np.int32))
    max_abs, rel = check(o, ref, cfg.dtype, cfg.name)
    say(f"  decode: max abs {max_abs:.3e} rel L2 {rel:.3e}")


# ---------------------------------------------------------------------------
# Edge shapes: ragged tails, one row, S_q != S_kv, every head dim, both dtypes
# ---------------------------------------------------------------------------
EDGE = [
    # B, H, S_q, S_kv, D, causal
    (1, 1, 1, 1, 128, True),
    (1, 2, 7, 7, 64, True),
    (2, 3, 63, 63, 128, True),
    (1, 2, 65, 65, 32, True),
    (1, 1, 127, 127, 128, True),
    (2, 1, 129, 129, 64, True),
    (1, 2, 1000, 1000, 128, True),
    (1, 2, 200, 300, 128, True),     # queries are the last 200 of 300 positions
    (2, 2, 129, 77, 64, False),      # more queries than keys, no mask
    (1, 3, 257, 257, 128, False),
    (1, 1, 1, 513, 128, True),       # one query at the end
    (3, 5, 33, 95, 32, True),
]


@pytest.mark.parametrize("dtype", ALL_DTYPES, ids=DTYPE_IDS)
@pytest.mark.parametrize("shape", EDGE, ids=lambda s: "x".join(map(str, s)))
def test_edge_shapes(attn, shape, dtype):
    B, H, S_q, S_kv, D, causal = shape
    say(f"edge {shape} {dtype}")
    q, k, v = workloads.make_prefill_shape(7, dtype, B, H, S_q, S_kv, D)
    o = attn.attn_fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal)
    torch.cuda.synchronize()
    check(o, oracle.attn_fwd(q, k, v, causal), dtype, str(shape))


@pytest.mark.parametrize("shape", [(1, 2, 300, 300, 128, True), (2, 1, 130, 200, 64, True),
                                   (1, 1, 77, 77, 32, False)], ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
def test_16bit_row_kernel_cross_check(attn, shape, dtype, monkeypatch):
    """ATTN_ALGO=row runs the per-query kernel on 16-bit storage: both kernels meet the bar."""
    B, H, S_q, S_kv, D, causal = shape
    q, k, v = workloads.make_prefill_shape(9, dtype, B, H, S_q, S_kv, D)
    ref = oracle.attn_fwd(q, k, v, causal)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    code = attn.ATTN_BF16 if dtype == torch.bfloat16 else attn.ATTN_F16
    monkeypatch.setenv("ATTN_ALGO", "row")
    assert attn.attn_fwd_plan(B, H, S_q, S_kv, D, causal, code).kernel == 2
    o_row = attn.attn_fwd(qc, kc, vc, causal=causal)
    monkeypatch.setenv("ATTN_ALGO", "tile")
    assert attn.attn_fwd_plan(B, H, S_q, S_kv, D, causal, code).kernel == 1
    o_tile = attn.attn_fwd(qc, kc, vc, causal=causal)
    torch.cuda.synchronize()
    check(o_row, ref, dtype, "row")
    check(o_tile, ref, dtype, "tile")


# ---------------------------------------------------------------------------
# Invariants the definition fixes exactly
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ALL_DTYPES, ids=DTYPE_IDS)
@pytest.mark.parametrize("D", [32, 64, 128])
def test_identity_values_expose_probabilities(attn, dtype, D):
    """V = I (S_kv = D) makes O = P: masked entries exactly 0, rows sum to 1."""
    S = D
    g = torch.Generator().manual_seed(100 + D)
    q = (torch.randn(1, S, 2, D, generator=g) * 2).to(dtype)
    k = (torch.randn(1, S, 2, D, generator=g) * 2).to(dtype)
    v = torch.eye(D).reshape(1, S, 1, D).expand(1, S, 2, D).contiguous().to(dtype)
    o = attn.attn_fwd(q.cuda(), k.cuda(), v.cuda(), causal=True).float().cpu()
    i = torch.arange(S)[:, None]
    j = torch.arange(D)[None, :]
    masked = (j > i).expand(2, S, D).permute(1, 0, 2)[None]
    assert torch.all(o[masked] == 0.0)
    tol = {torch.float32: 1e-4, torch.float16: 2e-3, torch.bfloat16: 2e-2}[dtype]
    assert torch.max(torch.abs(o.sum(-1) - 1.0)) <= tol
    check(o.to(dtype).cuda(), oracle.attn_fwd(q, k, v, True), dtype, "V=I")


@pytest.mark.parametrize("dtype", ALL_DTYPES, ids=DTYPE_IDS)
def test_row_zero_is_value_row_zero_bitwise(attn, dtype):
    q, k, v = workloads.make_prefill_shape(11, dtype, 2, 4, 300, 300, 128, qk_std=4.0)
    o = attn.attn_fwd(q.cuda(), k.cuda(), v.cuda(), causal=True).cpu()
    assert torch.equal(o[:, 0], v[:, 0])


def test_deterministic_across_runs(attn):
    q, k, v = (t.cuda() for t in workloads.make_prefill_shape(12, torch.bfloat16, 1, 8, 2048, 2048, 128))
    o1 = attn.attn_fwd(q, k, v, causal=True)
    o2 = attn.attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_guard_bands_untouched(attn):
    """NaN around every input and a sentinel around the output: an out-of-bounds
    read would poison the output, an out-of-bounds write would change a guard."""
    B, H, S, D = 1, 3, 129, 128
    q, k, v = workloads.make_prefill_shape(13, torch.bfloat16, B, H, S, S, D)
    n = q.numel()
    pad = 4096

    def guarded(t, fill):
        buf = torch.full((n + 2 * pad,), fill, dtype=t.dtype, device="cuda")
        view = buf[pad:pad + n].view(t.shape)
        view.copy_(t.cuda())
        return buf, view

    _, qg = guarded(q, float("nan"))
    _, kg = guarded(k, float("nan"))
    _, vg = guarded(v, float("nan"))
    obuf, og = guarded(torch.zeros_like(q), 1234.0)
    attn.attn_fwd(qg, kg, vg, og, causal=True)
    torch.cuda.synchronize()
    assert torch.all(obuf[:pad] == 1234.0) and torch.all(obuf[pad + n:] == 1234.0)
    check(og, oracle.attn_fwd(q, k, v, True), torch.bfloat16, "guarded")


# ---------------------------------------------------------------------------
# Decode edge cases
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ALL_DTYPES, ids=DTYPE_IDS)
@pytest.mark.parametrize("D", [64, 128, 32])
def test_decode_lengths(attn, dtype, D):
    S_cap = 600
    lens = [1, S_cap, 0, -3, S_cap + 5, 255, 256, 257, 511, 513, 64, 2]
    B, H = len(lens), 3
    g = torch.Generator().manual_seed(200 + D)
    q = torch.randn(B, 1, H, D, generator=g).to(dtype)
    kc = torch.randn(B, S_cap, H, D, generator=g).to(dtype)
    vc = torch.randn(B, S_cap, H, D, generator=g).to(dtype)
    for b, n in enumerate(lens):
        n = max(0, min(n, S_cap))
        kc[b, n:] = float("nan")
        vc[b, n:] = float("nan")
    sl = torch.tensor(lens, dtype=torch.int32)
    o = attn.attn_decode(q.cuda(), kc.cuda(), vc.cuda(), sl.cuda()).cpu()
    assert torch.all(o[2] == 0) and torch.all(o[3] == 0)
    assert torch.equal(o[0, 0], vc[0, 0])                # one key: its value row, bitwise
    ref = oracle.attn_decode(q, kc, vc, sl.numpy())
    check(o.cuda(), ref, dtype, f"decode D={D}")


# The split cuts the sequences' valid keys, laid end to end, into 256 equal
# ranges: short and empty sequences put several sequences into one range and
# leave ranges empty; more than 1024 sequences take the path that rescans the
# lengths in memory instead of LDS.
DECODE_SEGMENTS = [
    # seed, B, H, S_cap, D, length range
    (401, 5, 2, 16, 32, (0, 8)),          # 13-ish keys in all: one key per workgroup, most idle
    (402, 300, 2, 8, 64, (-1, 4)),        # about 2 keys per sequence: ranges span many sequences
    (403, 1100, 2, 40, 32, (-2, 45)),     # beyond the LDS length scan
    (404, 3, 4, 3000, 128, (2500, 3000)), # long sequences: several ranges each
    (405, 4, 2, 80, 32, (64, 70)),        # 257-280 keys: pair spans of 3 (2 for the even workgroup, 1 for the odd)
    (406, 130, 2, 4, 64, (1, 3)),         # ~260 keys over many sequences, spans of 3 crossing sequences
]


@pytest.mark.parametrize("dtype", ALL_DTYPES, ids=DTYPE_IDS)
@pytest.mark.parametrize("case", DECODE_SEGMENTS, ids=lambda c: f"B{c[1]}_S{c[3]}")
def test_decode_balanced_segments(attn, case, dtype):
    seed, B, H, S_cap, D, (lo, hi) = case
    say(f"decode segments seed={seed} B={B} H={H} S_cap={S_cap} D={D} {dtype}")
    g = torch.Generator().manual_seed(seed)
    sl = torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int32)
    q = torch.randn(B, 1, H, D, generator=g).to(dtype)
    kc = torch.randn(B, S_cap, H, D, generator=g).to(dtype)
    vc = torch.randn(B, S_cap, H, D, generator=g).to(dtype)
    for b in range(B):
        n = max(0, min(int(sl[b]), S_cap))
        kc[b, n:] = float("nan")
        vc[b, n:] = float("nan")
    o = attn.attn_decode(q.cuda(), kc.cuda(), vc.cuda(), sl.cuda())
    torch.cuda.synchronize()
    oc = o.cpu()
    empty = sl <= 0
    assert torch.all(oc[empty] == 0)
    ref = oracle.attn_decode(q, kc, vc, sl.numpy())
    check(o, ref, dtype, f"decode segments B={B}")
    o2 = attn.attn_decode(q.cuda(), kc.cuda(), vc.cuda(), sl.cuda())
    assert torch.equal(o2.cpu(), oc)   # fixed merge order: the same bits every run


def test_decode_workspace_reused_across_shapes_ignores_stale_contents(attn):
    """One workspace buffer, sized for the largest call and filled with NaN
    bytes first, serves calls of different shapes in turn: whatever an
    earlier call (or the fill) left in it never reaches a result. Each
    result matches the oracle and the rows of empty sequences are zero."""
    shapes = [  # seed, B, H, S_cap, D, dtype, length range
        (411, 16, 32, 300, 128, torch.bfloat16, (0, 300)),
        (412, 5, 8, 64, 64, torch.float32, (-1, 64)),
        (413, 300, 2, 8, 32, torch.float16, (0, 8)),
        (414, 16, 32, 300, 128, torch.bfloat16, (200, 300)),
    ]
    need = max(attn.attn_decode_workspace_bytes(B, H, S, D) for _, B, H, S, D, _, _ in shapes)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    for seed, B, H, S_cap, D, dtype, (lo, hi) in shapes:
        say(f"decode workspace reuse seed={seed} B={B} H={H} S_cap={S_cap} D={D} {dtype}")
        g = torch.Generator().manual_seed(seed)
        sl = torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int32)
        q = torch.randn(B, 1, H, D, generator=g).to(dtype)
        kc = torch.randn(B, S_cap, H, D, generator=g).to(dtype)
        vc = torch.randn(B, S_cap, H, D, generator=g).to(dtype)
        o = torch.full((B, 1, H, D), float("nan"), dtype=dtype, device="cuda")
        attn.attn_decode(q.cuda(), kc.cuda(), vc.cuda(), sl.cuda(), o=o, workspace=ws)
        torch.cuda.synchronize()
        check(o, oracle.attn_decode(q, kc, vc, sl.numpy()), dtype, f"decode reuse seed={seed}")
        assert torch.all(o.cpu()[sl <= 0] == 0)


def _decode_case(seed, B, H, S_cap, D, dtype, lens):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, 1, H, D, generator=g).to(dtype)
    kc = torch.randn(B, S_cap, H, D, generator=g).to(dtype)
    vc = torch.randn(B, S_cap, H, D, generator=g).to(dtype)
    return torch.tensor(lens, dtype=torch.int32), q, kc, vc


def test_decode_leaves_every_merge_flag_zero(attn):
    """A sequence cut into several segments is merged after its segments
    raise per-call flags in the workspace; the merging workgroup resets them.
    Garbage in flag words (here 0xFF bytes) is never taken for a raised flag,
    and from a zeroed flag area every call leaves all flags zero again, so a
    later call, or a replay of the same launch, never finds one left raised."""
    B, H, S_cap, D = 6, 8, 3000, 128
    lens = [3000, 1, 2999, 0, 1500, 2048]   # long ones span several workgroups each
    sl, q, kc, vc = _decode_case(420, B, H, S_cap, D, torch.bfloat16, lens)
    need = attn.attn_decode_workspace_bytes(B, H, S_cap, D)
    records_bytes = (256 + B - 1) * H * (D + 4) * 4   # the flags follow the records
    assert need == records_bytes + (256 + B - 1) * H * 8
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    ref = oracle.attn_decode(q, kc, vc, sl.numpy())
    flags = ws[records_bytes:].view(torch.int64)
    for it in range(4):
        say(f"decode flags reset, call {it}")
        o = attn.attn_decode(q.cuda(), kc.cuda(), vc.cuda(), sl.cuda(), workspace=ws)
        torch.cuda.synchronize()
        check(o, ref, torch.bfloat16, f"decode flags call {it}")
        if it == 0:
            flags.zero_()
            torch.cuda.synchronize()
        else:
            assert int((flags != 0).sum()) == 0


def test_decode_graph_replays_with_new_lengths(attn):
    """The decode launch captured once in a HIP graph and replayed with new
    lengths written into the same seqlens buffer between replays (the
    per-call flag value is frozen into the graph): every replay matches the
    eager call on the same lengths, bitwise."""
    B, H, S_cap, D = 8, 8, 2048, 128
    g = torch.Generator().manual_seed(421)
    q = torch.randn(B, 1, H, D, generator=g).bfloat16().cuda()
    kc = torch.randn(B, S_cap, H, D, generator=g).bfloat16().cuda()
    vc = torch.randn(B, S_cap, H, D, generator=g).bfloat16().cuda()
    sl = torch.zeros(B, dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    ws = torch.zeros(attn.attn_decode_workspace_bytes(B, H, S_cap, D), dtype=torch.uint8, device="cuda")
    sl.copy_(torch.randint(1, S_cap + 1, (B,), generator=g, dtype=torch.int32))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm-up outside capture
        attn.attn_decode(q, kc, vc, sl, o=o, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        attn.attn_decode(q, kc, vc, sl, o=o, workspace=ws)
    for it in range(4):
        lens = torch.randint(1, S_cap + 1, (B,), generator=g, dtype=torch.int32)
        if it == 2:
            lens[:] = S_cap   # every sequence long: all cut into segments
        say(f"decode graph replay {it}: lens {lens.tolist()}")
        sl.copy_(lens)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = o.clone()
        eager = attn.attn_decode(q, kc, vc, sl)
        torch.cuda.synchronize()
        assert torch.equal(got, eager), f"replay {it} differs from the eager call"


def test_decode_binding_rejects_bad_output_and_workspace(attn):
    """The Python binding checks a caller's o and workspace before any launch."""
    B, H, S_cap, D = 2, 2, 64, 64
    sl, q, kc, vc = _decode_case(422, B, H, S_cap, D, torch.bfloat16, [10, 64])
    q, kc, vc, sl = q.cuda(), kc.cuda(), vc.cuda(), sl.cuda()
    need = attn.attn_decode_workspace_bytes(B, H, S_cap, D)
    with pytest.raises(ValueError):
        attn.attn_decode(q, kc, vc, sl, o=torch.empty(B, 1, H, D, dtype=torch.bfloat16))   # CPU o
    with pytest.raises(ValueError):
        attn.attn_decode(q, kc, vc, sl, o=torch.empty(B, 1, H, D // 2, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        attn.attn_decode(q, kc, vc, sl, o=torch.empty(B, 1, H, D, dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):
        attn.attn_decode(q, kc, vc, sl, workspace=torch.empty(need, dtype=torch.uint8))   # CPU workspace
    with pytest.raises(attn.AttnError) as e:
        attn.attn_decode(q, kc, vc, sl, workspace=torch.empty(need - 16, dtype=torch.uint8, device="cuda"))
    assert e.value.status == attn.ATTN_ERR_WORKSPACE
    with pytest.raises(ValueError):
        attn.attn_decode(q, kc, vc, sl, workspace=torch.empty(2, need, dtype=torch.uint8, device="cuda")[:, 0])
    o = attn.attn_decode(q, kc, vc, sl, workspace=torch.empty(need, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    check(o, oracle.attn_decode(q.cpu(), kc.cpu(), vc.cpu(), sl.cpu().numpy()), torch.bfloat16, "binding")


def test_decode_matches_forward_with_one_query(attn):
    """attn_decode row b equals attn_fwd(S_q = 1, S_kv = len_b) on the same data."""
    B, H, S_cap, D = 4, 4, 700, 128
    lens = [700, 1, 333, 257]
    g = torch.Generator().manual_seed(300)
    q = torch.randn(B, 1, H, D, generator=g).bfloat16().cuda()
    kc = torch.randn(B, S_cap, H, D, generator=g).bfloat16().cuda()
    vc = torch.randn(B, S_cap, H, D, generator=g).bfloat16().cuda()
    o = attn.attn_decode(q, kc, vc, torch.tensor(lens, dtype=torch.int32).cuda())
    for b, n in enumerate(lens):
        of = attn.attn_fwd(q[b:b + 1], kc[b:b + 1, :n].contiguous(), vc[b:b + 1, :n].contiguous(), causal=True)
        d = (of.float() - o[b:b + 1].float()).abs().max().item()
        assert d <= 2e-2, (b, n, d)


@pytest.mark.parametrize("shape", [(1, 2, 300, 300, 128, True), (2, 3, 130, 200, 64, True),
                                   (1, 1, 77, 77, 32, False), (1, 2, 33, 1000, 64, True)],
                         ids=lambda s: "x".join(map(str, s)))
def test_fp32_mfma_kernel_against_row_kernel(attn, shape, monkeypatch):
    """fp32: the MFMA kernel (default) and the row kernel (ATTN_ALGO=row) both meet the 1e-4 bar."""
    B, H, S_q, S_kv, D, causal = shape
    say(f"fp32 mfma vs row {shape}")
    q, k, v = workloads.make_prefill_shape(11, torch.float32, B, H, S_q, S_kv, D)
    ref = oracle.attn_fwd(q, k, v, causal)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    assert attn.attn_fwd_plan(B, H, S_q, S_kv, D, causal, attn.ATTN_F32).kernel == 3
    o_mfma = attn.attn_fwd(qc, kc, vc, causal=causal)
    monkeypatch.setenv("ATTN_ALGO", "row")
    assert attn.attn_fwd_plan(B, H, S_q, S_kv, D, causal, attn.ATTN_F32).kernel == 2
    o_row = attn.attn_fwd(qc, kc, vc, causal=causal)
    torch.cuda.synchronize()
    check(o_mfma, ref, torch.float32, "mfma")
    check(o_row, ref, torch.float32, "row")


# ---------------------------------------------------------------------------
# KV-cache prefill (chunk of queries, per-entry lengths) and its log-sum-exp.
# LSE bars: the kernels add up the probabilities as rounded for P.V, so in
# bf16 the row sum carries a relative error up to 2^-9 and the log of it an
# absolute error up to about 2e-3 (plus fp32 rounding of the scores): bar
# 4e-3; in fp16 the relative error is up to 2^-11, the log error about 5e-4:
# bar 1e-3. fp32 inputs go through the fp32 MFMA kernel (fp32 throughout): bar 1e-5.
# ---------------------------------------------------------------------------
LSE_ATOL = {torch.bfloat16: 4e-3, torch.float16: 1e-3, torch.float32: 1e-5}


def check_lse(got: torch.Tensor, ref: np.ndarray, dtype: torch.dtype, what: str = ""):
    g = got.detach().cpu().double().numpy()
    assert g.shape == ref.shape, what
    assert np.array_equal(np.isneginf(g), np.isneginf(ref)), f"{what}: -inf rows differ"
    fin = np.isfinite(ref)
    assert np.all(np.isfinite(g[fin])), f"{what}: non-finite lse"
    err = float(np.abs(g[fin] - ref[fin]).max()) if fin.any() else 0.0
    assert err <= LSE_ATOL[dtype], f"{what}: lse max abs err {err:.3e} > {LSE_ATOL[dtype]}"
    return err


def test_kvcache_workload(attn):
    cfg = workloads.BF16_KVCACHE
    sl, q, kc, vc = workloads.make_kvcache_prefill(cfg, nan_fill=True)
    say(f"kvcache {cfg.name} B={cfg.B} S_q={cfg.S_q} S_cap={cfg.S_cap} lengths {sl.tolist()}")
    o, lse = attn.attn_fwd_kvcache(q.cuda(), kc.cuda(), vc.cuda(), sl.cuda(), causal=True, return_lse=True)
    torch.cuda.synchronize()
    ro, rlse = oracle.attn_fwd_kvcache(q, kc, vc, sl.numpy(), causal=True)
    ma, rel = check(o, ro, torch.bfloat16, "kvcache workload")
    le = check_lse(lse, rlse, torch.bfloat16, "kvcache workload")
    say(f"kvcache: max abs {ma:.2e}, rel L2 {rel:.2e}, lse max abs {le:.2e}")


KV_EDGE = [  # (B, H, S_q, S_cap, D, causal, lengths)
    (4, 2, 65, 200, 128, True, [200, 130, 64, 1]),          # entries shorter than the chunk
    (3, 1, 129, 129, 64, True, [0, 129, 300]),              # empty entry, clamped length
    (2, 3, 7, 90, 32, True, [90, 7]),
    (3, 2, 130, 400, 128, False, [400, 129, 5]),
    (2, 2, 1, 77, 128, True, [77, 33]),                      # one query = decode
    (1, 4, 300, 1000, 128, True, [999]),
]


@pytest.mark.parametrize("dtype", ALL_DTYPES, ids=DTYPE_IDS)
@pytest.mark.parametrize("case", KV_EDGE, ids=lambda c: "x".join(map(str, c[:6])))
def test_kvcache_edge_cases(attn, case, dtype):
    B, H, S_q, S_cap, D, causal, lens = case
    say(f"kvcache edge {case} {dtype}")
    cfg = workloads.KVCachePrefill("edge", dtype, B, H, S_q, S_cap, D, 400 + D, 1, S_cap, causal)
    sl, q, kc, vc = workloads.make_kvcache_prefill(cfg, nan_fill=True, seqlens=lens)
    o, lse = attn.attn_fwd_kvcache(q.cuda(), kc.cuda(), vc.cuda(), sl.cuda(), causal=causal, return_lse=True)
    ro, rlse = oracle.attn_fwd_kvcache(q, kc, vc, sl.numpy(), causal=causal)
    check(o, ro, dtype, f"kvcache {case}")
    check_lse(lse, rlse, dtype, f"kvcache {case}")
    # rows that see no key come out exactly 0
    empty = np.isneginf(rlse).all(axis=1)          # B, S_q
    assert torch.all(o.cpu()[torch.from_numpy(empty)] == 0)


@pytest.mark.parametrize("dtype", ALL_DTYPES, ids=DTYPE_IDS)
@pytest.mark.parametrize("B,H,S_q", [(70, 3, 200), (130, 1, 300)], ids=["140_classes", "390_classes"])
def test_kvcache_many_entries(attn, B, H, S_q, dtype):
    """Many entries: up to 256 (entry, block) classes are ranked by cost in
    LDS, beyond that the entries keep the launch order; both orders place
    every item once. H = 3 and 1 are not multiples of the 8 XCDs."""
    S_cap, D = 320, 64
    say(f"kvcache many entries B={B} H={H} S_q={S_q} {dtype}")
    cfg = workloads.KVCachePrefill("many", dtype, B, H, S_q, S_cap, D, 450 + B, 1, S_cap, True)
    lens = [int(x) for x in torch.randint(0, S_cap + 1, (B,), generator=torch.Generator().manual_seed(B))]
    sl, q, kc, vc = workloads.make_kvcache_prefill(cfg, nan_fill=True, seqlens=lens)
    o, lse = attn.attn_fwd_kvcache(q.cuda(), kc.cuda(), vc.cuda(), sl.cuda(), causal=True, return_lse=True)
    ro, rlse = oracle.attn_fwd_kvcache(q, kc, vc, sl.numpy(), causal=True)
    check(o, ro, dtype, f"kvcache many entries B={B}")
    check_lse(lse, rlse, dtype, f"kvcache many entries B={B}")


@pytest.mark.parametrize("dtype", ALL_DTYPES, ids=DTYPE_IDS)
def test_kvcache_without_lengths_is_attn_fwd_bitwise(attn, dtype):
    q, k, v = workloads.make_prefill_shape(500, dtype, 2, 4, 200, 333, 128)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    for causal in (True, False):
        o1 = attn.attn_fwd(q, k, v, causal=causal)
        o2, lse = attn.attn_fwd_kvcache(q, k, v, None, causal=causal, return_lse=True)
        o3 = attn.attn_fwd_kvcache(q, k, v, torch.full((2,), 333, dtype=torch.int32, device="cuda"), causal=causal)
        assert torch.equal(o1, o2) and torch.equal(o1, o3)
        _, rlse = oracle.attn_fwd_kvcache(q.cpu(), k.cpu(), v.cpu(), None, causal=causal)
        check_lse(lse, rlse, dtype, f"lse causal={causal}")


# ---------------------------------------------------------------------------
# Key-padding mask (attn_fwd_mask) and its log-sum-exp
# ---------------------------------------------------------------------------
MASK_CASES = [  # (B, H, S_q, S_kv, D, causal, pattern)
    (3, 2, 200, 200, 128, True, "random"),
    (2, 3, 129, 300, 64, True, "right_pad"),      # padded tail of each entry
    (2, 2, 65, 130, 32, False, "left_pad"),       # padded head of each entry
    (4, 2, 77, 77, 128, True, "edge_entries"),    # an entry fully hidden, one with only its last key
    (1, 4, 1000, 1000, 128, True, "random"),
    (2, 1, 33, 513, 128, False, "random"),
    (2, 2, 300, 300, 64, True, "right_pad"),      # causal, paired blocks, trailing tiles skipped
    (3, 2, 300, 300, 128, True, "left_pad"),      # causal, leading tiles skipped
    (2, 2, 200, 256, 64, True, "tile_pad"),       # visible keys end on a tile boundary
    (2, 3, 150, 300, 128, False, "right_pad_hole"),   # right padding and one hidden key inside
    (2, 2, 129, 300, 128, True, "right_pad_hole"),
]


def _make_mask(pattern, B, S_kv, seed):
    g = torch.Generator().manual_seed(seed)
    if pattern == "random":
        m = torch.rand(B, S_kv, generator=g) < 0.6
    elif pattern == "right_pad":
        n = torch.randint(1, S_kv + 1, (B,), generator=g)
        m = torch.arange(S_kv)[None, :] < n[:, None]
    elif pattern == "tile_pad":
        n = 64 * torch.randint(1, S_kv // 64 + 1, (B,), generator=g)
        m = torch.arange(S_kv)[None, :] < n[:, None]
    elif pattern == "right_pad_hole":
        n = torch.randint(2, S_kv + 1, (B,), generator=g)
        m = torch.arange(S_kv)[None, :] < n[:, None]
        m[torch.arange(B), n // 2] = False
    elif pattern == "left_pad":
        n = torch.randint(0, S_kv, (B,), generator=g)
        m = torch.arange(S_kv)[None, :] >= n[:, None]
    else:
        m = torch.rand(B, S_kv, generator=g) < 0.5
        m[0] = False
        m[1] = False
        m[1, -1] = True
    return m


@pytest.mark.parametrize("dtype", ALL_DTYPES, ids=DTYPE_IDS)
@pytest.mark.parametrize("case", MASK_CASES, ids=lambda c: "x".join(map(str, c[:6])) + "_" + c[6])
def test_key_mask_against_oracle(attn, case, dtype):
    B, H, S_q, S_kv, D, causal, pattern = case
    say(f"key mask {case} {dtype}")
    q, k, v = workloads.make_prefill_shape(600 + D, dtype, B, H, S_q, S_kv, D)
    m = _make_mask(pattern, B, S_kv, 700 + S_kv)
    o, lse = attn.attn_fwd_mask(q.cuda(), k.cuda(), v.cuda(), m.cuda(), causal=causal, return_lse=True)
    torch.cuda.synchronize()
    ro, rlse = oracle.attn_fwd_mask(q, k, v, m.numpy(), causal)
    check(o, ro, dtype, f"mask {case}")
    check_lse(lse, rlse, dtype, f"mask {case}")
    empty = np.isneginf(rlse).all(axis=1)          # B, S_q: rows with no visible key
    assert torch.all(o.cpu()[torch.from_numpy(empty)] == 0)


@pytest.mark.parametrize("dtype", ALL_DTYPES, ids=DTYPE_IDS)
def test_key_mask_absent_or_all_visible_is_attn_fwd(attn, dtype):
    """No mask is the attn_fwd kernel itself, and an all-visible mask hides no
    key, so the key-mask instantiation runs the same unmasked steps in the
    same order: both bitwise equal to attn_fwd."""
    for D in (128, 64, 32):
        q, k, v = (t.cuda() for t in workloads.make_prefill_shape(610 + D, dtype, 2, 3, 300, 300, D))
        for causal in (True, False):
            ref = attn.attn_fwd(q, k, v, causal=causal)
            o1 = attn.attn_fwd_mask(q, k, v, None, causal=causal)
            o2 = attn.attn_fwd_mask(q, k, v, torch.ones(2, 300, dtype=torch.bool, device="cuda"), causal=causal)
            assert torch.equal(o1, ref)
            assert torch.equal(o2, ref), f"all-visible mask D={D} causal={causal}"


@pytest.mark.parametrize("dtype", ALL_DTYPES, ids=DTYPE_IDS)
def test_key_mask_right_padding_is_a_key_length(attn, dtype):
    """A mask that hides only a suffix of each entry is that entry's key
    length: without the causal rule the result is bitwise that of
    attn_fwd_kvcache with the same lengths (the same steps over keys [0, n)),
    whatever the padding slots hold."""
    B, H, S, D = 3, 2, 300, 128
    q, k, v = workloads.make_prefill_shape(670, dtype, B, H, S, S, D)
    n = torch.tensor([300, 1, 193], dtype=torch.int32)
    m = torch.arange(S)[None, :] < n[:, None].long()
    kp, vp = _poison_hidden(k, m), _poison_hidden(v, m)
    o, lse = attn.attn_fwd_mask(q.cuda(), kp.cuda(), vp.cuda(), m.cuda(), causal=False, return_lse=True)
    ok, lsek = attn.attn_fwd_kvcache(q.cuda(), kp.cuda(), vp.cuda(), n.cuda(), causal=False, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o, ok) and torch.equal(lse, lsek)


NAN_PAD_CASES = [  # (B, H, S_q, S_kv, D, causal, pattern)
    (3, 2, 200, 200, 128, True, "random"),
    (2, 3, 129, 300, 64, False, "right_pad"),
    (2, 2, 65, 131, 32, True, "left_pad"),     # odd S_kv: mask rows start at every address mod 4
    (2, 2, 300, 300, 128, False, "right_pad"),
]


def _poison_hidden(t, m):
    """K or V with every row of a hidden key (all heads) set to NaN, +inf or
    -inf in turn: the contents of an unwritten padding slot."""
    t = t.clone()
    bad = torch.tensor([float("nan"), float("inf"), float("-inf")], dtype=t.dtype)
    idx = (~m).nonzero()
    for n, (b, j) in enumerate(idx.tolist()):
        t[b, j] = bad[n % 3]
    return t


@pytest.mark.parametrize("dtype", ALL_DTYPES, ids=DTYPE_IDS)
@pytest.mark.parametrize("case", NAN_PAD_CASES, ids=lambda c: "x".join(map(str, c[:6])) + "_" + c[6])
def test_key_mask_ignores_nan_in_padding(attn, case, dtype):
    """Hidden keys' K and V rows never reach the result: with NaN and +-inf in
    every padding slot the output and log-sum-exp are bitwise those of the
    same call on finite padding, and match the oracle on the finite data."""
    B, H, S_q, S_kv, D, causal, pattern = case
    say(f"NaN padding {case} {dtype}")
    q, k, v = workloads.make_prefill_shape(640 + D, dtype, B, H, S_q, S_kv, D)
    m = _make_mask(pattern, B, S_kv, 650 + S_kv)
    kp, vp = _poison_hidden(k, m), _poison_hidden(v, m)
    assert torch.isnan(kp.float()).any() and torch.isinf(vp.float()).any()
    o, lse = attn.attn_fwd_mask(q.cuda(), k.cuda(), v.cuda(), m.cuda(), causal=causal, return_lse=True)
    op, lsep = attn.attn_fwd_mask(q.cuda(), kp.cuda(), vp.cuda(), m.cuda(), causal=causal, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(op, o) and torch.equal(lsep, lse)
    ro, rlse = oracle.attn_fwd_mask(q, k, v, m.numpy(), causal)
    check(op, ro, dtype, f"NaN padding {case}")
    check_lse(lsep, rlse, dtype, f"NaN padding {case}")


def test_key_mask_ignores_nan_in_padding_row_kernel(attn, monkeypatch):
    """The same for the per-query row kernel (the cross-check path)."""
    B, H, S, D = 2, 2, 150, 64
    q, k, v = workloads.make_prefill_shape(660, torch.bfloat16, B, H, S, S, D)
    m = _make_mask("right_pad", B, S, 661)
    kp, vp = _poison_hidden(k, m), _poison_hidden(v, m)
    monkeypatch.setenv("ATTN_ALGO", "row")
    o = attn.attn_fwd_mask(q.cuda(), kp.cuda(), vp.cuda(), m.cuda(), causal=True)
    torch.cuda.synchronize()
    check(o, oracle.attn_fwd_mask(q, k, v, m.numpy(), True)[0], torch.bfloat16, "NaN padding row kernel")


def test_key_mask_unaligned_rows_and_long_rows(attn):
    """A mask that starts 1-3 bytes past an aligned address, rows longer than
    one pass of the kernel's visibility scan (16 bytes per thread, up to
    40,000 keys), and 300 entries of a ragged 65-key row."""
    for (B, H, S_q, S_kv, D, causal, pattern, off) in [(3, 2, 130, 257, 128, True, "random", 3),
                                                       (1, 2, 64, 9001, 64, False, "left_pad", 1),
                                                       (2, 1, 40, 8500, 32, False, "right_pad", 2),
                                                       (2, 1, 32, 40000, 64, False, "right_pad", 1),
                                                       (300, 1, 16, 65, 32, True, "random", 2)]:
        say(f"mask at offset {off}: {(B, H, S_q, S_kv, D, causal, pattern)}")
        q, k, v = workloads.make_prefill_shape(670 + D, torch.bfloat16, B, H, S_q, S_kv, D)
        m = _make_mask(pattern, B, S_kv, 671 + S_kv)
        buf = torch.zeros(off + B * S_kv + 5, dtype=torch.uint8, device="cuda")
        mv = buf[off:off + B * S_kv].view(B, S_kv)
        mv.copy_(m.to(torch.uint8).cuda())
        assert mv.data_ptr() % 4 == off % 4
        o, lse = attn.attn_fwd_mask(q.cuda(), k.cuda(), v.cuda(), mv, causal=causal, return_lse=True)
        torch.cuda.synchronize()
        ro, rlse = oracle.attn_fwd_mask(q, k, v, m.numpy(), causal)
        check(o, ro, torch.bfloat16, f"mask offset {off}")
        check_lse(lse, rlse, torch.bfloat16, f"mask offset {off}")


def test_key_mask_row_kernel_cross_check(attn, monkeypatch):
    B, H, S, D = 2, 2, 150, 64
    q, k, v = workloads.make_prefill_shape(620, torch.bfloat16, B, H, S, S, D)
    m = _make_mask("random", B, S, 621)
    ro, _ = oracle.attn_fwd_mask(q, k, v, m.numpy(), True)
    monkeypatch.setenv("ATTN_ALGO", "row")
    o_row = attn.attn_fwd_mask(q.cuda(), k.cuda(), v.cuda(), m.cuda(), causal=True)
    monkeypatch.setenv("ATTN_ALGO", "tile")
    o_tile = attn.attn_fwd_mask(q.cuda(), k.cuda(), v.cuda(), m.cuda(), causal=True)
    torch.cuda.synchronize()
    check(o_row, ro, torch.bfloat16, "mask row kernel")
    check(o_tile, ro, torch.bfloat16, "mask tile kernel")


def test_fp16_prefill_full_size(attn):
    """The fp16_s2048 workload (the bf16_s2048 shape, B=1 H=32 S=2048 D=128,
    causal, in fp16) at full size, the data and launch bench.py times."""
    q, k, v = workloads.make_prefill(workloads.FP16_S2048)
    say("fp16 prefill B=1 H=32 S=2048 D=128")
    o = attn.attn_fwd(q.cuda(), k.cuda(), v.cuda(), causal=True)
    torch.cuda.synchronize()
    max_abs, rel = check(o, oracle.attn_fwd(q, k, v, True), torch.float16, "fp16 s2048")
    say(f"  fp16 s2048: max abs {max_abs:.3e} rel L2 {rel:.3e}")


def test_noncausal_prefill_full_size(attn):
    """The bf16_s2048 data without the causal rule, the launch bench.py times
    (two query blocks per workgroup, every block walking all 32 key tiles)."""
    q, k, v = workloads.make_prefill(workloads.BF16_S2048)
    say("bf16 non-causal prefill B=1 H=32 S=2048 D=128")
    o = attn.attn_fwd(q.cuda(), k.cuda(), v.cuda(), causal=False)
    torch.cuda.synchronize()
    max_abs, rel = check(o, oracle.attn_fwd(q, k, v, False), torch.bfloat16, "non-causal s2048")
    say(f"  non-causal s2048: max abs {max_abs:.3e} rel L2 {rel:.3e}")


def test_keypad_prefill_full_size(attn):
    """The bf16_keypad workload (B=8 right-padded entries of S=1024, H=32,
    D=128, no causal rule) at full size, the data and launch bench.py times,
    with its log-sum-exp."""
    cfg = workloads.BF16_KEYPAD
    lens, mask, q, k, v = workloads.make_keypad_prefill(cfg)
    say(f"key-padding prefill full size, lengths {lens.tolist()}")
    o, lse = attn.attn_fwd_mask(q.cuda(), k.cuda(), v.cuda(), mask.cuda(), causal=False, return_lse=True)
    torch.cuda.synchronize()
    ro, rlse = oracle.attn_fwd_mask(q, k, v, mask.numpy(), False)
    max_abs, rel = check(o, ro, torch.bfloat16, "keypad full size")
    check_lse(lse, rlse, torch.bfloat16, "keypad full size")
    say(f"  keypad: max abs {max_abs:.3e} rel L2 {rel:.3e}")


# ---------------------------------------------------------------------------
# Q/K/V projection GEMM (attn_qkv_proj)
# ---------------------------------------------------------------------------
QKV_CASES = [  # (B, S, E, H, D)
    (1, 300, 128, 2, 64),       # M not a multiple of the 256-row tile
    (2, 130, 256, 3, 32),       # 3N = 288: one 384-column tile, its last wave column past 3N
    (1, 512, 512, 4, 128),      # 384-column tiles straddle the Q/K and K/V boundaries
    (1, 1, 32, 1, 32),          # one row, one K step
    (1, 100, 96, 2, 32),        # three K steps: the loop's second half runs once less
    (1, 100, 192, 2, 32),
    (3, 77, 1024, 8, 64),
]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("case", QKV_CASES, ids=lambda c: "x".join(map(str, c)))
def test_qkv_proj_against_oracle(attn, case, dtype):
    B, S, E, H, D = case
    say(f"qkv proj {case} {dtype}")
    cfg = workloads.QkvProj("edge", dtype, B, S, E, H, D, 900 + E)
    x, w = workloads.make_qkv_proj(cfg)
    q, k, v = attn.qkv_proj(x.cuda(), w.cuda(), H, D)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.qkv_proj(x, w, H, D)
    for name, got, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        check(got, ref, dtype, f"qkv {case} {name}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
def test_qkv_proj_identity_weights_copy_x_bitwise(attn, dtype):
    """W_Q = I, W_K = 2I, W_V = I: fp32 sums of one nonzero product round back exactly."""
    B, S, H, D = 2, 300, 4, 64
    E = H * D
    x = torch.randn(B, S, E, generator=torch.Generator().manual_seed(910)).to(dtype)
    eye = torch.eye(E)
    w = torch.cat([eye, 2 * eye, eye], 0).to(dtype)
    q, k, v = attn.qkv_proj(x.cuda(), w.cuda(), H, D)
    xs = x.reshape(B, S, H, D)
    assert torch.equal(q.cpu(), xs) and torch.equal(v.cpu(), xs) and torch.equal(k.cpu(), (2 * xs.float()).to(dtype))


def test_qkv_proj_full_size_sampled_rows(attn):
    """The bf16_qkv workload at full size, in the launch bench.py times; the
    oracle checks a sample of rows (each row of the output depends on one
    row of X only)."""
    cfg = workloads.BF16_QKV
    say(f"qkv proj full size M={cfg.B * cfg.S} E={cfg.E} N={cfg.H * cfg.D}")
    x, w = workloads.make_qkv_proj(cfg)
    q, k, v = attn.qkv_proj(x.cuda(), w.cuda(), cfg.H, cfg.D)
    torch.cuda.synchronize()
    rows = [0, 1, 255, 256, 777, 1024, 1535, 2046, 2047]
    rq, rk, rv = oracle.qkv_proj(x[:, rows], w, cfg.H, cfg.D)
    for name, got, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        check(got[:, rows], ref, torch.bfloat16, f"qkv full {name}")


# ---------------------------------------------------------------------------
# Sinusoidal position encoding (attn_sinusoidal_pe)
# Bar: fp32 sin/cos of an angle reduced to [-pi, pi] in fp64 are within
# about 1 ulp (1.2e-7) plus the rounding of the reduced angle to fp32 (up to
# 1.9e-7 rad); the fp64 angle itself (in the kernel and in the oracle) is off
# by up to about 1.1e-16 * pos rad. So: 3e-7 + 2.5e-16 * largest position.
# ---------------------------------------------------------------------------
PE_CASES = [  # (S, d_model, pos0)
    (1, 2, 0),
    (37, 64, 0),
    (300, 4096, 0),          # the model width of the bf16_s2048 layer
    (17, 128, 100_000),      # an offset block of positions (decode steps)
    (6, 8, (1 << 31) - 6),   # the largest positions the interface allows
    (9, 6, 5),               # an odd number of pairs: the last thread has one
    (5, 10, 3),              # rows not 16-byte aligned: 8-byte stores
]


@pytest.mark.parametrize("case", PE_CASES, ids=lambda c: "x".join(map(str, c)))
def test_sinusoidal_pe_against_oracle(attn, case):
    S, d, pos0 = case
    say(f"pe {case}")
    pe = attn.sinusoidal_pe(S, d, pos0).cpu().double().numpy()
    ref = oracle.sinusoidal_pe(S, d, pos0)
    bar = 3e-7 + 2.5e-16 * (pos0 + S)
    err = float(np.abs(pe - ref).max())
    assert err <= bar, f"pe {case}: max abs err {err:.3e} > {bar:.3e}"


def test_sinusoidal_pe_full_size(attn):
    """The table bench.py times: 4096 positions x d_model 4096."""
    S, d = workloads.PE_S, workloads.PE_D
    say(f"pe full size {S} x {d}")
    pe = attn.sinusoidal_pe(S, d).cpu().double().numpy()
    ref = oracle.sinusoidal_pe(S, d, 0)
    bar = 3e-7 + 2.5e-16 * S
    err = float(np.abs(pe - ref).max())
    assert err <= bar, f"pe full size: max abs err {err:.3e} > {bar:.3e}"


def test_sinusoidal_pe_output_aligned_to_8_bytes_only(attn):
    """A d_model that allows 16-byte row stores, written into a buffer that
    is only 8-byte aligned: the kernel takes its 8-byte store path."""
    S, d = 7, 64
    buf = torch.full((S * d + 2,), float("nan"), dtype=torch.float32, device="cuda")
    view = buf[2:].view(S, d)
    assert view.data_ptr() % 16 == 8
    attn.sinusoidal_pe(S, d, 11, out=view)
    torch.cuda.synchronize()
    ref = oracle.sinusoidal_pe(S, d, 11)
    assert float(np.abs(view.cpu().double().numpy() - ref).max()) <= 3e-7 + 2.5e-16 * (11 + S)
    assert torch.isnan(buf[:2].cpu()).all()   # nothing written before the table


def test_sinusoidal_pe_position_zero_is_exact(attn):
    pe = attn.sinusoidal_pe(1, 512).cpu()
    assert torch.all(pe[0, 0::2] == 0.0) and torch.all(pe[0, 1::2] == 1.0)


# ---------------------------------------------------------------------------
# Standalone masked softmax (attn_masked_softmax)
# Bars: the check() bars above; the probabilities lie in [0, 1], so the fp32
# bar is loose (fp32 exp2 and one division give a few ulp) and the 16-bit bars
# cover the output rounding (half an ulp of p <= 1). Masked entries must be 0
# exactly, whatever the input holds there.
# ---------------------------------------------------------------------------
SM_CASES = [  # (B, H, S_q, S_kv, causal, scale, std)
    (1, 1, 1, 8, True, 1.0, 1.0),               # one row, one chunk
    (2, 3, 37, 64, True, 0.125, 8.0),           # S_q < S_kv; 222 rows: the last workgroup holds 2
    (1, 2, 64, 64, False, 1.0, 1.0),
    (1, 1, 100, 40, True, 0.5, 2.0),            # S_q > S_kv: the first 60 rows see no key
    (1, 2, 300, 1024, True, 0.088, 11.3),       # 4 KiB fp32 rows: the largest small-register variant
    (1, 1, 130, 2048, True, 0.088, 11.3),       # 4 KiB 16-bit rows / 8 KiB fp32 rows
    (1, 1, 50, 2056, True, 1.0, 30.0),          # one chunk past 4 KiB (16-bit); logits to +-100
    (1, 1, 64, "max", True, 0.088, 11.3),       # 16 KiB rows: the largest the interface takes
    (1, 1, 19, "max", False, 0.088, 11.3),
]


def _sm_skv(S_kv, dtype):
    return (16384 // torch.empty(0, dtype=dtype).element_size()) if S_kv == "max" else S_kv


def _draw_scores(seed, dtype, B, H, S_q, S_kv, std):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(B, H, S_q, S_kv, generator=g) * std).to(dtype)


def _visible(S_q, S_kv, causal):
    i = torch.arange(S_q)[:, None]
    j = torch.arange(S_kv)[None, :]
    return (j <= i + (S_kv - S_q)) if causal else torch.ones(S_q, S_kv, dtype=torch.bool)


@pytest.mark.parametrize("dtype", ALL_DTYPES, ids=DTYPE_IDS)
@pytest.mark.parametrize("case", SM_CASES, ids=lambda c: "x".join(map(str, c[:5])))
def test_masked_softmax_against_oracle(attn, case, dtype):
    B, H, S_q, S_kv, causal, scale, std = case
    S_kv = _sm_skv(S_kv, dtype)
    say(f"masked softmax {(B, H, S_q, S_kv, causal)} {dtype}")
    s = _draw_scores(1100 + S_q, dtype, B, H, S_q, S_kv, std)
    p = attn.masked_softmax(s.cuda(), scale, causal).cpu()
    ref = oracle.masked_softmax(s, scale, causal)
    check(p, ref, dtype, f"softmax {case}")
    vis = _visible(S_q, S_kv, causal).expand(B, H, S_q, S_kv)
    assert torch.all(p[~vis] == 0), "masked entries must be exactly 0"
    sums = p.double().sum(-1)
    has = vis.any(-1)
    tol = 1e-5 if dtype == torch.float32 else 2e-2
    assert torch.all(sums[~has] == 0) and torch.allclose(sums[has], torch.ones_like(sums[has]), atol=tol)


@pytest.mark.parametrize("dtype", ALL_DTYPES, ids=DTYPE_IDS)
def test_masked_softmax_ignores_masked_inputs_and_runs_in_place(attn, dtype):
    """NaN and +inf above the causal limit are never read; p may be s itself."""
    B, H, S_q, S_kv = 2, 2, 48, 64
    s = _draw_scores(1180, dtype, B, H, S_q, S_kv, 3.0)
    ref = oracle.masked_softmax(s, 0.5, True)
    vis = _visible(S_q, S_kv, True)
    poisoned = s.clone()
    poisoned[..., ~vis] = float("nan")
    poisoned[..., 0, -1] = float("inf")
    g = poisoned.cuda()
    clean = attn.masked_softmax(s.cuda(), 0.5, True)
    out = attn.masked_softmax(g, 0.5, True, out=g)
    torch.cuda.synchronize()
    assert out.data_ptr() == g.data_ptr()
    check(out, ref, dtype, "in place, poisoned")
    assert torch.equal(out.cpu(), clean.cpu()), "the masked inputs changed the result"


def test_masked_softmax_full_size_sampled_rows(attn):
    """The bf16_softmax workload at full size, in the launch bench.py times.
    Row i of a head depends only on its own visible scores, so the oracle
    takes each sampled row alone as a one-query softmax over keys 0..i."""
    cfg = workloads.BF16_SOFTMAX
    say(f"masked softmax full size {cfg}")
    s = workloads.make_scores(cfg)
    p = attn.masked_softmax(s.cuda(), cfg.scale, cfg.causal)
    torch.cuda.synchronize()
    samples = [(0, 0), (0, 2047), (5, 1), (13, 640), (31, 2046), (31, 2047), (17, 1023), (22, 1024)]
    p_rows = p[0, [h for h, _ in samples], [i for _, i in samples]].cpu()
    for k, (h, i) in enumerate(samples):
        ref = oracle.masked_softmax(s[0, h, i, : i + 1].reshape(1, 1, 1, i + 1), cfg.scale, True)
        check(p_rows[k, : i + 1].reshape(1, 1, 1, i + 1), ref, torch.bfloat16, f"row ({h}, {i})")
        assert torch.all(p_rows[k, i + 1:] == 0)


# ---------------------------------------------------------------------------
# Error paths through the binding on a live device
# ---------------------------------------------------------------------------
def test_length_check_env_rejects_clamped_lengths(attn, monkeypatch):
    """ATTN_CHECK=1: lengths the kernels would clamp (below 0, above the cache
    capacity) are rejected on the host before any launch; valid lengths give
    the same bits as without the check."""
    B, H, S_cap, D = 3, 2, 40, 64
    g = torch.Generator().manual_seed(420)
    q = torch.randn(B, 1, H, D, generator=g).to(torch.bfloat16).cuda()
    kc = torch.randn(B, S_cap, H, D, generator=g).to(torch.bfloat16).cuda()
    vc = torch.randn(B, S_cap, H, D, generator=g).to(torch.bfloat16).cuda()
    good = torch.tensor([0, 17, S_cap], dtype=torch.int32, device="cuda")
    plain = attn.attn_decode(q, kc, vc, good)
    qs = torch.randn(B, 8, H, D, generator=g).to(torch.bfloat16).cuda()
    plain_kv = attn.attn_fwd_kvcache(qs, kc, vc, good, causal=True)
    monkeypatch.setenv("ATTN_CHECK", "1")
    checked = attn.attn_decode(q, kc, vc, good)
    checked_kv = attn.attn_fwd_kvcache(qs, kc, vc, good, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(plain.cpu(), checked.cpu()) and torch.equal(plain_kv.cpu(), checked_kv.cpu())
    for bad in ([5, -1, 3], [5, S_cap + 1, 3]):
        lens = torch.tensor(bad, dtype=torch.int32, device="cuda")
        with pytest.raises(attn.AttnError) as e:
            attn.attn_decode(q, kc, vc, lens)
        assert e.value.status == attn.ATTN_ERR_INVALID_ARG and "ATTN_CHECK" in str(e.value)
        with pytest.raises(attn.AttnError) as e:
            attn.attn_fwd_kvcache(qs, kc, vc, lens, causal=True)
        assert e.value.status == attn.ATTN_ERR_INVALID_ARG and "length[1]" in str(e.value)


def test_error_paths_on_device(attn):
    q = torch.zeros(1, 8, 2, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(attn.AttnError) as e:
        attn.attn_fwd(q, q, q, q, causal=True)            # output aliases the inputs
    assert e.value.status == attn.ATTN_ERR_INVALID_ARG
    sl = torch.ones(1, dtype=torch.int32, device="cuda")
    qd = torch.zeros(1, 1, 2, 128, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(1, 16, 2, 128, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(attn.AttnError) as e:
        attn.attn_decode(qd, kc, kc, sl, workspace=ws)
    assert e.value.status == attn.ATTN_ERR_WORKSPACE
