"""Pins for the fp64 oracle: it is checked against things other than itself.

Each test names the passage or the mathematical fact it relies on. The
oracle follows the "Hand-written Masked Multi-Head Attention CUDA kernel"
page (section 2: A = softmax(QK^T/sqrt(d_k) + M), O = A.V; section 2.1:
[B,S,H,D] layout; section 2.2: key j visible iff j <= i) and the "Week-4
CUDA notes" page, section 2.2 (-inf mask gives exp = 0; subtract the max).

What each kind of mistake would trip:
  dropped or wrong scale, transposed operand, wrong stride  -> library and golden pins
  diagonal hidden or mask off by one                        -> row-0, golden, masked-zero pins
  wrong S_q != S_kv alignment                               -> golden bottom-right case
  missing normalisation / max subtraction overflow          -> row sums, large-logit test
  decode reading past the length                            -> NaN-filled cache test
  log-sum-exp without the max, or ignoring the entry lengths -> golden, SDPA/logsumexp, merge pins
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "geometric_weights.json")


def rnd(seed, *shape, std=1.0):
    g = np.random.default_rng(seed)
    return g.standard_normal(shape) * std


def sdpa_f64(q, k, v, causal):
    """torch's scaled_dot_product_attention on the CPU in float64.

    For causal with S_q != S_kv the mask is passed explicitly as a boolean
    matrix (visible iff j <= i + S_kv - S_q) because torch's is_causal aligns
    top-left.
    """
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).permute(0, 2, 1, 3)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3)
    S_q, S_kv = q.shape[1], k.shape[1]
    if causal and S_q == S_kv:
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    elif causal:
        i = torch.arange(S_q)[:, None]
        j = torch.arange(S_kv)[None, :]
        mask = j <= i + (S_kv - S_q)
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    else:
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)
    return o.permute(0, 2, 1, 3).contiguous().numpy()


# --------------------------------------------------------------------------
# Library special case: torch SDPA in float64
# --------------------------------------------------------------------------
@pytest.mark.parametrize("B,H,S_q,S_kv,D,causal", [
    (1, 1, 1, 1, 8, True),
    (1, 2, 64, 64, 32, True),
    (2, 3, 37, 37, 16, True),
    (2, 2, 19, 53, 64, True),      # chunked prefill: queries are the last 19 positions
    (1, 2, 1, 70, 128, True),      # one query at the end = decode
    (2, 2, 33, 47, 32, False),
    (1, 1, 130, 130, 128, True),
])
def test_matches_sdpa_float64(B, H, S_q, S_kv, D, causal):
    q = rnd(1, B, S_q, H, D)
    k = rnd(2, B, S_kv, H, D)
    v = rnd(3, B, S_kv, H, D)
    got = oracle.attn_fwd(q, k, v, causal)
    ref = sdpa_f64(q, k, v, causal)
    assert np.max(np.abs(got - ref)) <= 1e-12


# --------------------------------------------------------------------------
# Exact closed forms (tests/golden/geometric_weights.json, written from
# fractions by tests/golden/make_golden.py, not by the oracle)
# --------------------------------------------------------------------------
def test_golden_geometric_weights():
    doc = json.load(open(GOLDEN))
    assert "section 2" in doc["citation"]
    for case in doc["cases"]:
        q = np.array(case["q"], dtype=np.float64)
        k = np.array(case["k"], dtype=np.float64)
        v = np.array(case["v"], dtype=np.float64)
        exact = np.vectorize(lambda s: float(Fraction(s)))(np.array(case["o_exact"], dtype=object))
        lse_exact = np.array([[[float(x) for x in row] for row in hb] for hb in case["lse_exact"]])
        if "seqlens" not in case:
            got = oracle.attn_fwd(q, k, v, case["causal"])
            assert got.shape == exact.shape
            np.testing.assert_allclose(got, exact.astype(np.float64), rtol=1e-13, atol=1e-14,
                                       err_msg=case["name"])
        # the KV-cache form, with the case's lengths or none (all rows valid)
        o2, lse = oracle.attn_fwd_kvcache(q, k, v, case.get("seqlens"), case["causal"])
        np.testing.assert_allclose(o2, exact.astype(np.float64), rtol=1e-13, atol=1e-14, err_msg=case["name"])
        assert np.array_equal(np.isneginf(lse), np.isneginf(lse_exact)), case["name"]
        fin = np.isfinite(lse_exact)
        np.testing.assert_allclose(lse[fin], lse_exact[fin], rtol=1e-13, atol=1e-13, err_msg=case["name"])


def test_two_keys_is_a_logistic_blend():
    """Two visible keys: weight of key 1 is 1/(1+exp(-(s1-s0))) (sigmoid)."""
    D = 1  # scale 1
    q = np.array([[[[0.7]], [[-1.3]]]])              # [1, 2, 1, 1]
    k = np.array([[[[0.5]], [[2.0]]]])
    v = np.array([[[[3.0]], [[-5.0]]]])
    o = oracle.attn_fwd(q, k, v, causal=True)
    assert o[0, 0, 0, 0] == 3.0
    w1 = 1.0 / (1.0 + math.exp(-(-1.3 * 2.0 - (-1.3 * 0.5))))
    assert abs(o[0, 1, 0, 0] - (3.0 * (1 - w1) + -5.0 * w1)) <= 1e-15
    del D


# --------------------------------------------------------------------------
# Brute force in pure Python, log-sum-exp formulation with exact summation
# --------------------------------------------------------------------------
def brute_force(q, k, v, causal):
    B, S_q, H, D = q.shape
    S_kv = k.shape[1]
    off = S_kv - S_q
    out = np.zeros_like(q)
    for b in range(B):
        for h in range(H):
            for i in range(S_q):
                vis = [j for j in range(S_kv) if not causal or j <= i + off]
                s = [math.fsum(q[b, i, h, d] * k[b, j, h, d] for d in range(D)) / math.sqrt(D)
                     for j in vis]
                top = max(s)
                lse = top + math.log(math.fsum(math.exp(x - top) for x in s))
                w = [math.exp(x - lse) for x in s]
                for d in range(D):
                    out[b, i, h, d] = math.fsum(wj * v[b, j, h, d] for wj, j in zip(w, vis))
    return out


@pytest.mark.parametrize("B,H,S_q,S_kv,D,causal", [
    (1, 1, 5, 5, 3, True), (2, 2, 7, 7, 4, True), (1, 3, 4, 9, 8, True),
    (2, 1, 6, 6, 5, False), (1, 2, 16, 16, 8, True),
])
def test_brute_force_tiny(B, H, S_q, S_kv, D, causal):
    q = rnd(11, B, S_q, H, D, std=2.0)
    k = rnd(12, B, S_kv, H, D, std=2.0)
    v = rnd(13, B, S_kv, H, D)
    got = oracle.attn_fwd(q, k, v, causal)
    assert np.max(np.abs(got - brute_force(q, k, v, causal))) <= 1e-13


# --------------------------------------------------------------------------
# Invariants
# --------------------------------------------------------------------------
def test_rows_sum_to_one_and_masked_entries_are_exactly_zero():
    B, H, S_q, S_kv, D = 2, 3, 40, 57, 16
    q, k, v = rnd(21, B, S_q, H, D, std=3), rnd(22, B, S_kv, H, D, std=3), rnd(23, B, S_kv, H, D)
    _, p = oracle.attn_fwd(q, k, v, causal=True, return_p=True)
    assert np.max(np.abs(p.sum(-1) - 1.0)) <= 1e-12
    i = np.arange(S_q)[:, None]
    j = np.arange(S_kv)[None, :]
    masked = np.broadcast_to(j > i + (S_kv - S_q), p.shape)
    assert np.all(p[masked] == 0.0)
    assert np.all(p[~masked] > 0.0)


def test_row_zero_returns_value_row_zero_exactly():
    B, H, S, D = 2, 4, 33, 32
    q, k, v = rnd(31, B, S, H, D), rnd(32, B, S, H, D), rnd(33, B, S, H, D)
    o = oracle.attn_fwd(q, k, v, causal=True)
    assert np.array_equal(o[:, 0], v[:, 0])


def test_equal_keys_give_prefix_means():
    """All keys equal -> uniform weights over the visible prefix -> O_i = mean(V_0..V_i)."""
    B, H, S, D = 1, 2, 50, 8
    q = rnd(41, B, S, H, D)
    k = np.broadcast_to(rnd(42, B, 1, H, D), (B, S, H, D)).copy()
    v = rnd(43, B, S, H, D)
    o = oracle.attn_fwd(q, k, v, causal=True)
    prefix = np.cumsum(v, axis=1) / np.arange(1, S + 1)[None, :, None, None]
    assert np.max(np.abs(o - prefix)) <= 1e-13


def test_constant_values_pass_through():
    B, H, S, D = 1, 2, 31, 16
    q, k = rnd(51, B, S, H, D, std=4), rnd(52, B, S, H, D, std=4)
    c = rnd(53, 1, 1, H, D)
    v = np.broadcast_to(c, (B, S, H, D)).copy()
    o = oracle.attn_fwd(q, k, v, causal=True)
    assert np.max(np.abs(o - v)) <= 1e-14


def test_shift_of_all_keys_leaves_output_unchanged():
    """k_j + c for one c: every score of row i moves by q_i.c/sqrt(D); softmax ignores it."""
    B, H, S, D = 1, 2, 45, 32
    q, k, v = rnd(61, B, S, H, D), rnd(62, B, S, H, D), rnd(63, B, S, H, D)
    c = rnd(64, 1, 1, H, D, std=3.0)
    o1 = oracle.attn_fwd(q, k, v, causal=True)
    o2 = oracle.attn_fwd(q, k + c, v, causal=True)
    assert np.max(np.abs(o1 - o2)) <= 1e-12


def test_large_logits_stay_finite_and_match_lse_brute_force():
    """Logits with spreads in the thousands overflow exp unless the row max is subtracted."""
    B, H, S, D = 1, 1, 12, 4
    q, k, v = rnd(71, B, S, H, D, std=30), rnd(72, B, S, H, D, std=30), rnd(73, B, S, H, D)
    o = oracle.attn_fwd(q, k, v, causal=True)
    assert np.all(np.isfinite(o))
    assert np.max(np.abs(o - brute_force(q, k, v, True))) <= 1e-12


def test_causal_prefix_consistency_is_exact():
    B, H, S, D = 1, 2, 60, 16
    q, k, v = rnd(81, B, S, H, D), rnd(82, B, S, H, D), rnd(83, B, S, H, D)
    full = oracle.attn_fwd(q, k, v, causal=True)
    for Sp in (1, 17, 59):
        part = oracle.attn_fwd(q[:, :Sp], k[:, :Sp], v[:, :Sp], causal=True)
        assert np.array_equal(full[:, :Sp], part)


def test_non_causal_key_permutation_invariance():
    B, H, S_q, S_kv, D = 1, 2, 9, 23, 8
    q, k, v = rnd(91, B, S_q, H, D), rnd(92, B, S_kv, H, D), rnd(93, B, S_kv, H, D)
    perm = np.random.default_rng(5).permutation(S_kv)
    o1 = oracle.attn_fwd(q, k, v, causal=False)
    o2 = oracle.attn_fwd(q, k[:, perm], v[:, perm], causal=False)
    assert np.max(np.abs(o1 - o2)) <= 1e-14


def test_heads_and_batches_are_independent():
    B, H, S, D = 2, 3, 20, 8
    q, k, v = rnd(101, B, S, H, D), rnd(102, B, S, H, D), rnd(103, B, S, H, D)
    o1 = oracle.attn_fwd(q, k, v, causal=True)
    k2, v2 = k.copy(), v.copy()
    k2[1, :, 2] += 5.0
    v2[1, :, 2] *= -3.0
    o2 = oracle.attn_fwd(q, k2, v2, causal=True)
    changed = np.zeros_like(o1, dtype=bool)
    changed[1, :, 2] = True
    assert np.array_equal(o1[~changed], o2[~changed])
    assert not np.allclose(o1[changed], o2[changed])


# --------------------------------------------------------------------------
# Decode: the S_q = 1 special case of the forward, never reading past len
# --------------------------------------------------------------------------
def test_decode_equals_forward_with_one_query_and_ignores_slots_past_len():
    B, H, S_cap, D = 4, 3, 40, 16
    seqlens = np.array([1, 17, 40, 5], dtype=np.int32)
    q, kc, vc = rnd(111, B, 1, H, D), rnd(112, B, S_cap, H, D), rnd(113, B, S_cap, H, D)
    for b in range(B):
        kc[b, seqlens[b]:] = np.nan
        vc[b, seqlens[b]:] = np.nan
    o = oracle.attn_decode(q, kc, vc, seqlens)
    assert np.all(np.isfinite(o))
    for b in range(B):
        n = seqlens[b]
        ref = oracle.attn_fwd(q[b:b + 1], kc[b:b + 1, :n], vc[b:b + 1, :n], causal=True)
        assert np.array_equal(o[b:b + 1], ref)
        ref2 = sdpa_f64(q[b:b + 1], kc[b:b + 1, :n], vc[b:b + 1, :n], causal=False)
        assert np.max(np.abs(o[b:b + 1] - ref2)) <= 1e-12
    assert np.array_equal(o[0, 0], vc[0, 0])  # one key: the value row itself


def test_decode_empty_and_overlong_lengths():
    B, H, S_cap, D = 3, 2, 10, 8
    q, kc, vc = rnd(121, B, 1, H, D), rnd(122, B, S_cap, H, D), rnd(123, B, S_cap, H, D)
    o = oracle.attn_decode(q, kc, vc, np.array([0, -4, 99], dtype=np.int32))
    assert np.all(o[0] == 0.0) and np.all(o[1] == 0.0)
    full = oracle.attn_decode(q, kc, vc, np.array([10, 10, 10], dtype=np.int32))
    assert np.array_equal(o[2], full[2])


# --------------------------------------------------------------------------
# KV-cache prefill with per-entry lengths and the log-sum-exp output
# --------------------------------------------------------------------------
def _kvcache_reference(q, kc, vc, seqlens, causal):
    """torch float64: SDPA per entry over its valid rows with the explicit
    bottom-right mask, and logsumexp of the explicitly scaled scores."""
    B, S_q, H, D = q.shape
    o = np.zeros_like(q)
    lse = np.full((B, H, S_q), -np.inf)
    for b in range(B):
        n = int(min(max(seqlens[b], 0), kc.shape[1]))
        if n == 0:
            continue
        qt = torch.from_numpy(q[b]).permute(1, 0, 2)            # H, S_q, D
        kt = torch.from_numpy(kc[b, :n]).permute(1, 0, 2)
        vt = torch.from_numpy(vc[b, :n]).permute(1, 0, 2)
        i = torch.arange(S_q)[:, None]
        j = torch.arange(n)[None, :]
        mask = (j <= i + (n - S_q)) if causal else torch.ones(S_q, n, dtype=torch.bool)
        rows = mask.any(dim=1)                                   # rows that see a key
        s = (qt @ kt.transpose(1, 2)) / math.sqrt(D)
        s = s.masked_fill(~mask, -math.inf)
        lse[b][:, rows.numpy()] = torch.logsumexp(s[:, rows], dim=-1).numpy()
        if rows.any():
            ob = torch.nn.functional.scaled_dot_product_attention(qt[:, rows], kt, vt, attn_mask=mask[rows])
            o[b][rows.numpy()] = ob.permute(1, 0, 2).numpy()
    return o, lse


@pytest.mark.parametrize("causal", [True, False])
def test_kvcache_matches_sdpa_and_logsumexp_float64(causal):
    B, S_q, S_cap, H, D = 4, 21, 50, 2, 32
    seqlens = np.array([50, 33, 9, 0], dtype=np.int32)   # 9 < S_q: early rows see no key
    q, kc, vc = rnd(201, B, S_q, H, D), rnd(202, B, S_cap, H, D), rnd(203, B, S_cap, H, D)
    for b in range(B):   # rows past the length are never read
        kc[b, seqlens[b]:] = np.nan
        vc[b, seqlens[b]:] = np.nan
    o, lse = oracle.attn_fwd_kvcache(q, kc, vc, seqlens, causal)
    ro, rlse = _kvcache_reference(q, kc, vc, seqlens, causal)
    assert np.all(np.isfinite(o))
    assert np.max(np.abs(o - ro)) <= 1e-12
    assert np.array_equal(np.isneginf(lse), np.isneginf(rlse))
    fin = np.isfinite(rlse)
    assert np.max(np.abs(lse[fin] - rlse[fin])) <= 1e-12


def test_kvcache_without_lengths_is_the_forward():
    B, S_q, S_cap, H, D = 2, 13, 29, 3, 16
    q, kc, vc = rnd(211, B, S_q, H, D), rnd(212, B, S_cap, H, D), rnd(213, B, S_cap, H, D)
    for causal in (True, False):
        o, lse = oracle.attn_fwd_kvcache(q, kc, vc, None, causal)
        assert np.array_equal(o, oracle.attn_fwd(q, kc, vc, causal))
        o2, lse2 = oracle.attn_fwd_kvcache(q, kc, vc, np.full(B, S_cap, dtype=np.int32), causal)
        assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_lse_merges_results_over_disjoint_key_sets():
    """softmax over keys A u B equals the two partial softmaxes weighted by
    exp(lse_A - lse) and exp(lse_B - lse), lse = ln(exp(lse_A) + exp(lse_B))."""
    B, S_q, H, D, n, m = 2, 7, 2, 16, 40, 15
    q, kc, vc = rnd(221, B, S_q, H, D, std=2.0), rnd(222, B, n, H, D, std=2.0), rnd(223, B, n, H, D)
    o, lse = oracle.attn_fwd_kvcache(q, kc, vc, None, causal=False)
    oa, la = oracle.attn_fwd_kvcache(q, kc[:, :m].copy(), vc[:, :m].copy(), None, causal=False)
    ob, lb = oracle.attn_fwd_kvcache(q, kc[:, m:].copy(), vc[:, m:].copy(), None, causal=False)
    lt = np.logaddexp(la, lb)
    assert np.max(np.abs(lse - lt)) <= 1e-12
    wa = np.exp(la - lt).transpose(0, 2, 1)[..., None]   # B, S_q, H, 1
    wb = np.exp(lb - lt).transpose(0, 2, 1)[..., None]
    assert np.max(np.abs(o - (wa * oa + wb * ob))) <= 1e-12


def test_kvcache_rows_that_see_no_key():
    B, S_q, S_cap, H, D = 3, 6, 8, 2, 8
    q, kc, vc = rnd(231, B, S_q, H, D), rnd(232, B, S_cap, H, D), rnd(233, B, S_cap, H, D)
    o, lse = oracle.attn_fwd_kvcache(q, kc, vc, np.array([0, 2, 99], dtype=np.int32), causal=True)
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(lse[0]))
    # entry 1: queries at positions -4..1; rows 0..3 see nothing, row 4 sees key 0 only
    assert np.all(o[1, :4] == 0.0) and np.all(np.isneginf(lse[1, :, :4]))
    assert np.array_equal(o[1, 4], vc[1, 0])
    np.testing.assert_allclose(lse[1, :, 4], (q[1, 4] * kc[1, 0]).sum(-1) / math.sqrt(D), rtol=1e-14)
    # entry 2: the length is clamped to S_cap
    full, _ = oracle.attn_fwd_kvcache(q, kc, vc, np.array([8, 8, 8], dtype=np.int32), causal=True)
    assert np.array_equal(o[2], full[2])


# ---------------------------------------------------------------------------
# Key-padding mask ("Week-4 CUDA notes" page, section 2.2: a padded position's
# score is set to -inf so that its exponential is exactly 0)
# ---------------------------------------------------------------------------
def _mask_reference(q, k, v, key_mask, causal):
    """torch float64 SDPA with the explicit boolean mask (key mask AND the
    bottom-right causal rule) and logsumexp of the explicitly scaled scores;
    rows that see no key stay 0 / -inf."""
    B, S_q, H, D = q.shape
    S_kv = k.shape[1]
    o = np.zeros_like(q)
    lse = np.full((B, H, S_q), -np.inf)
    i = torch.arange(S_q)[:, None]
    j = torch.arange(S_kv)[None, :]
    for b in range(B):
        vis = torch.from_numpy(np.asarray(key_mask[b]) != 0)[None, :].expand(S_q, S_kv)
        if causal:
            vis = vis & (j <= i + (S_kv - S_q))
        rows = vis.any(dim=1)
        qt = torch.from_numpy(q[b]).permute(1, 0, 2)
        kt = torch.from_numpy(k[b]).permute(1, 0, 2)
        vt = torch.from_numpy(v[b]).permute(1, 0, 2)
        s = ((qt @ kt.transpose(1, 2)) / math.sqrt(D)).masked_fill(~vis, -math.inf)
        if rows.any():
            lse[b][:, rows.numpy()] = torch.logsumexp(s[:, rows], dim=-1).numpy()
            ob = torch.nn.functional.scaled_dot_product_attention(qt[:, rows], kt, vt, attn_mask=vis[rows])
            o[b][rows.numpy()] = ob.permute(1, 0, 2).numpy()
    return o, lse


@pytest.mark.parametrize("S_q,S_kv,causal", [(23, 23, True), (9, 31, True), (17, 40, False), (40, 17, False)])
def test_key_mask_matches_sdpa_and_logsumexp_float64(S_q, S_kv, causal):
    B, H, D = 3, 2, 16
    q, k, v = rnd(241, B, S_q, H, D), rnd(242, B, S_kv, H, D), rnd(243, B, S_kv, H, D)
    g = np.random.default_rng(244)
    km = (g.random((B, S_kv)) < 0.6).astype(np.uint8)
    km[1, :] = 0
    km[1, S_kv - 1] = 1            # entry 1: only its last key (causal: only the last query sees it)
    km[2, :] = 0                   # entry 2: nothing visible at all
    o, lse = oracle.attn_fwd_mask(q, k, v, km, causal)
    ro, rlse = _mask_reference(q, k, v, km, causal)
    assert np.all(np.isfinite(o))
    assert np.max(np.abs(o - ro)) <= 1e-12
    assert np.array_equal(np.isneginf(lse), np.isneginf(rlse))
    fin = np.isfinite(rlse)
    assert np.max(np.abs(lse[fin] - rlse[fin])) <= 1e-12
    assert np.all(o[2] == 0.0) and np.all(np.isneginf(lse[2]))


def test_key_mask_equals_deleting_the_keys():
    """Without the causal rule, hiding keys is the same as removing their rows
    from K and V (the plain forward on the remaining keys)."""
    B, S_q, S_kv, H, D = 3, 11, 26, 2, 8
    q, k, v = rnd(251, B, S_q, H, D, std=1.5), rnd(252, B, S_kv, H, D, std=1.5), rnd(253, B, S_kv, H, D)
    g = np.random.default_rng(254)
    km = (g.random((B, S_kv)) < 0.5).astype(np.uint8)
    km[:, 3] = 1
    o, _ = oracle.attn_fwd_mask(q, k, v, km, causal=False)
    for b in range(B):
        keep = np.nonzero(km[b])[0]
        ref = oracle.attn_fwd(q[b:b + 1], k[b:b + 1, keep].copy(), v[b:b + 1, keep].copy(), causal=False)
        assert np.max(np.abs(o[b:b + 1] - ref)) <= 1e-12


def test_key_mask_with_equal_keys_gives_means_of_the_visible_values():
    """All keys equal: every visible key has the same weight, so row i is the
    plain mean of the values of the keys it may see (closed form)."""
    B, S, H, D = 2, 19, 2, 8
    q, v = rnd(261, B, S, H, D), rnd(262, B, S, H, D)
    k = np.broadcast_to(rnd(263, B, 1, H, D), (B, S, H, D)).copy()
    km = np.ones((B, S), dtype=np.uint8)
    km[0, [0, 4, 5, 11]] = 0
    km[1, 1::2] = 0
    o, _ = oracle.attn_fwd_mask(q, k, v, km, causal=True)
    for b in range(B):
        for i in range(S):
            vis = [j for j in range(i + 1) if km[b, j]]
            if vis:
                np.testing.assert_allclose(o[b, i], v[b, vis].mean(axis=0), rtol=0, atol=1e-13)
            else:
                assert np.all(o[b, i] == 0.0)


def test_key_mask_absent_or_all_visible_is_the_forward():
    B, S, H, D = 2, 15, 3, 16
    q, k, v = rnd(271, B, S, H, D), rnd(272, B, S, H, D), rnd(273, B, S, H, D)
    for causal in (True, False):
        ref = oracle.attn_fwd(q, k, v, causal)
        o1, l1 = oracle.attn_fwd_mask(q, k, v, None, causal)
        o2, l2 = oracle.attn_fwd_mask(q, k, v, np.ones((B, S), dtype=np.uint8), causal)
        assert np.array_equal(o1, ref) and np.array_equal(o2, ref) and np.array_equal(l1, l2)


# ---------------------------------------------------------------------------
# Q, K, V projections as one stacked GEMM (MMHA page, section 2; Week-4
# notes, section 2.1)
# ---------------------------------------------------------------------------
def test_qkv_proj_matches_numpy_matmul_float64():
    B, S, E, H, D = 2, 5, 48, 3, 16
    x = rnd(281, B, S, E)
    w = rnd(282, 3 * H * D, E)
    q, k, v = oracle.qkv_proj(x, w, H, D)
    ref = x.reshape(B * S, E) @ w.T            # [M, 3*H*D], library GEMM in float64
    got = np.concatenate([t.reshape(B * S, H * D) for t in (q, k, v)], axis=1)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_qkv_proj_identity_and_permutation_weights_are_exact():
    """W_Q = I gives Q = X, W_K = 2I gives K = 2X, W_V a permutation gives V =
    the permuted columns of X: exact in any arithmetic."""
    B, S, H, D = 2, 3, 2, 4
    E = H * D
    x = rnd(283, B, S, E)
    perm = np.random.default_rng(284).permutation(E)
    w = np.concatenate([np.eye(E), 2.0 * np.eye(E), np.eye(E)[perm]], axis=0)
    q, k, v = oracle.qkv_proj(x, w, H, D)
    assert np.array_equal(q.reshape(B, S, E), x)
    assert np.array_equal(k.reshape(B, S, E), 2.0 * x)
    assert np.array_equal(v.reshape(B, S, E), x[..., perm])


def test_qkv_proj_brute_force_exact_rationals():
    """Small integers: every dot product is exact, checked with Fractions."""
    M, E, H, D = 3, 5, 1, 2
    g = np.random.default_rng(285)
    x = g.integers(-4, 5, (M, E)).astype(np.float64)
    w = g.integers(-4, 5, (3 * H * D, E)).astype(np.float64)
    q, k, v = oracle.qkv_proj(x, w, H, D)
    for c, out in enumerate((q, k, v)):
        for m in range(M):
            for n in range(H * D):
                exact = sum(Fraction(int(x[m, e])) * Fraction(int(w[c * H * D + n, e])) for e in range(E))
                assert out[m].reshape(-1)[n] == float(exact)


def test_qkv_proj_is_linear_in_the_input():
    M, E, H, D = 7, 32, 2, 8
    x1, x2 = rnd(286, M, E), rnd(287, M, E)
    w = rnd(288, 3 * H * D, E)
    a = oracle.qkv_proj(2.5 * x1 + x2, w, H, D)
    b1 = oracle.qkv_proj(x1, w, H, D)
    b2 = oracle.qkv_proj(x2, w, H, D)
    for t, u1, u2 in zip(a, b1, b2):
        assert np.max(np.abs(t - (2.5 * u1 + u2))) <= 1e-12


# ---------------------------------------------------------------------------
# Sinusoidal position encoding (Week-4 notes page, section 2.3)
# ---------------------------------------------------------------------------
def test_pe_position_zero_and_first_pair():
    """pos 0: every sine is 0 and every cosine 1; dims 0/1 have frequency 1, so
    they are sin(pos), cos(pos) (math library, float64)."""
    pe = oracle.sinusoidal_pe(37, 64)
    assert np.all(pe[0, 0::2] == 0.0) and np.all(pe[0, 1::2] == 1.0)
    pos = np.arange(37, dtype=np.float64)
    assert np.max(np.abs(pe[:, 0] - [math.sin(p) for p in pos])) <= 1e-15
    assert np.max(np.abs(pe[:, 1] - [math.cos(p) for p in pos])) <= 1e-15


def test_pe_frequencies_and_unit_pairs():
    """Pair i oscillates with angular frequency 10000^(-2i/d): the angle
    atan2(sin, cos) of pair i at position 1 is that frequency (all < pi);
    every (sin, cos) pair has unit length."""
    d = 128
    pe = oracle.sinusoidal_pe(5, d)
    for i in range(d // 2):
        w = 10000.0 ** (-2.0 * i / d)
        assert abs(math.atan2(pe[1, 2 * i], pe[1, 2 * i + 1]) - w) <= 1e-15
    assert np.max(np.abs(pe[:, 0::2] ** 2 + pe[:, 1::2] ** 2 - 1.0)) <= 1e-15


def test_pe_shift_is_a_rotation():
    """PE(pos + k) is PE(pos) rotated pair by pair by the angle PE(k) holds
    (the relative-position property): sin(a+b) = sin a cos b + cos a sin b,
    cos(a+b) = cos a cos b - sin a sin b."""
    d, k = 96, 17
    pe = oracle.sinusoidal_pe(60, d)
    s, c = pe[:-k, 0::2], pe[:-k, 1::2]
    sk, ck = pe[k, 0::2], pe[k, 1::2]
    assert np.max(np.abs(pe[k:, 0::2] - (s * ck + c * sk))) <= 1e-12
    assert np.max(np.abs(pe[k:, 1::2] - (c * ck - s * sk))) <= 1e-12


def test_pe_offset_rows_are_the_later_rows():
    full = oracle.sinusoidal_pe(50, 32)
    assert np.array_equal(oracle.sinusoidal_pe(20, 32, pos0=30), full[30:])


# ---------------------------------------------------------------------------
# Standalone masked softmax (MMHA page, section 1; Week-4 notes, section 2.2)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("S_q,S_kv,causal", [(19, 19, True), (7, 30, True), (12, 9, False)])
def test_masked_softmax_matches_torch_softmax_float64(S_q, S_kv, causal):
    B, H, scale = 2, 3, 0.37
    s = rnd(291, B, H, S_q, S_kv, std=3.0)
    p = oracle.masked_softmax(s, scale, causal)
    t = torch.from_numpy(s) * scale
    if causal:
        i = torch.arange(S_q)[:, None]
        j = torch.arange(S_kv)[None, :]
        t = t.masked_fill(j > i + (S_kv - S_q), -math.inf)
    ref = torch.softmax(t, dim=-1).numpy()
    assert np.max(np.abs(p - ref)) <= 1e-15


def test_masked_softmax_is_the_attention_probabilities():
    """The probabilities the attention oracle forms from Q K^T / sqrt(D) are the
    masked softmax of those scores (scores from a float64 numpy matmul)."""
    B, S, H, D = 2, 23, 2, 16
    q, k, v = rnd(292, B, S, H, D), rnd(293, B, S, H, D), rnd(294, B, S, H, D)
    _, P = oracle.attn_fwd(q, k, v, True, return_p=True)
    scores = np.einsum("bihd,bjhd->bhij", q, k)
    p = oracle.masked_softmax(scores, 1.0 / math.sqrt(D), True)
    assert np.max(np.abs(p - P)) <= 1e-14


def test_masked_softmax_ignores_masked_scores_and_row_shifts():
    B, H, S = 1, 2, 11
    s = rnd(295, B, H, S, S)
    p = oracle.masked_softmax(s, 1.0, True)
    t = s.copy()
    t[..., np.triu_indices(S, 1)[0], np.triu_indices(S, 1)[1]] = np.nan   # masked scores are never read
    t += 5.0                                                              # a constant per row changes nothing
    q = oracle.masked_softmax(t, 1.0, True)
    assert np.all(np.isfinite(q)) and np.max(np.abs(q - p)) <= 1e-15
    assert np.all(p[..., np.triu_indices(S, 1)[0], np.triu_indices(S, 1)[1]] == 0.0)
    assert np.max(np.abs(p.sum(-1) - 1.0)) <= 1e-15


def test_rejects_invalid_arguments():
    q = rnd(1, 1, 4, 1, 8)
    with pytest.raises(ValueError):
        oracle.attn_fwd(q, q[:, :2], q[:, :2], causal=True)   # causal with S_q > S_kv


# --------------------------------------------------------------------------
# The workloads themselves (shapes and the decode lengths the recipe fixes)
# --------------------------------------------------------------------------
def test_workload_recipe():
    sl, q, kc, vc = workloads.make_decode(workloads.BF16_DECODE, S_cap=8)
    assert sl.tolist() == [1764, 1316, 2324, 1626, 376, 361, 133, 372, 1003, 3498, 32, 479,
                           3036, 3120, 1054, 3810]
    assert q.dtype == torch.bfloat16 and kc.shape == (16, 8, 32, 128)
    assert workloads.BF16_S2048.flops() == 34_376_515_584
    assert workloads.BF16_S4096.flops() == 137_472_507_904
    assert workloads.FP32_TINY.flops() == 532_480
    assert workloads.decode_kv_bytes(sl.tolist(), 32, 128, 2, 4096) == 398_196_736 + 262_144
