"""The oracle's pins must catch plausible mistakes planted in the oracle.

Each case compiles a copy of ``oracle/attn_oracle.c`` with one edit (a
dropped scale, a diagonal hidden, a transposed layout, ...) into a temporary
directory, points the oracle module at it and checks that at least one pin
of ``test_oracle.py`` fails. Runs on the CPU only; the real oracle is never
modified.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
from tests import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")

MUTANTS = {
    "diagonal_hidden": ("(causal && j > i + off)", "(causal && j >= i + off)"),
    "alignment_top_left": ("const long off = S_kv - S_q;", "const long off = 0;"),
    "alignment_sign": ("const long off = S_kv - S_q;", "const long off = S_q - S_kv;"),
    "mask_ignored": ("(causal && j > i + off)", "(0 && j > i + off)"),
    "scale_dropped": ("row[j] = dot * scale;", "row[j] = dot;"),
    "scale_is_1_over_d": ("1.0 / sqrt((double)D)", "1.0 / (double)D"),
    "values_replaced_by_keys": ("const double* vrow = v + at(", "const double* vrow = k + at("),
    "no_normalisation": ("for (long j = 0; j < S_kv; ++j) row[j] = row[j] / l;", ""),
    "no_max_subtraction": ("row[j] = exp(row[j] - m);", "row[j] = exp(row[j]);"),
    "layout_bhsd": ("return (size_t)(((b * S + s) * H + h) * D + d);",
                    "return (size_t)(((b * H + h) * S + s) * D + d);"),
    "decode_reads_full_cache": ("if (n > S_cap) n = S_cap;", "n = S_cap;"),
    "query_key_swapped": ("dot += q[at(b, i, h, d, S_qdim, H, D)] * k[at(b, j, h, d, S_kdim, H, D)];",
                          "dot += q[at(b, i, h, d, S_qdim, H, D)] * q[at(b, j % S_q, h, d, S_qdim, H, D)];"),
    "max_over_first_key_only": ("if (row[j] > m) m = row[j];", "if (j == 0) m = row[j];"),
    "lse_without_max": ("= m + log(l);", "= log(l);"),
    "lse_log2": ("= m + log(l);", "= m + log2(l);"),
    "kvcache_ignores_lengths": ("long n = seqlens ? seqlens[b] : S_cap;", "long n = S_cap;"),
    "empty_rows_not_zero": ("if (m == -INFINITY) {", "if (0) {"),
    "key_mask_ignored": ("(kmask && kmask[j] == 0)", "(0)"),
    "key_mask_inverted": ("kmask[j] == 0", "kmask[j] != 0"),
    "key_mask_on_queries": ("(kmask && kmask[j] == 0)", "(kmask && kmask[i % S_kv] == 0)"),
    "key_mask_of_entry_0_for_all": ("key_mask ? key_mask + (size_t)b * (size_t)S_kv : NULL", "key_mask"),
    "qkv_weight_read_transposed": ("for (long e = 0; e < E; ++e) acc += xrow[e] * wrow[e];",
                                   "for (long e = 0; e < E; ++e) acc += xrow[e] * w[(size_t)e * 3 * N + (size_t)c * N + n];"),
    "qkv_q_and_k_swapped": ("double* out[3] = {q, k, v};", "double* out[3] = {k, q, v};"),
    "pe_sin_cos_swapped": ("+ (size_t)(2 * i)] = sin(angle);", "+ (size_t)(2 * i)] = cos(angle);"),
    "pe_exponent_over_i": ("(double)(2 * i) / (double)d_model", "(double)(i) / (double)d_model"),
    "pe_base_1000": ("pow(10000.0,", "pow(1000.0,"),
    "pe_offset_ignored": ("const double pos = (double)pos0 + (double)s;", "const double pos = (double)s;"),
    "softmax_mask_off_by_one": ("long n = causal ? i + off + 1 : S_kv;", "long n = causal ? i + off : S_kv;"),
    "softmax_scale_after_max": ("prow[j] = exp(scale * srow[j] - m);", "prow[j] = exp(srow[j] - m);"),
    "qkv_dropped_last_term": ("for (long e = 0; e < E; ++e) acc += xrow[e] * wrow[e];",
                              "for (long e = 0; e + 1 < E; ++e) acc += xrow[e] * wrow[e];"),
}

PINS = [
    lambda: pins.test_matches_sdpa_float64(2, 2, 19, 53, 64, True),
    lambda: pins.test_matches_sdpa_float64(2, 3, 37, 37, 16, True),
    lambda: pins.test_matches_sdpa_float64(2, 2, 33, 47, 32, False),
    pins.test_golden_geometric_weights,
    pins.test_two_keys_is_a_logistic_blend,
    lambda: pins.test_brute_force_tiny(1, 3, 4, 9, 8, True),
    pins.test_rows_sum_to_one_and_masked_entries_are_exactly_zero,
    pins.test_row_zero_returns_value_row_zero_exactly,
    pins.test_equal_keys_give_prefix_means,
    pins.test_constant_values_pass_through,
    pins.test_large_logits_stay_finite_and_match_lse_brute_force,
    pins.test_decode_equals_forward_with_one_query_and_ignores_slots_past_len,
    pins.test_decode_empty_and_overlong_lengths,
    lambda: pins.test_kvcache_matches_sdpa_and_logsumexp_float64(True),
    pins.test_lse_merges_results_over_disjoint_key_sets,
    pins.test_kvcache_rows_that_see_no_key,
    lambda: pins.test_key_mask_matches_sdpa_and_logsumexp_float64(9, 31, True),
    pins.test_key_mask_equals_deleting_the_keys,
    pins.test_key_mask_with_equal_keys_gives_means_of_the_visible_values,
    pins.test_qkv_proj_matches_numpy_matmul_float64,
    pins.test_qkv_proj_identity_and_permutation_weights_are_exact,
    pins.test_pe_position_zero_and_first_pair,
    pins.test_pe_frequencies_and_unit_pairs,
    pins.test_pe_offset_rows_are_the_later_rows,
    lambda: pins.test_masked_softmax_matches_torch_softmax_float64(7, 30, True),
    pins.test_masked_softmax_is_the_attention_probabilities,
]


ORACLE_FUNCTIONS = ("oracle_attn_fwd_f64", "oracle_attn_decode_f64", "oracle_attn_fwd_kvcache_f64",
                    "oracle_attn_fwd_mask_f64", "oracle_qkv_proj_f64", "oracle_sinusoidal_pe_f64",
                    "oracle_masked_softmax_f64", "oracle_num_threads")


def test_every_exported_oracle_function_is_listed():
    import re
    text = open(SRC).read()
    exported = set(re.findall(r"^int (oracle_\w+)\(", text, re.M))
    assert exported == set(ORACLE_FUNCTIONS)


def _compile(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) >= 1, f"mutation anchor for {name} not found"
    src = tmp_path / f"{name}.c"
    src.write_text(text.replace(old, new))
    lib = tmp_path / f"{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", str(src), "-o",
                    str(lib), "-lm"], check=True)
    return str(lib)


def _failures():
    failed = 0
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError):
            failed += 1
    return failed


def test_unmutated_oracle_passes_every_pin():
    assert _failures() == 0


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path, monkeypatch):
    real = oracle._load()
    path = _compile(tmp_path, name, *MUTANTS[name])
    mutant = ctypes.CDLL(path)
    # every function of the oracle: same argument and result types
    for fn in ORACLE_FUNCTIONS:
        f, g = getattr(mutant, fn), getattr(real, fn)
        f.argtypes, f.restype = g.argtypes, g.restype
    monkeypatch.setattr(oracle, "_lib", mutant)
    assert _failures() >= 1, f"no pin catches mutant {name}"
