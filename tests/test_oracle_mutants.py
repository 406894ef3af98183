"""Planted mistakes in a copy of the oracle must be caught by the pins.

Each case edits one line of a copy of oracle/oracle.c (on the CPU, in a
temporary directory), builds it with gcc, points the oracle module at the
copy, runs the pin tests of test_oracle.py against it and requires at least
one of them to fail.  The real oracle is restored afterwards.  No edit makes
the copy read outside its buffers.
"""
import os
import subprocess

import pytest
import torch

import oracle
from tests import test_oracle as pins
from tests import test_oracle_bwd as bpins
from tests import test_oracle_decode as dpins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "causal_off_by_one": ("causal ? i + 1 : N", "causal ? i : N"),
    "scale_by_D": ("s[j] = dot / root_d;", "s[j] = dot / (double)D;"),
    "scale_dropped": ("s[j] = dot / root_d;", "s[j] = dot;"),
    "transposed_key": ("dot += qi[d] * kj[d];", "dot += qi[d] * k[d * N + j];"),
    "lse_log2": ("*lse_out = m + log(l);", "*lse_out = m + log2(l);"),
    "lse_without_max": ("*lse_out = m + log(l);", "*lse_out = log(l);"),
    "k_used_as_v": ("const double *vj = v + j * D;", "const double *vj = k + j * D;"),
    "attn_min_not_max": ("for (int64_t j = 1; j < nkeys; ++j)\n        if (s[j] > m)",
                         "for (int64_t j = 1; j < nkeys; ++j)\n        if (s[j] < m)"),
    "attn_no_max_subtraction": ("s[j] = exp(s[j] - m);", "s[j] = exp(s[j]);"),
    "attn_not_normalised": ("s[j] = s[j] / l;", "s[j] = s[j];"),
    "heads_mixed": ("const int64_t head = bh * jb->N * jb->D;", "const int64_t head = 0;"),
    "softmax_no_max_subtraction": ("y[j] = exp(x[j] - m);", "y[j] = exp(x[j]);"),
    "softmax_min_not_max": ("for (int64_t j = 1; j < N; ++j)\n        if (x[j] > m)",
                            "for (int64_t j = 1; j < N; ++j)\n        if (x[j] < m)"),
    "softmax_not_normalised": ("y[j] = y[j] / d;", "y[j] = y[j];"),
    "softmax_rows_shifted": ("softmax_row(jb->x + src * jb->N", "softmax_row(jb->x + (src / 2) * jb->N"),
    # paged decode (every edit keeps the reads inside the buffers)
    "dec_slot_off_by_one": ("dot += qr[d] * cache_at(jb, page, 0, t % jb->T, kvh, d);",
                            "dot += qr[d] * cache_at(jb, page, 0, (t + 1) % jb->T, kvh, d);"),
    "dec_head_interleaved": ("const int64_t kvh = h / (jb->Hq / jb->Hkv);",
                             "const int64_t kvh = h % jb->Hkv;"),
    "dec_v_read_from_k": ("o_row[d] += s[t] * cache_at(jb, page, 1,",
                          "o_row[d] += s[t] * cache_at(jb, page, 0,"),
    "dec_drops_last_token": ("const int64_t len = jb->lengths[b];",
                             "const int64_t len = jb->lengths[b] > 1 ? jb->lengths[b] - 1 : jb->lengths[b];"),
    "dec_first_page_only": ("const int64_t page = jb->block_table[b * jb->max_pages + t / jb->T];\n            double dot",
                            "const int64_t page = jb->block_table[b * jb->max_pages];\n            double dot"),
    "dec_scale_dropped": ("s[t] = dot / root_d;", "s[t] = dot;"),
    "dec_query_of_head0": ("const double *qr = jb->q + flat * jb->D;",
                           "const double *qr = jb->q + b * jb->Hq * jb->D;"),
    "dec_bf16_read_as_fp16": ("jb->is_bf16 ? bf16_bits_to_double(jb->cache[idx]) : half_bits_to_double(jb->cache[idx])",
                              "half_bits_to_double(jb->cache[idx])"),
    "half_subnormal_scale": ("v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);"),
    # attention backward
    "bwd_no_d_term": ("const double ds = s[j] * (dp[j] - dd);  /* dS_ij */",
                      "const double ds = s[j] * dp[j];  /* dS_ij */"),
    "bwd_dq_unscaled": ("dqi[d] /= root_d;", "dqi[d] /= 1.0;"),
    "bwd_dk_unscaled": ("dkj[d] /= root_d;", "dkj[d] /= 1.0;"),
    "bwd_dv_uses_ds": ("dvj[d] += p * doi[d];", "dvj[d] += ds * doi[d];"),
    "bwd_dp_uses_k": ("pdot += doi[d] * vj[d];", "pdot += doi[d] * kj[d];"),
    "bwd_causal_skips_diagonal": ("for (int64_t i = jb->causal ? j : 0; i < N; ++i) {",
                                  "for (int64_t i = jb->causal ? j + 1 : 0; i < N; ++i) {"),
    "bwd_dk_uses_k": ("dkj[d] += ds * qi[d];", "dkj[d] += ds * kj[d];"),
    "bwd_p_not_normalised": ("const double p = exp(sdot / root_d - jb->m[i]) / jb->l[i];",
                             "const double p = exp(sdot / root_d - jb->m[i]);"),
    "half_exponent_bias": ("v = ldexp((double)(1024 + m), e - 25);", "v = ldexp((double)(1024 + m), e - 24);"),
}

PIN_CALLS = [
    (pins.test_stage1_picks_one_key_column, {"D": 16}),
    (pins.test_stage1_causal_key_count_and_prefix, {}),
    (pins.test_single_key_returns_v0, {"D": 64}),
    (pins.test_identical_keys_give_prefix_mean, {"causal": True}),
    (pins.test_zero_queries_give_uniform_weights, {"causal": False}),
    (pins.test_two_keys_logistic, {"a": 7.0}),
    (pins.test_large_logits_stay_finite, {}),
    (pins.test_wide_logit_spread_needs_the_row_max, {}),
    (pins.test_key_shift_invariance, {"causal": True}),
    (pins.test_causal_prefix_property, {}),
    (pins.test_linear_in_v_and_weights_convex, {}),
    (pins.test_heads_and_batches_are_independent, {}),
    (pins.test_lse_normalises_the_scores, {"causal": True}),
    (pins.test_matches_torch_sdpa_float64, {"N": 33, "D": 64, "causal": True}),
    (pins.test_softmax_rows_sum_to_one_and_shift_invariant, {}),
    (pins.test_softmax_all_zero_is_uniform, {}),
    (pins.test_softmax_special_last_element_closed_form, {}),
    (pins.test_softmax_matches_library_routines, {}),
    (bpins.test_matches_torch_autograd_float64, {"shape": (1, 2, 9, 8), "causal": True}),
    (bpins.test_central_differences_of_the_forward_oracle, {"causal": True}),
    (bpins.test_key_gradients_sum_to_zero_and_dv_to_the_dout_sum, {"causal": True}),
    (bpins.test_single_key_and_identical_keys, {}),
    (bpins.test_causal_dependency_structure_is_exact, {}),
    (dpins.test_fp16_bits_decode_exactly, {}),
    (dpins.test_bf16_bits_decode_exactly, {}),
    (dpins.test_equals_last_causal_row_of_attention, {"dtype": torch.float16, "T": 4, "Hkv": 2}),
    (dpins.test_equals_last_causal_row_of_attention, {"dtype": torch.bfloat16, "T": 16, "Hkv": 4}),
    (dpins.test_matches_torch_sdpa_float64, {}),
    (dpins.test_single_token_returns_v0_and_its_logit, {}),
    (dpins.test_identical_keys_give_the_mean_of_v, {}),
    (dpins.test_physical_page_order_does_not_matter, {}),
    (dpins.test_heads_of_a_group_share_their_kv_head, {}),
    (dpins.test_invalid_requests_get_nan_and_others_are_unaffected, {}),
]


def _failures():
    failed = []
    for fn, kw in PIN_CALLS:
        try:
            fn(**kw)
        except Exception:  # a failing assertion, a NaN comparison, an error return
            failed.append(fn.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation site vanished: %r" % old
    mutated = src.replace(old, new, 1)
    c_path = tmp_path / "mutant.c"
    c_path.write_text(mutated)
    so_path = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", str(c_path),
                    "-o", str(so_path), "-lm"], check=True)
    oracle.swap_library(str(so_path))
    try:
        failed = _failures()
    finally:
        oracle.swap_library(None)
    assert failed, "planted mistake %s passed every pin" % name


def test_unmodified_copy_passes_every_pin(tmp_path):
    so_path = tmp_path / "libcopy.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", SRC,
                    "-o", str(so_path), "-lm"], check=True)
    oracle.swap_library(str(so_path))
    try:
        failed = _failures()
    finally:
        oracle.swap_library(None)
    assert failed == []


def test_gqa_pin_catches_wrong_head_map(monkeypatch):
    """Planted in the oracle's Python head map: h % Hkv (interleaved groups) in
    place of h // g.  The torch enable_gqa pin must reject it."""
    from tests.test_oracle import gqa_sdpa_check, rand
    q = rand(1, 4, 9, 8, scale=2.0)
    k, v = rand(1, 2, 9, 8, scale=2.0), rand(1, 2, 9, 8)
    assert gqa_sdpa_check(q, k, v, True) <= 1e-12
    monkeypatch.setattr(oracle, "kv_head", lambda h, H, Hkv: h % Hkv)
    assert gqa_sdpa_check(q, k, v, True) > 1e-3


def test_gqa_backward_pins_catch_wrong_head_map_and_missing_group_sum(monkeypatch):
    """Planted in the oracle's Python layer: (a) h % Hkv in place of h // g for
    the K/V head of a query head; (b) dK, dV of a shared head taken from the
    first query head of its group instead of summed over the group.  The
    autograd pin rejects both."""
    import numpy as np
    kw = {"shape": (1, 4, 2, 17, 8), "causal": True}
    bpins.test_gqa_matches_torch_autograd_float64(**kw)
    with monkeypatch.context() as m:
        m.setattr(oracle, "kv_head", lambda h, H, Hkv: h % Hkv)
        with pytest.raises(AssertionError):
            bpins.test_gqa_matches_torch_autograd_float64(**kw)
    real = oracle.attn_bwd_gqa

    def first_head_only(q, k, v, dout, causal, kv_heads=None, nthreads=None):
        B, H, N, D = q.shape
        Hkv = k.shape[1]
        dq, dk_h, dv_h = oracle.attn_bwd(q, oracle._kv_for_query_heads(k, H),
                                         oracle._kv_for_query_heads(v, H), dout, causal)
        g = H // Hkv
        return (dq, np.ascontiguousarray(dk_h[:, ::g]), np.ascontiguousarray(dv_h[:, ::g]))

    with monkeypatch.context() as m:
        m.setattr(oracle, "attn_bwd_gqa", first_head_only)
        with pytest.raises(AssertionError):
            bpins.test_gqa_matches_torch_autograd_float64(**kw)
    assert oracle.attn_bwd_gqa is real
