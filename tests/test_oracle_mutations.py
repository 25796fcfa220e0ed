"""Mutation proofs for the oracle's pins.

Each case plants one plausible mistake in a copy of the oracle's C source
(on the CPU), builds it, and runs the pins against that build: at least one
pin must fail, or the pins could not tell that mistake from the definition.
The unmutated copy, built the same way, must pass every pin (so the harness
itself fails nothing).  This is the discipline of vllm.cpp PR #2556, section
"Gates, read literally": each mutation is built successfully before it is run,
and must turn the suite red.
"""
import os

import numpy as np
import pytest

import oracle
from oracle import build as obuild

import test_oracle_brute as tb
import test_oracle_invariants as ti
import test_oracle_math as tm
import test_oracle_moe as tmoe

SRC = os.path.join(os.path.dirname(obuild.__file__), "dro.c")
HDR = os.path.join(os.path.dirname(obuild.__file__), "dro.h")


def _pins_logits():
    tb.test_logits_match_exact_rounding("normal", 3)
    tb.test_logits_match_exact_rounding("cancel", 2)
    tb.test_logits_match_exact_rounding("zeros", 4)
    tb.test_tree_grouping_is_distinguished()
    tb.test_fma_not_mul_add()
    tb.test_single_block_is_one_sequential_chain()
    ti.test_integer_inputs_give_exact_integer_matmul()
    ti.test_zero_rows_give_positive_zero()


def _pins_selection():
    for k, vals, want in ti._golden_tiebreak():
        ti.test_golden_tiebreak(k, vals, want)
    tb.test_selection_and_margin_bruteforce(6, 3)
    tb.test_selection_and_margin_bruteforce(8, 2)
    ti.test_constructed_ties_resolve_to_lowest_index()


def _pins_margin():
    for a, b, want in ti._golden_ulps():
        ti.test_golden_ulps(a, b, want)
    tm.test_ulps_closed_forms()
    tb.test_selection_and_margin_bruteforce(5, 5)
    tb.test_selection_and_margin_bruteforce(8, 7)


def _pins_weights():
    tb.test_weights_against_float64_softmax()
    tb.test_weights_exact_tree_denominator()
    tm.test_expf_special_values()


def _pins_exp():
    tm.test_expf_accuracy_strided_sweep()
    tm.test_expf_special_values()


def _pins_bf16():
    tm.test_bf16_rne_against_torch_and_exact_rounding()
    tb.test_bf16_logit_mode_selects_on_rounded_values()


def _pins_batch():
    ti.test_row_independent_of_batch_mates()
    ti.test_thread_count_does_not_change_bits()


def _pins_permute():
    for case in ((5, 2, 4), (19, 8, 256), (300, 8, 64)):
        tmoe.test_permute_matches_stable_argsort(*case)
    tmoe.test_permute_closed_forms()


def _pins_combine():
    for kind in ("normal", "cancel", "tiny"):
        tmoe.test_combine_matches_exact_rounding(kind)
    tmoe.test_combine_does_not_depend_on_slot_order()
    tmoe.test_combine_integer_inputs_are_exact()
    tmoe.test_combine_zero_sum_is_positive_zero()
    tmoe.test_combine_shared_term_comes_last()
    tmoe.test_combine_ascending_expert_order_is_distinguished()


def _pins_grouped():
    tmoe.test_grouped_gemm_ref_matches_numpy_per_group()
    tmoe.test_grouped_gemm_ref_exact_on_integers_and_rows_equal_pregathered()


# (name, text in dro.c, replacement, pins that must catch it)
MUTATIONS = [
    ("tie_break_highest_index",
     "return (a->i < b->i) ? -1 : (a->i > b->i ? 1 : 0);",
     "return (a->i > b->i) ? -1 : (a->i < b->i ? 1 : 0);",
     _pins_selection),
    ("ulps_twos_complement",
     "return (b & 0x8000u) ? -mag : mag;",
     "return (int32_t)(int16_t)b;",
     _pins_margin),
    ("ulps_drop_sign",
     "return (b & 0x8000u) ? -mag : mag;",
     "return mag;",
     _pins_margin),
    ("tree_left_to_right",
     "for (int64_t i = 0; i < half; ++i) v[i] = v[2 * i] + v[2 * i + 1];\n    if (n & 1) v[half] = v[n - 1];\n    n = half + (n & 1);",
     "for (int64_t i = 1; i < n; ++i) v[0] = v[0] + v[i];\n    n = 1;",
     _pins_logits),
    ("mul_then_add",
     "for (int64_t kk = k0; kk < k1; ++kk) p = fmaf(x_at(x, x_is_bf16, K, m, kk), W[kk * E + e], p);\n    part[b] = p;",
     "for (int64_t kk = k0; kk < k1; ++kk) { float t = x_at(x, x_is_bf16, K, m, kk) * W[kk * E + e]; p = p + t; }\n    part[b] = p;",
     _pins_logits),
    ("block_chain_starts_at_minus_zero",
     "    int64_t k1 = k0 + kblock < K ? k0 + kblock : K;\n    float p = 0.0f;",
     "    int64_t k1 = k0 + kblock < K ? k0 + kblock : K;\n    float p = -0.0f;",
     _pins_logits),
    ("drop_last_block",
     "  int64_t nb = (K + kblock - 1) / kblock;\n  for (int64_t b = 0; b < nb; ++b) {\n    int64_t k0 = b * kblock;",
     "  int64_t nb = K / kblock > 0 ? K / kblock : 1;\n  for (int64_t b = 0; b < nb; ++b) {\n    int64_t k0 = b * kblock;",
     _pins_logits),
    ("margin_rejected_off_by_one",
     "float rej = (k < E) ? ent[k].v : -INFINITY;",
     "float rej = (k < E) ? ent[k - 1].v : -INFINITY;",
     _pins_margin),
    ("bf16_truncate",
     "if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;",
     "(void)lower;",
     _pins_bf16),
    ("exp_degree_six",
     "  float p = INV_FACT_F[7];\n  for (int i = 6; i >= 0; --i)",
     "  float p = INV_FACT_F[6];\n  for (int i = 5; i >= 0; --i)",
     _pins_exp),
    ("softmax_denominator_sequential",
     "    float s = pairwise_tree(tmp, E);",
     "    float s = 0.0f;\n    for (int64_t e = 0; e < E; ++e) s = s + tmp[e];",
     _pins_weights),
    ("row_depends_on_batch_size",
     "      raw[e] = canonical_dot(j->x, j->x_is_bf16, j->W, j->K, E, m, e, j->kblock, part);",
     "      raw[e] = canonical_dot(j->x, j->x_is_bf16, j->W, j->K, E, m, e, j->M > 1 ? j->kblock / 2 : j->kblock, part);",
     _pins_batch),
    ("permute_tokens_descending",
     "    for (int64_t m = 0; m < M; ++m)\n      for (int32_t j = 0; j < k; ++j)\n        if (ids[m * k + j] == e) {",
     "    for (int64_t m = M - 1; m >= 0; --m)\n      for (int32_t j = 0; j < k; ++j)\n        if (ids[m * k + j] == e) {",
     _pins_permute),
    ("permute_offsets_inclusive",
     "    offsets[e] = (int32_t)p;\n    for (int64_t m = 0; m < M; ++m)\n      for (int32_t j = 0; j < k; ++j)\n        if (ids[m * k + j] == e) {\n          rows[p] = (int32_t)m;\n          pos[m * k + j] = (int32_t)p;\n          ++p;\n        }\n  }",
     "    for (int64_t m = 0; m < M; ++m)\n      for (int32_t j = 0; j < k; ++j)\n        if (ids[m * k + j] == e) {\n          rows[p] = (int32_t)m;\n          pos[m * k + j] = (int32_t)p;\n          ++p;\n        }\n    offsets[e] = (int32_t)p;\n  }",
     _pins_permute),
    ("combine_in_slot_order",
     "      if (es > et || (es == et && s > t)) {",
     "      if (s > t) {",
     _pins_combine),
    ("combine_starts_at_minus_zero",
     "    float acc = 0.0f;\n    for (int32_t i = 0; i < k; ++i) {",
     "    float acc = -0.0f;\n    for (int32_t i = 0; i < k; ++i) {",
     _pins_combine),
    ("combine_mul_then_add",
     "      acc = fmaf(c->weights[m * k + s], yv, acc);",
     "      acc = acc + c->weights[m * k + s] * yv;",
     _pins_combine),
    ("grouped_next_expert",
     "    for (int64_t p = offsets[e]; p < offsets[e + 1]; ++p) expert_of[p] = (int32_t)e;",
     "    for (int64_t p = offsets[e]; p < offsets[e + 1]; ++p) expert_of[p] = (int32_t)((e + 1) % E);",
     _pins_grouped),
    ("grouped_ignores_rows",
     "  const int64_t r = j->src_rows ? j->src_rows[p] : p;",
     "  const int64_t r = p < j->K ? p : 0;",
     _pins_grouped),
    ("combine_shared_first",
     "    float acc = 0.0f;\n    for (int32_t i = 0; i < k; ++i) {\n      int32_t s = order[i];\n      float yv = elem_at(c->y, c->y_is_bf16, (int64_t)c->pos[m * k + s] * c->D + d);\n      acc = fmaf(c->weights[m * k + s], yv, acc);\n    }\n    if (c->shared) acc = fmaf(c->gate[m], elem_at(c->shared, c->shared_is_bf16, m * c->D + d), acc);",
     "    float acc = 0.0f;\n    if (c->shared) acc = fmaf(c->gate[m], elem_at(c->shared, c->shared_is_bf16, m * c->D + d), acc);\n    for (int32_t i = 0; i < k; ++i) {\n      int32_t s = order[i];\n      float yv = elem_at(c->y, c->y_is_bf16, (int64_t)c->pos[m * k + s] * c->D + d);\n      acc = fmaf(c->weights[m * k + s], yv, acc);\n    }",
     _pins_combine),
]


def _build_variant(tmp_path, text: str, name: str) -> str:
    d = tmp_path / name
    d.mkdir()
    (d / "dro.h").write_text(open(HDR).read())
    (d / "dro.c").write_text(text)
    return obuild.compile_source(str(d / "dro.c"), str(d / "libdro.so"))


@pytest.fixture
def swap_oracle(monkeypatch):
    def use(path):
        monkeypatch.setattr(oracle, "_lib", oracle.bind(path))
    return use


def test_unmutated_copy_passes_every_pin(tmp_path, swap_oracle):
    swap_oracle(_build_variant(tmp_path, open(SRC).read(), "control"))
    for pins in {m[3] for m in MUTATIONS}:
        pins()


@pytest.mark.parametrize("name,old,new,pins", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(tmp_path, swap_oracle, name, old, new, pins):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    swap_oracle(_build_variant(tmp_path, src.replace(old, new), name))
    with pytest.raises(AssertionError):
        pins()
