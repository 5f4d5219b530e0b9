"""The oracle's pins must catch plausible mistakes in the oracle itself.

Each case edits one spot of a copy of ``oracle/qsa_oracle.c`` (a dropped term,
a wrong sign, index or operand, a reversed order), compiles it on the CPU and
runs the pins against it: at least one pin has to fail. The real oracle is
never edited.
"""
import os

import pytest

import oracle
import test_oracle_attention as A
import test_oracle_scores as S
import test_oracle_topk as T

SCORE_PINS = [
    S.test_hand_example,
    lambda lib: S.test_one_hot_keys_pick_a_coordinate(lib, 3),
    S.test_nonnegative_inputs_reduce_to_gemv,
    S.test_all_negative_dots_give_exact_zero,
    S.test_single_head_weight_isolates_that_head,
    S.test_mean_relu_matches_half_normal_closed_form,
    S.test_scores_at_matches_full,
]

TOPK_PINS = [
    lambda lib: T.test_hand_cases(lib, "topk_sort"),
    lambda lib: T.test_hand_cases(lib, "topk_rule"),
    lambda lib: T.test_brute_force_tiny(lib, 2),
    lambda lib: T.test_increasing_keys_take_the_last_blocks(lib, "topk_sort", 4, 2047),
    lambda lib: T.test_increasing_keys_take_the_last_blocks(lib, "topk_rule", 4, 2047),
    lambda lib: T.test_invariants_on_prompt_like_rows(lib, "q64"),
    lambda lib: T.test_cells_hand_cases(lib, "topk_sort_cells"),
    lambda lib: T.test_cells_hand_cases(lib, "topk_rule_cells"),
    lambda lib: T.test_cells_brute_force_tiny(lib, 3),
]

ATTN_PINS = [
    A.test_single_cell_returns_its_value,
    A.test_equal_logits_average_the_values,
    A.test_two_cells_are_a_logistic_mix,
    lambda lib: A.test_full_selection_is_dense_attention(lib, 8, 2),
    A.test_order_padding_and_foreign_ids_do_not_matter,
    A.test_empty_selection,
    A.test_group_sharing_uses_consecutive_heads,
]

# (name, original text, planted mistake, pins expected to notice)
MUTANTS = [
    ("relu dropped", "double relu = dot > 0.0 ? dot : 0.0;", "double relu = dot;", SCORE_PINS),
    ("relu keeps negatives", "double relu = dot > 0.0 ? dot : 0.0;",
     "double relu = dot < 0.0 ? dot : 0.0;", SCORE_PINS),
    ("weight of head 0 for all heads", "total += (double)w[(int64_t)iq * heads + h] * relu;",
     "total += (double)w[(int64_t)iq * heads] * relu;", SCORE_PINS),
    ("weight not applied", "total += (double)w[(int64_t)iq * heads + h] * relu;",
     "total += relu;", SCORE_PINS),
    ("query layout [head][query]", "q + ((int64_t)iq * heads + h) * head_dim;",
     "q + ((int64_t)h * nq + iq) * head_dim;", SCORE_PINS),
    ("key row stride off by one", "k + (int64_t)b * head_dim;",
     "k + (int64_t)b * (head_dim - 1);", SCORE_PINS),
    ("last coordinate dropped", "for (int d = 0; d < head_dim; ++d)\n                    dot",
     "for (int d = 0; d < head_dim - 1; ++d)\n                    dot", SCORE_PINS),
    ("weight inside relu", "double relu = dot > 0.0 ? dot : 0.0;\n"
     "                total += (double)w[(int64_t)iq * heads + h] * relu;",
     "double wd = (double)w[(int64_t)iq * heads + h] * dot;\n"
     "                total += wd > 0.0 ? wd : 0.0;", SCORE_PINS),
    ("ties by highest cell", "return (a->cell > b->cell) - (a->cell < b->cell);",
     "return (a->cell < b->cell) - (a->cell > b->cell);", TOPK_PINS),
    ("keys ascending", "if (a->key > b->key)\n        return -1;",
     "if (a->key > b->key)\n        return 1;\n    if (a->key < b->key)\n        return -1;\n    if (0)\n        return -1;",
     TOPK_PINS),
    ("cell takes the next block's key", "cells[c].key = scores[(int64_t)iq * ld + c / block_size];",
     "cells[c].key = scores[(int64_t)iq * ld + (c + 1) / block_size];", TOPK_PINS),
    ("active count ignored", "    if (!active)\n        return n_blocks;",
     "    if (1)\n        return n_blocks;", TOPK_PINS),
    ("above counts ties", "if (ordered_image(row[b]) > T)", "if (ordered_image(row[b]) >= T)", TOPK_PINS),
    ("negative keys mapped by sign flip", "return (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);",
     "return (bits & 0x80000000u) ? (bits ^ 0x80000000u) : (bits | 0x80000000u);", TOPK_PINS),
    ("signed zeros not merged", "    if (bits == 0x80000000u)\n        bits = 0u;", "", TOPK_PINS),
    ("tie budget one too many", "} else if (key == T && budget > 0) {",
     "} else if (key == T && budget >= 0) {", TOPK_PINS),
    ("partial tail block counted whole", "    return rest < block_size ? rest : block_size;",
     "    return block_size;", TOPK_PINS),
    ("visible cell count ignored", "        return c < 0 ? 0 : (c > all ? all : c);",
     "        return all;", TOPK_PINS),
    ("visible cells rounded up to whole blocks", "        return c < 0 ? 0 : (c > all ? all : c);",
     "        c = (c + block_size - 1) / block_size * block_size;\n        return c < 0 ? 0 : (c > all ? all : c);",
     TOPK_PINS),
    ("attention scale dropped", "s[i] = scale * dot;", "s[i] = dot;", ATTN_PINS),
    ("attention key head by modulo", "const int g = h / group;", "const int g = h % kv_heads;", ATTN_PINS),
    ("attention not normalised", "o[d] /= total;", "o[d] /= 1.0;", ATTN_PINS),
    ("attention lse without the max", "lse[(int64_t)iq * n_heads + h] = top + log(total);",
     "lse[(int64_t)iq * n_heads + h] = log(total);", ATTN_PINS),
    ("attention reads keys as values", "const float *vrow = v + ((int64_t)list[i] * kv_heads + g) * head_dim;",
     "const float *vrow = k + ((int64_t)list[i] * kv_heads + g) * head_dim;", ATTN_PINS),
    ("attention drops the last listed cell", "            for (int i = 0; i < width; ++i) {\n                if (isnan(s[i]))",
     "            for (int i = 0; i < width - 1; ++i) {\n                if (isnan(s[i]))", ATTN_PINS),
    ("attention keeps foreign ids", "if (c < 0 || c >= n_cells) {", "if (c < 0) {", ATTN_PINS),
    ("attention weights without the exponential", "const double e = exp(s[i] - top);",
     "const double e = 1.0 + (s[i] - top);", ATTN_PINS),
    ("attention cell rows without the head stride", "k + ((int64_t)c * kv_heads + g) * head_dim;",
     "k + ((int64_t)c + g) * head_dim;", ATTN_PINS),
]


@pytest.mark.parametrize("name,orig,planted,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, orig, planted, pins):
    src = open(oracle.SOURCE).read()
    assert src.count(orig) >= 1, f"mutation site not found: {name}"
    lib_path = oracle.compile_source(src.replace(orig, planted), os.path.join(tmp_path, "mutant.so"))
    lib = oracle.Library(lib_path)
    caught = []
    for pin in pins:
        try:
            pin(lib)
        except (AssertionError, ValueError, IndexError):
            caught.append(getattr(pin, "__name__", "pin"))
            break
    assert caught, f"no pin noticed the planted mistake '{name}'"
