"""Each plausible mistake planted in a copy of the oracle (compiled to a
temporary library on the CPU) must fail at least one pin.  This shows that the
pins constrain the oracle, not just agree with it."""
import os
import subprocess

import pytest

import oracle
import pins

# (name, original text, replacement) -- each original must occur exactly once
MUTANTS = [
    ("lse_becomes_max", "  return m + log(s);\n}", "  (void)s;\n  return m;\n}"),
    ("intermediate_drops_second_child",
     "  for (int64_t r = 2 * j; r <= 2 * j + 1 && r < m_child; ++r) {\n    if (p->causal",
     "  for (int64_t r = 2 * j; r <= 2 * j && r < m_child; ++r) {\n    if (p->causal"),
    ("ties_go_to_higher_index",
     "  return (x->j < y->j) ? -1 : (x->j > y->j);\n}\n\nstatic int by_index",
     "  return (x->j > y->j) ? -1 : (x->j < y->j);\n}\n\nstatic int by_index"),
    ("leaf_causal_mask_off_by_one", "    if (p->causal && i > t) break;\n    buf[n++]",
     "    if (p->causal && i >= t) break;\n    buf[n++]"),
    ("leaf_mean_divides_by_C", "      pyr[j * D + d] = s / (double)(hi - lo);", "      pyr[j * D + d] = s / (double)C;"),
    ("gqa_uses_first_head_only", "        for (int32_t g = 0; g < G; ++g) {\n          int32_t hq = h * G + g;",
     "        for (int32_t g = 0; g < 1; ++g) {\n          int32_t hq = h * G + g;"),
    ("expansion_forgets_doubling",
     "        for (int64_t r = 2 * A[a].j; r <= 2 * A[a].j + 1 && r < m_child; ++r) {\n          next[nn].j = r;",
     "        for (int64_t r = A[a].j; r <= A[a].j + 1 && r < m_child; ++r) {\n          next[nn].j = r;"),
    ("leaf_score_unscaled", "    buf[n++] = dot_qk(q, k, p->dtype, qoff, kbase + i * p->D, p->D) * p->scale;",
     "    buf[n++] = dot_qk(q, k, p->dtype, qoff, kbase + i * p->D, p->D);"),
    ("attention_ignores_causal_mask", "          if (p->causal && i > t) break;\n          key[n] = i;",
     "          key[n] = i;"),
    ("block_start_one_level_off", "  return j * (int64_t)C * ((int64_t)1 << (l - 1));",
     "  return j * (int64_t)C * ((int64_t)1 << l);"),
    ("ragged_parent_halves_single_child", "      int64_t nch = (2 * j + 1 < mc) ? 2 : 1;",
     "      int64_t nch = 2;\n      if (2 * j + 1 >= mc) { for (int32_t d = 0; d < D; ++d) par[j * D + d] = child[2 * j * D + d] / 2.0; continue; }"),
    ("keeps_one_block_too_few", "      nI = K;\n", "      nI = K > 1 ? K - 1 : 1;\n"),
    ("flat_uses_first_head_only", "            for (int32_t g = 0; g < G; ++g) {\n              int64_t qoff",
     "            for (int32_t g = 0; g < 1; ++g) {\n              int64_t qoff"),
    ("backward_drops_row_term", "            const double ds = z[a] * (dp - Dt);", "            const double ds = z[a] * dp;"),
    ("child_dots_count_invalid_children",
     "              if (!(p->causal && block_start(r, p->C, l - 1) > t)) cnt[CNT_CHILD_DOTS] += 1;",
     "              cnt[CNT_CHILD_DOTS] += 1;"),
    ("leaf_key_dots_ignore_causal_mask", "            if (must_score) cnt[CNT_LEAF_KEY_DOTS] += (g == 0) ? nk : 0;",
     "            if (must_score) cnt[CNT_LEAF_KEY_DOTS] += (g == 0) ? p->C : 0;"),
    ("leaf_key_dots_counted_per_head", "            if (must_score) cnt[CNT_LEAF_KEY_DOTS] += (g == 0) ? nk : 0;",
     "            if (must_score) cnt[CNT_LEAF_KEY_DOTS] += nk;"),
    ("unscored_leaf_level_counted", "        if (must_score) {\n          if (l == 1) {",
     "        if (1) {\n          if (l == 1) {"),
    ("backward_dk_unscaled", "              dk[ko + d] += p->scale * ds * widen(q, p->dtype, qoff + d);",
     "              dk[ko + d] += ds * widen(q, p->dtype, qoff + d);"),
]


@pytest.fixture(scope="module")
def source():
    with open(os.path.join(os.path.dirname(oracle.__file__), "pisa_oracle.c")) as f:
        return f.read()


@pytest.mark.parametrize("name,orig,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_fails_a_pin(tmp_path, source, name, orig, repl):
    assert source.count(orig) == 1, f"mutation site for {name} not unique"
    src = tmp_path / f"{name}.c"
    src.write_text(source.replace(orig, repl))
    so = tmp_path / f"lib{name}.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", str(src), "-o", str(so), "-lm"])
    lib = oracle.load(str(so))
    caught = []
    for pin_name, check in pins.ALL_CHECKS:
        try:
            check(lib)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append(pin_name)
            break
    assert caught, f"mutant {name} passed every pin"
