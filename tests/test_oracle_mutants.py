"""Planted mistakes in the oracle must fail at least one pin.

Each case copies oracle/oracle.c, applies one textual change that a careless
reading of the pages could produce (a wrong comparison, a transposed operand,
a dropped term, an off-by-one row or uniform), compiles the copy with gcc on
the CPU and runs the whole pin suite against it in a subprocess.  The pins
are only trusted if every such mutant is caught.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "accept_with_le": ("if (!((double)u[i] < ratio)) j = i;",
                       "if (!((double)u[i] <= ratio)) j = i;"),
    "ratio_q_over_p": ("fmin(1.0, p / q)", "fmin(1.0, q / p)"),
    "residual_abs": ("r[t] = (p - q > 0.0) ? (p - q) : 0.0;", "r[t] = fabs(p - q);"),
    "residual_is_p": ("r[t] = (p - q > 0.0) ? (p - q) : 0.0;", "r[t] = p + 0.0 * q;"),
    "residual_q_minus_p": ("r[t] = (p - q > 0.0) ? (p - q) : 0.0;",
                           "r[t] = (q - p > 0.0) ? (q - p) : 0.0;"),
    "bonus_row_off_by_one": ("size_t prow = ((size_t)b * (K + 1) + j) * (size_t)V;",
                             "size_t prow = ((size_t)b * (K + 1) + (j == k && j > 0 ? j - 1 : j)) * (size_t)V;"),
    "final_uniform_is_u_j": ("double uf = (double)u[k];", "double uf = (double)u[j];"),
    "temperature_multiplies": ("exp((l - m) / T)", "exp((l - m) * T)"),
    "normaliser_ignores_T": ("z += exp((l - m) / T);", "z += exp(l - m);"),
    "cdf_with_le": ("if (target_mass < C)", "if (target_mass <= C)"),
    "argmax_ties_highest": ("if (l > bv) { bv = l; best = t; }",
                            "if (l >= bv) { bv = l; best = t; }"),
    "greedy_emits_draft": ("int32_t a_j = a[j];", "int32_t a_j = (j < k) ? xt[j] : a[j];"),
    "greedy_no_bonus": ("int32_t a_j = a[j];", "int32_t a_j = (j == k) ? -1 : a[j];"),
    "greedy_compares_next_row": ("if (xt[i] != a[i]) { j = i; break; }",
                                 "if (xt[i] != a[i + 1]) { j = i; break; }"),
    "q_zero_rejects": ("(q == 0.0) ? 1.0 :", "(q == 0.0) ? 0.0 :"),
    "last_draft_never_tested": ("for (int32_t i = 0; i < k; ++i) {\n            int32_t x = xt[i];",
                                "for (int32_t i = 0; i < k - 1; ++i) {\n            int32_t x = xt[i];"),
    "does_not_stop_at_first_rejection": ("if (j == k) { /* still on the path */", "if (1) {"),
    "rejected_draft_emitted": ("out[j] = tok;", "out[j] = (j < k) ? xt[j] : tok;"),
    "max_not_subtracted_in_prob": ("return exp((l - m) / T) / z;", "return exp(l / T) / z;"),
    "tested_excludes_rejected": ("if (i < k && i <= n) counters[(size_t)K + i] += 1;",
                                 "if (i < k && i < n) counters[(size_t)K + i] += 1;"),
    "accepted_counts_reached": ("if (i < n) counters[2 * (size_t)K + i] += 1;",
                                "if (i <= n && i < k) counters[2 * (size_t)K + i] += 1;"),
    "alpha_over_drafted": ("const double a = tested > 0.0 ? accepted / tested : 0.0;",
                           "const double a = drafted > 0.0 ? accepted / drafted : 0.0;"),
    "cost_counts_target_pass_twice": ("const double speedup = tokens / (1.0 + c * (double)k);",
                                      "const double speedup = tokens / (1.0 + c * (double)(k + 1));"),
    "tokens_without_extra_token": ("for (int32_t i = 0; i <= k; ++i) {\n            tokens += power;",
                                   "for (int32_t i = 1; i <= k; ++i) {\n            tokens += power;"),
    "ties_pick_larger_k": ("if (speedup > best) {", "if (speedup >= best) {"),
    "ngram_earliest_occurrence": ("for (int32_t e = L - 2; e >= n - 1; --e) {",
                                  "for (int32_t e = n - 1; e <= L - 2; ++e) {"),
    "ngram_shorter_first": ("for (int32_t n = n_max; n >= n_min && found_e < 0; --n) {",
                            "for (int32_t n = n_min; n <= n_max && found_e < 0; ++n) {"),
    "ngram_matches_itself": ("for (int32_t e = L - 2; e >= n - 1; --e) {",
                             "for (int32_t e = L - 1; e >= n - 1; --e) {"),
    "ngram_proposes_from_match_end": ("? c[found_e + 1 + i] : -1;", "? c[found_e + i] : -1;"),
    "ngram_no_run_in": ("kb = L - 1 - found_e;", "kb = L - 1 - found_e - 1;"),
    "tree_ignores_parent": ("acc[n] = parent_ok && tok[n] == amax[p + 1];",
                            "acc[n] = (parent_ok || 1) && tok[n] == amax[p + 1];"),
    "tree_own_row": ("acc[n] = parent_ok && tok[n] == amax[p + 1];",
                     "acc[n] = parent_ok && tok[n] == amax[n + 1];"),
    "tree_ties_last": ("if (acc[n] && depth[n] > end_depth) { end = n; end_depth = depth[n]; }",
                       "if (acc[n] && depth[n] >= end_depth) { end = n; end_depth = depth[n]; }"),
    "tree_bonus_from_parent": ("out[end_depth] = amax[end + 1];",
                               "out[end_depth] = amax[end >= 0 && par[end] >= 0 ? par[end] + 1 : 0];"),
    "mask_excludes_self": ("for (int32_t j = i; j >= 0; j = par[j]) m[",
                           "for (int32_t j = par[i]; j >= 0; j = par[j]) m["),
    "mask_parent_only": ("for (int32_t j = i; j >= 0; j = par[j]) m[",
                         "for (int32_t j = i; j >= 0 && j >= par[i]; j = par[j]) m["),
    "mask_transposed": ("m[(size_t)i * N + j] = 1;", "m[(size_t)j * N + i] = 1;"),
    "depth_zero_based": ("d[i] = par[i] < 0 ? 1 : d[par[i]] + 1;", "d[i] = par[i] < 0 ? 0 : d[par[i]] + 1;"),
    "topk_off_by_one": ("? s[top_k - 1] : -INFINITY;", "? s[top_k] : -INFINITY;"),
    "topp_strict": ("if (cum >= w) {", "if (cum > w) {"),
    "topp_over_all_tokens": ("for (int32_t i = 0; i < V && s[i] >= theta_k; ++i) zk +=",
                             "for (int32_t i = 0; i < V; ++i) zk +="),
    "topp_without_temperature": ("zk += exp((s[i] - m) / T);", "zk += exp(s[i] - m);"),
    "topp_floor_next_value": ("                    fl = v;\n", "                    fl = i < V ? s[i] : v;\n"),
    "topp_ignores_topk": ("        double fl = theta_k, mg = INFINITY;", "        double fl = -INFINITY, mg = INFINITY;"),
    "tree_first_accepted_not_deepest": ("if (acc[n] && depth[n] > end_depth) { end = n; end_depth = depth[n]; }",
                                        "if (acc[n] && end < 0) { end = n; end_depth = depth[n]; }"),
}

RUNNER = r"""
import sys
sys.path.insert(0, %(root)r)
import oracle
from tests import pins
o = oracle.Oracle(%(lib)r)
for pin in pins.ALL_PINS:
    try:
        pin(o)
    except AssertionError as e:
        print("CAUGHT_BY", pin.__name__)
        sys.exit(3)
print("NOT_CAUGHT")
sys.exit(0)
"""


def test_mutants_patch_cleanly():
    src = open(oracle.SOURCE).read()
    for name, (old, new) in MUTANTS.items():
        assert src.count(old) >= 1, name


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert old in src, "mutation anchor missing: %s" % name
    mutated = src.replace(old, new)
    csrc = tmp_path / "oracle_mutant.c"
    csrc.write_text(mutated)
    lib = str(tmp_path / "liboracle_mutant.so")
    oracle.compile_source(str(csrc), lib)
    env = dict(os.environ, OMP_NUM_THREADS="4")
    proc = subprocess.run([sys.executable, "-c", RUNNER % {"root": ROOT, "lib": lib}],
                          capture_output=True, text=True, timeout=300, env=env)
    out = proc.stdout + proc.stderr
    assert "NOT_CAUGHT" not in out, "planted mistake %r passed every pin" % name
    assert proc.returncode != 0, out[-2000:]
