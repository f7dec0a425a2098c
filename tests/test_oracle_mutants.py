"""Mutation tests for the oracle's pins.

Each case copies the oracle source, plants one plausible mistake (a dropped
term, a wrong comparison, a swapped operand), builds it on the CPU, and checks
that at least one pin fails on the planted build.  The oracle itself is never
modified and the GPU is never touched.
"""
import numpy as np
import pytest

import oracle
import test_oracle_bf16_router_pins as hf_pins
import test_oracle_channel_topk_pins as ck_pins
import test_oracle_pins as pins
import test_oracle_shared_pins as shared_pins

MUTANTS = {
    "tie break takes the higher index":
        ("if (best < 0 || p[e] > p[best])", "if (best < 0 || p[e] >= p[best])"),
    "top-k2 mass drops the first term":
        ("for (int32_t r = 0; r < K2; ++r)\n            M = M + p[rank_id[r]];",
         "for (int32_t r = 1; r < K2; ++r)\n            M = M + p[rank_id[r]];"),
    "no-renormalisation branch only for k2 > E":
        ("if (k2 >= E) {", "if (k2 > E) {"),
    "mass over top-k1 instead of top-k2":
        ("int32_t K2 = k2 < E ? k2 : E;", "int32_t K2 = k1;"),
    "ln2 low part dropped":
        ("r = fmaf(-n, g_ln2_lo, r);", "r = r;"),
    "Taylor polynomial one degree short":
        ("float q = g_inv_fact[7];", "float q = 0.0f;"),
    "no max subtraction":
        ("p[e] = oracle_exp_spec(l[e] - m);", "p[e] = oracle_exp_spec(l[e] - m + 1.0f);"),
    "sequential instead of pairwise sum":
        ("float S = pairwise_sum(p, 0, next_pow2(E), E);",
         "float S = 0.0f; for (int32_t q = 0; q < E; ++q) S += p[q];"),
    "multiply by reciprocal instead of divide":
        ("p[e] = p[e] / S;", "p[e] = p[e] * (1.0f / S);"),
    "silu on the up projection":
        ("a[c] = silu(g) * u;", "a[c] = g * silu(u);"),
    "weights not applied in the combine":
        ("acc[h] += wr * z;", "acc[h] += z;"),
    "router bias dropped":
        ("s += (double)br[e];", "s += 0.0;"),
    "gate and up read the same row":
        ("u += load_elem(Wu, wt, row + h) * xv[h];", "u += load_elem(Wg, wt, row + h) * xv[h];"),
    "bf16 rounding truncates":
        ("double m = nearbyint(ldexp(d, -q));", "double m = trunc(ldexp(d, -q));"),
    "bf16 rounding sends ties away from zero":
        ("double m = nearbyint(ldexp(d, -q));", "double m = round(ldexp(d, -q));"),
    "bf16 rounding keeps one bit too many":
        ("int q = ex - 8;", "int q = ex - 9;"),
    "bf16 logits left in fp32":
        ("logits[t * E + e] = round_bf16(s);", "logits[t * E + e] = (float)s;"),
    "bf16 router weights not cast":
        ("w[i] = round_bf16((double)w[i]);", "w[i] = w[i];"),
    "shared expert gate not applied":
        ("ys[t * H + h] = (float)(g * z);", "ys[t * H + h] = (float)z;"),
    "shared expert gate with the wrong sign":
        ("g = 1.0 / (1.0 + exp(-z));", "g = 1.0 / (1.0 + exp(z));"),
    "shared expert silu on the up projection":
        ("a[c] = silu(gg) * u;", "a[c] = gg * silu(u);"),
    "shared expert gate and up read the same row":
        ("u += load_elem(Su, wt, row + h) * xv[h];", "u += load_elem(Sg, wt, row + h) * xv[h];"),
    "channel select takes the higher index on ties":
        ("if (best < 0 || s[j] > s[best])", "if (best < 0 || s[j] >= s[best])"),
    "channel score without the down-column norm":
        ("(float)((double)w[t * k1 + r] * (double)dn[e * I + c] * fabs(a));",
         "(float)((double)w[t * k1 + r] * fabs(a));"),
    "channel score on the signed activation":
        ("(float)((double)w[t * k1 + r] * (double)dn[e * I + c] * fabs(a));",
         "(float)((double)w[t * k1 + r] * (double)dn[e * I + c] * a);"),
    "column norm without the square root":
        ("dn[e * I + c] = (float)sqrt(s);", "dn[e * I + c] = (float)s;"),
    "kept channels not weighted":
        ("double a = silu(g) * u * (double)w[t * k1 + r];", "double a = silu(g) * u;"),
}

PIN_CHECKS = [
    pins.test_golden_closed_forms,
    lambda: pins.test_topk_matches_brute_force_on_tiny_E(5),
    lambda: pins.test_k1_equal_k2_is_standard_renormalisation_bitwise(128, 8),
    lambda: pins.test_k2_at_least_E_gives_probabilities_bitwise(128, 4),
    lambda: pins.test_weight_sum_is_topk1_mass_over_topk2_mass(128, 4, 16),
    pins.test_tie_break_takes_lower_index,
    pins.test_exp_spec_sampled_against_numpy,
    lambda: pins.test_softmax_sums_to_one_and_matches_fp64(128),
    pins.test_softmax_sum_order_and_division,
    pins.test_softmax_max_subtraction_is_shift_invariant,
    lambda: pins.test_each_expert_matches_numpy_fp64(False),
    pins.test_single_expert_case,
    pins.test_router_bias_is_added,
    hf_pins.test_round_bf16_matches_torch_cast_from_fp32,
    hf_pins.test_bf16_logits_are_the_exact_dot_product_rounded_once,
    lambda: hf_pins.test_bf16_router_at_k1_eq_k2_is_stock_bitwise(128, 8),
    lambda: shared_pins.test_shared_matches_numpy_fp64(False, True),
    shared_pins.test_zero_gate_vector_halves_the_expert,
    ck_pins.test_down_column_norms_match_numpy,
    ck_pins.test_scores_match_numpy_fp64,
    lambda: ck_pins.test_select_matches_a_lexicographic_sort(50),
    ck_pins.test_kept_layer_matches_numpy_masked_fp64,
]


def run_pins():
    failed = 0
    for check in PIN_CHECKS:
        try:
            check()
        except (AssertionError, oracle.OracleError):
            failed += 1
    return failed


def test_pins_pass_on_the_real_oracle():
    assert run_pins() == 0


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = oracle.SRC.read_text()
    assert src.count(old) == 1, f"mutation site for '{name}' not found once"
    mut = tmp_path / "oracle_mut.c"
    mut.write_text(src.replace(old, new))
    so = oracle.build(src=mut, out=tmp_path / "liboracle_mut.so")
    with oracle.using_library(so):
        failed = run_pins()
    assert failed > 0, f"no pin caught the planted mistake: {name}"
