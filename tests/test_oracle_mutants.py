"""Mutation check of the oracle's pins (no GPU).

Each case plants one plausible slip in a copy of oracle.c (the committed
oracle is untouched), builds it into a temporary library, and runs the pins
of tests/test_oracle_pins.py against it: at least one pin must fail.
"""
import os
import subprocess

import pytest

import oracle
import test_oracle_accept as acc
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

ROUTE = [lambda: pins.test_route_matches_brute_force(16, 4, 2, 4, 256),
         lambda: pins.test_route_matches_brute_force(256, 8, 4, 8, 128),
         pins.test_route_textbook_special_case, pins.test_route_group_score_is_top2_sum,
         pins.test_route_excluded_groups_never_selected, pins.test_route_ties_go_to_lower_index,
         pins.test_route_weights_use_unbiased_scores]
QUANT = [pins.test_quant_round_half_even_by_hand, pins.test_quant_closed_forms]
DOTS = [pins.test_code_layout_by_hand] + \
       [lambda b=b: pins.test_block_dots_brute_force(b) for b in (2, 4, 8)] + \
       [lambda b=b: pins.test_matvec_equals_dequantised_matmul(b) for b in (2, 4, 8)]
LAYER = [pins.test_single_expert_layer_is_dense_swiglu, pins.test_layer_linear_in_rsf_and_shared_alone,
         pins.test_layer_equals_sum_of_experts]
MISC = [pins.test_rmsnorm_closed_forms, pins.test_permute_is_stable_sort, pins.test_permute_skips_dropped_assignments]
TOPP = [lambda: pins.test_top_p_keeps_the_shortest_prefix_reaching_p(0.7), pins.test_top_p_off_and_single_expert,
        pins.test_top_p_boundary_is_inclusive, pins.test_top_p_follows_selection_order_not_weight,
        pins.test_top_p_layer_with_one_expert_per_token]
ACCEPT = [acc.test_sampled_first_token_is_lossless, acc.test_acceptance_rate_is_one_minus_total_variation,
          acc.test_second_and_bonus_tokens_follow_their_rows, acc.test_no_drafts_is_inverse_cdf_sampling_of_p,
          acc.test_identical_draft_and_target_keep_every_draft, acc.test_greedy_equals_plain_greedy_decoding,
          acc.test_temperature_enters_both_distributions]
ALL = ROUTE + QUANT + DOTS + LAYER + MISC + TOPP + ACCEPT

MUTANTS = {
    "group score = max only": ("gscore[g] = (m >= 2) ? b1 + b2 : b1;", "gscore[g] = b1;"),
    "group ties to higher index": ("gscore[g] > gscore[best]", "gscore[g] >= gscore[best]"),
    "expert ties to higher index": ("!taken[e] && (best < 0 || c[e] > c[best])",
                                    "!taken[e] && (best < 0 || c[e] >= c[best])"),
    "weights from biased score": ("(float)(s[idx[(size_t)t * k + i]] / sum",
                                  "(float)(c[idx[(size_t)t * k + i]] / sum"),
    "rsf dropped": ("/ sum * sh->rsf)", "/ sum)"),
    "sigmoid sign": ("s[e] = 1.0 / (1.0 + exp(-z));", "s[e] = 1.0 / (1.0 + exp(z));"),
    "gate weight transposed": ("gate_w[(size_t)e * H + j]", "gate_w[(size_t)j * E + e]"),
    "round half away": ("rintf(xb[j] / db)", "roundf(xb[j] / db)"),
    "reciprocal multiply": ("rintf(xb[j] / db)", "rintf(xb[j] * (1.0f / db))"),
    "scale over 128": ("amax / 127.0f", "amax / 128.0f"),
    "nibble order": ("(j & 1) ? (row[j >> 1] >> 4) : (row[j >> 1] & 15)",
                     "(j & 1) ? (row[j >> 1] & 15) : (row[j >> 1] >> 4)"),
    "int4 offset not two's complement": ("return nib >= 8 ? nib - 16 : nib;", "return nib - 8;"),
    "int2 field order": ("int f = (row[j >> 2] >> (2 * (j & 3))) & 3;",
                         "int f = (row[j >> 2] >> (6 - 2 * (j & 3))) & 3;"),
    "wrong activation block scale": ("acc += (double)d[(size_t)t * nb + b] * (double)blk;",
                                     "acc += (double)d[(size_t)t * nb] * (double)blk;"),
    "silu -> sigmoid": ("double silu = gz / (1.0 + exp(-gz));", "double silu = 1.0 / (1.0 + exp(-gz));"),
    "gate and up swapped": ("h[i] = (float)(silu * (double)u[i]);",
                            "h[i] = (float)((double)u[i] / (1.0 + exp(-(double)u[i])) * gz);"),
    "shared scaled by rsf": ("if (y_shared) acc += (double)y_shared[(size_t)t * H + r];",
                             "if (y_shared) acc += sh->rsf * (double)y_shared[(size_t)t * H + r];"),
    "rmsnorm eps outside sqrt": ("sqrt(ss / H + eps)", "(sqrt(ss / H) + eps)"),
    "top-p boundary exclusive": ("if (cum >= sh->top_p) break;", "if (cum > sh->top_p) break;"),
    "top-p not renormalised": ("            sum = 0.0;\n            for (int i = 0; i < kept; i++)",
                               "            for (int i = 0; i < kept; i++) if (0)"),
    "top-p counts one short": ("                kept++;\n                if (cum >= sh->top_p) break;",
                               "                if (cum >= sh->top_p) break;\n                kept++;"),
    "permute keeps dropped": ("        if (idx[a] == -1) continue;                 /* dropped by top-p: no row */\n",
                              "        if (idx[a] == -1) { off[1]++; continue; }\n"),
    "permute not stable": ("int row = fill[idx[a]]++;",
                           "int row = off[idx[a]] + off[idx[a] + 1] - 1 - fill[idx[a]]++;"),
    "draft test ratio inverted": ("const double lhs = ub[i] * Q[x], rhs = P[x];",
                                  "const double lhs = ub[i] * P[x], rhs = Q[x];"),
    "residual q - p": ("Q[y] = P[y] > Q[y] ? P[y] - Q[y] : 0.0;", "Q[y] = Q[y] > P[y] ? Q[y] - P[y] : 0.0;"),
    "residual not clipped": ("Q[y] = P[y] > Q[y] ? P[y] - Q[y] : 0.0;", "Q[y] = P[y] - Q[y];"),
    "residual from p": ("nx = inverse_cdf(R > 0.0 ? Q : P, V, ub[D], &m2);", "nx = inverse_cdf(P, V, ub[D], &m2);"),
    "draft rows off by one": ("softmax_row(pb + (size_t)i * V, V, tau, P);",
                              "softmax_row(pb + (size_t)(i + 1) * V, V, tau, P);"),
    "inverse cdf unscaled": ("const double t = u * W;", "const double t = u;"),
    "inverse cdf reuses a draw": ("nx = inverse_cdf(P, V, ub[D], &m2);", "nx = inverse_cdf(P, V, ub[0], &m2);"),
    "argmax ties to higher index": ("if (z[x] > z[a]) a = x;", "if (z[x] >= z[a]) a = x;"),
    "greedy against draft logits": ("const int a = argmax_row(pb + (size_t)i * V, V);",
                                    "const int a = argmax_row(qb + (size_t)i * V, V);"),
    "temperature ignored": ("out[x] = exp(((double)z[x] - (double)m) / tau);",
                            "out[x] = exp((double)z[x] - (double)m);"),
}


@pytest.fixture
def mutant_lib(tmp_path):
    saved = (oracle.LIB, oracle._lib)

    def make(old, new):
        src = open(SRC).read()
        assert src.count(old) == 1, "mutation anchor not unique: %r" % old
        d = tmp_path / "m"
        d.mkdir(exist_ok=True)
        (d / "oracle.c").write_text(src.replace(old, new))
        (d / "oracle.h").write_text(open(SRC[:-1] + "h").read())
        so = str(d / "liboracle_mut.so")
        subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
                        "-ffp-contract=off", str(d / "oracle.c"), "-o", so, "-lm"], check=True)
        oracle.LIB, oracle._lib = so, None
        oracle.lib()

    yield make
    oracle.LIB, oracle._lib = saved


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, mutant_lib):
    mutant_lib(*MUTANTS[name])
    caught = []
    for pin in ALL:
        try:
            pin()
        except (AssertionError, ValueError, RuntimeError, IndexError):
            caught.append(getattr(pin, "__name__", "pin"))
    assert caught, "no pin caught the mutant %r" % name


def test_unmutated_copy_passes(mutant_lib):
    mutant_lib("static size_t row_bytes", "static size_t row_bytes")
    for pin in ALL:
        pin()
