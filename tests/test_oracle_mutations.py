"""Mutation controls for the oracle's pins.

Each case plants one plausible mistake in a copy of oracle/oracle.cpp (built
into a temporary directory, on the CPU) and checks that at least one of the
named pins in test_oracle_pins.py turns red against the mutant.  This shows
the pins can see the mistakes they are meant to catch.
"""
import importlib.util
import os
import shutil

import pytest

import test_oracle_pins as pins

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")

MUTATIONS = {
    "nibble_order_swapped": (
        "(kk & 1) ? (byte >> 4) : (byte & 0xf)", "(kk & 1) ? (byte & 0xf) : (byte >> 4)",
        ["test_dequant_golden"]),
    "scale_on_wrong_axis": (
        "s[n * (K / 32) + kk / 32]", "s[(kk / 32) * 0 + n * (K / 32) + (n % (K / 32))]",
        ["test_dequant_golden"]),
    "offset_seven": ("(double)(nib - 8)", "(double)(nib - 7)", ["test_dequant_golden"]),
    "tie_goes_to_higher_index": ("L[e] > L[best]", "L[e] >= L[best]",
                                 ["test_topk_brute_force_with_ties"]),
    "denominator_drops_last_pick": (
        "for (int64_t j = 0; j < k; ++j) den +=", "for (int64_t j = 0; j + 1 < k; ++j) den +=",
        ["test_weights_sum_and_ratio"]),
    "unstable_bucket_order": (
        "std::vector<int64_t> cur(off, off + E);\n  for (int64_t s = 0; s < S; ++s) {",
        "std::vector<int64_t> cur(off, off + E);\n  for (int64_t s = S - 1; s >= 0; --s) {",
        ["test_permute_matches_stable_sort"]),
    "dropped_pick_counted": ("if (valid(s)) cnt[idx[s]]++;", "if (idx[s] >= 0) cnt[idx[s] % E]++;",
                             ["test_permute_drops_out_of_range_picks"]),
    "dropped_pick_keeps_a_row": ("      row_of[s] = -1;\n      continue;", "      row_of[s] = 0;\n      continue;",
                                 ["test_permute_drops_out_of_range_picks"]),
    "silu_dropped": ("h[n] = g * sigmoid(g) * u;", "h[n] = g * u;",
                     ["test_expert_closed_form_uniform_planes"]),
    "down_reads_gate_row_count": (
        "acc += weight(fmt, qd, sd, I, n, kk) * h[kk];",
        "acc += weight(fmt, qd, sd, I, n, kk) * h[0];",
        ["test_expert_down_plane_orientation"]),
    "shared_gate_ignored": ("gw = sigmoid(a);", "gw = 1.0;", ["test_layer_shared_expert_gate"]),
    "e2m1_exponent_bias_zero": ("std::ldexp(1.0 + 0.5 * man, ex - 1)", "std::ldexp(1.0 + 0.5 * man, ex)",
                                ["test_e2m1_golden", "test_dequant_mxfp4_golden"]),
    "e2m1_subnormal_read_as_normal": ("(ex == 0) ? 0.5 * man", "(ex == 0) ? 1.0 * man",
                                      ["test_e2m1_golden"]),
    "e8m0_bias_128": ("std::ldexp(1.0, (int)e - 127)", "std::ldexp(1.0, (int)e - 128)",
                      ["test_e8m0_matches_library"]),
    "mxfp4_nibble_order_swapped": (
        "(kk & 1) ? (byte >> 4) : (byte & 0xf);\n  return e2m1_to_double(nib)",
        "(kk & 1) ? (byte & 0xf) : (byte >> 4);\n  return e2m1_to_double(nib)",
        ["test_dequant_mxfp4_golden"]),
    "mxfp4_scale_group_of_64": ("e8m0_to_double(s[n * (K / 32) + kk / 32])",
                                "e8m0_to_double(s[n * (K / 32) + kk / 64])",
                                ["test_dequant_mxfp4_golden"]),
    "mxfp4_scale_stride_two_bytes": ("return fmt == 1 ? 1 : 2;", "return 2;",
                                     ["test_layer_mxfp4_equals_dense_library_mixture"]),
    "bf16_rounded_through_fp32": ("const double a = std::fabs(v);",
                                  "const double a = (double)(float)std::fabs(v);",
                                  ["test_bf16_rounding_golden"]),
    "bf16_truncates": ("std::nearbyint(std::ldexp(a, -q))", "std::trunc(std::ldexp(a, -q))",
                       ["test_bf16_rounding_golden"]),
    "rms_eps_outside_root": ("std::sqrt(ss / (double)H + eps)", "(std::sqrt(ss / (double)H) + eps)",
                             ["test_add_rmsnorm_special_cases"]),
    "rms_mean_over_h_plus_one": ("std::sqrt(ss / (double)H + eps)",
                                 "std::sqrt(ss / (double)(H + 1) + eps)",
                                 ["test_add_rmsnorm_matches_library_rms_norm"]),
    "rms_weight_dropped": ("* inv * (double)g[h]", "* inv", ["test_add_rmsnorm_matches_library_rms_norm"]),
    "top_p_counts_the_pick_itself": (
        "    if (!(above / all < top_p)) break;\n    const double ex = std::exp((double)L[idx[j]] - l0);\n    above += ex;",
        "    const double ex = std::exp((double)L[idx[j]] - l0);\n    above += ex;\n    if (!(above / all < top_p)) break;",
        ["test_top_p_closed_form"]),
    "top_p_mass_over_picks_only": ("all += std::exp((double)L[e] - l0);",
                                   "all += (e < k) ? std::exp((double)L[idx[e]] - l0) : 0.0;",
                                   ["test_top_p_closed_form", "test_top_p_prefix_property"]),
    "top_p_weights_not_renormalised": ("w[j] = scale * std::exp((double)L[idx[j]] - l0) / kept_den;",
                                       "w[j] = scale * std::exp((double)L[idx[j]] - l0) / all;",
                                       ["test_top_p_closed_form"]),
    "variant_weights_from_keys": ("for (int64_t j = 0; j < k; ++j) den += s[idx[j]];\n  for (int64_t j = 0; j < k; ++j) w[j] = scale * s[idx[j]] / den;",
                                  "for (int64_t j = 0; j < k; ++j) den += key[idx[j]];\n  for (int64_t j = 0; j < k; ++j) w[j] = scale * key[idx[j]] / den;",
                                  ["test_sigmoid_gate_and_bias_closed_form"]),
    "sigmoid_of_negated_logit": ("s[e] = sigmoid((double)L[e]);", "s[e] = sigmoid(-(double)L[e]);",
                                 ["test_sigmoid_gate_and_bias_closed_form"]),
    "variant_tie_to_higher_index": ("if (best < 0 || key[e] > key[best]) best = e;",
                                    "if (best < 0 || key[e] >= key[best]) best = e;",
                                    ["test_variant_ties_lower_index"]),
    "group_score_top1_only": ("gscore[g] = gsz >= 2 ? kg[0] + kg[1] : kg[0];", "gscore[g] = kg[0];",
                              ["test_grouped_closed_form", "test_grouped_brute_force"]),
    "group_tie_to_higher_index": ("if (best < 0 || gscore[g] > gscore[best]) best = g;",
                                  "if (best < 0 || gscore[g] >= gscore[best]) best = g;",
                                  ["test_grouped_brute_force"]),
    "masked_experts_keyed_zero": ("for (int64_t e = 0; e < E; ++e) pickable[e] = kept[e / gsz];",
                                  "for (int64_t e = 0; e < E; ++e) if (!kept[e / gsz]) key[e] = 0.0;",
                                  ["test_grouped_closed_form"]),
    "groups_strided": ("for (int64_t e = 0; e < E; ++e) pickable[e] = kept[e / gsz];",
                       "for (int64_t e = 0; e < E; ++e) pickable[e] = kept[e % n_group];",
                       ["test_grouped_closed_form", "test_grouped_brute_force"]),
    "folded_router_first_row_only": ("oracle_router_logits(n_out, wr, nullptr, T, H, E, logits);",
                                     "oracle_router_logits(n_out, wr, nullptr, 1, H, E, logits);",
                                     ["test_add_rmsnorm_router_one_hot_rows"]),
    "folded_router_rows_off_by_one": ("oracle_router_logits(n_out, wr, nullptr, T, H, E, logits);",
                                       "oracle_router_logits(n_out, wr + H, nullptr, T, H, E - 1, logits);",
                                       ["test_add_rmsnorm_router_one_hot_rows"]),
    "combine_uses_first_weight": ("acc[h] += w[j] * o[h];", "acc[h] += w[0] * o[h];",
                                  ["test_layer_equals_dense_masked_mixture"]),
}


def _load_mutant(tmp_path, name, old, new):
    d = tmp_path / name
    shutil.copytree(ORACLE_DIR, d, ignore=shutil.ignore_patterns("*.so", "__pycache__", "*.tmp*"))
    src = (d / "oracle.cpp").read_text()
    assert old in src, "mutation anchor not found: %s" % name
    (d / "oracle.cpp").write_text(src.replace(old, new, 1))
    spec = importlib.util.spec_from_file_location("oracle_mut_" + name, d / "__init__.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.build(force=True)
    mod.lib()
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(tmp_path, name):
    old, new, tests = MUTATIONS[name]
    mut = _load_mutant(tmp_path, name, old, new)
    caught = []
    for t in tests:
        try:
            getattr(pins, t)(mut)
        except AssertionError:
            caught.append(t)
    assert caught, "no pin caught mutation %s" % name
