"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake into a copy of oracle/moe_oracle.cpp (on the CPU,
in a temporary directory), builds it, and runs the pin suite
(tests/test_oracle.py) against that library; the suite must fail.  The
original oracle is never modified.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.cpp")

# (name, original text, mistaken text)
MUTANTS = [
    ("bias_dropped", "      if (bias) acc += static_cast<double>(bias[e]);", "      (void)bias;"),
    ("tie_to_higher_id", "      if (best < 0 || key[e] > key[best]) best = e;",
     "      if (best < 0 || key[e] >= key[best]) best = e;"),
    ("no_renormalisation", "  for (int k = 0; k < K; ++k) w[k] = renorm ? s[ids[k]] / total : s[ids[k]];",
     "  for (int k = 0; k < K; ++k) w[k] = s[ids[k]];"),
    ("sigmoid_sign", "    for (int e = 0; e < E; ++e) s[e] = 1.0 / (1.0 + std::exp(-z[e]));",
     "    for (int e = 0; e < E; ++e) s[e] = 1.0 / (1.0 + std::exp(z[e]));"),
    ("softmax_missing_denominator", "  for (int e = 0; e < E; ++e) s[e] = std::exp(z[e] - m) / denom;",
     "  for (int e = 0; e < E; ++e) s[e] = std::exp(z[e] - m);"),
    ("dispatch_token_major", "  for (int e = e_begin; e < e_end; ++e) {\n    for (int t = 0; t < T; ++t) {",
     "  for (int t = 0; t < T; ++t) {\n    for (int e = e_begin; e < e_end; ++e) {"),
    ("offsets_inclusive", "  for (int j = 0; j < n_loc; ++j) offsets[j + 1] = offsets[j] + counts[e_begin + j];",
     "  for (int j = 0; j < n_loc; ++j) offsets[j + 1] = offsets[j] + counts[e_begin + j] + (j == 0);"),
    ("nonlocal_rows_not_cleared", "  for (int a = 0; a < T * K; ++a) row_of[a] = -1;", "  (void)0;"),
    ("silu_sign", "double silu(double z) { return z / (1.0 + std::exp(-z)); }",
     "double silu(double z) { return z / (1.0 + std::exp(z)); }"),
    ("gate_up_swapped", "      h[j] = silu(g) * u;", "      h[j] = silu(u) * g;"),
    ("down_transposed", "      const size_t base = (e * d + c) * (size_t)I;\n      for (int j = 0; j < I; ++j) acc += h[j] * value_at(w_down, base + j, dt_w);",
     "      for (int j = 0; j < I; ++j) acc += h[j] * value_at(w_down, (e * I + j) * (size_t)d + c, dt_w);"),
    ("combine_ignores_shared", "      for (int s = 0; s < n_shared; ++s)\n        acc += value_at(y_shared, ((size_t)s * T + t) * d + c, dt_y);",
     "      (void)n_shared;"),
    ("combine_weight_index", "        acc += value_at(weights, t * K + k, dt_w) * value_at(y_sorted, (size_t)r * d + c, dt_y);",
     "        acc += value_at(weights, (size_t)k * T + t, dt_w) * value_at(y_sorted, (size_t)r * d + c, dt_y);"),
    ("split_without_padding", "  const int t_pad = (T + pad - 1) / pad * pad;", "  const int t_pad = T;"),
    ("bf16_round_truncates", "      r = std::ldexp(std::nearbyint(std::ldexp(v, -q)), q);",
     "      r = std::ldexp(std::trunc(std::ldexp(v, -q)), q);"),
    ("e4m3_ties_away", "  const double r = std::nearbyint(a / q) * q;  // round to nearest, ties to even",
     "  const double r = std::round(a / q) * q;"),
    ("mx_scale_one_binade_low", "        s = std::min(127, std::max(-127, e - 1 - 8));",
     "        s = std::min(127, std::max(-127, e - 8));"),
    ("mx_no_clamp", "        codes[(size_t)r * cols + b * 32 + i] = oracle_e4m3_encode(std::min(448.0, std::max(-448.0, v)));",
     "        codes[(size_t)r * cols + b * 32 + i] = oracle_e4m3_encode(v);"),
    ("mx_forward_payload_not_encoded",
     "    oracle_mxfp8_dequantize(rows, cols, codes.data(), scales.data(), v.data());",
     "    for (size_t i = 0; i < v.size(); ++i) v[i] = value_at(m, i, t);"),
    ("mx_forward_h_not_encoded",
     "  const std::vector<double> hq = decoded(n_rows, I, ODT_F64, hh.data());",
     "  const std::vector<double> hq = hh;"),
    ("dbo_boundary_ties_high",
     "    split = (split - below <= above - split) ? below : above;",
     "    split = (split - below < above - split) ? below : above;"),
    ("e4m3_subnormal_step", "  if (ef == 0) return sign * std::ldexp((double)m, -9);",
     "  if (ef == 0) return sign * std::ldexp((double)m, -8);"),
    ("invalid_ids_not_counted", "    if (e < 0 || e >= E) ++bad;\n    else ++counts[e];",
     "    if (e < 0 || e >= E) (void)bad;\n    else ++counts[e];"),
    ("dispatch_slot_major",
     "    for (int t = 0; t < T; ++t) {\n      for (int k = 0; k < K; ++k) {\n        if (ids[(size_t)t * K + k] != e) continue;",
     "    for (int k = 0; k < K; ++k) {\n      for (int t = 0; t < T; ++t) {\n        if (ids[(size_t)t * K + k] != e) continue;"),
    ("softmax_without_max_shift",
     "  for (int e = 0; e < E; ++e) denom += std::exp(z[e] - m);\n  for (int e = 0; e < E; ++e) s[e] = std::exp(z[e] - m) / denom;",
     "  for (int e = 0; e < E; ++e) denom += std::exp(z[e]);\n  for (int e = 0; e < E; ++e) s[e] = std::exp(z[e]) / denom;"),
    ("combine_weights_shared_rows",
     "        acc += value_at(y_shared, ((size_t)s * T + t) * d + c, dt_y);",
     "        acc += value_at(weights, t * K, dt_w) * value_at(y_shared, ((size_t)s * T + t) * d + c, dt_y);"),
    ("select_on_scores", "    topk_of_row(key.data(), E, K, ids + (size_t)t * K);",
     "    topk_of_row(s.data(), E, K, ids + (size_t)t * K);"),
    ("score_kind_ignored", "  if (score == OSCORE_SIGMOID) {\n    for (int e = 0; e < E; ++e) s[e] = 1.0 / (1.0 + std::exp(-z[e]));",
     "  if (score != OSCORE_SIGMOID) {\n    for (int e = 0; e < E; ++e) s[e] = 1.0 / (1.0 + std::exp(-z[e]));"),
    ("mx_shared_first_stack_only",
     "      for (int t = 0; t < T; ++t) sh_expert[t] = s;\n      oracle_expert_mlp_mxfp8(",
     "      for (int t = 0; t < T; ++t) sh_expert[t] = 0;\n      oracle_expert_mlp_mxfp8("),
]


@pytest.mark.parametrize("name,orig,bad", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, orig, bad, tmp_path):
    src = open(SRC).read()
    assert src.count(orig) == 1, f"mutation site for {name} not found exactly once"
    mutant = os.path.join(tmp_path, "moe_oracle_mutant.cpp")
    with open(mutant, "w") as f:
        f.write(src.replace(orig, bad))
    lib = os.path.join(tmp_path, "liboracle_mutant.so")
    subprocess.run(["g++", "-O1", "-std=c++17", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    mutant, "-o", lib], check=True)
    env = dict(os.environ, ORACLE_LIBRARY=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"the oracle pins did not catch mutant {name}:\n{r.stdout[-2000:]}"
