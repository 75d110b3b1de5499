"""Planted mistakes in the oracle must each fail at least one pin.

Every mutation below is a plausible slip (a dropped term, a wrong sign, a
wrong index or operand, a flipped tie-break). The test compiles a mutated
copy of oracle.c on the CPU, runs the whole pin suite against it and
requires at least one pin to fail. The committed oracle is never modified.
"""
import os
import subprocess

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTATIONS = {
    "bf16_shift": ("(uint32_t)bits << 16", "(uint32_t)bits << 15"),
    "bias_dropped": ("l[e] += (double)bias[e];", "l[e] += 0.0;"),
    "router_row_stride": ("wg + (int64_t)e * H, H);", "wg + (int64_t)e, H);"),
    "topk_tie_to_higher": ("if (best < 0 || v > best_v) {", "if (best < 0 || v >= best_v) {"),
    "topk_ascending": ("if (best < 0 || v > best_v) {", "if (best < 0 || v < best_v) {"),
    "softmax_sign": ("w[(int64_t)t * k + j] = exp(l[idx[(int64_t)t * k + j]] - m) / den;",
                     "w[(int64_t)t * k + j] = exp(m - l[idx[(int64_t)t * k + j]]) / den;"),
    "softmax_not_normalised": ("w[(int64_t)t * k + j] = exp(l[idx[(int64_t)t * k + j]] - m) / den;",
                               "w[(int64_t)t * k + j] = exp(l[idx[(int64_t)t * k + j]] - m);"),
    "silu_on_up": ("double s = g / (1.0 + exp(-g));\n    return s * u;",
                   "double s = u / (1.0 + exp(-u));\n    return s * g;"),
    "sigmoid_not_silu": ("double s = g / (1.0 + exp(-g));", "double s = 1.0 / (1.0 + exp(-g));"),
    "silu_exp_sign": ("double s = g / (1.0 + exp(-g));", "double s = g / (1.0 + exp(g));"),
    "token_index": (
        "int32_t t = (int32_t)(p / k);\n            int64_t e = idx[p];\n            const uint16_t *xt = x + (int64_t)t * H;\n            double g = dot_bf16(",
        "int32_t t = (int32_t)(p % M);\n            int64_t e = idx[p];\n            const uint16_t *xt = x + (int64_t)t * H;\n            double g = dot_bf16("),
    "fp8_token_index": (
        "int32_t t = (int32_t)(p / k);\n            int64_t e = idx[p];\n            const uint16_t *xt = x + (int64_t)t * H;\n            double g = dot_e4m3(",
        "int32_t t = (int32_t)(p % M);\n            int64_t e = idx[p];\n            const uint16_t *xt = x + (int64_t)t * H;\n            double g = dot_e4m3("),
    "down_wrong_expert": ("y[p * H + r] = dot_bf16_f64(wdown + (e * H + r) * I, a + p * I, I);",
                          "y[p * H + r] = dot_bf16_f64(wdown + ((int64_t)idx[0] * H + r) * I, a + p * I, I);"),
    "down_transposed_rows": ("y[p * H + r] = dot_bf16_f64(wdown + (e * H + r) * I, a + p * I, I);",
                             "y[p * H + r] = dot_bf16_f64(wdown + e * H * I + r, a + p * I, I - r / I);"),
    "combine_unweighted": ("s += w[p] * y[p * H + r];", "s += y[p * H + r];"),
    "combine_last_slot_dropped": (
        "for (int32_t j = 0; j < k; ++j) {\n                int64_t p = (int64_t)t * k + j;\n                s +=",
        "for (int32_t j = 0; j + 1 < k; ++j) {\n                int64_t p = (int64_t)t * k + j;\n                s +="),
    "fp8_combine_last_slot_dropped": (
        "for (int32_t j = 0; j < k; ++j) {\n                int64_t p = (int64_t)t * k + j;\n                int64_t e",
        "for (int32_t j = 0; j + 1 < k; ++j) {\n                int64_t p = (int64_t)t * k + j;\n                int64_t e"),
    "argmax_tie_to_higher": ("if (zv > best_v) {", "if (zv >= best_v) {"),
    "argmax_skips_last": ("for (int32_t v = 1; v < V; ++v) {", "for (int32_t v = 1; v + 1 < V; ++v) {"),
    "lmhead_row_stride": ("wlm + (int64_t)v * H, H);", "wlm + (int64_t)v, H);"),
    "e4m3_bias_8": ("ldexp(1.0 + (double)m / 8.0, e - 7);", "ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "e4m3_subnormal_scale": ("? ldexp((double)m / 8.0, -6)", "? ldexp((double)m / 8.0, -7)"),
    "e4m3_mantissa_16": ("ldexp(1.0 + (double)m / 8.0, e - 7);", "ldexp(1.0 + (double)m / 16.0, e - 7);"),
    "fp8_down_scale_dropped": ("double sd = sdown[e * H + r], y = 0.0;", "double sd = 1.0, y = 0.0;"),
    "fp8_gate_scale_wrong_row": ("sgate[e * I + i], xt, H);", "sgate[e * I], xt, H);"),
    "fp8_lm_scale_dropped": ("z[v] = dot_e4m3(qlm + (int64_t)v * H, slm[v], h + (int64_t)t * H, H);",
                             "z[v] = dot_e4m3(qlm + (int64_t)v * H, 1.0, h + (int64_t)t * H, H);"),
    "rms_mean_over_h_minus_1": ("double ms = ss / (double)H + eps;", "double ms = ss / (double)(H - 1) + eps;"),
    "rms_eps_dropped": ("double ms = ss / (double)H + eps;", "double ms = ss / (double)H;"),
    "rms_no_sqrt": ("double inv = 1.0 / sqrt(ms);", "double inv = 1.0 / ms;"),
    "rms_gain_dropped": ("oracle_bf16_value(row[i]) * oracle_bf16_value(gamma[i]) * inv;",
                         "oracle_bf16_value(row[i]) * inv;"),
    "rms_truncating_round": ("double r = ldexp(nearbyint(ldexp(v, -q)), q);",
                             "double r = ldexp(trunc(ldexp(v, -q)), q);"),
    "rms_ties_away": ("double r = ldexp(nearbyint(ldexp(v, -q)), q);",
                      "double r = ldexp(round(ldexp(v, -q)), q);"),
    "rms_wrong_binade": ("    int q = e - 8;", "    int q = e - 9;"),
    "verdict_same_position": ("if (tokens[i] != tok[i - 1])", "if (tokens[i] != tok[i])"),
    "verdict_no_stop": ("            break;\n        n = i;", "            continue;\n        n = i;"),
    "verdict_bonus_from_chain": ("accept[1] = tok[n];", "accept[1] = tokens[n];"),
    "verdict_no_bonus": ("accept[0] = n + 1;", "accept[0] = n;"),
    "gap_wrong_rank": ("*gap_sel = (k < n) ? s[k - 1] - s[k] : INFINITY;",
                       "*gap_sel = (k < n) ? s[0] - s[k] : INFINITY;"),
}


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, source, tmp_path):
    old, new = MUTATIONS[name]
    assert source.count(old) == 1, f"mutation anchor for {name} not unique"
    src = tmp_path / "oracle.c"
    src.write_text(source.replace(old, new))
    (tmp_path / "oracle.h").write_text(open(SRC[:-1] + "h").read())
    lib = str(tmp_path / "liboracle_mut.so")
    oracle.build(out=lib, src=str(src))
    o = oracle.Oracle(lib)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(o)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {name}"
