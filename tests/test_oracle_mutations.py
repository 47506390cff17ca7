"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of oracle/eta_oracle.c (on the CPU),
builds it, and runs the pin suites (test_oracle_hand_example.py,
test_oracle_properties.py, test_oracle_gqa.py, test_oracle_prefill.py) against the mutant through
ETA_ORACLE_LIB.  Every
mutant must make at least one pin fail; the unmodified source must pass.
"""
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PINS = [os.path.join(HERE, "test_oracle_hand_example.py"),
        os.path.join(HERE, "test_oracle_properties.py"),
        os.path.join(HERE, "test_oracle_gqa.py"),
        os.path.join(HERE, "test_oracle_prefill.py")]

MUTANTS = {
    "prefill_diagonal_gated": ("double l = (s == t) ? S : S * m;", "double l = S * m;"),
    "prefill_density_over_t": ("dens[row] = msum / (double)(t + 1);",
                               "dens[row] = msum / (double)(t > 0 ? t : 1);"),
    "prefill_density_skips_diagonal": ("msum += m;", "if (s != t) msum += m;"),
    "prefill_wrong_kv_head": ("kv = (int)((uq % Hq) / G);", "kv = (int)((uq % Hq) % Hkv);"),
    "prefill_key_t_excluded": ("for (int s = 0; s <= t; ++s) {", "for (int s = 0; s < t; ++s) {", 2),
    "sample_variance": ("var[(size_t)j * d + i] = s / b;", "var[(size_t)j * d + i] = s / (b - 1);"),
    "mean_over_d": ("mu[(size_t)j * d + i] = s / b;", "mu[(size_t)j * d + i] = s / d;"),
    "maxnorm_squared": ("double n = sqrt(n2);", "double n = n2;"),
    "moment_uses_abs_q": ("mom += qi * qi * var[i];", "mom += fabs(qi) * var[i];"),
    "z_sign_flipped": ("double probabilistic = dot + z * sqrt(mom);",
                       "double probabilistic = dot - z * sqrt(mom);"),
    "z_ignored": ("double probabilistic = dot + z * sqrt(mom);",
                  "double probabilistic = dot + sqrt(mom);"),
    "ceiling_without_norm_sqrt": ("double geometric = sqrt(qq) * maxnorm;",
                                  "double geometric = qq * maxnorm;"),
    "score_unscaled": ("return scale * (probabilistic < geometric ? probabilistic : geometric);",
                       "return (probabilistic < geometric ? probabilistic : geometric);"),
    "max_instead_of_min": ("return scale * (probabilistic < geometric ? probabilistic : geometric);",
                           "return scale * (probabilistic > geometric ? probabilistic : geometric);"),
    "strict_admission": ("j < nbc && score[j] >= tau_screen", "j < nbc && score[j] > tau_screen"),
    "last_block_not_forced": ("int on = (j == nb - 1) ||", "int on = 0 ||"),
    "diagonal_key_gated": ("if (mode == ORC_GATED && s != T - 1)", "if (mode == ORC_GATED)"),
    "gate_sign_flipped": ("exp(-beta * (S - tau))", "exp(beta * (S - tau))"),
    "gate_on_weight_not_logit": ("l = S * (1.0 / (1.0 + exp(-beta * (S - tau))));",
                                 "l = S + log(1.0 / (1.0 + exp(-beta * (S - tau))));"),
    "mask_ignored": ("    if (!active[s / b]) continue;\n", "", 2),
    "predictor_bias_dropped": ("double t = (double)bias_or_c[h];\n      if (W) {",
                               "double t = W ? 0.0 : (double)bias_or_c[h];\n      if (W) {"),
    "predictor_W_transposed": ("(double)W[(size_t)j * H + h]", "(double)W[(size_t)h * H * d + j]"),
    "adjustment_sign": ("tau_screen[bb * H + h] = t - a;", "tau_screen[bb * H + h] = t + a;"),
    "calibration_off_by_one": ("c = 0.5 * (x[k - 1] + x[k]);", "c = 0.5 * (x[k] + x[k + 1 < (long long)n ? k + 1 : k]);"),
    "calibration_forced_ignored": ("double want = (rho * total - forced) / b;",
                                   "double want = (rho * total) / b;"),
    "index_round_half_up": ("return ldexp(nearbyint(ldexp(m, 8)), e - 8);",
                            "return ldexp(floor(ldexp(m, 8) + 0.5), e - 8);"),
    "index_seven_bits": ("return ldexp(nearbyint(ldexp(m, 8)), e - 8);",
                         "return ldexp(nearbyint(ldexp(m, 7)), e - 7);"),
    "gqa_wrong_kv_head": ("int bb = uq / Hq, kv = (uq % Hq) / G;",
                          "int bb = uq / Hq, kv = (uq % Hq) % Hkv;", 2),
    "gqa_union_counts_first_head": ("for (int g = 0; g < G; ++g) on |= active",
                                    "for (int g = 0; g < 1; ++g) on |= active"),
    "gqa_union_intersection": ("uint8_t on = 0;\n      for (int g = 0; g < G; ++g) on |= active",
                               "uint8_t on = 1;\n      for (int g = 0; g < G; ++g) on &= active"),
    "values_from_keys": ("out[i] += w * elem(V, dtype, (size_t)s * d + i);",
                         "out[i] += w * elem(K, dtype, (size_t)s * d + i);", 2),
    "attend_unscaled": ("    S *= scale;\n    double l = S;", "    double l = S;"),
    "dense_unscaled": ("S[s] = scale * x;", "S[s] = x;"),
    "attend_denominator_counts_keys": ("    double w = exp(logit[s] - top);\n    den += w;",
                                       "    double w = exp(logit[s] - top);\n    den += 1.0;"),
    "predictor_first_sequence_only": ("(double)q[(size_t)bb * H * d + j]", "(double)q[(size_t)j]"),
    "calibration_count_rounded_down": ("long long k = (long long)floor(want + 0.5);",
                                       "long long k = (long long)floor(want);"),
    "ceiling_norm_from_mean": ("qq += qi * qi;", "qq += qi * mu[i];"),
    "maxnorm_of_last_key": ("if (n > best) best = n;", "best = n;"),
    "variance_about_zero": ("double x = elem(K, dtype, (size_t)(j * b + r) * d + i) - m;",
                            "double x = elem(K, dtype, (size_t)(j * b + r) * d + i);"),
    "meta_partial_block_counted": ("int nbc = T / b;\n  for (int j = 0; j < nbc; ++j) {",
                                   "int nbc = (T + b - 1) / b;\n  for (int j = 0; j < nbc; ++j) {"),
    "prefill_values_from_keys": ("o[i] += w * elem(Vu, dtype, (size_t)s * d + i);",
                                 "o[i] += w * elem(Ku, dtype, (size_t)s * d + i);"),
    "prefill_unscaled": ("      S *= scale;\n      double m =", "      double m ="),
    "prefill_gate_on_raw_dot": ("double m = 1.0 / (1.0 + exp(-beta * (S - tt)));",
                                "double m = 1.0 / (1.0 + exp(-beta * (S / scale - tt)));"),
    "prefill_threshold_of_next_row": ("double tt = tau[row];",
                                      "double tt = tau[t + 1 < T ? row + 1 : row];"),
}


def _run_pins(lib_path):
    env = dict(os.environ, ETA_ORACLE_LIB=lib_path)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *PINS], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


def _build_variant(tmp_path, name, src):
    c = tmp_path / f"{name}.c"
    c.write_text(src)
    so = str(tmp_path / f"lib_{name}.so")
    oracle.build(out=so, src=str(c))
    return so


def test_unmodified_oracle_passes_pins(tmp_path):
    src = open(oracle._SRC).read()
    rc, out = _run_pins(_build_variant(tmp_path, "orig", src))
    assert rc == 0, out


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    old, new, *n = MUTANTS[name]
    src = open(oracle._SRC).read()
    assert src.count(old) == (n[0] if n else 1), f"mutation site for {name} not as expected"
    rc, out = _run_pins(_build_variant(tmp_path, name, src.replace(old, new)))
    assert rc != 0, f"mutant {name} passed every pin:\n{out}"
