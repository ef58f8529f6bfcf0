"""Planted mistakes in copies of oracle.c must each trip at least one pin.

Every mutant is a plausible slip (a dropped term, a wrong sign, an index off
by one, a transposed operand); it is built from a copy of the source on the
CPU, run through the pins of tests/test_oracle.py, and must fail one of them.
The real oracle is untouched.
"""
import os
import shutil

import pytest

import oracle
from tests.test_oracle import PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "score_drops_scale": ("s[j] = scale * acc;", "s[j] = acc;"),
    "score_transposed_channel": ("acc += qi[c] * kj[c];", "acc += qi[c] * kj[d - 1 - c];"),
    "causal_off_by_one": ("return (i + 1 < nk) ? i + 1 : nk;", "return (i < nk) ? (i > 0 ? i : 1) : nk;"),
    "value_index_shift": ("for (int c = 0; c < d; ++c) o[c] += w * vj[c];",
                          "for (int c = 0; c < d; ++c) o[c] += w * vj[c > 0 ? c - 1 : 0];"),
    "normaliser_drops_last_key": ("      l += w;\n", "      if (j + 1 < n) l += w;\n"),
    "kbar_wrong_count": ("kbar[c] /= (double)nk;", "kbar[c] /= (double)(nk + 1);"),
    "kbar_drops_last_key": ("for (int64_t j = 0; j < nk; ++j)\n    for (int c = 0; c < d; ++c) kbar[c]",
                            "for (int64_t j = 0; j < nk - 1; ++j)\n    for (int c = 0; c < d; ++c) kbar[c]"),
    "centering_sign": ("const double t = k[j * (int64_t)d + c] - kbar[c];",
                       "const double t = k[j * (int64_t)d + c] + kbar[c];"),
    "bound_drops_log2e": ("bound = max_keep_nan(bound, c2 * qn * kappa);",
                          "bound = max_keep_nan(bound, scale * qn * kappa);"),
    "vmax_drops_abs": ("vmax = max_keep_nan(vmax, fabs(v[j]));", "vmax = max_keep_nan(vmax, v[j]);"),
    "ceil_log2_is_floor_plus_one": ("return (f == 0.5) ? e - 1 : e;", "return e;"),
    "cap_drops_margin": ("ceil(u_acc - (double)A) - 1.0;", "ceil(u_acc - (double)A);"),
    "cap_ignores_headroom": ("const double c_acc = ceil(u_acc - (double)A) - 1.0;",
                             "const double c_acc = ceil(u_acc) - 1.0;"),
    "strict_compare": ("bound <= (double)C) ? 1 : 0;", "bound < (double)C - 0.5) ? 1 : 0;"),
    "mu_drops_log2e": ("mu[r] = c2 * dot;", "mu[r] = scale * dot;"),
    "mu_sign": ("mu[r] = c2 * dot;", "mu[r] = -c2 * dot;"),
    "online_forgets_rescale": ("      l *= alpha;\n", "      l *= 1.0;\n"),
    "online_rescale_wrong_way": ("const double alpha = exp2(m - mn);", "const double alpha = exp2(mn - m);"),
    "lazy_stabilizer_never_moves": ("const double mn = (mb > m + tau) ? mb : m;",
                                    "const double mn = (m == -INFINITY) ? mb : m;"),
    "lse_log2_not_ln": ("lse[t] = m + log(sum);", "lse[t] = m + log2(sum);"),
    "lse_drops_shift": ("for (int64_t j = 0; j < n; ++j) sum += exp(s[j] - m);",
                        "for (int64_t j = 0; j < n; ++j) sum += exp(s[j]);"),
    "partial_ignores_start": ("for (int64_t j = k0; j < end; ++j) {", "for (int64_t j = 0; j < end; ++j) {"),
    "partial_ignores_causal": ("const int64_t end = k1 < n ? k1 : n;", "const int64_t end = k1 < nk ? k1 : nk;"),
    "partial_mu_sign": ("const double p = exp2(c2 * dot - mu[i]);", "const double p = exp2(c2 * dot + mu[i]);"),
    "kappa_drops_sqrt": ("kappa = max_keep_nan(kappa, sqrt(ss));", "kappa = max_keep_nan(kappa, ss);"),
    "qnorm_drops_sqrt": ("const double qn = sqrt(ss);", "const double qn = ss;"),
    "qmax_first_row_only": ("double qmax = 0.0, bound = 0.0;\n  for (int64_t r = 0; r < nq; ++r) {",
                            "double qmax = 0.0, bound = 0.0;\n  for (int64_t r = 0; r < 1; ++r) {"),
    "keys_exponent_is_floor": ("const int32_t L = ceil_log2_exact((double)nk);",
                               "const int32_t L = (int32_t)floor(log2((double)nk));"),
    "G_without_floor_of_one": ("ceil_log2_exact(vmax > 1.0 ? vmax : 1.0)", "ceil_log2_exact(vmax)"),
    "fixed_mu_uses_row0_mu": ("const double x = c2 * s[j] - mu[i];", "const double x = c2 * s[j] - mu[0];"),
    "fixed_mu_drops_log2e": ("const double x = c2 * s[j] - mu[i];", "const double x = scale * s[j] - mu[i];"),
    "max_drops_nan_argument": ("if (isnan(acc) || isnan(x)) return NAN;", "if (isnan(acc)) return NAN;"),
}


def _any_pin_fails():
    for pin in PINS:
        try:
            pin()
        except Exception:  # an assertion, or a crash of the mutant's output checks
            return True
    return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    so = oracle.compile_source(str(path), str(tmp_path / "mutant.so"))
    with oracle.using_library(so):
        assert _any_pin_fails(), f"no pin caught the planted mistake {name}"


def test_unmutated_copy_passes(tmp_path):
    path = tmp_path / "copy.c"
    shutil.copy(SRC, path)
    so = oracle.compile_source(str(path), str(tmp_path / "copy.so"))
    with oracle.using_library(so):
        assert not _any_pin_fails()
