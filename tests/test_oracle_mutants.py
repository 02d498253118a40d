"""Plants plausible mistakes in copies of oracle.c (on the CPU) and checks that
the pins catch every one of them. This tests the pin set, not the library."""
import os

import pytest

import oracle
import pins

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("drop_logvar_term", "log(2.0 * M_PI) + log_var[c * d + j] + diff", "log(2.0 * M_PI) + diff"),
    ("variance_not_inverted", "diff * diff / s2", "diff * diff * s2"),
    ("prior_ignored", "double logp = logit_pi[c] - lse_pi;", "double logp = 0.0;"),
    ("eps_dropped", "out[i * dv + e] = num / (den + eps);", "out[i * dv + e] = num / den;"),
    ("causal_excludes_self",
     "const int write = causal || pass == 0;\n      const int read = causal || pass == 1;",
     "const int write = 0;\n      const int read = causal || pass == 1;\n      if (causal && i > 0) {"
     " gma_posterior(k + (i - 1) * d, d, K, mu, log_var, logit_pi, gk); for (int64_t c = 0; c < K; ++c) {"
     " for (int64_t e = 0; e < dv; ++e) vt[c * dv + e] += gk[c] * v[(i - 1) * dv + e]; zt[c] += gk[c]; } }"
     "\n      if (!causal && pass == 0) { gma_posterior(k + i * d, d, K, mu, log_var, logit_pi, gk);"
     " for (int64_t c = 0; c < K; ++c) { for (int64_t e = 0; e < dv; ++e) vt[c * dv + e] += gk[c] * v[i * dv + e];"
     " zt[c] += gk[c]; } }"),
    ("decay_after_add", "S[a * dv + e] = g[t] * S[a * dv + e] + kt[a] * vt[e];",
     "S[a * dv + e] = g[t] * (S[a * dv + e] + kt[a] * vt[e]);"),
    ("cov_unbiased", "const double cnt = (double)(t0 + t + 1);",
     "const double cnt = (double)(t0 + t > 0 ? t0 + t : 1);"),
    ("state_count_ignored", "const double cnt = (double)(t0 + t + 1);", "const double cnt = (double)(t + 1);"),
    ("state_key_sum_not_carried", "memcpy(m, st_in + dk * dv + dk * dk, sizeof(double) * (size_t)dk);", ""),
    ("state_decay_not_applied", "S[a * dv + e] = g[t] * S[a * dv + e] + kt[a] * vt[e];",
     "S[a * dv + e] = (t == 0 && st_in ? 1.0 : g[t]) * S[a * dv + e] + kt[a] * vt[e];"),
    ("gma_state_normaliser_not_carried", "memcpy(zt, mem_in + K * dv, sizeof(double) * (size_t)K);", ""),
    ("glv_decay_by_value_feature", "S[a * dv + e] = gs[t * dk + a] * S[a * dv + e]",
     "S[a * dv + e] = gs[t * dk + (e % dk)] * S[a * dv + e]"),
    ("glv_decay_of_previous_token", "S[a * dv + e] = gs[t * dk + a] * S[a * dv + e]",
     "S[a * dv + e] = (t > 0 ? gs[(t - 1) * dk + a] : 1.0) * S[a * dv + e]"),
    ("glv_state_not_carried", "if (st_in) memcpy(S, st_in + s * dk * dv, sizeof(double) * (size_t)(dk * dv));", ""),
    ("gma_state_out_missing_z", "memcpy(mem_out + K * dv, zt, sizeof(double) * (size_t)K);", ""),
    ("cov_mean_term_dropped", "(M[a * dk + c] / cnt - mu[a] * mu[c]) * qt[c]", "(M[a * dk + c] / cnt) * qt[c]"),
    ("lambda_sign", "qc[a] = qt[a] - lam * sq;", "qc[a] = qt[a] + lam * sq;"),
    ("gate_bias_sign", "double z = bias;\n      for (int64_t a = 0; a < dk; ++a) z += w[a] * qt[a];",
     "double z = -bias;\n      for (int64_t a = 0; a < dk; ++a) z += w[a] * qt[a];"),
    ("state_transposed_read", "acc += S[a * dv + e] * qc[a];", "acc += S[e * dv + a] * qc[a];"),
    ("chunk_intra_decay_off_by_one", "for (int64_t s = j + 1; s <= i; ++s) dec *= g[s];",
     "for (int64_t s = j; s <= i; ++s) dec *= g[s];"),
    ("chunk_inter_decay_missing", "out[i * dv + e] = decay_in * acc;", "out[i * dv + e] = acc;"),
    ("delta_error_sign", "r[e] = pred - vt[e];", "r[e] = vt[e] - pred;"),
    ("delta_no_decay", "for (int64_t e = 0; e < dv; ++e) S[a * dv + e] *= g[t];", ""),
    ("delta_error_from_undecayed_state", "pred += S[a * dv + e] * kt[a];", "pred += S[a * dv + e] / g[t] * kt[a];"),
    ("delta_transposed_prediction", "pred += S[a * dv + e] * kt[a];", "pred += S[e * dv + a % dv] * kt[a];"),
    ("delta_beta_on_value_only", "S[a * dv + e] -= beta[t] * kt[a] * r[e];",
     "S[a * dv + e] -= kt[a] * (r[e] + (1.0 - beta[t]) * vt[e]);"),
    ("delta_beta_squared", "S[a * dv + e] -= beta[t] * kt[a] * r[e];",
     "S[a * dv + e] -= beta[t] * beta[t] * kt[a] * r[e];"),
    ("delta_plain_write", "  if (beta) {\n      /* state: decay, then one gradient step",
     "  if (0) {\n      /* state: decay, then one gradient step"),
]


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, source, name, old, new):
    assert source.count(old) >= 1, "mutation anchor not found in oracle.c: %s" % name
    src = tmp_path / ("mut_%s.c" % name)
    src.write_text(source.replace(old, new, 1))
    lib = oracle.compile_library(str(src), str(tmp_path / ("mut_%s.so" % name)))
    orc = oracle.Oracle(lib)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "mutant %s passed every pin" % name
