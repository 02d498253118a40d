/*
 * oracle.c -- plain, slow, fp64 CPU reference of the sequence-mixer forward pass.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark may build, load or call this file. The HIP
 * library never links or calls it, and the two share no code, header, table or
 * helper. Every function evaluates the plain definition with loops, in the order
 * the pages state it. There is no blocking, fusion or algebraic rewriting beyond
 * what the definition itself says.
 *
 * Sources (web pages, cited by title and section):
 *  [GMA] "Gaussian Mixture Attention: Linear-Time Sequence Mixing via
 *        Probabilistic Latent Routing" (gist.science explainer), technical
 *        summary, "Method: Gaussian Mixture Attention" -> "Core mechanism"
 *        (probabilistic latent routing; latent memory routing: write phase and
 *        read phase) and "Variants and training" (bidirectional / causal
 *        prefix sums; softplus / softmax reparameterisation).
 *  [CCQ] "Don't Read Everything: A Curvature-Conditioned Query for Linear
 *        Attention" (gist.science explainer), technical summary, section 2
 *        "Method": theoretical derivation (second-order expansion of the
 *        softmax log-partition, Hessian = running key covariance), mechanism
 *        (contracted query and its gate), integration (read-only change,
 *        output = state times cleaned query).
 *  [LIN] allinfo.ai.kr post on linear attention without a KV cache, sections
 *        "Key messages" and "Easy explanation": a matrix state that
 *        accumulates key-value outer products, decay gates in (0,1), and
 *        the chunkwise-parallel form (intra-chunk matrix products + state
 *        handed over at chunk boundaries), which gives the same result as
 *        the recurrence. The same sections read the state update as one
 *        step of gradient descent on a squared-error regression from keys
 *        to values, and name the delta rule (erase the value bound to the
 *        current key, write the new one) as the companion of the decay gate.
 *
 * Layouts: q, k [B,H,N,d]; v, out [B,H,N,dv]; per-head parameters [H,...];
 * decays g [B,H,N]. All arrays are row-major float64. Nothing is allocated
 * on behalf of the caller except per-thread scratch, which is freed before
 * return.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef M_PI
#define M_PI 3.14159265358979323846
#endif

/* ------------------------------------------------------------------------ */
/* GMA: responsibilities                                                     */
/* ------------------------------------------------------------------------ */

/*
 * Posterior responsibility of every component for one routing vector x [d]:
 * gamma_k = p(z=k | x) for a mixture with means mu_k, diagonal covariances
 * sigma^2_k = exp(log_var_k) and priors pi = softmax(logit_pi)  [GMA, core
 * mechanism; priors by softmax, variances kept positive by construction, per
 * "Variants and training"]. The log-density is the textbook diagonal-Gaussian
 * one, written term by term:
 *   log N(x; mu, diag s2) = -1/2 sum_j [ log(2 pi) + log s2_j + (x_j-mu_j)^2 / s2_j ].
 * The posterior normalises prior times likelihood over k (log-sum-exp with
 * the maximum taken out for range only).
 */
static void gma_posterior(const double* x, int64_t d, int64_t K, const double* mu,
                          const double* log_var, const double* logit_pi, double* gamma) {
  /* log pi = logit_pi - log sum exp(logit_pi) */
  double lmax = -INFINITY;
  for (int64_t c = 0; c < K; ++c) lmax = fmax(lmax, logit_pi[c]);
  double lsum = 0.0;
  for (int64_t c = 0; c < K; ++c) lsum += exp(logit_pi[c] - lmax);
  const double lse_pi = lmax + log(lsum);

  double best = -INFINITY;
  for (int64_t c = 0; c < K; ++c) {
    double logp = logit_pi[c] - lse_pi;
    for (int64_t j = 0; j < d; ++j) {
      const double s2 = exp(log_var[c * d + j]);
      const double diff = x[j] - mu[c * d + j];
      logp += -0.5 * (log(2.0 * M_PI) + log_var[c * d + j] + diff * diff / s2);
    }
    gamma[c] = logp;
    best = fmax(best, logp);
  }
  double z = 0.0;
  for (int64_t c = 0; c < K; ++c) {
    gamma[c] = exp(gamma[c] - best);
    z += gamma[c];
  }
  for (int64_t c = 0; c < K; ++c) gamma[c] /= z;
}

/* Responsibilities for N vectors of one head: x [N,d] -> gamma [N,K]. */
void oracle_gma_responsibilities(const double* x, int64_t N, int64_t d, int64_t K,
                                 const double* mu, const double* log_var,
                                 const double* logit_pi, double* gamma) {
  for (int64_t i = 0; i < N; ++i)
    gma_posterior(x + i * d, d, K, mu, log_var, logit_pi, gamma + i * K);
}

/* ------------------------------------------------------------------------ */
/* GMA: associative (linear-time) forward                                    */
/* ------------------------------------------------------------------------ */

/*
 * One (b,h) slice of GMA [GMA, latent memory routing + variants]:
 *   write:  Vtil = Gamma_K^T V  (K x dv),   Z = Gamma_K^T 1  (K)
 *   read:   O = (Gamma_Q Vtil) / (Gamma_Q Z + eps), row by row.
 * Causal: Vtil and Z are prefix sums, so row i reads the memory built from
 * keys j <= i (the current token included). Bidirectional: the whole
 * sequence is written first, then every row is read.
 * row_mask (optional, length N): when non-NULL only rows with a nonzero flag
 * are read and written to out; the memory is still built from every key.
 */
static void gma_slice(const double* q, const double* k, const double* v, const double* mu,
                      const double* log_var, const double* logit_pi, double* out, int64_t N,
                      int64_t d, int64_t K, int64_t dv, int causal, double eps,
                      const uint8_t* row_mask, const double* mem_in, double* mem_out) {
  double* vt = (double*)calloc((size_t)(K * dv), sizeof(double));
  double* zt = (double*)calloc((size_t)K, sizeof(double));
  /* causal: the memory may start from an earlier prefix (Vtil, Z) */
  if (mem_in) {
    memcpy(vt, mem_in, sizeof(double) * (size_t)(K * dv));
    memcpy(zt, mem_in + K * dv, sizeof(double) * (size_t)K);
  }
  double* gk = (double*)malloc(sizeof(double) * (size_t)K);
  double* gq = (double*)malloc(sizeof(double) * (size_t)K);

  for (int64_t pass = causal ? 1 : 0; pass < 2; ++pass) {
    for (int64_t i = 0; i < N; ++i) {
      const int write = causal || pass == 0;
      const int read = causal || pass == 1;
      if (write) {
        gma_posterior(k + i * d, d, K, mu, log_var, logit_pi, gk);
        for (int64_t c = 0; c < K; ++c) {
          for (int64_t e = 0; e < dv; ++e) vt[c * dv + e] += gk[c] * v[i * dv + e];
          zt[c] += gk[c];
        }
      }
      if (read && (row_mask == NULL || row_mask[i])) {
        gma_posterior(q + i * d, d, K, mu, log_var, logit_pi, gq);
        double den = 0.0;
        for (int64_t c = 0; c < K; ++c) den += gq[c] * zt[c];
        for (int64_t e = 0; e < dv; ++e) {
          double num = 0.0;
          for (int64_t c = 0; c < K; ++c) num += gq[c] * vt[c * dv + e];
          out[i * dv + e] = num / (den + eps);
        }
      }
    }
  }
  if (mem_out) {
    memcpy(mem_out, vt, sizeof(double) * (size_t)(K * dv));
    memcpy(mem_out + K * dv, zt, sizeof(double) * (size_t)K);
  }
  free(vt);
  free(zt);
  free(gk);
  free(gq);
}

/*
 * mem_in, mem_out (optional, causal only): per (b,h) memory [Vtil (K x dv) | Z (K)]
 * before the first token and after the last [GMA, variants: the causal form
 * is a running prefix sum, so a sequence can be continued from its memory].
 */
void oracle_gma_forward(const double* q, const double* k, const double* v, const double* mu,
                        const double* log_var, const double* logit_pi, double* out, int64_t B,
                        int64_t H, int64_t N, int64_t d, int64_t K, int64_t dv, int causal,
                        double eps, const uint8_t* row_mask, const double* mem_in,
                        double* mem_out) {
  int64_t BH = B * H;
  const int64_t ms = K * dv + K;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t s = 0; s < BH; ++s) {
    const int64_t h = s % H;
    gma_slice(q + s * N * d, k + s * N * d, v + s * N * dv, mu + h * K * d, log_var + h * K * d,
              logit_pi + h * K, out + s * N * dv, N, d, K, dv, causal, eps,
              row_mask ? row_mask + s * N : NULL, mem_in ? mem_in + s * ms : NULL,
              mem_out ? mem_out + s * ms : NULL);
  }
}

/*
 * Brute-force GMA: materialise the implicit affinity A = Gamma_Q Gamma_K^T
 * (N x N, non-negative, rank <= K) [GMA, core mechanism and key contributions],
 * keep j <= i when causal, and form O = (A V) / (A 1 + eps). The same numbers
 * as oracle_gma_forward by associativity; used on small N only.
 * affinity (optional): receives A [N,N] of the last slice processed.
 */
void oracle_gma_brute(const double* q, const double* k, const double* v, const double* mu,
                      const double* log_var, const double* logit_pi, double* out, int64_t B,
                      int64_t H, int64_t N, int64_t d, int64_t K, int64_t dv, int causal,
                      double eps, double* affinity) {
  double* gq = (double*)malloc(sizeof(double) * (size_t)(N * K));
  double* gk = (double*)malloc(sizeof(double) * (size_t)(N * K));
  double* a = (double*)malloc(sizeof(double) * (size_t)(N * N));
  for (int64_t s = 0; s < B * H; ++s) {
    const int64_t h = s % H;
    oracle_gma_responsibilities(q + s * N * d, N, d, K, mu + h * K * d, log_var + h * K * d,
                                logit_pi + h * K, gq);
    oracle_gma_responsibilities(k + s * N * d, N, d, K, mu + h * K * d, log_var + h * K * d,
                                logit_pi + h * K, gk);
    for (int64_t i = 0; i < N; ++i)
      for (int64_t j = 0; j < N; ++j) {
        double acc = 0.0;
        if (!causal || j <= i)
          for (int64_t c = 0; c < K; ++c) acc += gq[i * K + c] * gk[j * K + c];
        a[i * N + j] = acc;
      }
    for (int64_t i = 0; i < N; ++i) {
      double den = 0.0;
      for (int64_t j = 0; j < N; ++j) den += a[i * N + j];
      for (int64_t e = 0; e < dv; ++e) {
        double num = 0.0;
        for (int64_t j = 0; j < N; ++j) num += a[i * N + j] * v[s * N * dv + j * dv + e];
        out[s * N * dv + i * dv + e] = num / (den + eps);
      }
    }
    if (affinity) memcpy(affinity, a, sizeof(double) * (size_t)(N * N));
  }
  free(gq);
  free(gk);
  free(a);
}

/* ------------------------------------------------------------------------ */
/* Gated linear attention and CCQ: recurrent definitions                     */
/* ------------------------------------------------------------------------ */

/*
 * One slice of decayed linear attention / CCQ, token by token.
 *   state write [LIN, decay gates; CCQ integration, write rule unchanged]:
 *       S_t = g_t S_{t-1} + k_t v_t^T          (S is dk x dv, S_0 = 0)
 *   running key statistics [CCQ, derivation + mechanism]:
 *       mu_t = (1/t) sum_{j<=t} k_j,
 *       Sigma_t = (1/t) sum_{j<=t} k_j k_j^T - mu_t mu_t^T
 *     (the Hessian at q = 0 of log sum_{j<=t} exp(k_j^T q), i.e. the key
 *      covariance under uniform weights 1/t; no decay enters it)
 *   gate and contraction [CCQ, mechanism]:
 *       lambda_t = sigmoid(w . q_t + b),  q_clean = q_t - lambda_t Sigma_t q_t
 *   read [CCQ, integration]: o_t = S_t^T q_clean  (plain linear attention
 *   reads with q_t itself).
 *   gated delta write (beta != NULL) [LIN, key messages + easy explanation:
 *   the update is one gradient step on the squared error of predicting v_t
 *   from k_t, and the delta rule overwrites the value bound to k_t; the
 *   decay gate forgets first]:
 *       S' = g_t S_{t-1},  r_t = S'^T k_t - v_t  (prediction error),
 *       S_t = S' - beta_t k_t r_t^T
 *   i.e. S' minus beta_t times the gradient of 1/2 ||S^T k_t - v_t||^2 at S'.
 *   The CCQ read is unchanged on this write rule [CCQ, integration: the read
 *   does not depend on the write rule].
 */
static void linattn_slice(const double* q, const double* k, const double* v, const double* g,
                          const double* beta, const double* w, double bias, double* out, int64_t N,
                          int64_t dk, int64_t dv, int ccq, int64_t t0, const double* st_in,
                          double* st_out) {
  double* S = (double*)calloc((size_t)(dk * dv), sizeof(double));
  double* M = ccq ? (double*)calloc((size_t)(dk * dk), sizeof(double)) : NULL;
  double* m = ccq ? (double*)calloc((size_t)dk, sizeof(double)) : NULL;
  /* state [S (dk x dv) | M (dk x dk) | m (dk)] after t0 earlier tokens */
  if (st_in) {
    memcpy(S, st_in, sizeof(double) * (size_t)(dk * dv));
    if (ccq) {
      memcpy(M, st_in + dk * dv, sizeof(double) * (size_t)(dk * dk));
      memcpy(m, st_in + dk * dv + dk * dk, sizeof(double) * (size_t)dk);
    }
  }
  double* mu = ccq ? (double*)malloc(sizeof(double) * (size_t)dk) : NULL;
  double* qc = (double*)malloc(sizeof(double) * (size_t)dk);
  double* r = beta ? (double*)malloc(sizeof(double) * (size_t)dv) : NULL;

  for (int64_t t = 0; t < N; ++t) {
    const double* qt = q + t * dk;
    const double* kt = k + t * dk;
    const double* vt = v + t * dv;
    if (beta) {
      /* state: decay, then one gradient step of size beta_t on the error */
      for (int64_t a = 0; a < dk; ++a)
        for (int64_t e = 0; e < dv; ++e) S[a * dv + e] *= g[t];
      for (int64_t e = 0; e < dv; ++e) {
        double pred = 0.0;
        for (int64_t a = 0; a < dk; ++a) pred += S[a * dv + e] * kt[a];
        r[e] = pred - vt[e];
      }
      for (int64_t a = 0; a < dk; ++a)
        for (int64_t e = 0; e < dv; ++e) S[a * dv + e] -= beta[t] * kt[a] * r[e];
    } else {
      /* state: decay, then add the current outer product */
      for (int64_t a = 0; a < dk; ++a)
        for (int64_t e = 0; e < dv; ++e) S[a * dv + e] = g[t] * S[a * dv + e] + kt[a] * vt[e];
    }

    for (int64_t a = 0; a < dk; ++a) qc[a] = qt[a];
    if (ccq) {
      const double cnt = (double)(t0 + t + 1);
      for (int64_t a = 0; a < dk; ++a) {
        m[a] += kt[a];
        for (int64_t c = 0; c < dk; ++c) M[a * dk + c] += kt[a] * kt[c];
      }
      for (int64_t a = 0; a < dk; ++a) mu[a] = m[a] / cnt;
      double z = bias;
      for (int64_t a = 0; a < dk; ++a) z += w[a] * qt[a];
      const double lam = 1.0 / (1.0 + exp(-z));
      for (int64_t a = 0; a < dk; ++a) {
        double sq = 0.0; /* (Sigma_t q_t)_a */
        for (int64_t c = 0; c < dk; ++c) sq += (M[a * dk + c] / cnt - mu[a] * mu[c]) * qt[c];
        qc[a] = qt[a] - lam * sq;
      }
    }
    for (int64_t e = 0; e < dv; ++e) {
      double acc = 0.0;
      for (int64_t a = 0; a < dk; ++a) acc += S[a * dv + e] * qc[a];
      out[t * dv + e] = acc;
    }
  }
  if (st_out) {
    memcpy(st_out, S, sizeof(double) * (size_t)(dk * dv));
    if (ccq) {
      memcpy(st_out + dk * dv, M, sizeof(double) * (size_t)(dk * dk));
      memcpy(st_out + dk * dv + dk * dk, m, sizeof(double) * (size_t)dk);
    }
  }
  free(S);
  free(M);
  free(m);
  free(mu);
  free(qc);
  free(r);
}

/*
 * st_in, st_out (optional): per (b,h) state [S (dk x dv)] before the first token
 * and after the last [LIN, recurrent form: the state is all a later token
 * needs, so a sequence can be continued, one token at a time, from it].
 */
void oracle_gla_forward(const double* q, const double* k, const double* v, const double* g,
                        double* out, int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv,
                        const double* st_in, double* st_out) {
  int64_t BH = B * H;
  const int64_t ss = dk * dv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t s = 0; s < BH; ++s)
    linattn_slice(q + s * N * dk, k + s * N * dk, v + s * N * dv, g + s * N, NULL, NULL, 0.0,
                  out + s * N * dv, N, dk, dv, 0, 0, st_in ? st_in + s * ss : NULL,
                  st_out ? st_out + s * ss : NULL);
}

/*
 * t0, st_in, st_out: the running key statistics belong to the state too
 * [CCQ, integration: they are kept by the same recurrent machinery], so the
 * per (b,h) state is [S (dk x dv) | M = sum k k^T (dk x dk) | m = sum k (dk)],
 * and t0 is the number of tokens it already holds (0 without st_in).
 */
void oracle_ccq_forward(const double* q, const double* k, const double* v, const double* g,
                        const double* w, const double* b, double* out, int64_t B, int64_t H,
                        int64_t N, int64_t dk, int64_t dv, int64_t t0, const double* st_in,
                        double* st_out) {
  int64_t BH = B * H;
  const int64_t ss = dk * dv + dk * dk + dk;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t s = 0; s < BH; ++s) {
    const int64_t h = s % H;
    linattn_slice(q + s * N * dk, k + s * N * dk, v + s * N * dv, g + s * N, NULL, w + h * dk,
                  b[h], out + s * N * dv, N, dk, dv, 1, t0, st_in ? st_in + s * ss : NULL,
                  st_out ? st_out + s * ss : NULL);
  }
}

/*
 * Gated delta write rule with the plain read [LIN, key messages + easy
 * explanation]: beta [B,H,N] is the step size of each token's gradient step.
 * st_in / st_out as for oracle_gla_forward (S, dk x dv).
 */
void oracle_deltanet_forward(const double* q, const double* k, const double* v, const double* g,
                             const double* beta, double* out, int64_t B, int64_t H, int64_t N,
                             int64_t dk, int64_t dv, const double* st_in, double* st_out) {
  int64_t BH = B * H;
  const int64_t ss = dk * dv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t s = 0; s < BH; ++s)
    linattn_slice(q + s * N * dk, k + s * N * dk, v + s * N * dv, g + s * N, beta + s * N, NULL,
                  0.0, out + s * N * dv, N, dk, dv, 0, 0, st_in ? st_in + s * ss : NULL,
                  st_out ? st_out + s * ss : NULL);
}

/*
 * The CCQ read over the gated delta write rule [CCQ, integration: the read
 * attaches to any write rule; Gated DeltaNet is the second backbone the page
 * names]. State [S | M | m] and t0 as for oracle_ccq_forward.
 */
void oracle_ccq_deltanet_forward(const double* q, const double* k, const double* v,
                                 const double* g, const double* beta, const double* w,
                                 const double* b, double* out, int64_t B, int64_t H, int64_t N,
                                 int64_t dk, int64_t dv, int64_t t0, const double* st_in,
                                 double* st_out) {
  int64_t BH = B * H;
  const int64_t ss = dk * dv + dk * dk + dk;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t s = 0; s < BH; ++s) {
    const int64_t h = s % H;
    linattn_slice(q + s * N * dk, k + s * N * dk, v + s * N * dv, g + s * N, beta + s * N,
                  w + h * dk, b[h], out + s * N * dv, N, dk, dv, 1, t0,
                  st_in ? st_in + s * ss : NULL, st_out ? st_out + s * ss : NULL);
  }
}

/*
 * Decayed linear attention with a decay gate per key feature [LIN, decay gates:
 * the forget rate may be set per channel]:
 *     S_t[a][e] = g_t[a] S_{t-1}[a][e] + k_t[a] v_t[e],   o_t = S_t^T q_t
 * g [B,H,N,dk]. With g_t[a] the same for every a this is oracle_gla_forward.
 */
void oracle_glv_forward(const double* q, const double* k, const double* v, const double* g,
                        double* out, int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv,
                        const double* st_in, double* st_out) {
  int64_t BH = B * H;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t s = 0; s < BH; ++s) {
    const double* qs = q + s * N * dk;
    const double* ks = k + s * N * dk;
    const double* vs = v + s * N * dv;
    const double* gs = g + s * N * dk;
    double* os = out + s * N * dv;
    double* S = (double*)calloc((size_t)(dk * dv), sizeof(double));
    /* optional state S (dk x dv) before the first token */
    if (st_in) memcpy(S, st_in + s * dk * dv, sizeof(double) * (size_t)(dk * dv));
    for (int64_t t = 0; t < N; ++t) {
      for (int64_t a = 0; a < dk; ++a)
        for (int64_t e = 0; e < dv; ++e)
          S[a * dv + e] = gs[t * dk + a] * S[a * dv + e] + ks[t * dk + a] * vs[t * dv + e];
      for (int64_t e = 0; e < dv; ++e) {
        double acc = 0.0;
        for (int64_t a = 0; a < dk; ++a) acc += S[a * dv + e] * qs[t * dk + a];
        os[t * dv + e] = acc;
      }
    }
    if (st_out) memcpy(st_out + s * dk * dv, S, sizeof(double) * (size_t)(dk * dv));
    free(S);
  }
}

/* ------------------------------------------------------------------------ */
/* Chunkwise-parallel forms                                                  */
/* ------------------------------------------------------------------------ */

/*
 * The chunkwise form of the same recurrences [LIN, key messages and easy
 * explanation]: cut the sequence into chunks of C tokens; inside a chunk,
 * the contributions of the chunk's own keys are formed directly (pairwise
 * products with the decay accumulated between the two positions); the
 * state from earlier chunks is read once per row and handed to the next
 * chunk only at the boundary. Decay products are kept as plain products
 * of the g values (no log-space). For CCQ the running key sums are carried
 * across chunk boundaries the same way and completed inside the chunk with
 * the chunk's own keys up to the current row [CCQ, mechanism: the
 * covariance is kept by the same recurrent or chunkwise machinery].
 * This function exists so that tests can check that the chunkwise and
 * token-by-token forms give the same numbers.
 */
static void chunk_slice(const double* q, const double* k, const double* v, const double* g,
                        const double* w, double bias, double* out, int64_t N, int64_t dk,
                        int64_t dv, int64_t C, int ccq) {
  double* S = (double*)calloc((size_t)(dk * dv), sizeof(double)); /* state at chunk start */
  double* M = ccq ? (double*)calloc((size_t)(dk * dk), sizeof(double)) : NULL;
  double* m = ccq ? (double*)calloc((size_t)dk, sizeof(double)) : NULL;
  double* Mi = ccq ? (double*)malloc(sizeof(double) * (size_t)(dk * dk)) : NULL;
  double* mi = ccq ? (double*)malloc(sizeof(double) * (size_t)dk) : NULL;
  double* qc = (double*)malloc(sizeof(double) * (size_t)dk);
  double* Snew = (double*)malloc(sizeof(double) * (size_t)(dk * dv));

  for (int64_t c0 = 0; c0 < N; c0 += C) {
    const int64_t c1 = c0 + C < N ? c0 + C : N;
    for (int64_t i = c0; i < c1; ++i) {
      const double* qi = q + i * dk;
      for (int64_t a = 0; a < dk; ++a) qc[a] = qi[a];
      if (ccq) {
        /* running statistics at row i: carried sums + this chunk's keys j <= i */
        memcpy(Mi, M, sizeof(double) * (size_t)(dk * dk));
        memcpy(mi, m, sizeof(double) * (size_t)dk);
        for (int64_t j = c0; j <= i; ++j)
          for (int64_t a = 0; a < dk; ++a) {
            mi[a] += k[j * dk + a];
            for (int64_t c = 0; c < dk; ++c) Mi[a * dk + c] += k[j * dk + a] * k[j * dk + c];
          }
        const double cnt = (double)(i + 1);
        double z = bias;
        for (int64_t a = 0; a < dk; ++a) z += w[a] * qi[a];
        const double lam = 1.0 / (1.0 + exp(-z));
        for (int64_t a = 0; a < dk; ++a) {
          double sq = 0.0;
          for (int64_t c = 0; c < dk; ++c)
            sq += (Mi[a * dk + c] / cnt - (mi[a] / cnt) * (mi[c] / cnt)) * qi[c];
          qc[a] = qi[a] - lam * sq;
        }
      }
      /* inter-chunk part: decay from the chunk start through row i */
      double decay_in = 1.0;
      for (int64_t s = c0; s <= i; ++s) decay_in *= g[s];
      for (int64_t e = 0; e < dv; ++e) {
        double acc = 0.0;
        for (int64_t a = 0; a < dk; ++a) acc += S[a * dv + e] * qc[a];
        out[i * dv + e] = decay_in * acc;
      }
      /* intra-chunk part: keys j <= i of this chunk, decayed by g_{j+1..i} */
      for (int64_t j = c0; j <= i; ++j) {
        double dec = 1.0;
        for (int64_t s = j + 1; s <= i; ++s) dec *= g[s];
        double score = 0.0;
        for (int64_t a = 0; a < dk; ++a) score += qc[a] * k[j * dk + a];
        for (int64_t e = 0; e < dv; ++e) out[i * dv + e] += dec * score * v[j * dv + e];
      }
    }
    /* hand the state over the boundary */
    double decay_all = 1.0;
    for (int64_t s = c0; s < c1; ++s) decay_all *= g[s];
    for (int64_t a = 0; a < dk; ++a)
      for (int64_t e = 0; e < dv; ++e) Snew[a * dv + e] = decay_all * S[a * dv + e];
    for (int64_t j = c0; j < c1; ++j) {
      double dec = 1.0;
      for (int64_t s = j + 1; s < c1; ++s) dec *= g[s];
      for (int64_t a = 0; a < dk; ++a)
        for (int64_t e = 0; e < dv; ++e) Snew[a * dv + e] += dec * k[j * dk + a] * v[j * dv + e];
    }
    memcpy(S, Snew, sizeof(double) * (size_t)(dk * dv));
    if (ccq)
      for (int64_t j = c0; j < c1; ++j)
        for (int64_t a = 0; a < dk; ++a) {
          m[a] += k[j * dk + a];
          for (int64_t c = 0; c < dk; ++c) M[a * dk + c] += k[j * dk + a] * k[j * dk + c];
        }
  }
  free(S);
  free(M);
  free(m);
  free(Mi);
  free(mi);
  free(qc);
  free(Snew);
}

void oracle_gla_chunkwise(const double* q, const double* k, const double* v, const double* g,
                          double* out, int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv,
                          int64_t C) {
  for (int64_t s = 0; s < B * H; ++s)
    chunk_slice(q + s * N * dk, k + s * N * dk, v + s * N * dv, g + s * N, NULL, 0.0,
                out + s * N * dv, N, dk, dv, C, 0);
}

void oracle_ccq_chunkwise(const double* q, const double* k, const double* v, const double* g,
                          const double* w, const double* b, double* out, int64_t B, int64_t H,
                          int64_t N, int64_t dk, int64_t dv, int64_t C) {
  for (int64_t s = 0; s < B * H; ++s) {
    const int64_t h = s % H;
    chunk_slice(q + s * N * dk, k + s * N * dk, v + s * N * dv, g + s * N, w + h * dk, b[h],
                out + s * N * dv, N, dk, dv, C, 1);
  }
}

/* Number of OpenMP threads a parallel region would use (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
