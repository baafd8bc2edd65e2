/*
 * drgrpo_oracle.c - plain, slow, binary64 CPU reference of the Dr. GRPO update
 * loss and its gradient with respect to the policy logits.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no code,
 * header or constant with the GPU library: every step is written out here
 * from the pages' definitions, one loop per step, in the pages' order.
 *
 * Sources (page title, section):
 *   [DG]  "Making Dr GRPO go brrr": sections "PPO", "GRPO", "Dr. GRPO",
 *         "The completion mask", "compute_logprobs", "The loss",
 *         "Putting it together".
 *   [QL]  "The Quiet Library" / "GRPO efficiency starts before the kernel":
 *         "The sparse-reward bottleneck".
 *
 * Readings taken where the pages leave a step open (each is listed in the
 * design notes):
 *   - the logits handed in are already the completion slice, so row t scores
 *     token t of the completion ([DG] "compute_logprobs": the slice that
 *     starts one position before the completion);
 *   - the token sum is divided by a caller-supplied constant kappa ([DG]
 *     "Dr. GRPO": a sum, optionally divided by a fixed constant); the GRPO
 *     normalisations the same section removes (group standard deviation,
 *     per-response mean) and the token mean are kept as variants;
 *   - the KL term is the k3 estimator exp(d) - d - 1, d = logp_ref - logp,
 *     summed into the same masked token sum (the pages name the penalty but
 *     not its estimator);
 *   - a token whose loss term is identically zero (masked out, or zero
 *     advantage with beta = 0) contributes exactly 0 to the loss and to the
 *     gradient whatever its logits hold;
 *   - the advantage is formed in binary32 as a sequential group sum, one
 *     division by G and one subtraction.
 *
 * Element types of the logits: 0 = binary32, 1 = bfloat16 (upper half of a
 * binary32), 2 = binary64.  Every element is widened exactly to binary64.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

enum { OR_F32 = 0, OR_BF16 = 1, OR_F64 = 2 };

static double or_elem(const void* base, int dtype, int64_t i) {
  if (dtype == OR_F32) return (double)((const float*)base)[i];
  if (dtype == OR_F64) return ((const double*)base)[i];
  /* bfloat16: the 16 stored bits are the high half of a binary32 */
  uint32_t u = (uint32_t)((const uint16_t*)base)[i] << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* [DG] "The completion mask": the mask is 1 for real tokens up to and
 * including the first EOS and 0 after it; a row with no EOS at all counts
 * every token.  Returned as a length: len = (index of first EOS) + 1, or C. */
int oracle_completion_len(const int64_t* tokens, int64_t N, int64_t C, int64_t eos_id,
                          int32_t* len) {
  if (!tokens || !len || N < 0 || C < 0) return -1;
  for (int64_t i = 0; i < N; ++i) {
    int64_t L = C;
    for (int64_t t = 0; t < C; ++t) {
      if (tokens[i * C + t] == eos_id) {
        L = t + 1;
        break;
      }
    }
    len[i] = (int32_t)L;
  }
  return 0;
}

/* [DG] "Dr. GRPO" and "Putting it together": the advantage of completion i is
 * its reward minus the mean reward of its group, with no division by the
 * group's standard deviation.  Groups are G consecutive rows.  Arithmetic is
 * binary32: sequential sum in row order, divide by G, subtract. */
int oracle_group_advantage(const float* rewards, int64_t N, int64_t G, float* adv) {
  if (!rewards || !adv || G <= 0 || N < 0 || N % G != 0) return -1;
  for (int64_t b = 0; b < N / G; ++b) {
    volatile float s = 0.0f;
    for (int64_t j = 0; j < G; ++j) s = s + rewards[b * G + j];
    volatile float mu = s / (float)G;
    for (int64_t j = 0; j < G; ++j) adv[b * G + j] = rewards[b * G + j] - mu;
  }
  return 0;
}

/* [DG] "GRPO": the advantage is the reward minus the group mean, divided by
 * the group's standard deviation.  Readings: the standard deviation is the
 * sample one (divisor G - 1, what torch's Tensor.std computes), and a group
 * whose rewards are all equal has advantage 0 (it carries no contrast and the
 * quotient would be 0/0).  Binary32 throughout: the mean as in
 * oracle_group_advantage, then the sequential sum of squared deviations
 * (each square rounded, then added), one division by G - 1, a correctly
 * rounded square root, and one division per completion. */
int oracle_group_advantage_zscore(const float* rewards, int64_t N, int64_t G, float* adv) {
  if (!rewards || !adv || G <= 0 || N < 0 || N % G != 0) return -1;
  for (int64_t b = 0; b < N / G; ++b) {
    int same = 1;
    for (int64_t j = 1; j < G; ++j)
      if (!(rewards[b * G + j] == rewards[b * G])) same = 0;
    if (same) {
      for (int64_t j = 0; j < G; ++j) adv[b * G + j] = 0.0f;
      continue;
    }
    volatile float s = 0.0f;
    for (int64_t j = 0; j < G; ++j) s = s + rewards[b * G + j];
    volatile float mu = s / (float)G;
    volatile float q = 0.0f;
    for (int64_t j = 0; j < G; ++j) {
      volatile float d = rewards[b * G + j] - mu;
      volatile float d2 = d * d;
      q = q + d2;
    }
    volatile float var = q / (float)(G - 1);
    volatile float sd = sqrtf(var);
    for (int64_t j = 0; j < G; ++j) {
      volatile float d = rewards[b * G + j] - mu;
      adv[b * G + j] = d / sd;
    }
  }
  return 0;
}

/* Aggregation: the loss is L = sum_i (sum_t lambda[i,t]) / div_i, with one
 * divisor per completion:
 *   agg 0, [DG] "Dr. GRPO": the token sum over the batch divided by a fixed
 *          constant, div_i = kappa;
 *   agg 1, [DG] "Dr. GRPO" (length bias): the original GRPO loss averages each
 *          response's token sum over its |o_i| tokens, div_i = kappa * len_i
 *          (kappa = N gives the mean over completions);
 *   agg 2, [DG] "Dr. GRPO" pseudo-code ("not token_mean"): the mean over
 *          every counted token of the batch, div_i = kappa * sum_j len_j. */
int oracle_row_divisor(const int32_t* len, int64_t N, int agg, double kappa, double* div) {
  if (!len || !div || N < 0 || agg < 0 || agg > 2) return -1;
  double total = 0.0;
  for (int64_t i = 0; i < N; ++i) total += (double)len[i];
  for (int64_t i = 0; i < N; ++i) {
    if (agg == 0) div[i] = kappa;
    else if (agg == 1) div[i] = kappa * (double)len[i];
    else div[i] = kappa * total;
  }
  return 0;
}

/* [QL] "The sparse-reward bottleneck": a group has no reward contrast when
 * every reward in it is equal.  Returns the number of such groups. */
int64_t oracle_nocontrast_groups(const float* rewards, int64_t N, int64_t G) {
  if (!rewards || G <= 0 || N % G != 0) return -1;
  int64_t n = 0;
  for (int64_t b = 0; b < N / G; ++b) {
    int same = 1;
    for (int64_t j = 1; j < G; ++j)
      if (!(rewards[b * G + j] == rewards[b * G])) same = 0;
    n += same;
  }
  return n;
}

/* [DG] "compute_logprobs": log_softmax over the vocabulary followed by a
 * gather at the sampled token.  For each of `rows` rows of V logits:
 *   M = max_v x_v,  S = sum_v exp(x_v - M),  lse = M + ln S,
 *   logp = x_y - lse with y = tokens[r].
 * A NaN logit makes lse and logp NaN.  A token outside [0, V) makes logp NaN
 * and is counted; the return value is that count (or -1 on bad arguments). */
int64_t oracle_row_logprob(const void* logits, int dtype, int64_t V, const int64_t* tokens,
                           int64_t rows, double* lse, double* logp) {
  if (!logits || !tokens || !lse || !logp || V <= 0 || rows < 0) return -1;
  if (dtype != OR_F32 && dtype != OR_BF16 && dtype != OR_F64) return -1;
  int64_t bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : bad)
  for (int64_t r = 0; r < rows; ++r) {
    const int64_t base = r * V;
    int has_nan = 0;
    double M = -INFINITY;
    for (int64_t v = 0; v < V; ++v) {
      double x = or_elem(logits, dtype, base + v);
      if (isnan(x)) has_nan = 1;
      if (x > M) M = x;
    }
    double S = 0.0;
    for (int64_t v = 0; v < V; ++v) S += exp(or_elem(logits, dtype, base + v) - M);
    double l = has_nan ? NAN : M + log(S);
    lse[r] = l;
    int64_t y = tokens[r];
    if (y < 0 || y >= V) {
      logp[r] = NAN;
      bad += 1;
    } else {
      logp[r] = or_elem(logits, dtype, base + y) - l;
    }
  }
  return bad;
}

/* Per-token loss term and its derivative, for a [N, C] batch.
 *
 * [DG] "PPO": importance ratio r = exp(logp - logp_old); clipped surrogate
 *   s = min(r*A, clip(r, 1-eps, 1+eps)*A), the clip applied to the ratio
 *   before the multiply ([DG] "The loss").
 * KL term (reading above): d = logp_ref - logp, k3 = exp(d) - d - 1.
 * [DG] "Dr. GRPO" pseudo-code: the loss is the negated surrogate plus beta
 *   times the KL term, so lambda = -s + beta*k3 per token.
 * The mask multiplies the per-token loss, not the ratio ([DG] "The loss").
 *
 * Gradient of lambda with respect to logp, g = dlambda/dlogp, following the
 * subgradient that automatic differentiation of the printed expression takes
 * (clamp passes its gradient on the closed interval, a tie of the two
 * surrogates splits it evenly, which sums to the unclipped branch):
 *   chi = 0 if (A > 0 and r > 1+eps) or (A < 0 and r < 1-eps), else 1
 *   g   = -A*r*chi + beta*(1 - exp(d)).
 * The loss is L = sum_i (sum over mask=1 tokens of row i of lambda) / div_i
 * (div from oracle_row_divisor; div_i = kappa for the Dr. GRPO token sum), so
 * the gradient of L with respect to the logits of token (i,t) is
 *   dL/dx_v = (g/div_i) * ([v = y] - softmax_v) = coef * (softmax_v - [v = y])
 * with coef = -g / div_i.
 *
 * Inactive tokens (t >= len_i, or A_i = 0 with beta = 0) get lambda = 0 and
 * coef = 0 without reading logp.  stats (nullable, int64[2]) receives the
 * number of active tokens whose ratio lies outside [1-eps, 1+eps] and the
 * number whose surrogate gradient is cut by the clip (chi = 0, A != 0).
 * logp_ref may be NULL only when beta == 0. */
int oracle_token_terms(const double* logp, const float* logp_old, const float* logp_ref,
                       const float* adv, const int32_t* len, int64_t N, int64_t C, double eps,
                       double beta, const double* div, double* lambda, double* coef,
                       int64_t* stats) {
  if (!logp || !logp_old || !adv || !len || !div || !lambda || !coef || N < 0 || C < 0)
    return -1;
  if (beta != 0.0 && !logp_ref) return -1;
  int64_t n_out = 0, n_cut = 0;
  for (int64_t i = 0; i < N; ++i) {
    const double A = (double)adv[i];
    for (int64_t t = 0; t < C; ++t) {
      const int64_t k = i * C + t;
      if (t >= len[i] || (A == 0.0 && beta == 0.0)) {
        lambda[k] = 0.0;
        coef[k] = 0.0;
        continue;
      }
      const double r = exp(logp[k] - (double)logp_old[k]);
      /* clamp to [1-eps, 1+eps]; a NaN ratio stays NaN */
      const double c = r < 1.0 - eps ? 1.0 - eps : (r > 1.0 + eps ? 1.0 + eps : r);
      const double u = r * A;
      const double v = c * A;
      const double s = (u < v || isnan(u)) ? u : v;
      double k3 = 0.0, dk3 = 0.0;
      if (beta != 0.0) {
        const double d = (double)logp_ref[k] - logp[k];
        k3 = exp(d) - d - 1.0;
        dk3 = 1.0 - exp(d);
      }
      const int cut = (A > 0.0 && r > 1.0 + eps) || (A < 0.0 && r < 1.0 - eps);
      const double g = -A * r * (cut ? 0.0 : 1.0) + beta * dk3;
      lambda[k] = -s + beta * k3;
      coef[k] = -g / div[i];
      if (r < 1.0 - eps || r > 1.0 + eps) n_out += 1;
      if (cut && A != 0.0) n_cut += 1;
    }
  }
  if (stats) {
    stats[0] = n_out;
    stats[1] = n_cut;
  }
  return 0;
}

/* [DG] "Dr. GRPO": token-sum aggregation; each completion's token sum is
 * divided by its divisor (oracle_row_divisor) and the quotients are added.
 * lambda is zero at masked positions, so the plain sum over a row is the
 * masked sum. */
double oracle_loss(const double* lambda, const double* div, int64_t N, int64_t C) {
  double s = 0.0;
  for (int64_t i = 0; i < N; ++i) {
    double row = 0.0;
    for (int64_t t = 0; t < C; ++t) row += lambda[i * C + t];
    s += row / div[i];
  }
  return s;
}

/* Gradient rows: out[r, v] = coef_r * (exp(x_v - lse_r) - [v = y_r]); a row
 * with coef_r = 0 is exactly zero (its logits are not read). */
int oracle_dlogits_rows(const void* logits, int dtype, int64_t V, const int64_t* tokens,
                        const double* lse, const double* coef, int64_t rows, double* out) {
  if (!logits || !tokens || !lse || !coef || !out || V <= 0 || rows < 0) return -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < rows; ++r) {
    double* o = out + r * V;
    if (coef[r] == 0.0) {
      for (int64_t v = 0; v < V; ++v) o[v] = 0.0;
      continue;
    }
    for (int64_t v = 0; v < V; ++v) {
      double p = exp(or_elem(logits, dtype, r * V + v) - lse[r]);
      o[v] = coef[r] * (p - (v == tokens[r] ? 1.0 : 0.0));
    }
  }
  return 0;
}
