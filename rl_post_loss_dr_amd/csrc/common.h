/*
 * common.h - pieces shared by the raw-logits path (drgrpo.hip) and the fused
 * lm_head path (lmhead.hip): per-token flags, the per-token loss term and
 * gradient coefficient, the completion-mask / advantage kernel, the
 * fixed-order finishing reduction, and host-side argument helpers.
 * Definitions are those of include/drgrpo.h.
 */
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "drgrpo.h"

namespace {

// per-token flags
constexpr uint8_t TF_OUTSIDE = 1;  // ratio outside [1-eps, 1+eps]
constexpr uint8_t TF_CUT = 2;      // clip cuts the surrogate gradient (A != 0)
constexpr uint8_t TF_BADTOK = 4;   // token outside [0, V) at a mask=1 position
// per-row flags
constexpr uint8_t RF_NOEOS = 1;      // row has no EOS
constexpr uint8_t RF_NOCONTRAST = 2; // first row of a group whose rewards are all equal

constexpr int32_t kStatusTokenRange = 1;

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }


// ------------------------------------------------------- per-token epilogue
// Loss term and gradient coefficient of one counted token ("Making Dr GRPO go
// brrr", sections "PPO" and "The loss": clipped surrogate of the ratio; the
// pseudo-code of "Dr. GRPO": negated surrogate plus beta times the KL term,
// here the k3 estimator).  Binary64 throughout.
struct TokenTerms {
  double lam;    // -min(r*A, clip(r)*A) + beta*k3
  double coef;   // dL/dlogp / -1: dlogits = coef * (softmax - onehot)
  uint8_t flags; // TF_OUTSIDE | TF_CUT
};

__device__ inline TokenTerms token_terms(double logp, float old, float ref, float A, float eps_f,
                                         float beta_f, double kappa) {
  const double Ad = (double)A;
  const double eps = (double)eps_f;
  const double beta = (double)beta_f;
  const double r = exp(logp - (double)old);
  const double lo = 1.0 - eps, hi = 1.0 + eps;
  const double c = r < lo ? lo : (r > hi ? hi : r);  // a NaN ratio stays NaN
  const double u = r * Ad;
  const double v = c * Ad;
  const double sur = (u < v || isnan(u)) ? u : v;
  double k3 = 0.0, dk3 = 0.0;
  if (beta != 0.0) {
    const double d = (double)ref - logp;
    const double ed = exp(d);
    k3 = ed - d - 1.0;
    dk3 = 1.0 - ed;
  }
  // the clip cuts the surrogate's gradient when the clipped branch is the
  // minimum and the ratio lies outside the range
  const bool cut = (Ad > 0.0 && r > hi) || (Ad < 0.0 && r < lo);
  const double g = -Ad * r * (cut ? 0.0 : 1.0) + beta * dk3;
  TokenTerms t;
  t.lam = -sur + beta * k3;
  t.coef = -g / kappa;
  t.flags = (uint8_t)(((r < lo || r > hi) ? TF_OUTSIDE : 0) | ((cut && Ad != 0.0) ? TF_CUT : 0));
  return t;
}

// ------------------------------------------------------------------- k_prep
// One wavefront per completion row i.
// adv_mode: DRGRPO_ADV_CENTER or DRGRPO_ADV_ZSCORE (include/drgrpo.h).
// zero2 (nullable): two words, [0] and [64], set to zero by completion 0
// (the loss's ticket counters, ahead of the row kernel on the stream).
__global__ void __launch_bounds__(64)
k_prep(const int64_t* __restrict__ tokens, int64_t C, int64_t eos_id,
       const float* __restrict__ rewards, int64_t G, int adv_mode, int32_t* __restrict__ len,
       float* __restrict__ adv, uint8_t* __restrict__ row_flags, int32_t* __restrict__ aux_len,
       uint8_t* __restrict__ aux_mask, float* __restrict__ aux_adv,
       int32_t* __restrict__ nocontrast_count, uint32_t* __restrict__ zero2) {
  const int64_t i = blockIdx.x;
  const int lane = threadIdx.x;
  if (zero2 && i == 0 && lane == 0) {
    zero2[0] = 0u;
    zero2[64] = 0u;
  }
  int64_t first = C;
  if (tokens) {
    const int64_t* row = tokens + i * C;
    for (int64_t base = 0; base < C; base += 64) {
      const int64_t t = base + lane;
      const bool hit = t < C && row[t] == eos_id;
      const unsigned long long b = __ballot(hit);
      if (b) {
        first = base + __ffsll(b) - 1;
        break;
      }
    }
    const int32_t L = first < C ? (int32_t)(first + 1) : (int32_t)C;
    if (aux_mask)
      for (int64_t t = lane; t < C; t += 64) aux_mask[i * C + t] = t < L ? 1 : 0;
    if (lane == 0) {
      if (len) len[i] = L;
      if (aux_len) aux_len[i] = L;
    }
  }
  if (rewards && lane == 0) {
    // A_i = R_i - (sequential binary32 group sum) / G ("Dr. GRPO"); the GRPO
    // variant divides by the group's sample standard deviation (sequential
    // sum of rounded squares, / (G-1), correctly rounded sqrt and division),
    // and gives 0 to a group whose rewards are all equal.  No contraction:
    // every product and sum is rounded on its own, bit-identical to a plain
    // binary32 evaluation in this order.
#pragma clang fp contract(off)
    const int64_t g0 = (i / G) * G;
    const float r0 = rewards[g0];
    float s = 0.0f;
    bool same = true;
    for (int64_t j = 0; j < G; ++j) {
      const float r = rewards[g0 + j];
      s = s + r;
      same = same && (r == r0);
    }
    const float mu = s / (float)G;
    float a = rewards[i] - mu;
    if (adv_mode == DRGRPO_ADV_ZSCORE) {
      if (same) {
        a = 0.0f;
      } else {
        float q = 0.0f;
        for (int64_t j = 0; j < G; ++j) {
          const float d = rewards[g0 + j] - mu;
          const float d2 = d * d;
          q = q + d2;
        }
        const float sd = sqrtf(q / (float)(G - 1));
        a = a / sd;
      }
    }
    if (adv) adv[i] = a;
    if (aux_adv) aux_adv[i] = a;
    const bool group_head = (i == g0) && same;
    if (row_flags)
      row_flags[i] = (uint8_t)((tokens && first == C ? RF_NOEOS : 0) |
                               (group_head ? RF_NOCONTRAST : 0));
    if (nocontrast_count && group_head) atomicAdd(nocontrast_count, 1);
  }
}

__global__ void k_zero_i32(int32_t* p) { *p = 0; }

// Divisor of completion i's token sum for the aggregation `agg`
// (include/drgrpo.h, drgrpo_variant_t): kappa (token sum), kappa*len_i
// (per-response mean), kappa * total counted tokens (token mean).
__device__ inline double row_divisor(int agg, double kappa, int32_t len_i,
                                     const int64_t* total_len) {
  if (agg == DRGRPO_AGG_SEQ_MEAN) return kappa * (double)len_i;
  if (agg == DRGRPO_AGG_TOKEN_MEAN) return kappa * (double)*total_len;
  return kappa;
}

// Total counted tokens (sum of len) for the token mean: one workgroup,
// integer sum (exact, order-free).
__global__ void __launch_bounds__(1024)
k_total_len(const int32_t* __restrict__ len, int64_t N, int64_t* __restrict__ total) {
  __shared__ long long sh[16];
  long long s = 0;
  for (int64_t i = threadIdx.x; i < N; i += 1024) s += len[i];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    long long t = 0;
    for (int w = 0; w < 16; ++w) t += sh[w];
    *total = (int64_t)t;
  }
}

// ----------------------------------------------------------------- k_finish
__device__ inline double wave_sum_d(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
__device__ inline int wave_sum_i(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// tok_loss holds each token's term already divided by its row divisor, so
// the loss is their plain sum (fixed order).  Counters: drgrpo_aux_t.stats
// and drgrpo_loss_opts_t.token_counts.
__global__ void __launch_bounds__(1024)
k_finish(const double* __restrict__ tok_loss, const uint8_t* __restrict__ tok_flags, int64_t T,
         const uint8_t* __restrict__ row_flags, const int32_t* __restrict__ len,
         const float* __restrict__ adv, float beta, int64_t N, float* __restrict__ out_loss,
         int32_t* __restrict__ status, int32_t* __restrict__ aux_stats,
         int64_t* __restrict__ aux_counts) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  double s = 0.0;
  int n_out = 0, n_cut = 0, n_bad = 0, n_trunc = 0, n_noc = 0;
  long long n_len = 0, n_act = 0;
  // each thread sums tokens tid, tid + 1024, ... in that order (coalesced
  // across the wavefront; the loads of 8 of them go out before their adds),
  // then the wavefront butterflies and the 16 wavefront partials in order: a
  // fixed summation order, bitwise reproducible
  for (int64_t k = tid; k < T; k += 8 * 1024) {
    double v[8];
    uint8_t f[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t kk = k + (int64_t)u * 1024;
      v[u] = kk < T ? tok_loss[kk] : 0.0;
      f[u] = kk < T ? tok_flags[kk] : (uint8_t)0;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      s += v[u];
      n_out += (f[u] & TF_OUTSIDE) ? 1 : 0;
      n_cut += (f[u] & TF_CUT) ? 1 : 0;
      n_bad += (f[u] & TF_BADTOK) ? 1 : 0;
    }
  }
  for (int64_t k = tid; k < N; k += 1024) {
    const uint8_t f = row_flags[k];
    n_trunc += (f & RF_NOEOS) ? 1 : 0;
    n_noc += (f & RF_NOCONTRAST) ? 1 : 0;
    n_len += len[k];
    n_act += (adv[k] != 0.0f || beta != 0.0f) ? len[k] : 0;
  }
  s = wave_sum_d(s);
  n_out = wave_sum_i(n_out);
  n_cut = wave_sum_i(n_cut);
  n_bad = wave_sum_i(n_bad);
  n_trunc = wave_sum_i(n_trunc);
  n_noc = wave_sum_i(n_noc);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    n_len += __shfl_xor(n_len, off);
    n_act += __shfl_xor(n_act, off);
  }
  __shared__ double sh_s[16];
  __shared__ int sh_i[5][16];
  __shared__ long long sh_l[2][16];
  if (lane == 0) {
    sh_s[wave] = s;
    sh_i[0][wave] = n_out;
    sh_i[1][wave] = n_cut;
    sh_i[2][wave] = n_bad;
    sh_i[3][wave] = n_trunc;
    sh_i[4][wave] = n_noc;
    sh_l[0][wave] = n_len;
    sh_l[1][wave] = n_act;
  }
  __syncthreads();
  if (tid == 0) {
    double tot = 0.0;
    int64_t c[5] = {0, 0, 0, 0, 0};
    int64_t nl = 0, na = 0;
    for (int w = 0; w < 16; ++w) {
      tot += sh_s[w];
      for (int q = 0; q < 5; ++q) c[q] += sh_i[q][w];
      nl += sh_l[0][w];
      na += sh_l[1][w];
    }
    *out_loss = (float)tot;
    status[0] = c[2] ? kStatusTokenRange : 0;
    status[1] = (int32_t)c[3];
    status[2] = (int32_t)c[4];
    if (aux_stats) {  // each count is at most the token rows, below 2^31
      aux_stats[0] = (int32_t)c[4];
      aux_stats[1] = (int32_t)c[3];
      aux_stats[2] = (int32_t)c[0];
      aux_stats[3] = (int32_t)c[1];
    }
    if (aux_counts) {
      aux_counts[0] = nl;
      aux_counts[1] = na;
    }
  }
}

// ------------------------------------------------------------ host helpers
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

bool finite_f(float x) { return x == x && x - x == 0.0f; }

// Validated variant (NULL = Dr. GRPO: centred advantage, token sum).
bool read_variant(const drgrpo_variant_t* v, int* adv_mode, int* agg) {
  *adv_mode = v ? v->adv_mode : DRGRPO_ADV_CENTER;
  *agg = v ? v->agg_mode : DRGRPO_AGG_TOKEN_SUM;
  return (*adv_mode == DRGRPO_ADV_CENTER || *adv_mode == DRGRPO_ADV_ZSCORE) &&
         (*agg == DRGRPO_AGG_TOKEN_SUM || *agg == DRGRPO_AGG_SEQ_MEAN ||
          *agg == DRGRPO_AGG_TOKEN_MEAN);
}

int launch_status() { return hipGetLastError() == hipSuccess ? DRGRPO_OK : DRGRPO_ERR_HIP; }


}  // namespace
