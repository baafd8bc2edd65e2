/*
 * drgrpo.hip - fused Dr. GRPO update loss, forward and backward, for gfx950.
 *
 * Definitions are those of include/drgrpo.h ("Making Dr GRPO go brrr":
 * "The completion mask", "compute_logprobs", "PPO", "Dr. GRPO", "The loss").
 *
 * One call is three (four) stream-ordered launches:
 *   k_prep    one wavefront per completion: first-EOS length (ballot over 64
 *             tokens at a time), group advantage, per-row flags; zeroes the
 *             row kernel's ticket counters.
 *   k_plan    one workgroup, only for the ticket order at 256 or more
 *             completions or for the token mean: prefix of active rows per
 *             completion, counted tokens.
 *   k_rows    one 1024-thread workgroup per token row (rows of at least
 *             192 KB taken in the ticket order of ticket_row: each class of
 *             rows, active or zero, in memory order by an arrival counter;
 *             smaller ones by a fixed stride): streams the row's V
 *             logits from HBM once with 16-byte loads, keeps them in
 *             registers (19 chunks of 16 B per lane covers a bf16 row of up
 *             to 155,648 entries), reduces max / sum-of-exp with wavefront
 *             shuffles and one LDS exchange, evaluates the per-token surrogate
 *             and KL in binary64, then writes dlogits = coef*(softmax - onehot)
 *             from the same registers.  Rows longer than one register tile
 *             are swept tile by tile, last tile first; the write pass starts
 *             from the first tile, still in the registers, and re-reads only
 *             the rest.  Tokens
 *             whose loss term is identically zero only write zeros.
 *   k_finish  one workgroup: fixed-order binary64 sum of the per-token terms
 *             (each already divided by its completion's aggregation divisor:
 *             norm_const for the Dr. GRPO token sum), counters and the
 *             status word.
 * No floating-point atomics: results are bitwise reproducible.
 */
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "drgrpo.h"
#include "common.h"

namespace {

constexpr int kThreads = 1024;          // largest token-row workgroup (rows that
                                        // need more than one register tile)
constexpr int kNch = 19;                // register-resident 16-byte chunks per lane
constexpr float kLog2e = 1.4426950408889634f;
constexpr double kLog2eD = 1.4426950408889634074;

// Workspace carve-up (offsets from a 256-byte aligned base).
struct Ws {
  int32_t* status;     // [64]: [0] status word
  int32_t* len;        // [N]
  float* adv;          // [N]
  uint8_t* row_flags;  // [N]
  int64_t* total_len;  // [1] counted tokens (token-mean aggregation)
  double* tok_loss;    // [T] per-token term / row divisor
  uint8_t* tok_flags;  // [T]
  uint32_t* plan;      // row plan of the ticket order: two counters and the
                       // prefix of active rows per completion (kPlan* offsets)
};

// Offsets (in 32-bit words) into the row plan: the two ticket counters sit
// 256 bytes apart, so their atomics do not share a cache line; the prefix
// holds N + 1 entries.
constexpr uint32_t kPlanActive = 0;
constexpr uint32_t kPlanZero = 64;
constexpr uint32_t kPlanPrefix = 128;

size_t ws_carve(void* base, int64_t N, int64_t T, Ws* ws) {
  size_t off = 0;
  char* b = static_cast<char*>(base);
  auto take = [&](size_t bytes) {
    char* p = b ? b + off : nullptr;
    off += align256(bytes);
    return p;
  };
  Ws w;
  w.status = reinterpret_cast<int32_t*>(take(256));
  w.len = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * N));
  w.adv = reinterpret_cast<float*>(take(sizeof(float) * N));
  w.row_flags = reinterpret_cast<uint8_t*>(take(N));
  w.total_len = reinterpret_cast<int64_t*>(take(sizeof(int64_t)));
  w.tok_loss = reinterpret_cast<double*>(take(sizeof(double) * T));
  w.tok_flags = reinterpret_cast<uint8_t*>(take(T));
  w.plan = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * (kPlanPrefix + N + 1)));
  if (ws) *ws = w;
  return off;
}

// ----------------------------------------------------------------- element IO
// Row data moves in 16-byte chunks (bf16 x 8 or f32 x 4).  Loads are
// nontemporal global loads: every byte is read once.  Stores go through a
// buffer descriptor spanning exactly the output row (the hardware drops any
// access past it) with the nontemporal + sc1 cache policy, which measured
// 2-5% faster than plain nontemporal stores for this write-heavy stream.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// cache-policy immediate of a buffer store on gfx950: sc1 (16) | nt (2)
constexpr int kStorePolicy = 16 | 2;
// third descriptor word of a raw (byte-addressed, unswizzled) buffer
constexpr int kRawBufferWord3 = 0x00020000;

struct RowOut {
  __amdgpu_buffer_rsrc_t rsrc;  // the output row, bounded by its byte size
};

__device__ inline RowOut row_out(char* row, uint32_t bytes) {
  return RowOut{__builtin_amdgcn_make_buffer_rsrc(row, (short)0, (int)bytes, kRawBufferWord3)};
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// a and b rounded to bfloat16 (nearest even), a in the low half: one
// v_cvt_pk_bf16_f32 (a vector conversion; scalar ones take one each)
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <int DT, int VEC>
struct Io;

// bfloat16, 8 per 16-byte chunk
template <>
struct Io<DRGRPO_BF16, 8> {
  using chunk = u32x4;
  static constexpr int kBytes = 2;
  __device__ static chunk load(const char* row, uint32_t c) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row) + c);
  }
  __device__ static void unpack(const chunk& v, float (&f)[8]) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
    f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
  }
  // `sign` (0 or all ones) flips the sign bit of every packed value
  __device__ static chunk pack(const float (&f)[8], uint32_t sign) {
    const uint32_t m = sign & 0x80008000u;
    return u32x4{pack_bf16x2(f[0], f[1]) ^ m, pack_bf16x2(f[2], f[3]) ^ m,
                 pack_bf16x2(f[4], f[5]) ^ m, pack_bf16x2(f[6], f[7]) ^ m};
  }
  __device__ static void store(const RowOut& o, uint32_t c, const chunk& v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, o.rsrc, (int)(c * 16u), 0, kStorePolicy);
  }
  __device__ static chunk splat(float val) {
    const uint32_t w = pack_bf16x2(val, val);
    return u32x4{w, w, w, w};
  }
  // element idx of the row set to val (rounded to nearest even)
  __device__ static void store_one(const RowOut& o, int64_t idx, float val) {
    const __bf16 h = (__bf16)val;
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, h), o.rsrc, (int)(idx * 2),
                                          0, kStorePolicy);
  }
};

// binary32, 4 per 16-byte chunk
template <>
struct Io<DRGRPO_F32, 4> {
  using chunk = u32x4;
  static constexpr int kBytes = 4;
  __device__ static chunk load(const char* row, uint32_t c) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row) + c);
  }
  __device__ static void unpack(const chunk& v, float (&f)[4]) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
  __device__ static chunk pack(const float (&f)[4], uint32_t sign) {
    const uint32_t m = sign & 0x80000000u;
    return u32x4{__float_as_uint(f[0]) ^ m, __float_as_uint(f[1]) ^ m,
                 __float_as_uint(f[2]) ^ m, __float_as_uint(f[3]) ^ m};
  }
  __device__ static void store(const RowOut& o, uint32_t c, const chunk& v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, o.rsrc, (int)(c * 16u), 0, kStorePolicy);
  }
  __device__ static chunk splat(float val) {
    const uint32_t w = __float_as_uint(val);
    return u32x4{w, w, w, w};
  }
  __device__ static void store_one(const RowOut& o, int64_t idx, float val) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val), o.rsrc, (int)(idx * 4), 0,
                                          kStorePolicy);
  }
};

// bfloat16, one element per access (rows not 16-byte aligned)
template <>
struct Io<DRGRPO_BF16, 1> {
  using chunk = uint16_t;
  static constexpr int kBytes = 2;
  __device__ static chunk load(const char* row, uint32_t c) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(row) + c);
  }
  __device__ static void unpack(const chunk& v, float (&f)[1]) {
    f[0] = __uint_as_float((uint32_t)v << 16);
  }
  __device__ static chunk pack(const float (&f)[1], uint32_t sign) {
    const __bf16 h = (__bf16)f[0];
    return (uint16_t)(__builtin_bit_cast(uint16_t, h) ^ (sign & 0x8000u));
  }
  __device__ static void store(const RowOut& o, uint32_t c, const chunk& v) {
    __builtin_amdgcn_raw_buffer_store_b16(v, o.rsrc, (int)(c * 2u), 0, kStorePolicy);
  }
  __device__ static chunk splat(float val) {
    const __bf16 h = (__bf16)val;
    return __builtin_bit_cast(uint16_t, h);
  }
  __device__ static void store_one(const RowOut& o, int64_t idx, float val) {
    store(o, (uint32_t)idx, splat(val));
  }
};

// binary32, one element per access (rows not 16-byte aligned)
template <>
struct Io<DRGRPO_F32, 1> {
  using chunk = float;
  static constexpr int kBytes = 4;
  __device__ static chunk load(const char* row, uint32_t c) {
    return __builtin_nontemporal_load(reinterpret_cast<const float*>(row) + c);
  }
  __device__ static void unpack(const chunk& v, float (&f)[1]) { f[0] = v; }
  __device__ static chunk pack(const float (&f)[1], uint32_t sign) {
    return __uint_as_float(__float_as_uint(f[0]) ^ (sign & 0x80000000u));
  }
  __device__ static void store(const RowOut& o, uint32_t c, const chunk& v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), o.rsrc, (int)(c * 4u), 0,
                                          kStorePolicy);
  }
  __device__ static chunk splat(float val) { return val; }
  __device__ static void store_one(const RowOut& o, int64_t idx, float val) {
    store(o, (uint32_t)idx, val);
  }
};

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// (max, sum of exp(x - max)) pair merge; empty sides have max = -inf, sum = 0.
__device__ inline void lse_merge(float& m, float& s, float m2, float s2) {
  const float nm = fmaxf(m, m2);
  if (nm == -INFINITY) return;
  s = s * fast_exp2((m - nm) * kLog2e) + s2 * fast_exp2((m2 - nm) * kLog2e);
  m = nm;
}

// ------------------------------------------------------------------- k_rows
struct RowArgs {
  const void* logits;
  void* dlogits;
  const int64_t* tokens;
  const float* logp_old;
  const float* logp_ref;
  const int32_t* len;
  const float* adv;
  int64_t C;
  int64_t V;
  float eps;
  float beta;
  double kappa;
  int agg;                   // drgrpo_agg_mode_t
  const int64_t* total_len;  // counted tokens of the batch (token mean only)
  double* tok_loss;
  uint8_t* tok_flags;
  float* aux_logp;
  float* aux_tok_loss;
  float* out_logp;  // forward-only mode: log-prob of every token
  uint32_t* plan;   // row plan (k_plan) of the ticket order
  uint32_t row_stride;  // workgroup b handles row (b * row_stride) mod T; gcd(row_stride, T) = 1
  uint32_t T;
  uint32_t N;
};

// The ticket order of the full-size rows.  Each row is of one of two
// classes: active (counted token of a completion whose term is not
// identically zero: it reads the row and writes its gradient) or zero (it
// only writes zeros).  Workgroup b takes the class of row (b * row_stride)
// mod T, so the workgroups in flight mix the classes in the batch's
// proportion, and then the next row of that class in memory order from the
// class's counter, so the rows in flight at once sit next to each other in
// memory.  Against every workgroup owning row (b * row_stride) mod T, with
// rows of 297 KB: 10% faster at 16K rows of which 30% are active, 8% with
// all of them active, even at 64K rows (55% active), 1% faster at 128K rows
// (two thirds active).  The k-th active row lies in the completion i with
// P[i] <= k < P[i+1] (P the exclusive prefix of active rows), the k-th zero
// row in the completion with i*C - P[i] <= k < (i+1)*C - P[i+1]: both keys
// are nondecreasing in i.  One wavefront finds i: for N < 256 the whole
// prefix sits in its registers (4 entries a lane), formed before the ticket
// is taken, and i + 1 is the number of entries j <= N with key(j) <= k;
// larger batches narrow [lo, hi) 63-fold per round.  Returns -1 for a
// ticket past the class's rows (never, when len, adv and the prefix agree:
// they are the same values).
__device__ int64_t ticket_row(const RowArgs& a, int lane) {
  const uint32_t C = (uint32_t)a.C, N = a.N;
  const uint32_t r0 = (uint32_t)(((uint64_t)blockIdx.x * a.row_stride) % a.T);
  const uint32_t i0 = r0 / C;
  const bool act =
      (int32_t)(r0 - i0 * C) < a.len[i0] && (a.adv[i0] != 0.0f || a.beta != 0.0f);
  const uint32_t* P = a.plan + kPlanPrefix;
  auto key = [&](uint32_t j, uint32_t p) { return act ? p : j * C - p; };
  // N < 256: the wavefront forms P[j], j = lane*4 .. lane*4+3, itself from
  // len and adv (the same values and test as the class above); larger
  // batches read the prefix k_plan wrote
  uint32_t pv[4];
  uint32_t active_rows;
  if (N < 256) {
    uint32_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t j = (uint32_t)lane * 4u + u;
      v[u] = (j < N && (a.adv[j] != 0.0f || a.beta != 0.0f)) ? (uint32_t)a.len[j] : 0u;
    }
    const uint32_t own = v[0] + v[1] + v[2] + v[3];
    uint32_t incl = own;  // inclusive scan of the lanes' sums
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t y = (uint32_t)__shfl_up((int)incl, off);
      if (lane >= off) incl += y;
    }
    uint32_t run = incl - own;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      pv[u] = run;
      run += v[u];
    }
    active_rows = (uint32_t)__shfl((int)incl, 63);
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) pv[u] = 0u;
    active_rows = P[N];
  }
  uint32_t k = 0;
  if (lane == 0) k = atomicAdd(a.plan + (act ? kPlanActive : kPlanZero), 1u);
  k = __shfl(k, 0);
  if (k >= (act ? active_rows : a.T - active_rows)) return -1;
  uint32_t i, p0, p1;
  if (N < 256) {
    uint32_t n = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t j = (uint32_t)lane * 4u + u;
      n += (uint32_t)__popcll(__ballot(j <= N && key(j, pv[u]) <= k));
    }
    i = n - 1;  // key(0) = 0 <= k and key(N) > k: 0 <= i < N
    auto pick = [&](uint32_t e) {
      const uint32_t u = e & 3u;
      const uint32_t v = u == 0 ? pv[0] : u == 1 ? pv[1] : u == 2 ? pv[2] : pv[3];
      return (uint32_t)__shfl((int)v, (int)(e >> 2));
    };
    p0 = pick(i);
    p1 = pick(i + 1);
  } else {
    uint32_t lo = 0, hi = N;  // key(lo) <= k < key(hi)
    for (;;) {
      // lanes 0..63 probe lo, lo + step, ... up to hi (loaded clamped to hi),
      // so the lane after the last passing one holds the next entry
      const uint32_t step = (hi - lo + 62) / 63;
      const uint32_t j = lo + (uint32_t)lane * step;
      const uint32_t p = P[min(j, hi)];
      // keys are nondecreasing and the probe at lo passes: the passing lanes
      // are a prefix, the last of them brackets the answer
      const uint64_t m = __ballot(j < hi && key(j, p) <= k);
      const int L = 63 - __clzll(m);
      if (step == 1) {  // hi - lo <= 63: lane L holds P[i], lane L + 1 P[i + 1]
        i = lo + (uint32_t)L;
        p0 = (uint32_t)__shfl((int)p, L);
        p1 = (uint32_t)__shfl((int)p, L + 1);
        break;
      }
      lo += (uint32_t)L * step;
      hi = min(lo + step, hi);
    }
  }
  return (int64_t)i * C + (act ? k - p0 : (p1 - p0) + (k - (i * C - p0)));
}

// Merge one chunk of values into a lane's running (max, sum of exp(x - max)).
// A lane past the end of the row holds a copy of the row's last chunk (its
// load is clamped there): the copy cannot raise the maximum, and its sum is
// dropped (live = false) with one select instead of overwriting its values
// (against -inf in each entry: 8 fewer VALU instructions a chunk, measured
// 3% faster on an all-active batch, 0.5-1.6% on the others).
template <int VEC>
__device__ inline void lse_chunk(float& m, float& s, const float (&f)[VEC], bool live) {
  float cm = f[0];
#pragma unroll
  for (int e = 1; e < VEC; ++e) cm = fmaxf(cm, f[e]);
  const float nm = fmaxf(m, cm);
  const float base = nm == -INFINITY ? 0.0f : nm;  // nothing finite seen yet
  // exp(x - base) with the difference taken first: exact for the entries
  // near the maximum that dominate the sum, and exactly 1 at the maximum (so
  // a one-entry vocabulary gives log-prob 0 exactly; a fused x*log2e -
  // base*log2e would leave that product's rounding)
  float cs = fast_exp2((f[0] - base) * kLog2e);
#pragma unroll
  for (int e = 1; e < VEC; ++e) cs += fast_exp2((f[e] - base) * kLog2e);
  s = s * fast_exp2((m - base) * kLog2e) + (live ? cs : 0.0f);
  m = nm;
}

// Two chunks merged in one step: one rescale of the running sum for both
// (against one chunk a step: 1.7% faster on an all-active batch, 0.3-0.6% on
// the others).
template <int VEC>
__device__ inline void lse_pair(float& m, float& s, const float (&f)[VEC], const float (&g)[VEC],
                                bool live_f, bool live_g) {
  float cm = f[0];
#pragma unroll
  for (int e = 1; e < VEC; ++e) cm = fmaxf(cm, f[e]);
#pragma unroll
  for (int e = 0; e < VEC; ++e) cm = fmaxf(cm, g[e]);
  const float nm = fmaxf(m, cm);
  const float base = nm == -INFINITY ? 0.0f : nm;
  float cf = fast_exp2((f[0] - base) * kLog2e);
#pragma unroll
  for (int e = 1; e < VEC; ++e) cf += fast_exp2((f[e] - base) * kLog2e);
  float cg = fast_exp2((g[0] - base) * kLog2e);
#pragma unroll
  for (int e = 1; e < VEC; ++e) cg += fast_exp2((g[e] - base) * kLog2e);
  s = s * fast_exp2((m - base) * kLog2e) + (live_f ? cf : 0.0f) + (live_g ? cg : 0.0f);
  m = nm;
}

// Pass 2 of a row: dlogits = coef * (softmax - onehot), with |coef| folded
// into the exponent and the sign of coef applied to the packed result bits:
// |coef| * exp(x - lse) = exp2((x - M)*log2e - off2) with M the row maximum
// (lse = M + ln S) and off2 = log2 S - log2|coef|.  Binary32 results take the
// difference first (x - M is exact for the entries that matter, accurate to
// ~1e-6 relative whatever the logits' magnitude); bfloat16 results take one
// fused step, exp2(x*log2e + c2) with c2 = -M*log2e - off2 formed in binary64
// and rounded once, which scales the row by one factor 2^d, |d| <= 2^-24 |c2|
// (below 1e-4 relative for |M| up to 10^4, under the bfloat16 rounding).
// Each register tile is
// converted in place and stored in two bursts of 16-byte stores (the stores
// of a half tile leave back to back: one store per converted chunk measured
// 2-3% slower than one burst, two bursts 1-3% faster than one).
template <typename IO, int VEC, int NT>
__device__ __attribute__((always_inline)) inline void write_dlogits(
    typename IO::chunk (&buf)[kNch], const char* in, const RowOut& out, uint32_t nchunks,
    uint32_t ntiles, int tid, float mrow, float off2, float c2, float dy, bool neg, int64_t y) {
  const uint32_t tile = (uint32_t)kNch * NT;
  const uint32_t last = nchunks - 1;
  const uint32_t cy = (uint32_t)(y / VEC);
  const uint32_t sign = neg ? 0xFFFFFFFFu : 0u;
  for (uint32_t k = 0; k < ntiles; ++k) {
    const uint32_t tb = k * tile;
    if (k > 0) {  // tile 0 is still in the registers from pass 1
#pragma unroll
      for (int j = 0; j < kNch; ++j) {
        const uint32_t c = tb + (uint32_t)j * NT + tid;
        buf[j] = IO::load(in, c < nchunks ? c : last);
      }
    }
    // slot and lane holding the sampled token's chunk in this tile
    const bool here = cy >= tb && cy - tb < tile;
    const int owner = here ? (int)((cy - tb) % NT) : -1;
    auto convert = [&](int j) {
      if (tb + (uint32_t)j * NT < nchunks) {
        float f[VEC];
        IO::unpack(buf[j], f);
        if constexpr (IO::kBytes == 2) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) f[e] = fast_exp2(fmaf(f[e], kLog2e, c2));
        } else {
#pragma unroll
          for (int e = 0; e < VEC; ++e) f[e] = fast_exp2(fmaf(f[e] - mrow, kLog2e, -off2));
        }
        buf[j] = IO::pack(f, sign);
      }
    };
    auto store = [&](int j) {
      const uint32_t c = tb + (uint32_t)j * NT + tid;
      if (c < nchunks) IO::store(out, c, buf[j]);
    };
    // two bursts: the first half of the tile is converted and stored, then
    // the rest, so the stores start while the second half is converted
    // (against one burst: 1-3% faster on every loss batch)
    constexpr int kBurst = (kNch + 1) / 2;
#pragma unroll
    for (int j = 0; j < kBurst; ++j) convert(j);
#pragma unroll
    for (int j = 0; j < kBurst; ++j) store(j);
#pragma unroll
    for (int j = kBurst; j < kNch; ++j) convert(j);
#pragma unroll
    for (int j = kBurst; j < kNch; ++j) store(j);
    // the sampled token's entry, coef * (p_y - 1), rewritten by the lane that
    // stored its chunk (its later store to the same address lands last), so
    // no lane pays a select per entry
    if (tid == owner) IO::store_one(out, y, dy);
  }
}

// One workgroup of NT threads per token row.  Every lane issues all of its
// kNch 16-byte loads of a tile before touching any of them (tail lanes
// re-read the last chunk and drop its sum), so a row's 297 KB are in flight at
// once; each pair of chunks is merged into the lane's running (max, sum) as they
// arrive.  NT is 256 when a 256-thread register tile holds the whole row
// (up to 38,912 bfloat16 entries), so four such workgroups share a CU and
// overlap their phases; 1024 otherwise.  (512 threads for rows up to twice
// that measured 10-25% faster on an all-active batch but 5-17% slower on a
// sparse one: not used.)
template <int DT, int VEC, bool kFwdOnly, int NT, bool kOrd = false>
__global__ void __launch_bounds__(NT) k_rows(RowArgs a) {
  static_assert(!kOrd || (!kFwdOnly && NT == kThreads), "the ticket order: the loss's 1024-thread rows");
  using IO = Io<DT, VEC>;
  constexpr int kWaves = NT / 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // consecutive workgroups take rows far apart, so the workgroups in flight
  // mix rows of every reward group (active rows and zero rows interleave);
  // the loss's rows of at least kTicketMinRowBytes go by the ticket order
  // (ticket_row)
  constexpr bool kTicket = kOrd;
  int64_t row;
  if constexpr (kTicket) {
    __shared__ int64_t sh_row;
    if (wave == 0) {
      const int64_t r = ticket_row(a, lane);
      if (lane == 0) sh_row = r;
    }
    __syncthreads();
    row = sh_row;
    if (row < 0) return;
  } else if (kFwdOnly) {
    // the forward-only pass reads every row: in index order the rows in
    // flight are neighbours (against the stride order: 1-4% faster)
    row = (int64_t)blockIdx.x;
  } else {
    row = (int64_t)(((uint64_t)blockIdx.x * a.row_stride) % a.T);
  }
  const int64_t i = row / a.C;
  const int64_t t = row - i * a.C;
  const int64_t V = a.V;
  const uint32_t nchunks = (uint32_t)(V / VEC);  // < 2^31 (checked on the host)
  const uint32_t last = nchunks - 1;
  const char* in = static_cast<const char*>(a.logits) + row * V * IO::kBytes;
  const RowOut out =
      row_out(kFwdOnly ? nullptr : static_cast<char*>(a.dlogits) + row * V * IO::kBytes,
              kFwdOnly ? 0u : (uint32_t)(V * IO::kBytes));
  const int64_t y = a.tokens[row];

  bool in_mask = true;
  bool active = true;
  float A = 0.0f;
  if (!kFwdOnly) {
    in_mask = t < a.len[i];
    A = a.adv[i];
    active = in_mask && (A != 0.0f || a.beta != 0.0f);
  }
  const bool bad = in_mask && (y < 0 || y >= V);
  if (bad || !active) {
    if (kFwdOnly) {
      if (tid == 0) a.out_logp[row] = NAN;
      return;
    }
    const typename IO::chunk fillv = IO::splat(bad ? NAN : 0.0f);
    for (uint32_t c = tid; c < nchunks; c += NT) IO::store(out, c, fillv);
    if (tid == 0) {
      a.tok_loss[row] = bad ? (double)NAN : 0.0;
      a.tok_flags[row] = bad ? TF_BADTOK : 0;
      if (a.aux_logp) a.aux_logp[row] = bad ? NAN : 0.0f;
      if (a.aux_tok_loss) a.aux_tok_loss[row] = bad ? NAN : 0.0f;
    }
    return;
  }

  // the sampled token's logit and the per-token inputs, fetched early by the
  // wavefront that evaluates the epilogue (read before any store of the row)
  // (every wavefront issues the same few loads: no divergent branch, so the
  // compiler need not drain the load counter before the row loads)
  const typename IO::chunk xy_chunk = IO::load(in, (uint32_t)(y / VEC));
  const float old = kFwdOnly ? 0.0f : a.logp_old[row];
  const float ref = (!kFwdOnly && a.beta != 0.0f) ? a.logp_ref[row] : 0.0f;

  // ---- pass 1: running max / sum of exp per lane over register tiles
  typename IO::chunk buf[kNch];
  const uint32_t tile = (uint32_t)kNch * NT;
  const uint32_t ntiles = (nchunks + tile - 1) / tile;
  float m = -INFINITY;
  float s = 0.0f;
  // tiles in reverse order, so the first (full) tile is the one left in the
  // registers for pass 2, which re-reads only the others
  for (uint32_t kk = ntiles; kk-- > 0;) {
    const uint32_t tb = kk * tile;
#pragma unroll
    for (int j = 0; j < kNch; ++j) {
      const uint32_t c = tb + (uint32_t)j * NT + tid;
      buf[j] = IO::load(in, c < nchunks ? c : last);
    }
#pragma unroll
    for (int j = 0; j < kNch; j += 2) {
      const uint32_t sb = tb + (uint32_t)j * NT;  // first chunk of the slot (uniform)
      if (j + 1 < kNch && sb + NT < nchunks) {  // slot j full, slot j + 1 not empty
        float f[VEC], g[VEC];
        IO::unpack(buf[j], f);
        IO::unpack(buf[j + 1], g);
        lse_pair<VEC>(m, s, f, g, true, sb + NT + tid < nchunks);
      } else if (sb < nchunks) {
        float f[VEC];
        IO::unpack(buf[j], f);
        lse_chunk<VEC>(m, s, f, sb + tid < nchunks);
      }
    }
  }
  // wavefront merge (fixed butterfly order)
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off);
    const float s2 = __shfl_xor(s, off);
    lse_merge(m, s, m2, s2);
  }
  __shared__ float sh_m[kWaves];
  __shared__ float sh_s[kWaves];
  __shared__ float sh_coef, sh_m_row, sh_off2, sh_c2, sh_dy;
  __shared__ bool sh_neg;
  if (lane == 0) {
    sh_m[wave] = m;
    sh_s[wave] = s;
  }
  __syncthreads();

  if (wave == 0) {
    // merge the kWaves wavefront partials in binary64
    const float mw = lane < kWaves ? sh_m[lane] : -INFINITY;
    const float sw = lane < kWaves ? sh_s[lane] : 0.0f;
    float M = mw;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    double term = 0.0;
    if (lane < kWaves && sw != 0.0f) term = (double)sw * exp2(((double)mw - (double)M) * kLog2eD);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) term += __shfl_xor(term, off);
    const double lse = (double)M + log(term);
    float xy;
    {
      float f[VEC];
      IO::unpack(xy_chunk, f);
      const int ey = (int)(y % VEC);
      xy = f[0];
#pragma unroll
      for (int e = 1; e < VEC; ++e) xy = e == ey ? f[e] : xy;
    }
    const double logp = (double)xy - lse;
    if (kFwdOnly) {
      if (lane == 0) a.out_logp[row] = (float)logp;
    } else if (lane == 0) {
      const double div = row_divisor(a.agg, a.kappa, a.len[i], a.total_len);
      const TokenTerms tt = token_terms(logp, old, ref, A, a.eps, a.beta, div);
      const double lam = tt.lam;
      const double coef = tt.coef;
      a.tok_loss[row] = lam / div;
      a.tok_flags[row] = tt.flags;
      if (a.aux_logp) a.aux_logp[row] = (float)logp;
      if (a.aux_tok_loss) a.aux_tok_loss[row] = (float)lam;
      sh_coef = (float)coef;
      sh_neg = coef < 0.0;
      sh_m_row = M;
      sh_off2 = (float)(log2(term) - log2(fabs(coef)));
      sh_c2 = (float)(log2(fabs(coef)) - log2(term) - (double)M * (double)kLog2e);
      sh_dy = (float)(coef * expm1(logp));
    }
  }
  if (kFwdOnly) return;
  __syncthreads();

  // ---- pass 2: dlogits = coef * (softmax - onehot)
  const float coef = sh_coef;
  if (coef == 0.0f) {  // the clip cut the only gradient term: an exact zero row
    const typename IO::chunk zero = IO::splat(0.0f);
    for (uint32_t c = tid; c < nchunks; c += NT) IO::store(out, c, zero);
    return;
  }
  write_dlogits<IO, VEC, NT>(buf, in, out, nchunks, ntiles, tid, sh_m_row, sh_off2, sh_c2, sh_dy,
                         sh_neg, y);
}


// Row plan of the ticket order for 256 or more completions (the row kernel
// forms it itself below that), one workgroup: zeroes the two ticket
// counters and writes P[i] = sum over completions j < i of their active rows
// (len_j when adv_j != 0 or beta != 0, else 0), i = 0..N; with total_len
// non-null also the batch's counted tokens (sum of len) for the token mean.
// Integer sums: exact, order-free.
__global__ void __launch_bounds__(1024)
k_plan(const int32_t* __restrict__ len, const float* __restrict__ adv, float beta, int64_t N,
       uint32_t* __restrict__ plan, int64_t* __restrict__ total_len) {
  __shared__ uint32_t sh_w[16];
  __shared__ long long sh_l[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t* P = plan + kPlanPrefix;
  if (tid == 0) {
    plan[kPlanActive] = 0u;
    plan[kPlanZero] = 0u;
  }
  uint32_t carry = 0;  // at most T < 2^31
  long long lsum = 0;
  for (int64_t base = 0; base < N; base += 1024) {
    const int64_t i = base + tid;
    uint32_t v = 0;
    if (i < N) {
      const int32_t L = len[i];
      lsum += L;
      v = (adv[i] != 0.0f || beta != 0.0f) ? (uint32_t)L : 0u;
    }
    uint32_t x = v;  // inclusive scan over the wavefront
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) sh_w[wave] = x;
    __syncthreads();
    uint32_t before = 0, chunk = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const uint32_t sw = sh_w[w];
      before += w < wave ? sw : 0u;
      chunk += sw;
    }
    if (i < N) P[i] = carry + before + x - v;
    carry += chunk;
    __syncthreads();  // sh_w is rewritten by the next chunk
  }
  if (tid == 0) P[N] = carry;
  if (total_len) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) lsum += __shfl_xor(lsum, off);
    if (lane == 0) sh_l[wave] = lsum;
    __syncthreads();
    if (tid == 0) {
      long long t = 0;
      for (int w = 0; w < 16; ++w) t += sh_l[w];
      *total_len = (int64_t)t;
    }
  }
}

uint64_t gcd_u64(uint64_t a, uint64_t b) {
  while (b) {
    const uint64_t r = a % b;
    a = b;
    b = r;
  }
  return a;
}

// A stride coprime with T near T/phi^2 (Fibonacci hashing): every run of
// consecutive workgroups, the ~256 in flight at once included, then samples
// the batch evenly, so each resident set mixes active and zero rows in the
// batch's proportion whatever the batch size.  Against T/256 + 1 it measured
// 2.3% faster at T = 131,072 and 0.8% at 65,536, even at 16,384 and on an
// all-active batch; fixed strides swung from -2.5% to +24% with T.
uint32_t row_stride_for(int64_t T) {
  uint64_t s = (uint64_t)((double)T * 0.3819660112501051) | 1u;
  while (gcd_u64(s, (uint64_t)T) != 1) ++s;
  return (uint32_t)s;
}

// Rows move in 16-byte chunks when their byte size is a multiple of 16 and
// both bases are 16-byte aligned (dlogits NULL: the forward-only pass).
bool vector_path(const void* logits, const void* dlogits, int64_t V, drgrpo_dtype_t dtype) {
  const size_t esz = dtype == DRGRPO_BF16 ? 2 : 4;
  return ((size_t)V * esz) % 16 == 0 && reinterpret_cast<uintptr_t>(logits) % 16 == 0 &&
         reinterpret_cast<uintptr_t>(dlogits) % 16 == 0;
}

// 256 threads when their register tile holds the whole row, else 1024.
bool rows_fit_256(int64_t V, drgrpo_dtype_t dtype, bool vec) {
  const int64_t nch = V / (dtype == DRGRPO_BF16 ? (vec ? 8 : 1) : (vec ? 4 : 1));
  return nch <= (int64_t)kNch * 256;
}

// The ticket order pays from rows of about 192 KB: a shorter-lived workgroup
// spends relatively more on its start (the class, the prefix, the atomic).
// k_rows on the B=8, G=8, C=256 batch (30% active rows / all active):
// 128 KB rows 0.49 / 0.95 ms in the stride order against 0.58 / 0.97 in the
// ticket order, 160 KB 0.58 / 1.12 against 0.65 / 1.11, 195 KB 0.75 / 1.39
// against 0.74 / 1.30, 297 KB 1.16 / 2.05 against 1.03 / 1.82.
constexpr int64_t kTicketMinRowBytes = 196608;

// whether the loss's rows go by the ticket order (1024-thread rows of at
// least kTicketMinRowBytes)
bool rows_ticketed(int64_t V, drgrpo_dtype_t dtype, bool vec) {
  return !rows_fit_256(V, dtype, vec) &&
         V * (dtype == DRGRPO_BF16 ? 2 : 4) >= kTicketMinRowBytes;
}

// k_rows over T rows.  The loss's kernels in the ticket order need a.plan
// written by k_plan, or its counters zeroed by k_prep, earlier on the same
// stream.
template <bool kFwdOnly>
int launch_rows(RowArgs a, int64_t T, drgrpo_dtype_t dtype, hipStream_t st,
                hipEvent_t ev_begin = nullptr, hipEvent_t ev_end = nullptr) {
  a.T = (uint32_t)T;
  a.N = (uint32_t)(T / a.C);
  a.row_stride = row_stride_for(T);
  const bool vec = vector_path(a.logits, kFwdOnly ? nullptr : a.dlogits, a.V, dtype);
  const dim3 grid((unsigned)T);
  auto go = [&](auto kernel, int nt) {
    const dim3 block((unsigned)nt);
    if (ev_begin || ev_end)  // events stamped by the dispatch itself
      hipExtLaunchKernelGGL(kernel, grid, block, 0, st, ev_begin, ev_end, 0, a);
    else
      hipLaunchKernelGGL(kernel, grid, block, 0, st, a);
  };
  const bool small = rows_fit_256(a.V, dtype, vec);
  const bool ticket = !kFwdOnly && rows_ticketed(a.V, dtype, vec);
  if (ticket && !a.plan) return DRGRPO_ERR_PARAM;
  auto pick = [&](auto k256, auto k1024, auto k1024_ticket) {
    if (small)
      go(k256, 256);
    else if (ticket)
      go(k1024_ticket, kThreads);
    else
      go(k1024, kThreads);
  };
  constexpr bool F = kFwdOnly;
  if (dtype == DRGRPO_BF16) {
    if (vec)
      pick(k_rows<DRGRPO_BF16, 8, F, 256>, k_rows<DRGRPO_BF16, 8, F, kThreads>,
           k_rows<DRGRPO_BF16, 8, F, kThreads, !F>);
    else
      pick(k_rows<DRGRPO_BF16, 1, F, 256>, k_rows<DRGRPO_BF16, 1, F, kThreads>,
           k_rows<DRGRPO_BF16, 1, F, kThreads, !F>);
  } else {
    if (vec)
      pick(k_rows<DRGRPO_F32, 4, F, 256>, k_rows<DRGRPO_F32, 4, F, kThreads>,
           k_rows<DRGRPO_F32, 4, F, kThreads, !F>);
    else
      pick(k_rows<DRGRPO_F32, 1, F, 256>, k_rows<DRGRPO_F32, 1, F, kThreads>,
           k_rows<DRGRPO_F32, 1, F, kThreads, !F>);
  }
  return launch_status();
}

int check_shape(int64_t N, int64_t C, int64_t V, int64_t G, int64_t* T, int64_t* elems) {
  if (N <= 0 || C <= 0 || V <= 0 || G <= 0 || N % G != 0) return DRGRPO_ERR_SHAPE;
  if (V > (int64_t(1) << 28)) return DRGRPO_ERR_SHAPE;  // per-row offsets are 32-bit
  if (!mul_ok(N, C, T)) return DRGRPO_ERR_SHAPE;
  if (*T > INT32_MAX) return DRGRPO_ERR_SHAPE;  // one workgroup per token row
  // and a dispatch holds fewer than 2^32 work-items: T x 256 threads when a
  // 256-thread register tile holds every row whatever the path (V up to
  // kNch * 256 elements), else T x 1024
  const int64_t nt_max = V <= (int64_t)kNch * 256 ? 256 : kThreads;
  if (*T > (int64_t)UINT32_MAX / nt_max) return DRGRPO_ERR_SHAPE;
  if (!mul_ok(*T, V, elems)) return DRGRPO_ERR_SHAPE;
  int64_t bytes;
  if (!mul_ok(*elems, 4, &bytes)) return DRGRPO_ERR_SHAPE;
  return DRGRPO_OK;
}

}  // namespace

// ====================================================================== C ABI
extern "C" size_t drgrpo_workspace_bytes(int64_t N, int64_t C, int64_t V, int64_t G) {
  int64_t T, elems;
  if (check_shape(N, C, V, G, &T, &elems) != DRGRPO_OK) return 0;
  return ws_carve(nullptr, N, T, nullptr);
}

namespace {

// Host-side argument checks of the loss calls (everything but the workspace
// and the overlap of dlogits with logits, which come after it), before
// anything is enqueued.  On success *T and *elems hold N*C and N*C*V.
int check_loss_args(const void* logits, const int64_t* tokens, const float* rewards,
                    const float* logp_old, const float* logp_ref, int64_t G, float eps,
                    float beta, float norm_const, const float* out_loss, const void* out_dlogits,
                    int64_t N, int64_t C, int64_t V, drgrpo_dtype_t dtype,
                    const drgrpo_variant_t* variant, int64_t* T, int64_t* elems) {
  if (!logits || !tokens || !rewards || !logp_old || !out_loss || !out_dlogits)
    return DRGRPO_ERR_NULL;
  if (dtype != DRGRPO_F32 && dtype != DRGRPO_BF16) return DRGRPO_ERR_DTYPE;
  const int sh = check_shape(N, C, V, G, T, elems);
  if (sh != DRGRPO_OK) return sh;
  if (!finite_f(eps) || eps < 0.0f || !finite_f(beta) || beta < 0.0f || !finite_f(norm_const) ||
      norm_const <= 0.0f)
    return DRGRPO_ERR_PARAM;
  if (beta > 0.0f && !logp_ref) return DRGRPO_ERR_NULL;
  int adv_mode, agg;
  if (!read_variant(variant, &adv_mode, &agg)) return DRGRPO_ERR_PARAM;
  return DRGRPO_OK;
}

// out_dlogits is exactly logits (in place) or disjoint from it.
int check_alias(const void* logits, const void* out_dlogits, int64_t elems,
                drgrpo_dtype_t dtype) {
  const size_t esz = dtype == DRGRPO_BF16 ? 2 : 4;
  const uintptr_t lo = reinterpret_cast<uintptr_t>(logits);
  const uintptr_t dl = reinterpret_cast<uintptr_t>(out_dlogits);
  const uintptr_t nbytes = (uintptr_t)elems * esz;
  if (lo != dl && lo < dl + nbytes && dl < lo + nbytes) return DRGRPO_ERR_ALIAS;
  return DRGRPO_OK;
}

// The three launches of one loss call over a carved workspace (arguments
// already checked).
int enqueue_loss(const void* logits, const int64_t* tokens, int64_t eos_id, const float* rewards,
                 const float* logp_old, const float* logp_ref, int64_t G, float eps, float beta,
                 float norm_const, float* out_loss, void* out_dlogits, int64_t N, int64_t C,
                 int64_t V, int64_t T, drgrpo_dtype_t dtype, void* workspace, hipStream_t st,
                 const drgrpo_aux_t* aux, const drgrpo_loss_opts_t* opts) {
  const drgrpo_loss_opts_t no_opts = {};
  const drgrpo_loss_opts_t& o = opts ? *opts : no_opts;
  int adv_mode, agg;
  read_variant(o.variant, &adv_mode, &agg);
  Ws ws;
  ws_carve(workspace, N, T, &ws);
  const drgrpo_aux_t none = {};
  const drgrpo_aux_t& x = aux ? *aux : none;

  hipLaunchKernelGGL(k_prep, dim3((unsigned)N), dim3(64), 0, st, tokens, C, eos_id, rewards, G,
                     adv_mode, ws.len, ws.adv, ws.row_flags, x.len, x.mask, x.adv,
                     (int32_t*)nullptr, ws.plan);
  int rc = launch_status();
  if (rc != DRGRPO_OK) return rc;
  const bool ticket = rows_ticketed(V, dtype, vector_path(logits, out_dlogits, V, dtype));
  // the row kernel forms the prefix itself below 256 completions
  if ((ticket && N >= 256) || agg == DRGRPO_AGG_TOKEN_MEAN) {
    hipLaunchKernelGGL(k_plan, dim3(1), dim3(1024), 0, st, ws.len, ws.adv, beta, N, ws.plan,
                       agg == DRGRPO_AGG_TOKEN_MEAN ? ws.total_len : (int64_t*)nullptr);
    if ((rc = launch_status()) != DRGRPO_OK) return rc;
  }

  RowArgs a;
  a.logits = logits;
  a.dlogits = out_dlogits;
  a.tokens = tokens;
  a.logp_old = logp_old;
  a.logp_ref = logp_ref;
  a.len = ws.len;
  a.adv = ws.adv;
  a.C = C;
  a.V = V;
  a.eps = eps;
  a.beta = beta;
  a.kappa = (double)norm_const;
  a.agg = agg;
  a.total_len = ws.total_len;
  a.tok_loss = ws.tok_loss;
  a.tok_flags = ws.tok_flags;
  a.aux_logp = x.logp;
  a.aux_tok_loss = x.tok_loss;
  a.out_logp = nullptr;
  a.plan = ticket ? ws.plan : nullptr;
  rc = launch_rows<false>(a, T, dtype, st, static_cast<hipEvent_t>(o.rows_event_begin),
                         static_cast<hipEvent_t>(o.rows_event_end));
  if (rc != DRGRPO_OK) return rc;

  hipLaunchKernelGGL(k_finish, dim3(1), dim3(1024), 0, st, ws.tok_loss, ws.tok_flags, T,
                     ws.row_flags, ws.len, ws.adv, beta, N, out_loss, ws.status, x.stats,
                     o.token_counts);
  return launch_status();
}

}  // namespace

extern "C" int drgrpo_loss_fwd_bwd_opts(const void* logits, const int64_t* tokens,
                                        int64_t eos_id, const float* rewards,
                                        const float* logp_old, const float* logp_ref, int64_t G,
                                        float eps, float beta, float norm_const, float* out_loss,
                                        void* out_dlogits, int64_t N, int64_t C, int64_t V,
                                        drgrpo_dtype_t dtype, void* workspace,
                                        size_t workspace_bytes, void* stream,
                                        const drgrpo_aux_t* aux, const drgrpo_loss_opts_t* opts) {
  int64_t T, elems;
  const int rc = check_loss_args(logits, tokens, rewards, logp_old, logp_ref, G, eps, beta,
                                 norm_const, out_loss, out_dlogits, N, C, V, dtype,
                                 opts ? opts->variant : nullptr, &T, &elems);
  if (rc != DRGRPO_OK) return rc;
  if (!workspace || reinterpret_cast<uintptr_t>(workspace) % 256 != 0 ||
      workspace_bytes < ws_carve(nullptr, N, T, nullptr))
    return DRGRPO_ERR_WORKSPACE;
  if (check_alias(logits, out_dlogits, elems, dtype) != DRGRPO_OK) return DRGRPO_ERR_ALIAS;
  if (opts && opts->require_vector_path && !vector_path(logits, out_dlogits, V, dtype))
    return DRGRPO_ERR_ALIGN;
  return enqueue_loss(logits, tokens, eos_id, rewards, logp_old, logp_ref, G, eps, beta,
                      norm_const, out_loss, out_dlogits, N, C, V, T, dtype, workspace,
                      static_cast<hipStream_t>(stream), aux, opts);
}

extern "C" int drgrpo_loss_fwd_bwd_ex(const void* logits, const int64_t* tokens, int64_t eos_id,
                                      const float* rewards, const float* logp_old,
                                      const float* logp_ref, int64_t G, float eps, float beta,
                                      float norm_const, float* out_loss, void* out_dlogits,
                                      int64_t N, int64_t C, int64_t V, drgrpo_dtype_t dtype,
                                      void* workspace, size_t workspace_bytes, void* stream,
                                      const drgrpo_aux_t* aux) {
  return drgrpo_loss_fwd_bwd_opts(logits, tokens, eos_id, rewards, logp_old, logp_ref, G, eps,
                                  beta, norm_const, out_loss, out_dlogits, N, C, V, dtype,
                                  workspace, workspace_bytes, stream, aux, nullptr);
}

extern "C" int drgrpo_loss_fwd_bwd(const void* logits, const int64_t* tokens, int64_t eos_id,
                                   const float* rewards, const float* logp_old,
                                   const float* logp_ref, int64_t G, float eps, float beta,
                                   float norm_const, float* out_loss, void* out_dlogits,
                                   int64_t N, int64_t C, int64_t V, drgrpo_dtype_t dtype,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  return drgrpo_loss_fwd_bwd_opts(logits, tokens, eos_id, rewards, logp_old, logp_ref, G, eps,
                                  beta, norm_const, out_loss, out_dlogits, N, C, V, dtype,
                                  workspace, workspace_bytes, stream, nullptr, nullptr);
}

// ------------------------------------------------ no-allocation entry point
// The scratch of drgrpo_loss_fwd_bwd_noalloc: the same carve-up as a caller's
// workspace, in a static device array.  Every GPU the library runs on holds
// its own copy (at its own address) until the process ends.  In host code the
// name `scratch` is only a stand-in for the symbol: kernels and copies get the
// address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[DRGRPO_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, looked up once per device.
int current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DRGRPO_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DRGRPO_ERR_HIP;
    if (reinterpret_cast<uintptr_t>(p) % 256 != 0) return DRGRPO_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DRGRPO_OK;
}

}  // namespace

extern "C" int drgrpo_loss_fwd_bwd_noalloc(const void* logits, const int64_t* tokens,
                                           int64_t eos_id, const float* rewards,
                                           const float* logp_old, const float* logp_ref,
                                           int64_t G, float eps, float beta, float norm_const,
                                           float* out_loss, void* out_dlogits, int64_t N,
                                           int64_t C, int64_t V, drgrpo_dtype_t dtype,
                                           void* stream) {
  int64_t T, elems;
  int rc = check_loss_args(logits, tokens, rewards, logp_old, logp_ref, G, eps, beta, norm_const,
                           out_loss, out_dlogits, N, C, V, dtype, nullptr, &T, &elems);
  if (rc != DRGRPO_OK) return rc;
  if (ws_carve(nullptr, N, T, nullptr) > (size_t)DRGRPO_NOALLOC_SCRATCH_BYTES)
    return DRGRPO_ERR_SCRATCH_LIMIT;
  if (check_alias(logits, out_dlogits, elems, dtype) != DRGRPO_OK) return DRGRPO_ERR_ALIAS;
  void* ws = nullptr;
  if ((rc = current_scratch(&ws)) != DRGRPO_OK) return rc;
  // every scratch field is written before it is read within the call, so the
  // previous call's contents need no clearing
  return enqueue_loss(logits, tokens, eos_id, rewards, logp_old, logp_ref, G, eps, beta,
                      norm_const, out_loss, out_dlogits, N, C, V, T, dtype, ws,
                      static_cast<hipStream_t>(stream), nullptr, nullptr);
}

extern "C" int drgrpo_completion_mask(const int64_t* tokens, int64_t N, int64_t C,
                                      int64_t eos_id, int32_t* out_len, uint8_t* out_mask,
                                      void* stream) {
  if (!tokens || !out_len) return DRGRPO_ERR_NULL;
  int64_t T;
  if (N <= 0 || C <= 0 || !mul_ok(N, C, &T) || N > INT32_MAX) return DRGRPO_ERR_SHAPE;
  hipLaunchKernelGGL(k_prep, dim3((unsigned)N), dim3(64), 0, static_cast<hipStream_t>(stream),
                     tokens, C, eos_id, (const float*)nullptr, (int64_t)1, 0, (int32_t*)nullptr,
                     (float*)nullptr, (uint8_t*)nullptr, out_len, out_mask, (float*)nullptr,
                     (int32_t*)nullptr, (uint32_t*)nullptr);
  return launch_status();
}

extern "C" int drgrpo_group_advantage_ex(const float* rewards, int64_t N, int64_t G,
                                         int32_t adv_mode, float* out_adv,
                                         int32_t* out_nocontrast, void* stream) {
  if (!rewards || !out_adv) return DRGRPO_ERR_NULL;
  if (N <= 0 || G <= 0 || N % G != 0 || N > INT32_MAX) return DRGRPO_ERR_SHAPE;
  if (adv_mode != DRGRPO_ADV_CENTER && adv_mode != DRGRPO_ADV_ZSCORE) return DRGRPO_ERR_PARAM;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (out_nocontrast) {
    hipLaunchKernelGGL(k_zero_i32, dim3(1), dim3(1), 0, st, out_nocontrast);
    const int rc = launch_status();
    if (rc != DRGRPO_OK) return rc;
  }
  hipLaunchKernelGGL(k_prep, dim3((unsigned)N), dim3(64), 0, st, (const int64_t*)nullptr,
                     (int64_t)1, (int64_t)0, rewards, G, (int)adv_mode, (int32_t*)nullptr,
                     (float*)nullptr,
                     (uint8_t*)nullptr, (int32_t*)nullptr, (uint8_t*)nullptr, out_adv,
                     out_nocontrast, (uint32_t*)nullptr);
  return launch_status();
}

extern "C" int drgrpo_group_advantage(const float* rewards, int64_t N, int64_t G,
                                      float* out_adv, int32_t* out_nocontrast, void* stream) {
  return drgrpo_group_advantage_ex(rewards, N, G, DRGRPO_ADV_CENTER, out_adv, out_nocontrast,
                                   stream);
}

extern "C" int drgrpo_logprobs(const void* logits, const int64_t* tokens, int64_t N, int64_t C,
                               int64_t V, drgrpo_dtype_t dtype, float* out_logp, void* stream) {
  if (!logits || !tokens || !out_logp) return DRGRPO_ERR_NULL;
  if (dtype != DRGRPO_F32 && dtype != DRGRPO_BF16) return DRGRPO_ERR_DTYPE;
  int64_t T, elems;
  const int sh = check_shape(N, C, V, 1, &T, &elems);
  if (sh != DRGRPO_OK) return sh;
  RowArgs a = {};
  a.logits = logits;
  a.tokens = tokens;
  a.C = C;
  a.V = V;
  a.kappa = 1.0;
  a.out_logp = out_logp;
  return launch_rows<true>(a, T, dtype, static_cast<hipStream_t>(stream));
}

extern "C" int drgrpo_device_status(const void* workspace, void* stream) {
  if (!workspace) return DRGRPO_ERR_NULL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(st) != hipSuccess) return DRGRPO_ERR_HIP;
  int32_t word = 0;
  if (hipMemcpy(&word, workspace, sizeof word, hipMemcpyDeviceToHost) != hipSuccess)
    return DRGRPO_ERR_HIP;
  return word & kStatusTokenRange ? DRGRPO_ERR_TOKEN_RANGE : DRGRPO_OK;
}

extern "C" const char* drgrpo_status_string(int status) {
  switch (status) {
    case DRGRPO_OK: return "ok";
    case DRGRPO_ERR_NULL: return "a required pointer is NULL";
    case DRGRPO_ERR_SHAPE: return "invalid shape (N, C, V, G must be > 0, N % G == 0, sizes in range)";
    case DRGRPO_ERR_PARAM: return "invalid parameter (eps, beta finite and >= 0; norm_const finite and > 0)";
    case DRGRPO_ERR_DTYPE: return "unknown element type";
    case DRGRPO_ERR_WORKSPACE: return "workspace NULL, too small or not 256-byte aligned";
    case DRGRPO_ERR_ALIAS: return "out_dlogits partially overlaps logits";
    case DRGRPO_ERR_HIP: return "HIP launch or runtime error";
    case DRGRPO_ERR_TOKEN_RANGE: return "a token at a mask=1 position is outside [0, V)";
    case DRGRPO_ERR_ALIGN: return "a pointer lacks the alignment the call requires";
    case DRGRPO_ERR_SCRATCH_LIMIT:
      return "sizes exceed the static scratch of drgrpo_loss_fwd_bwd_noalloc";
    default: return "unknown status";
  }
}
