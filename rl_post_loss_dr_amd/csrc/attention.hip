/*
 * attention.hip - decode attention of the rollout step for gfx950: one new
 * query token per sequence against its KV cache, grouped-query heads.
 *
 * "Making Dr GRPO go brrr", section "What is RL post-training, and why is it
 * slow": the rollout runs one forward pass per generated token on a
 * (B*G, 1, hidden) input plus a growing KV cache; this is the attention of
 * that step (the scaled dot-product attention it replaces).  For sequence s,
 * query head h and its key/value head g = h / (Hq / Hkv):
 *
 *   x_j = scale * <q[s,h], K[s,g,j]>  (j < len_s),   o = sum_j softmax(x)_j V[s,g,j]
 *
 * The step is bound by reading the cache once (bfloat16 K and V) and, at
 * the sizes of a rollout, by the latency of that read, so a workgroup issues
 * all of its loads at once:
 *   k_attn_fused    a workgroup of 8 (or 16) wavefronts per (sequence,
 *                   key/value head, split of the cached positions); each
 *                   wavefront takes 32 positions per round, forms the scores
 *                   of every query head of the group and the weighted values
 *                   on MFMAs (details at the kernel) and keeps an online
 *                   softmax; the partials are merged in LDS.  With one split
 *                   (the usual decode batch) it writes the bfloat16 output
 *                   and the log-sum-exp itself; otherwise a partial
 *                   (unnormalised output, max, sum of exp) per split.  The
 *                   launch plan (attn_plan) picks the wavefront count and
 *                   the splits.
 *   k_attn_combine  merges the splits of each (sequence, query head) in
 *                   split order and writes the output and the log-sum-exp.
 *   k_rope_append   (drgrpo_decode_attention_rope) the step's attention
 *                   block before those: rotary embedding of the new token's
 *                   query and key heads from the q/k/v projection output and
 *                   the append of its key and value to the cache, one
 *                   workgroup per sequence.
 */
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "drgrpo.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

constexpr int kManyPairs = 512;                  // (sequence, KV head) pairs that fill the chip
constexpr int kGroupsPerSplit = 4;               // load groups per split when pairs are many
constexpr int kWaveKeys = 32;                    // cached positions per wavefront and round
constexpr int kMaxGroup = 16;                    // query heads per key/value head (one MFMA block)
constexpr int kTargetBlocks = 128;               // split workgroups aimed for
constexpr int kMaxSplit = 32;                    // splits of the cached positions at most
constexpr float kLog2eA = 1.4426950408889634f;

__device__ inline float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ inline uint16_t to_bf16(float x) {
  const __bf16 h = (__bf16)x;  // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

// Wavefront-wide max / sum: four DPP steps inside each 16-lane row (quad
// swaps, half-row and row mirrors: every lane ends with its row's value),
// then the four row values read as scalars.  Cheaper than LDS-routed
// shuffles on this serial path.
template <int CTRL>
__device__ inline float dpp_a(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ inline float row4(float v, int lane_of_row) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane_of_row));
}
__device__ inline float wave_max(float v) {
  v = fmaxf(v, dpp_a<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_a<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_a<0x141>(v));  // row half-mirror
  v = fmaxf(v, dpp_a<0x140>(v));  // row mirror
  return fmaxf(fmaxf(row4(v, 0), row4(v, 16)), fmaxf(row4(v, 32), row4(v, 48)));
}
__device__ inline float wave_sum(float v) {
  v += dpp_a<0xB1>(v);
  v += dpp_a<0x4E>(v);
  v += dpp_a<0x141>(v);
  v += dpp_a<0x140>(v);
  return (row4(v, 0) + row4(v, 16)) + (row4(v, 32) + row4(v, 48));
}

struct AttnArgs {
  const uint16_t* q;    // [S, Hq, D]
  const uint16_t* k;    // [S, Hkv, Lmax, D]
  const uint16_t* v;    // [S, Hkv, Lmax, D]
  const int32_t* lens;  // [S]
  int64_t S, Hq, Hkv, Lmax;
  float scale;
  int nsplit;           // splits of the cached positions
  int chunk;            // positions per split (a multiple of kWaveKeys)
  float* part;          // [S, Hq, nsplit, D + 2]: unnormalised output, max, sum of exp
  uint16_t* out;        // [S, Hq, D]
  float* out_lse;       // [S, Hq] or NULL
};

// cached length of sequence s, clamped to [0, Lmax]
__device__ inline int seq_len(const AttnArgs& a, int64_t s) {
  const int32_t L = a.lens[s];
  return L < 0 ? 0 : (L > a.Lmax ? (int)a.Lmax : (int)L);
}

template <int D>
__device__ inline int vswz(int key) {
  // 16-byte chunk permutation of a cached value row in LDS: the transposing
  // reads (4 keys x 2 chunks per 16-lane group, 32 lanes per LDS pass) then
  // touch every bank once
  return D == 128 ? 2 * (key & 7) : 2 * ((key >> 1) & 3);
}

template <int D>
constexpr int attn_rounds() { return D == 64 ? 2 : 1; }  // value slots per wavefront in LDS

// One workgroup of NW wavefronts (8 or 16) per (sequence, key/value head,
// split of the cached positions); wavefront w takes positions
// j0 + w*32 + 32*NW*n .. +31 for rounds n = 0, 1, ...  The loads of
// attn_rounds<D>() rounds (64 positions per wavefront at D = 64, 32 at
// D = 128) are issued together, so a load group costs one round trip to
// memory.  Per round of 32 positions a wavefront
//   - loads its keys straight into MFMA operands and forms the transposed
//     scores S^T = K Q^T for all query heads of the group (v_mfma_f32_16x16x32_bf16:
//     16 positions x 16 heads per block, binary32 accumulation of exact
//     bf16 products; the scale is applied to the binary32 scores),
//   - updates an online softmax per head: in S^T's accumulator layout a lane
//     holds 8 positions of one head, so a head's max and sum take two
//     cross-lane exchanges,
//   - forms O^T += V^T P^T: the weights' registers are the B operand as they
//     stand, because the 32 reduction slots may enumerate the positions in any
//     order as long as both operands agree; the values reach LDS through
//     direct loads and come back as the A operand through transposing LDS
//     reads in that same order.  P is split into bfloat16 high and low parts
//     (two MFMAs), so the weights keep about 17 bits.
// The NW partial softmaxes are merged through LDS at the end.
template <int D, int NW>
__global__ void __launch_bounds__(64 * NW) k_attn_fused(AttnArgs a) {
  constexpr int kAttnWaves = NW;
  constexpr int kAttnThreads = 64 * NW;
  static_assert(D == 64 || D == 128, "head size");
  constexpr int NCH = D / 8;                     // 16-byte chunks per cached row
  constexpr int NST = D / 32;                    // MFMA steps of one score block
  constexpr int NCB = D / 16;                    // 16-column blocks of the output
  constexpr int VW = kWaveKeys * D;              // bfloat16 of values per wavefront and round
  constexpr int kDma = VW / 8 / 64;              // 16-byte direct loads per lane and round
  constexpr int NR = attn_rounds<D>();           // rounds whose loads are issued together
  static_assert(NR * kAttnWaves * VW * 2 >= kAttnWaves * 16 * D * 4, "merge area fits the value area");
  __shared__ __attribute__((aligned(16))) uint16_t sv[NR * kAttnWaves * VW];
  __shared__ float sm[kAttnWaves][16], sl[kAttnWaves][16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g16 = lane >> 4, li = lane & 15;
  const int grp = (int)(a.Hq / a.Hkv);
  const int64_t b = blockIdx.x;
  const int split = (int)(b % a.nsplit);
  const int64_t sg = b / a.nsplit;  // (sequence, key/value head)
  const int64_t s = sg / a.Hkv;
  const int64_t g = sg - s * a.Hkv;
  const int L = seq_len(a, s);
  const int j0 = split * a.chunk;
  const int j1 = min(L, j0 + a.chunk);

  // queries, the B operand of S^T: lane (head li, dims 32*st + 8*g16 .. +7)
  bf16x8 qf[NST];
#pragma unroll
  for (int st = 0; st < NST; ++st) {
    u32x4 w = u32x4{0u, 0u, 0u, 0u};
    if (li < grp) w = *reinterpret_cast<const u32x4*>(a.q + (s * a.Hq + g * grp + li) * D + 32 * st + 8 * g16);
    qf[st] = __builtin_bit_cast(bf16x8, w);
  }

  const int64_t cache_off = (s * a.Hkv + g) * a.Lmax * D;
  const uint16_t* kb = a.k + cache_off;
  const auto vrsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.v + cache_off), 0,
                                                       (int)(a.Lmax * D * 2), 0x00020000);
  float m_run = -INFINITY, l_run = 0.0f;  // head li
  f32x4 o[NCB];                            // O^T[16*cb + 4*g16 + r][head li]
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) o[cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  constexpr int kRoundKeys = kAttnWaves * kWaveKeys;
  for (int base = j0 + wv * kWaveKeys; base < j1; base += NR * kRoundKeys) {
    // issue every load of these rounds: values into this wavefront's LDS slot
    // of the round (lane slot e of direct load p holds chunk (e % NCH) ^
    // vswz(key) of position key = e / NCH of the round), keys straight into
    // the A operands of S^T (lane: position 16*bk + li, dims 32*st + 8*g16 ..)
    bf16x8 kf[NR][2][NST];
#pragma unroll
    for (int n = 0; n < NR; ++n) {
      const int r0 = base + n * kRoundKeys;
      if (r0 >= j1) break;  // uniform across the wavefront
      const int klast = min(kWaveKeys, j1 - r0) - 1 + r0;  // later positions re-read it (weight 0)
      uint16_t* slot = sv + (n * kAttnWaves + wv) * VW;
#pragma unroll
      for (int p = 0; p < kDma; ++p) {
        const int e = 64 * p + lane;
        const int key = e / NCH;
        const int c = (e % NCH) ^ vswz<D>(key);
        const int kk = min(r0 + key, klast);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            vrsrc, (__attribute__((address_space(3))) void*)(slot + 64 * 8 * p), 16,
            (uint32_t)((kk * D + 8 * c) * 2), 0, 0, 0);
      }
#pragma unroll
      for (int bk = 0; bk < 2; ++bk) {
        const int kk = min(r0 + 16 * bk + li, klast);
#pragma unroll
        for (int st = 0; st < NST; ++st)
          kf[n][bk][st] = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(kb + (int64_t)kk * D + 32 * st + 8 * g16));
      }
    }
    // every value of these rounds has landed in this wavefront's LDS slots
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    asm volatile("" ::: "memory");
#pragma unroll
    for (int n = 0; n < NR; ++n) {
      const int r0 = base + n * kRoundKeys;
      if (r0 >= j1) break;
      const int nk = min(kWaveKeys, j1 - r0);  // >= 1
      const uint16_t* slot = sv + (n * kAttnWaves + wv) * VW;
      f32x4 sc[2];
#pragma unroll
      for (int bk = 0; bk < 2; ++bk) {
        sc[bk] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int st = 0; st < NST; ++st)
          sc[bk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[n][bk][st], qf[st], sc[bk], 0, 0, 0);
      }
      // lane holds positions 16*bk + 4*g16 + r of head li
      float x[8];
      float mx = -INFINITY;
#pragma unroll
      for (int bk = 0; bk < 2; ++bk)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = 16 * bk + 4 * g16 + r;
          x[4 * bk + r] = key < nk ? sc[bk][r] * a.scale : -INFINITY;
          mx = fmaxf(mx, x[4 * bk + r]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(m_run, mx);  // finite: position r0 is valid
      const float corr = m_run == -INFINITY ? 0.0f : exp2f((m_run - mn) * kLog2eA);
      float ps = 0.0f;
      bf16x8 phi, plo;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float pv = exp2f((x[i] - mn) * kLog2eA);  // exactly 0 past the round's end
        ps += pv;
        const __bf16 h = (__bf16)pv;
        phi[i] = h;
        plo[i] = (__bf16)(pv - (float)h);
      }
      ps += __shfl_xor(ps, 16);
      ps += __shfl_xor(ps, 32);
      l_run = fmaf(l_run, corr, ps);
      m_run = mn;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        // lane (4e + q) of a 16-lane group points at position k0 + e, columns
        // 16*cb + 4q .. +3; it receives positions k0 .. k0+3 of column 16*cb + li
        const int d = 16 * cb + 4 * (li & 3);
        const int k0a = 4 * g16 + (li >> 2), k0b = 16 + 4 * g16 + (li >> 2);
        const s16x4 ta = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(slot + (k0a * NCH + ((d >> 3) ^ vswz<D>(k0a))) * 8 + (d & 7)));
        const s16x4 tb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(slot + (k0b * NCH + ((d >> 3) ^ vswz<D>(k0b))) * 8 + (d & 7)));
        const bf16x8 va = __builtin_bit_cast(
            bf16x8, s16x8{ta[0], ta[1], ta[2], ta[3], tb[0], tb[1], tb[2], tb[3]});
        o[cb] *= corr;
        o[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, phi, o[cb], 0, 0, 0);
        o[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, plo, o[cb], 0, 0, 0);
      }
    }
    // the next group's direct loads overwrite the slots only after these
    // reads (their results feed the MFMAs above)
  }

  // merge the wavefronts' partial softmaxes; the value area is reused
  __syncthreads();
  float* so = reinterpret_cast<float*>(sv);  // [wave][head][D]
  if (g16 == 0) {
    sm[wv][li] = m_run;
    sl[wv][li] = l_run;
  }
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int r = 0; r < 4; ++r) so[(wv * 16 + li) * D + 16 * cb + 4 * g16 + r] = o[cb][r];
  __syncthreads();
  // thread t merges (head, column) pairs t, t + kAttnThreads, ... of the
  // 16 x D partial outputs
  const int64_t sh0 = s * a.Hq + g * grp;
  for (int idx = tid; idx < 16 * D; idx += kAttnThreads) {
    const int h = idx / D, c = idx % D;
    if (h >= grp) break;  // pairs are head-major: the rest belong to absent heads
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, sm[w][h]);
    float l = 0.0f, ov = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) {
        if (sm[w][h] == -INFINITY) continue;  // a wavefront without positions
        const float f = exp2f((sm[w][h] - M) * kLog2eA);
        l = fmaf(sl[w][h], f, l);
        ov = fmaf(so[(w * 16 + h) * D + c], f, ov);
      }
    }
    const int64_t sh = sh0 + h;
    if (a.nsplit == 1) {  // the whole cache in one split: normalise and write the output here
      const bool empty = M == -INFINITY;  // no cached key: an empty softmax
      a.out[sh * D + c] = to_bf16(empty ? NAN : ov / l);
      if (a.out_lse && c == 0) a.out_lse[sh] = empty ? NAN : M + logf(l);
    } else {  // partial of this split (an empty split: max -inf, sum 0)
      float* pp = a.part + (sh * a.nsplit + split) * (int64_t)(D + 2);
      pp[c] = ov;
      if (c == 0) {
        pp[D] = M;
        pp[D + 1] = l;
      }
    }
  }
}

// One workgroup per (sequence, key/value head, block of up to 1024 / D query
// heads of the group), a thread per (query head, column): merge the splits in
// split order.  Every partial a thread needs is loaded before any is used
// (one round trip to memory).  A separate launch, because publishing the
// partials across the XCDs' L2 caches inside one kernel would need a
// device-scope release per workgroup (an L2 write-back each), measured 10x
// slower than the second launch.
template <int D>
__global__ void __launch_bounds__(1024) k_attn_combine(AttnArgs a) {
  constexpr int kHeadsPerBlock = 1024 / D;
  const int grp = (int)(a.Hq / a.Hkv);
  const int nhb = (grp + kHeadsPerBlock - 1) / kHeadsPerBlock;
  const int64_t sg = blockIdx.x / nhb;  // s * Hkv + g
  const int h = (int)(blockIdx.x - sg * nhb) * kHeadsPerBlock + (int)(threadIdx.x / D);
  const int c = threadIdx.x % D;
  if (h >= grp) return;
  const int64_t sh = sg * grp + h;  // s * Hq + g * grp + h
  const int ns = a.nsplit;
  const float* pp = a.part + sh * ns * (D + 2);
  float mi[kMaxSplit], li[kMaxSplit], oi[kMaxSplit];
#pragma unroll
  for (int i = 0; i < kMaxSplit; ++i) {
    if (i < ns) {
      mi[i] = pp[i * (D + 2) + D];
      li[i] = pp[i * (D + 2) + D + 1];
      oi[i] = pp[i * (D + 2) + c];
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < kMaxSplit; ++i)
    if (i < ns) M = fmaxf(M, mi[i]);
  float o = 0.0f, l = 0.0f;
  if (M != -INFINITY) {
#pragma unroll
    for (int i = 0; i < kMaxSplit; ++i) {
      if (i < ns && mi[i] != -INFINITY) {  // an empty split contributes nothing
        const float w = exp2f((mi[i] - M) * kLog2eA);
        l = fmaf(li[i], w, l);
        o = fmaf(oi[i], w, o);
      }
    }
    o = o / l;
  } else {
    o = NAN;  // no cached key: the softmax is empty
  }
  a.out[sh * D + c] = to_bf16(o);
  if (a.out_lse && c == 0) a.out_lse[sh] = M != -INFINITY ? M + logf(l) : NAN;
}

int attn_launch_status() { return hipGetLastError() == hipSuccess ? DRGRPO_OK : DRGRPO_ERR_HIP; }

inline size_t attn_align(size_t x) { return (x + 255) & ~size_t(255); }  // 256-byte carve-up

template <int D>
void launch_combine(const AttnArgs& a, hipStream_t st) {
  constexpr int kHeadsPerBlock = 1024 / D;
  const int grp = (int)(a.Hq / a.Hkv);
  const int nhb = (grp + kHeadsPerBlock - 1) / kHeadsPerBlock;
  const int threads = (grp < kHeadsPerBlock ? grp : kHeadsPerBlock) * D;
  hipLaunchKernelGGL(k_attn_combine<D>, dim3((unsigned)(a.S * a.Hkv * nhb)), dim3(threads), 0,
                     st, a);
}

// Launch plan: 8-wavefront workgroups (two fit a CU, so one's loads overlap
// the other's products and merge), or 16 when that covers a cache of up to
// 1024 positions (D = 64) in one load group and there are few (sequence, KV
// head) pairs: a second launch (the combine) costs more than a bigger
// workgroup.  Positions per split: one load group, or kGroupsPerSplit of them
// when there are kManyPairs pairs anyway; at most kMaxSplit splits; more
// splits, down to 128 positions, while there are fewer than kTargetBlocks
// workgroups.
struct AttnPlan {
  int nw, nsplit, chunk;
};

AttnPlan attn_plan(int64_t S, int64_t Hkv, int64_t Lmax, int64_t D) {
  const int64_t pairs = S * Hkv;
  const int64_t per_wave = kWaveKeys * (D == 64 ? attn_rounds<64>() : attn_rounds<128>());
  AttnPlan p;
  p.nw = 8;
  if (D == 64 && pairs <= kTargetBlocks && Lmax > 8 * per_wave && Lmax <= 16 * per_wave) p.nw = 16;
  const int64_t group = p.nw * per_wave * (pairs >= kManyPairs ? kGroupsPerSplit : 1);
  int64_t ns = (Lmax + group - 1) / group;
  const int64_t ns_par = (kTargetBlocks + pairs - 1) / pairs;
  const int64_t ns_fine = (Lmax + 4 * kWaveKeys - 1) / (4 * kWaveKeys);
  const int64_t ns_more = ns_par < ns_fine ? ns_par : ns_fine;
  if (ns < ns_more) ns = ns_more;
  if (ns > kMaxSplit) ns = kMaxSplit;
  if (ns < 1) ns = 1;
  const int64_t per = ((Lmax + ns - 1) / ns + kWaveKeys - 1) / kWaveKeys * kWaveKeys;
  p.chunk = (int)per;
  p.nsplit = (int)((Lmax + per - 1) / per);
  return p;
}

int attn_check(int64_t S, int64_t Hq, int64_t Hkv, int64_t Lmax, int64_t D) {
  if (S <= 0 || Hq <= 0 || Hkv <= 0 || Lmax <= 0 || Hq % Hkv != 0 || Hq / Hkv > kMaxGroup)
    return DRGRPO_ERR_SHAPE;
  if (D != 64 && D != 128) return DRGRPO_ERR_SHAPE;
  // one (sequence, head) cache region is addressed with 32-bit byte offsets
  if (Lmax * D * 2 > INT32_MAX || S * Hkv > (int64_t(1) << 25) || S * Hq > INT32_MAX)
    return DRGRPO_ERR_SHAPE;
  return DRGRPO_OK;
}

// ------------------------------------------------- rotary embedding + append
// The attention block of the rollout step ("Making Dr GRPO go brrr", section
// "What is RL post-training, and why is it slow": one forward pass per
// generated token with a growing KV cache).  One workgroup per sequence: each
// query head vector of the projection output is rotated by the token's
// position into q_rot; each key head is rotated and written to the key cache
// at [s, g, pos_s]; each value head is copied to the value cache there;
// lens[s] = pos_s + 1.  Rotate-half form: pair i < D/2 is (x_i, x_{i+D/2})
// turned by the angle whose cosine and sine the tables hold, in binary32 with
// each product and the sum rounded separately (no fused steps), then rounded
// to bfloat16.  A position outside [0, Lmax) writes nothing, rotates the
// queries by angle 0 and gives lens = 0 (the attention output is then NaN).
template <int D>
__global__ void __launch_bounds__(256)
k_rope_append(const uint16_t* __restrict__ qkv, const float* __restrict__ rcos,
              const float* __restrict__ rsin, const int32_t* __restrict__ pos, int Hq, int Hkv,
              int64_t Lmax, uint16_t* __restrict__ q_rot, uint16_t* __restrict__ kc,
              uint16_t* __restrict__ vc, int32_t* __restrict__ lens) {
#pragma clang fp contract(off)
  constexpr int kHalf = D / 2;
  const int64_t s = blockIdx.x;
  const int32_t p = pos[s];
  const bool ok = p >= 0 && p < Lmax;
  const uint16_t* x = qkv + s * (Hq + 2 * Hkv) * D;
  if (threadIdx.x == 0) lens[s] = ok ? p + 1 : 0;
  for (int w = threadIdx.x; w < (Hq + Hkv) * kHalf; w += blockDim.x) {
    const int h = w / kHalf, i = w % kHalf;
    const float a = __uint_as_float((uint32_t)x[h * D + i] << 16);
    const float b = __uint_as_float((uint32_t)x[h * D + i + kHalf] << 16);
    const float c = ok ? rcos[p * kHalf + i] : 1.0f;
    const float sn = ok ? rsin[p * kHalf + i] : 0.0f;
    const float ac = a * c, bs = b * sn, bc = b * c, as = a * sn;
    const uint16_t lo = to_bf16(ac - bs), hi = to_bf16(bc + as);
    if (h < Hq) {
      uint16_t* dst = q_rot + (s * Hq + h) * D;
      dst[i] = lo;
      dst[i + kHalf] = hi;
    } else if (ok) {
      uint16_t* dst = kc + ((s * Hkv + (h - Hq)) * Lmax + p) * D;
      dst[i] = lo;
      dst[i + kHalf] = hi;
    }
  }
  if (ok) {
    for (int w = threadIdx.x; w < Hkv * D; w += blockDim.x) {
      const int g = w / D, e = w % D;
      vc[((s * Hkv + g) * Lmax + p) * D + e] = x[(Hq + Hkv + g) * D + e];
    }
  }
}

// The attention launches for checked arguments (plan, fused kernel, combine).
int attn_run(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* lens,
             int64_t S, int64_t Hq, int64_t Hkv, int64_t Lmax, int64_t D, float scale, float* part,
             uint16_t* out, float* out_lse, hipStream_t st) {
  AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.lens = lens;
  a.S = S;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Lmax = Lmax;
  a.scale = scale;
  const AttnPlan plan = attn_plan(S, Hkv, Lmax, D);
  a.nsplit = plan.nsplit;
  a.chunk = plan.chunk;
  a.part = part;
  a.out = out;
  a.out_lse = out_lse;
  const unsigned blocks = (unsigned)(S * Hkv * a.nsplit);
  if (D == 64 && plan.nw == 16)
    hipLaunchKernelGGL((k_attn_fused<64, 16>), dim3(blocks), dim3(64 * 16), 0, st, a);
  else if (D == 64)
    hipLaunchKernelGGL((k_attn_fused<64, 8>), dim3(blocks), dim3(64 * 8), 0, st, a);
  else
    hipLaunchKernelGGL((k_attn_fused<128, 8>), dim3(blocks), dim3(64 * 8), 0, st, a);
  if (attn_launch_status() != DRGRPO_OK) return DRGRPO_ERR_HIP;
  if (a.nsplit > 1) {
    if (D == 64)
      launch_combine<64>(a, st);
    else
      launch_combine<128>(a, st);
  }
  return attn_launch_status();
}

}  // namespace

// ====================================================================== C ABI
extern "C" size_t drgrpo_decode_attention_workspace_bytes(int64_t S, int64_t Hq, int64_t Hkv,
                                                          int64_t Lmax, int64_t D) {
  if (attn_check(S, Hq, Hkv, Lmax, D) != DRGRPO_OK) return 0;
  return (size_t)(S * Hq) * attn_plan(S, Hkv, Lmax, D).nsplit * (D + 2) * sizeof(float);
}

extern "C" int drgrpo_decode_attention(const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* lens, int64_t S, int64_t Hq, int64_t Hkv,
                                       int64_t Lmax, int64_t D, float scale, void* out,
                                       float* out_lse, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  if (!q || !k_cache || !v_cache || !lens || !out) return DRGRPO_ERR_NULL;
  const int sh = attn_check(S, Hq, Hkv, Lmax, D);
  if (sh != DRGRPO_OK) return sh;
  if (!(scale > 0.0f) || scale - scale != 0.0f) return DRGRPO_ERR_PARAM;
  const uintptr_t al = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_cache) |
                       reinterpret_cast<uintptr_t>(v_cache) | reinterpret_cast<uintptr_t>(out);
  if (al % 16 != 0) return DRGRPO_ERR_ALIGN;
  if (!workspace || reinterpret_cast<uintptr_t>(workspace) % 256 != 0 ||
      workspace_bytes < drgrpo_decode_attention_workspace_bytes(S, Hq, Hkv, Lmax, D))
    return DRGRPO_ERR_WORKSPACE;
  return attn_run(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
                  static_cast<const uint16_t*>(v_cache), lens, S, Hq, Hkv, Lmax, D, scale,
                  static_cast<float*>(workspace), static_cast<uint16_t*>(out), out_lse,
                  static_cast<hipStream_t>(stream));
}

extern "C" size_t drgrpo_decode_attention_rope_workspace_bytes(int64_t S, int64_t Hq, int64_t Hkv,
                                                               int64_t Lmax, int64_t D) {
  const size_t a = drgrpo_decode_attention_workspace_bytes(S, Hq, Hkv, Lmax, D);
  if (a == 0) return 0;
  return attn_align(a) + attn_align((size_t)(S * Hq * D) * 2) + attn_align((size_t)S * 4);
}

extern "C" int drgrpo_decode_attention_rope(const void* qkv, const float* rope_cos,
                                            const float* rope_sin, const int32_t* pos, int64_t S,
                                            int64_t Hq, int64_t Hkv, int64_t Lmax, int64_t D,
                                            float scale, void* k_cache, void* v_cache, void* out,
                                            float* out_lse, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  if (!qkv || !rope_cos || !rope_sin || !pos || !k_cache || !v_cache || !out)
    return DRGRPO_ERR_NULL;
  const int sh = attn_check(S, Hq, Hkv, Lmax, D);
  if (sh != DRGRPO_OK) return sh;
  if (!(scale > 0.0f) || scale - scale != 0.0f) return DRGRPO_ERR_PARAM;
  const uintptr_t al = reinterpret_cast<uintptr_t>(k_cache) |
                       reinterpret_cast<uintptr_t>(v_cache) | reinterpret_cast<uintptr_t>(out);
  if (al % 16 != 0 || reinterpret_cast<uintptr_t>(qkv) % 2 != 0) return DRGRPO_ERR_ALIGN;
  if (!workspace || reinterpret_cast<uintptr_t>(workspace) % 256 != 0 ||
      workspace_bytes < drgrpo_decode_attention_rope_workspace_bytes(S, Hq, Hkv, Lmax, D))
    return DRGRPO_ERR_WORKSPACE;
  char* w = static_cast<char*>(workspace);
  float* part = reinterpret_cast<float*>(w);
  w += attn_align(drgrpo_decode_attention_workspace_bytes(S, Hq, Hkv, Lmax, D));
  uint16_t* q_rot = reinterpret_cast<uint16_t*>(w);
  w += attn_align((size_t)(S * Hq * D) * 2);
  int32_t* lens = reinterpret_cast<int32_t*>(w);
  hipStream_t st = static_cast<hipStream_t>(stream);
  auto rope = D == 64 ? k_rope_append<64> : k_rope_append<128>;
  hipLaunchKernelGGL(rope, dim3((unsigned)S), dim3(256), 0, st, static_cast<const uint16_t*>(qkv),
                     rope_cos, rope_sin, pos, (int)Hq, (int)Hkv, Lmax, q_rot,
                     static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache), lens);
  if (attn_launch_status() != DRGRPO_OK) return DRGRPO_ERR_HIP;
  return attn_run(q_rot, static_cast<const uint16_t*>(k_cache),
                  static_cast<const uint16_t*>(v_cache), lens, S, Hq, Hkv, Lmax, D, scale, part,
                  static_cast<uint16_t*>(out), out_lse, st);
}
