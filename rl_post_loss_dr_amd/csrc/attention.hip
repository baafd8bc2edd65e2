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
 * The step is bound by reading the cache once (bfloat16 K and V), so the
 * work is split along the cached positions:
 *   k_attn_split    a 256-thread workgroup per (sequence, key/value head,
 *                   split of the cached positions).  Each K/V tile of 64
 *                   positions is read from HBM once with 16-byte loads (the
 *                   queries and the first tile requested together, the next
 *                   tile in flight while one is computed) into LDS and serves
 *                   every query head of the group.  A wavefront owns a fixed
 *                   set of query heads: as 64 keys (one per lane) it forms
 *                   binary32 scores and the online softmax state; as 64
 *                   head-dimension columns it accumulates the weighted values
 *                   (V is stored transposed in LDS, so a column's 64 keys are
 *                   eight 16-byte reads), so the rescale factors stay in its
 *                   registers and only the weights pass through LDS.  Writes
 *                   a partial (unnormalised output, max, sum of exp).
 *   k_attn_combine  merges the splits of each (sequence, query head) in
 *                   split order and writes the bfloat16 output and the
 *                   log-sum-exp.
 */
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "drgrpo.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kAttnThreads = 256;  // 4 wavefronts
constexpr int kTileKeys = 64;      // cached positions per LDS tile (one per lane)
constexpr int kMaxGroup = 16;      // query heads per key/value head
constexpr int kKeyPad = 8;         // bfloat16 of padding per K row in LDS (spreads banks)
constexpr int kTargetBlocks = 512;  // split workgroups aimed for (2 per CU; measured best)
constexpr int kMaxSplit = 32;      // splits of the cached positions at most
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
  int chunk;            // positions per split (a multiple of kTileKeys)
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
__global__ void __launch_bounds__(kAttnThreads) k_attn_split(AttnArgs a) {
  static_assert(D == 64 || D == 128, "head size");
  constexpr int KROW = D + kKeyPad;           // LDS row of one cached key
  constexpr int kWavesPerSet = D / 64;        // wavefronts sharing a head set (one per 64 columns)
  constexpr int kHeadStride = 4 / kWavesPerSet;
  constexpr int kSlots = kMaxGroup / kHeadStride;  // heads per wavefront at most
  __shared__ __attribute__((aligned(16))) float sq[kMaxGroup][D];  // scaled queries
  constexpr int VROW = kTileKeys + kKeyPad;   // LDS row of one value column (transposed tile)
  __shared__ __attribute__((aligned(16))) uint16_t sk[kTileKeys][KROW];
  __shared__ __attribute__((aligned(16))) uint16_t svt[D][VROW];
  __shared__ __attribute__((aligned(16))) float sp[kMaxGroup][kTileKeys];  // softmax weights

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = (int)(a.Hq / a.Hkv);
  const int64_t b = blockIdx.x;
  const int split = (int)(b % a.nsplit);
  const int64_t sg = b / a.nsplit;  // (sequence, key/value head)
  const int64_t s = sg / a.Hkv;
  const int64_t g = sg - s * a.Hkv;
  const int L = seq_len(a, s);
  const int j0 = split * a.chunk;
  const int j1 = min(L, j0 + a.chunk);

  // this wavefront's heads: h0, h0 + kHeadStride, ...; its value columns d
  const int h0 = wave / kWavesPerSet;
  const int d = (wave % kWavesPerSet) * 64 + lane;
  const bool writer = (wave % kWavesPerSet) == 0;  // one copy of the weights per head

  float m_run[kSlots], l_run[kSlots], acc[kSlots];
#pragma unroll
  for (int i = 0; i < kSlots; ++i) {
    m_run[i] = -INFINITY;
    l_run[i] = 0.0f;
    acc[i] = 0.0f;
  }

  const uint16_t* kbase = a.k + (s * a.Hkv + g) * a.Lmax * D;
  const uint16_t* vbase = a.v + (s * a.Hkv + g) * a.Lmax * D;
  constexpr int kVec = 8;  // bfloat16 per 16-byte load
  constexpr int kPer = kTileKeys * D / kVec / kAttnThreads;  // 16-byte loads per thread per tile
  // registers of one tile: thread slot e = tid + kAttnThreads * p covers key
  // r = e / (D / kVec), columns c .. c+7 with c = (e % (D / kVec)) * kVec;
  // positions past the tile's end are zero (their weights are 0 and must not
  // meet NaN bits)
  u32x4 kreg[kPer], vreg[kPer];
  auto load_tile = [&](int t0, int nk) {
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int e = tid + kAttnThreads * p;
      const int r = e / (D / kVec), c = (e - r * (D / kVec)) * kVec;
      kreg[p] = u32x4{0u, 0u, 0u, 0u};
      vreg[p] = u32x4{0u, 0u, 0u, 0u};
      if (r < nk) {
        const int64_t off = (int64_t)(t0 + r) * D + c;
        kreg[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + off));
        vreg[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vbase + off));
      }
    }
  };
  // the queries and the first tile are requested together
  constexpr int kQPer = (kMaxGroup * D + kAttnThreads - 1) / kAttnThreads;
  float qreg[kQPer];
#pragma unroll
  for (int p = 0; p < kQPer; ++p) {
    const int e = tid + kAttnThreads * p;
    qreg[p] = e < grp * D ? bf16f(a.q[(s * a.Hq + g * grp) * D + e]) * a.scale : 0.0f;
  }
  if (j0 < j1) load_tile(j0, min(kTileKeys, j1 - j0));
#pragma unroll
  for (int p = 0; p < kQPer; ++p) {
    const int e = tid + kAttnThreads * p;
    if (e < grp * D) sq[e / D][e % D] = qreg[p];
  }

  for (int t0 = j0; t0 < j1; t0 += kTileKeys) {
    const int nk = min(kTileKeys, j1 - t0);
    __syncthreads();  // the previous tile's K, V and weights are consumed (and sq is written)
    // K rows as they are; V transposed (column-major), so that the value
    // role reads a column's 64 keys as 16-byte vectors
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int e = tid + kAttnThreads * p;
      const int r = e / (D / kVec), c = (e - r * (D / kVec)) * kVec;
      *reinterpret_cast<u32x4*>(&sk[r][c]) = kreg[p];
      const uint32_t w[4] = {vreg[p].x, vreg[p].y, vreg[p].z, vreg[p].w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        svt[c + 2 * u][r] = (uint16_t)(w[u] & 0xFFFFu);
        svt[c + 2 * u + 1][r] = (uint16_t)(w[u] >> 16);
      }
    }
    __syncthreads();
    // the next tile's loads fly while this one is computed
    if (t0 + kTileKeys < j1) load_tile(t0 + kTileKeys, min(kTileKeys, j1 - t0 - kTileKeys));
    // scores of key `lane` for this wavefront's heads, online softmax
    float corr[kSlots];
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
      const int h = h0 + kHeadStride * i;
      corr[i] = 1.0f;
      if (h < grp) {  // uniform across the wavefront
        float x = -INFINITY;
        if (lane < nk) {
          float dot = 0.0f;
#pragma unroll
          for (int c = 0; c < D; c += kVec) {
            const u32x4 kk = *reinterpret_cast<const u32x4*>(&sk[lane][c]);
            const uint32_t w[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              dot = fmaf(sq[h][c + 2 * u], __uint_as_float(w[u] << 16), dot);
              dot = fmaf(sq[h][c + 2 * u + 1], __uint_as_float(w[u] & 0xFFFF0000u), dot);
            }
          }
          x = dot;
        }
        const float tm = wave_max(x);
        const float mn = fmaxf(m_run[i], tm);  // finite: the tile holds at least one key
        const float p = lane < nk ? exp2f((x - mn) * kLog2eA) : 0.0f;
        const float ps = wave_sum(p);
        corr[i] = m_run[i] == -INFINITY ? 0.0f : exp2f((m_run[i] - mn) * kLog2eA);
        l_run[i] = l_run[i] * corr[i] + ps;
        m_run[i] = mn;
        if (writer) sp[h][lane] = p;
      }
    }
    __syncthreads();  // weights visible
    // weighted values of column d for the same heads: the column's 64 keys
    // in eight 16-byte reads, the weights as broadcast 16-byte reads
    u32x4 vcol[kTileKeys / kVec];
#pragma unroll
    for (int c = 0; c < kTileKeys / kVec; ++c)
      vcol[c] = *reinterpret_cast<const u32x4*>(&svt[d][c * kVec]);
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
      const int h = h0 + kHeadStride * i;
      if (h < grp) {
        float o = acc[i] * corr[i];
#pragma unroll
        for (int c = 0; c < kTileKeys / kVec; ++c) {
          const float4 pa = *reinterpret_cast<const float4*>(&sp[h][c * kVec]);
          const float4 pb = *reinterpret_cast<const float4*>(&sp[h][c * kVec + 4]);
          const float pw[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
          const uint32_t w[4] = {vcol[c].x, vcol[c].y, vcol[c].z, vcol[c].w};
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            o = fmaf(pw[2 * u], __uint_as_float(w[u] << 16), o);
            o = fmaf(pw[2 * u + 1], __uint_as_float(w[u] & 0xFFFF0000u), o);
          }
        }
        acc[i] = o;
      }
    }
  }

  if (a.nsplit == 1) {  // the whole cache in one split: normalise and write the output here
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
      const int h = h0 + kHeadStride * i;
      if (h < grp) {
        const int64_t sh = s * a.Hq + g * grp + h;
        const bool empty = m_run[i] == -INFINITY;  // no cached key: an empty softmax
        a.out[sh * D + d] = to_bf16(empty ? NAN : acc[i] / l_run[i]);
        if (a.out_lse && writer && lane == 0)
          a.out_lse[sh] = empty ? NAN : m_run[i] + logf(l_run[i]);
      }
    }
    return;
  }
  // partial of every head of the group (an empty split: max -inf, sum 0)
  float* gpart = a.part + (s * a.Hq + g * grp) * (int64_t)a.nsplit * (D + 2);
#pragma unroll
  for (int i = 0; i < kSlots; ++i) {
    const int h = h0 + kHeadStride * i;
    if (h < grp) {
      float* pp = gpart + ((int64_t)h * a.nsplit + split) * (D + 2);
      pp[d] = acc[i];
      if (writer && lane == 0) {
        pp[D] = m_run[i];
        pp[D + 1] = l_run[i];
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

template <int D>
void launch_combine(const AttnArgs& a, hipStream_t st) {
  constexpr int kHeadsPerBlock = 1024 / D;
  const int grp = (int)(a.Hq / a.Hkv);
  const int nhb = (grp + kHeadsPerBlock - 1) / kHeadsPerBlock;
  const int threads = (grp < kHeadsPerBlock ? grp : kHeadsPerBlock) * D;
  hipLaunchKernelGGL(k_attn_combine<D>, dim3((unsigned)(a.S * a.Hkv * nhb)), dim3(threads), 0,
                     st, a);
}

// splits: about kTargetBlocks workgroups, whole tiles per split
void attn_splits(int64_t S, int64_t Hkv, int64_t Lmax, int* nsplit, int* chunk) {
  const int64_t tiles = (Lmax + kTileKeys - 1) / kTileKeys;
  int64_t ns = (kTargetBlocks + S * Hkv - 1) / (S * Hkv);
  if (ns > tiles) ns = tiles;
  if (ns > kMaxSplit) ns = kMaxSplit;
  if (ns < 1) ns = 1;
  const int64_t tiles_per = (tiles + ns - 1) / ns;
  *chunk = (int)(tiles_per * kTileKeys);
  *nsplit = (int)((tiles + tiles_per - 1) / tiles_per);
}

int attn_check(int64_t S, int64_t Hq, int64_t Hkv, int64_t Lmax, int64_t D) {
  if (S <= 0 || Hq <= 0 || Hkv <= 0 || Lmax <= 0 || Hq % Hkv != 0 || Hq / Hkv > kMaxGroup)
    return DRGRPO_ERR_SHAPE;
  if (D != 64 && D != 128) return DRGRPO_ERR_SHAPE;
  if (Lmax > (int64_t(1) << 30) || S * Hkv > (int64_t(1) << 25) || S * Hq > INT32_MAX)
    return DRGRPO_ERR_SHAPE;
  return DRGRPO_OK;
}

}  // namespace

// ====================================================================== C ABI
extern "C" size_t drgrpo_decode_attention_workspace_bytes(int64_t S, int64_t Hq, int64_t Hkv,
                                                          int64_t Lmax, int64_t D) {
  if (attn_check(S, Hq, Hkv, Lmax, D) != DRGRPO_OK) return 0;
  int nsplit, chunk;
  attn_splits(S, Hkv, Lmax, &nsplit, &chunk);
  return (size_t)(S * Hq) * nsplit * (D + 2) * sizeof(float);
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
  if (al % 16 != 0) return DRGRPO_ERR_ALIAS;
  if (!workspace || reinterpret_cast<uintptr_t>(workspace) % 256 != 0 ||
      workspace_bytes < drgrpo_decode_attention_workspace_bytes(S, Hq, Hkv, Lmax, D))
    return DRGRPO_ERR_WORKSPACE;
  AttnArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k_cache);
  a.v = static_cast<const uint16_t*>(v_cache);
  a.lens = lens;
  a.S = S;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Lmax = Lmax;
  a.scale = scale;
  attn_splits(S, Hkv, Lmax, &a.nsplit, &a.chunk);
  a.part = static_cast<float*>(workspace);
  a.out = static_cast<uint16_t*>(out);
  a.out_lse = out_lse;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const unsigned blocks = (unsigned)(S * Hkv * a.nsplit);
  if (D == 64) {
    hipLaunchKernelGGL(k_attn_split<64>, dim3(blocks), dim3(kAttnThreads), 0, st, a);
    if (attn_launch_status() != DRGRPO_OK) return DRGRPO_ERR_HIP;
    if (a.nsplit > 1) launch_combine<64>(a, st);
  } else {
    hipLaunchKernelGGL(k_attn_split<128>, dim3(blocks), dim3(kAttnThreads), 0, st, a);
    if (attn_launch_status() != DRGRPO_OK) return DRGRPO_ERR_HIP;
    if (a.nsplit > 1) launch_combine<128>(a, st);
  }
  return attn_launch_status();
}
