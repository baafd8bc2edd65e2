/*
 * lmhead.hip - fused lm_head variant of the Dr. GRPO loss for gfx950: the
 * policy's last hidden states and the unembedding W go in, the loss, dhidden
 * and dW come out; the [tokens, V] logits are never stored.
 *
 * Definitions are those of include/drgrpo.h with logits = hidden . W^T.
 * Only "active" tokens (counted, with a non-zero advantage or beta > 0)
 * have a non-zero gradient; they are compacted first and every GEMM runs over
 * them alone.  All products are C = A . B^T computed by one MFMA kernel
 * (v_mfma_f32_16x16x32_bf16, binary32 accumulation) with three epilogues:
 *
 *   GM_LSE    logits tile of H_a . W^T -> per-token (max, sum exp) over the
 *             tile's vocabulary columns and the sampled token's logit (the
 *             forward-only log-prob pass)
 *   GM_LSE_E  the same product for the loss: sums of exp(x - r_t) relative to
 *             a per-token reference r_t fixed before the product (the sampled
 *             token's logit), and E = exp(x - r_t) of every logit in bfloat16
 *   GM_ACC    dhidden = s_t * (E . W) over the whole vocabulary   (binary32)
 *   GM_STORE  dW_chunk = E_chunk^T . (s . H_a)                     (bfloat16)
 *
 * With one reference per token, every dlogits entry is a per-token factor
 * times E: D[t, v] = s_t E[t, v] with s_t = coef_t exp(r_t - lse_t), once the
 * sampled entry of E is replaced by exp(x_y - r_t) - exp(lse_t - r_t).  The
 * gradient products therefore read E as it is (no dlogits array): dhidden
 * applies s_t to its result rows, dW reads the hidden states scaled by s_t.
 * A row whose logits exceed its reference by more than a fixed window (its
 * exponentials would leave the binary32 range) flags the call; the forward
 * product then runs again with that row's maximum as its reference.
 * Transposed copies of the compacted hidden states and of W give the
 * products their reduction dimension contiguous; the
 * dhidden product reads E, whose reduction dimension (vocabulary) is strided
 * in the forward's accumulator order, through transposing LDS reads.  No
 * floating-point atomics: results are bitwise reproducible.
 */
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "drgrpo.h"
#include "common.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int GBM = 256;                   // workgroup tile rows (A rows)
constexpr int GBN = 256;                   // workgroup tile columns (B rows)
constexpr int GBK = 32;                    // reduction depth per LDS stage: one MFMA
constexpr int WM = 128, WN = 64;           // wavefront tile
constexpr int NWM = GBM / WM, NWN = GBN / WN;  // wavefront grid: 2 (rows) x 4 (columns)
constexpr int GT = 64 * NWM * NWN;         // 8 wavefronts, 2 per SIMD
constexpr int FM = WM / 16, FN = WN / 16;  // 8 x 4 MFMA blocks per wavefront
constexpr int kStages = 4;                 // LDS ring depth (3 stages of loads in flight)
constexpr int kStageElems = (GBM + GBN) * GBK;  // bfloat16 per LDS stage (32 KB)
constexpr int kDmaA = GBM / 16 / (GT / 64);  // 16-row direct loads of A per wavefront per stage
constexpr int kDmaB = GBN / 16 / (GT / 64);  // and of B
constexpr int kDmaPerThread = kDmaA + kDmaB;
static_assert(kDmaA * (GT / 64) * 16 == GBM && kDmaB * (GT / 64) * 16 == GBN,
              "the wavefronts split both operands' row groups evenly");
constexpr int kRingElems = kStages * kStageElems;
constexpr int kTableBytes = 4096;          // per-row epilogue tables (after the main loop)
// the tables sit past the ring when it leaves room, else in its last 4 KB
// (free once the main loop is over; the epilogue staging uses its first 128 KB)
constexpr int kLdsMax = 163840;            // gfx950: 160 KB of LDS per workgroup
constexpr bool kTablesInRing = kRingElems * 2 + kTableBytes > kLdsMax;
constexpr int kTableElem = kTablesInRing ? kRingElems - kTableBytes / 2 : kRingElems;
constexpr size_t kGemmLds = kRingElems * sizeof(uint16_t) + (kTablesInRing ? 0 : kTableBytes);
static_assert(kGemmLds <= (size_t)kLdsMax, "LDS ring too deep");
// The forward product's per-wavefront (max, sum exp) table sits past the row
// tables: its epilogue stages the exponentials in the ring.
constexpr int kRedElem = (int)(kGemmLds / sizeof(uint16_t));
constexpr size_t kRedBytes = sizeof(float2) * NWN * GBM;
constexpr size_t kGemmLdsLse = kGemmLds + kRedBytes;
static_assert(kGemmLdsLse <= (size_t)kLdsMax, "forward product's LDS");
static_assert(!kTablesInRing || kRingElems - kTableBytes / 2 >= (GT / 64) * WM * WN,
              "epilogue staging overlaps the tables");
static_assert((GT / 64) * WM * WN <= kRingElems, "epilogue staging exceeds the ring");
constexpr int kPad = 32;                   // token and vocabulary counts are padded to this
// vocabulary rows per dW launch: 128 row tiles (two full rounds on 256 CUs;
// measured against 8K, 16K and 24K)
constexpr int kChunkV = 32768;
constexpr float kL2E = 1.4426950408889634f;
constexpr double kL2ED = 1.4426950408889634074;
// How far (in nats) a token's logits may exceed its reference before the
// forward product runs again for it: E stays below e^48 (bfloat16 and
// binary32 hold up to e^88), its sum over any vocabulary below e^61 and the
// gradient products' sums far inside the binary32 range.
constexpr float kRefWindow = 48.0f;
constexpr float kRefSumMax = 7.0167e20f;  // e^kRefWindow (rounded down)
static_assert(kRefWindow == 48.0f, "kRefSumMax is e^48");

enum { GM_LSE = 0, GM_LSE_E = 1, GM_ACC = 2, GM_STORE = 3 };

// Tile shape of each product.  The forward product's output width is the
// vocabulary: 256 x 256 tiles, wavefronts of WM x WN = 128 x 64 in a 2 x 4
// grid (the constants above).  The two gradient products' output width is
// the hidden size, 896 = 4 x 224 at the Qwen2.5-0.5B shape: 256 x 224 tiles,
// wavefronts of 64 x 112 in a 4 x 2 grid, so no column of a tile is padding
// (256-column tiles spent 1/8 of their MFMAs on it).  Their LDS stages still
// hold 256 rows of B, the last 32 unused: the direct loads are the forward
// product's.
template <int MODE>
struct TileShape {
  static constexpr bool kFwd = MODE == GM_LSE || MODE == GM_LSE_E;
  static constexpr int BN = kFwd ? GBN : 224;  // output columns of a workgroup
  static constexpr int WM = kFwd ? 128 : 64;
  static constexpr int WN = kFwd ? 64 : 112;
};

// Layout of the forward product's exponentials E, the accumulators' own
// order: tile (tm, tn) of GBM x GBN at (tm * ntn + tn) * GBM * GBN; in it
// wavefront (wm, wn)'s WM x WN block at (wm * NWN + wn) * WM * WN; in that
// its 16 x 16 MFMA block (i, j) at (i * FN + j) * 256; in that lane l's four
// rows 4 * (l / 16) + r, r = 0..3, of column l % 16 at l * 4 + r.  Each lane
// stores its 4 values as one 8-byte store, so a wavefront's 16 x 16 block is
// 512 contiguous bytes.  Element (t, v) lies at ebk_offset(t, v, ntn).
// The gradient products read E in this order: for the dhidden product, 32
// vocabulary columns of a tile's 256 tokens are 16 runs of 1 KB (blocks
// j, j+1 of every (wm, i)); for the dW product, 32 tokens of its 256
// vocabulary rows are 4 runs of 4 KB (blocks i, i+1 of every wn).
// first element of E tile (tm, tn), ntn tiles along the vocabulary
__host__ __device__ inline int64_t etile(int64_t tm, int64_t tn, int64_t ntn) {
  return (tm * ntn + tn) * (GBM * GBN);
}
__host__ __device__ inline int64_t ebk_offset(int64_t t, int64_t v, int64_t ntn) {
  const int64_t tl = t % GBM, vl = v % GBN;
  const int64_t wm = tl / WM, i = (tl % WM) / 16, q = (tl % 16) / 4, r = tl % 4;
  const int64_t wn = vl / WN, j = (vl % WN) / 16, f = vl % 16;
  return etile(t / GBM, v / GBN, ntn) + (wm * NWN + wn) * (WM * WN) + (i * FN + j) * 256 +
         (q * 16 + f) * 4 + r;
}


struct GemmArgs {
  // Operands in bfloat16.  Element (r, k) of A sits at
  // A[r * ar + (k / 32) * ak + k % 32]: a row-major [M, ld] matrix has
  // ar = ld, ak = 32; a K-paneled one, stored as K/32 panels [rows][32],
  // has ar = 32, ak = rows * 32.  The same holds for B ([N, K]) with br, bk.
  // The gradient products' A is the forward product's E (ebk_offset order;
  // ar and ak unused): GM_ACC's element (t, k) is E[t, col_base + k], GM_STORE's
  // element (v, k) is E[k, col_base + v].
  const uint16_t* A;
  const uint16_t* B;
  int64_t ar, ak, br, bk;
  int64_t M, N, K;    // static bounds (grid); K a multiple of 8
  const int32_t* M_dev;  // if set: M = *M_dev (active-token count)
  const int32_t* K_dev;  // if set: K = *K_dev (padded active-token count)
  // GM_LSE / GM_LSE_E
  float2* part;          // [rows, ntn] per-token (reference, sum exp) of each column tile
  int64_t ntn;           // vocabulary tiles of the forward product (all products)
  float* xy;             // [rows] sampled token's logit
  const int32_t* ycol;   // [rows] sampled token id
  int64_t col_base;      // vocabulary id of column 0 (the gradient products: of the chunk)
  // GM_LSE_E: partial sums of exp(x - r_t), r_t = mref[t], and (E != NULL)
  // E = exp(x - r_t) of every logit in bfloat16, in the accumulators' own
  // order (ebk_offset); a row whose tile sum exceeds e^kRefWindow sets
  // rowmark[t] = 1 and raises *flag
  uint16_t* E;
  const float* mref;
  int32_t* rowmark;
  int32_t* flag;
  const int32_t* run_if;  // the rerun kernel: does nothing unless *run_if != 0
  // GM_ACC / GM_STORE
  float* Cf;             // [M, ldc] binary32 accumulator
  uint16_t* Cb;          // [M, ldc] bfloat16 result
  int64_t ldc;
  int accumulate;        // GM_ACC: add to Cf (else overwrite)
  const float* rscale;   // GM_ACC: row t's result is scaled by rscale[t]
};

template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

// Workgroup barrier for the LDS ring: the hardware barrier alone (the waits
// before it are explicit), fenced for the compiler so no memory access moves
// across it.
__device__ inline void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ inline uint16_t bf16_bits(float x) {
  const __bf16 h = (__bf16)x;  // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// two values rounded to bfloat16 (nearest even) in one packed conversion, a
// in the low half
__device__ inline uint32_t bf16x2_bits(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// Cross-lane moves within a DPP row of 16 lanes (lanes sharing l / 16).  A
// max or sum over the row takes four steps: swaps within quads (xor 1, xor 2),
// then across quad pairs (half-row mirror) and row halves (row mirror); every
// lane of the row ends with the result.  Every source lane of these patterns
// lies in the row, so bound_ctrl never applies; the compiler folds the move
// into the integer max and the float add that consume it.
template <int CTRL>
__device__ inline int dpp_i32(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ inline float dpp_f32(float v) {
  return __builtin_bit_cast(float, dpp_i32<CTRL>(__builtin_bit_cast(int, v)));
}
// An order-preserving map of non-NaN binary32 values to int32 (its own
// inverse): the magnitude bits of negative values are flipped, so the integer
// max is the float max (a float max would be canonicalised first and could
// not absorb the lane move).
__device__ inline int f32_ord(float x) {
  const int b = __builtin_bit_cast(int, x);
  return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ inline float ord_f32(int b) { return __builtin_bit_cast(float, b ^ ((b >> 31) & 0x7FFFFFFF)); }
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

// chunk permutation of LDS row r (see the main loop): rows of one parity
// among 8 consecutive, and rows equal mod 4 among 16, get distinct values
__device__ inline int swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

// chunk permutation within a 512-byte E block (one 16 x 16 MFMA block) of
// GM_ACC's A stage: LDS chunk 8q + y (16 bytes) holds the block's chunk
// 8q + (y ^ 2q), i.e. columns 2y', 2y'+1 of rows 4q .. 4q+3 with y' = y ^ 2q.
// One transposing read of a 16-lane group takes 4 consecutive columns of all
// four quads: 8 chunks that land on 8 distinct 16-byte positions of a
// 128-byte bank row, so the group touches every bank once.  Its own inverse.
__device__ inline int esw(int p) { return p ^ (2 * (p >> 3)); }

// the forward product's wavefront grid, under names the products' own tile
// shapes do not hide
constexpr int WM_F = WM, WN_F = WN, NWN_F = NWN;

// quad permutation of row c of an epilogue stage of kWM rows (kWM / 4
// quads): an even value below kWM / 4; 16 consecutive rows get distinct
// values (8 at kWM = 64), and 4 rows from a multiple of 4 distinct bits 2-3
// (the transposing reads)
template <int kWM>
__device__ inline int stage_swz(int c) {
  static_assert(kWM == 128 || kWM == 64, "stage heights");
  if constexpr (kWM == 128)
    return 2 * (((c & 3) << 1) | ((c >> 2) & 1) | (((c >> 3) & 1) << 3));
  else
    return 2 * (((c & 3) << 1) | ((c >> 2) & 1));
}

// 16-byte stores of a wavefront's staged kWM x kWN bfloat16 block, element
// (t, c) to out[t * rs + (c / 32) * ps + c % 32] (row-major: rs = ld, ps = 32;
// K-paneled over columns: rs = 32, ps = panel stride), for rows t < rows_lim
// and 8-column groups c < cols_lim (cols_lim a multiple of 8).  One
// instruction covers 16 rows x 32 columns: a contiguous 1 KB block when
// paneled (kWN = 112: the last covers 16 columns, the other lanes read a
// column of the block and store nothing).  The transposing LDS read gives lane li of a 16-lane group 4
// consecutive columns of row tb + li when lane 4e + q4 of the group points at
// quad tb/4 + q4 of stage row (first column + e).  The stores are
// nontemporal: a dlogits chunk and its transpose (1.9 GB at 32K columns) are
// far larger than any cache, and the hint made the dlogits product 2-3%
// faster without slowing the products that read the chunk back.
template <bool kFull, int kWM, int kWN>
__device__ inline void store_staged_rows(const uint16_t* stg, int lane, uint16_t* out, int64_t rs,
                                         int64_t ps, int rows_lim, int cols_lim) {
  static_assert(kWN % 16 == 0, "whole 16-column groups");
  const int grp = lane >> 4, li = lane & 15;
  const int e = li >> 2, q4 = li & 3;
#pragma unroll
  for (int sidx = 0; sidx < ((kWN + 31) / 32) * (kWM / 16); ++sidx) {
    const int tb = 16 * (sidx % (kWM / 16));
    const int cb = 32 * (sidx / (kWM / 16)) + 8 * grp;  // 8 columns of this group
    const int qq = (tb >> 2) + q4;
    // columns past the block (the last group at kWN = 112) read its last column
    const int ca = cb + e < kWN ? cb + e : kWN - 1, cc = cb + 4 + e < kWN ? cb + 4 + e : kWN - 1;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(stg + ca * kWM + 4 * (qq ^ stage_swz<kWM>(ca))));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(stg + cc * kWM + 4 * (qq ^ stage_swz<kWM>(cc))));
    const int t = tb + li;
    if ((kWN % 32 == 0 || cb < kWN) && (kFull || (t < rows_lim && cb < cols_lim))) {
      const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
      __builtin_nontemporal_store(u32x4{l2.x, l2.y, h2.x, h2.y},
                                  reinterpret_cast<u32x4*>(out + t * rs + (cb / 32) * ps + cb % 32));
    }
  }
}

// Stage column c = j*16 + (lane % 16) of the wavefront block, rows
// i*16 + 4*(lane/16) .. +3 (one MFMA accumulator quad, as bfloat16 bits:
// rows 0-1 in lo, 2-3 in hi, the lower row in the low half).
template <int kWM>
__device__ inline void stage_pair(uint16_t* stg, int lane, int i, int j, uint32_t lo, uint32_t hi) {
  const int q = i * 4 + (lane >> 4);
  const int c = j * 16 + (lane & 15);
  *reinterpret_cast<uint2*>(stg + c * kWM + 4 * (q ^ stage_swz<kWM>(c))) = make_uint2(lo, hi);
}

// GM_ACC's fragment reads within one step, in issue order: after the
// MFMAs of row block i (of 4), B fragments b_cum(i) .. b_cum(i+1)-1 of the
// next stage (all 7 within row blocks 0-2, so the last one has a row block of
// MFMAs to land), then the two transposing reads of A fragment i.  A
// wavefront's LDS reads complete in order, so "at most n outstanding" lands
// every read with n or more issued after it; the counts below follow.
namespace tr_reads {
constexpr int b_cum(int i) { return i <= 0 ? 0 : i == 1 ? 3 : i == 2 ? 5 : 7; }
constexpr int n(int i) { return b_cum(i + 1) - b_cum(i) + 2; }
constexpr int before(int i) { return i == 0 ? 0 : before(i - 1) + n(i - 1); }
constexpr int a_end(int i) { return before(i) + n(i) - 1; }  // A fragment i's last read
constexpr int b_last(int i) {                                   // the last B read
  return b_cum(i + 1) > b_cum(i) ? before(i) + b_cum(i + 1) - b_cum(i) - 1 : b_last(i - 1);
}
constexpr int kTotal = before(4);
// row block 0 needs every B fragment and A fragment 0 of the previous step
constexpr int kLand0 = b_last(3) > a_end(0) ? b_last(3) : a_end(0);
constexpr int kWait0 = kTotal - 1 - kLand0;
constexpr bool landed0(int i) { return a_end(i) <= kLand0; }
// A fragment i (not landed by then) before row block i: the previous step's
// reads after it and this step's reads of row blocks 0 .. i-1
constexpr int wait_a(int i) { return kTotal - 1 - a_end(i) + before(i); }
static_assert(b_cum(4) == 7 && kTotal == 15 && kWait0 == 4 && landed0(1) && !landed0(2) &&
                  wait_a(2) == 11 && wait_a(3) == 13,
              "GM_STORE read order");
}  // namespace tr_reads

// One output tile b of a product (the launch's workgroup id, or a tile a
// workgroup of the rerun kernel walks to).
template <int MODE>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, const int b) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  // this product's tile shape (for the forward product the same values as
  // the namespace constants these names hide)
  constexpr int BN = TileShape<MODE>::BN;
  constexpr int WM = TileShape<MODE>::WM, WN = TileShape<MODE>::WN;
  constexpr int NWM = GBM / WM, NWN = BN / WN;
  constexpr int FM = WM / 16, FN = WN / 16;
  static_assert(NWM * NWN * 64 == GT && BN <= GBN, "eight wavefronts; B rows within a stage");
  static_assert((GT / 64) * WM * WN <= kRingElems, "epilogue staging exceeds the ring");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / NWN, wn = wave % NWN;
  const int64_t M = g.M_dev ? (int64_t)*g.M_dev : g.M;
  const int64_t K = g.K_dev ? (int64_t)*g.K_dev : g.K;
  // tile order: each XCD (workgroup id mod 8) takes a contiguous run of one
  // linear order, so the workgroups sharing its L2 share operand tiles.  The
  // order runs along the operand that is small: column tiles fastest for
  // the products reducing over a dlogits chunk (A is the large operand).
  // The forward product walks groups of kColGroup column tiles row by row,
  // so the 32 workgroups an XCD runs at once share 4 row tiles and 8 column
  // tiles (12 distinct operand panels per reduction step instead of 33).
  // The grid covers the static row bound; only the tiles of the first M rows
  // (M read on the device) take part, spread evenly over the XCDs.
  // (32-bit index arithmetic: the host keeps the grid below 2^31 workgroups)
  const int ntm = (int)((M + GBM - 1) / GBM);
  const int ntn_t = (int)((g.N + BN - 1) / BN);
  const int total = ntm * ntn_t;
  if (b >= total) return;
  const int q8 = total / 8;
  const int v = b < 8 * q8 ? (b % 8) * q8 + b / 8 : b;
  int tm, tn;
  if constexpr (TileShape<MODE>::kFwd) {
    constexpr int kColGroup = 8;
    const int grouped = (ntn_t / kColGroup) * kColGroup * ntm;
    const int gw = v < grouped ? kColGroup : ntn_t % kColGroup;  // width of v's group
    const int w = v < grouped ? v % (kColGroup * ntm) : v - grouped;
    tm = w / gw;
    tn = (v < grouped ? v / (kColGroup * ntm) * kColGroup : grouped / ntm) + w % gw;
  } else {
    tm = v / ntn_t;
    tn = v % ntn_t;
  }
  const int64_t m0 = (int64_t)tm * GBM;
  const int64_t n0 = (int64_t)tn * BN;

  // ---- main loop: a ring of kStages LDS stages, each [A 256 x 32 | B 256 x 32]
  // bfloat16 (row r of A at r*32, of B at (256 + r)*32; 64-byte rows), filled
  // by direct global -> LDS loads issued kStages-1 stages ahead.  Each
  // wavefront loads kDmaA 1 KB pieces of A and kDmaB of B, through buffer
  // descriptors over the tile's part of the current 32-wide reduction step
  // (buffer loads: the compiler counts them on vmcnt alone, so the LDS
  // fragment reads keep fine-grained waits).
  // A paneled operand: one instruction moves 16 rows x 64 B (lane l: row
  // l/4, chunk l%4), a single contiguous 1 KB block.  Rows past M or N
  // re-read the last valid row (their results are never used).  K is a
  // multiple of 32.  The four 16-byte chunks of a row are stored
  // XOR-permuted by swz(row % 16), so the fragment reads (16 rows, one chunk)
  // spread over all LDS banks.
  // The gradient products' A is E in the forward's order (ebk_offset): one
  // instruction moves one 1 KB run, two 16 x 16 blocks.  GM_ACC (rows =
  // tokens, reduction over vocabulary) stages run (wm, i) of the forward tile
  // at 1 KB * (8 wm + i), its chunks permuted within each 512-byte block by
  // esw, and reads its fragments through transposing LDS reads.  GM_STORE
  // (rows = vocabulary, reduction over tokens) stages its four 4 KB runs
  // (one per wn) in order and reads each fragment as two 8-byte reads.
  constexpr bool kAT = MODE == GM_ACC;     // A through transposing reads
  constexpr bool kEA = MODE == GM_ACC || MODE == GM_STORE;  // A is E
  static_assert(!kEA || kDmaA == 2, "two E runs per wavefront and stage");
  const int64_t nk = K / GBK;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int64_t nvA = M - m0 < GBM ? M - m0 : GBM;    // >= 1: the tile exists
  const int64_t nvB = g.N - n0 < GBN ? g.N - n0 : GBN;
  const uint16_t* baseB = g.B + n0 * g.br;
  // the span one stage's loads address
  const int pbA = MODE == GM_ACC     ? 2 * (32768 + 7 * 1024 + 512)
                  : MODE == GM_STORE ? 2 * (3 * 8192 + 2048)
                                     : (int)(((nvA - 1) * g.ar + GBK) * 2);
  const int pbB = (int)(((nvB - 1) * g.br + GBK) * 2);
  const int dchunk = 8 * ((lane & 3) ^ swz(lane >> 2));
  uint32_t voffA[kDmaA], voffB[kDmaB];
#pragma unroll
  for (int p = 0; p < kDmaA; ++p) {
    if constexpr (MODE == GM_ACC) {
      // run (wm, i) = (wv / 4, 2 (wv % 4) + p); lane l: chunk esw(l % 32) of block l / 32
      voffA[p] = (uint32_t)(2 * ((wv >> 2) * 32768 + (2 * (wv & 3) + p) * 1024 +
                                 (lane >> 5) * 256 + esw(lane & 31) * 8));
    } else if constexpr (MODE == GM_STORE) {
      // run wn = wv / 2, its half wv % 2, 1 KB piece p
      voffA[p] = (uint32_t)(2 * ((wv >> 1) * 8192 + (wv & 1) * 1024 + p * 512 + lane * 8));
    } else {
      const int64_t r = (wv * kDmaA + p) * 16 + (lane >> 2);
      voffA[p] = (uint32_t)(((r < nvA ? r : nvA - 1) * g.ar + dchunk) * 2);
    }
  }
#pragma unroll
  for (int p = 0; p < kDmaB; ++p) {
    const int64_t r = (wv * kDmaB + p) * 16 + (lane >> 2);
    voffB[p] = (uint32_t)(((r < nvB ? r : nvB - 1) * g.br + dchunk) * 2);
  }
  // first element of stage kt's part of A
  auto a_stage = [&](int64_t kt) -> const uint16_t* {
    if constexpr (MODE == GM_ACC) {
      const int64_t v = g.col_base + kt * GBK;  // the step's first vocabulary column
      return g.A + etile(tm, v / GBN, g.ntn) + ((v % GBN) / WN_F) * (WM_F * WN_F) +
             ((v % WN_F) / 32) * 512;
    } else if constexpr (MODE == GM_STORE) {
      // tokens 32 kt ..: forward row tile kt / 8, its wavefront row block
      // (kt % 8) / 4, MFMA row blocks 2 (kt % 4), +1
      return g.A + etile(kt / 8, (g.col_base + m0) / GBN, g.ntn) +
             ((kt % 8) / 4) * (NWN_F * WM_F * WN_F) + (kt % 4) * 2048;
    } else {
      return g.A + m0 * g.ar + kt * g.ak;
    }
  };
  auto dma = [&](int64_t kt) {
    uint16_t* slot = smem + (kt % kStages) * kStageElems;
    const auto ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a_stage(kt)), 0, pbA,
                                                      0x00020000);
    const auto rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(baseB + kt * g.bk), 0,
                                                      pbB, 0x00020000);
#pragma unroll
    for (int p = 0; p < kDmaA; ++p)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (__attribute__((address_space(3))) void*)(slot + (wv * kDmaA + p) * 16 * GBK), 16,
          voffA[p], 0, 0, 0);
#pragma unroll
    for (int p = 0; p < kDmaB; ++p)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb, (__attribute__((address_space(3))) void*)(slot + (GBM + (wv * kDmaB + p) * 16) * GBK),
          16, voffB[p], 0, 0, 0);
  };
  const int fr = lane & 15;  // row (A) / column (B) within a 16 x 16 block
  // LDS position of the lane's 8 reduction indices 8*(lane/16) .. +7
  const int fk = 8 * ((lane >> 4) ^ swz(fr));
  // A fragments are reloaded in place, row block by row block, as soon as the
  // MFMAs of that block have issued; B fragments are double-buffered
  bf16x8 fa[FM], fb[2][FN];
  // GM_ACC reads every fragment through inline assembly: the compiler
  // models the transposing read's builtin as possibly aliasing the direct
  // loads in flight and would drain them all (vmcnt(0)) before each one.
  // The reads then issue in program order and the step waits for them
  // explicitly (lgkmcnt), naming the fragments as operands of the wait so no
  // instruction that reads them can move above it.
  auto lds_addr = [](const uint16_t* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint16_t*)p;
  };
  // GM_ACC's A fragment i: rows wm*WM + i*16 + fr are rows 4q + r of MFMA
  // block i' = 4 (wm % 2) + i of forward wavefront row block wm / 2, staged
  // as run 4 wm + i (1 KB each).  Lane 4e + q4 of 16-lane group g points at
  // quad q4 (4 rows) of column f = 8 (g % 2) + 4 hh + e of block g / 2 of the
  // run; the read hands lane fr of the group columns f - e .. +3 of row fr,
  // and the two reads (hh = 0, 1) give its 8 reduction indices 8g .. 8g+7.
  // Column f of quad q4 is chunk 8 q4 + f / 2 (half f % 2) of its block,
  // staged at chunk esw(8 q4 + f / 2).  In bytes from the stage:
  // 4096 wm + 1024 i + 512 (g / 2) + 16 esw(..) + 8 (e % 2): the lane- and
  // hh-dependent part is one base register per hh, 1024 i an offset.
  const int g4 = lane >> 4, e4 = (lane & 15) >> 2, q4 = lane & 3;
  const uint32_t offA[2] = {
      (uint32_t)(4096 * wm + 512 * (g4 >> 1) + 16 * esw(8 * q4 + 4 * (g4 & 1) + 0 + (e4 >> 1)) +
                 8 * (e4 & 1)),
      (uint32_t)(4096 * wm + 512 * (g4 >> 1) + 16 * esw(8 * q4 + 4 * (g4 & 1) + 2 + (e4 >> 1)) +
                 8 * (e4 & 1))};
  // GM_STORE's A fragment i: vocabulary rows wm*WM + i*16 + fr are column fr
  // of MFMA block (i_l, j = i) of forward wavefront column block wn = wm;
  // the lane's tokens 8 g4 .. +7 are quads 2 (g4 % 2), +1 of block i_l = g4 / 2,
  // two 8-byte reads 128 bytes apart
  const int offS = (4096 * wm + 2048 * (g4 >> 1) + 256 * (g4 & 1) + 8 * fr) / 2;
  const uint32_t offB = (uint32_t)(2 * ((wn * WN + fr) * GBK + fk));
  auto frag_a = [&](const uint16_t* As, int i) -> bf16x8 {
    if constexpr (kAT) {
      s16x4 t[2];
      asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                   : "=v"(t[0]) : "v"(lds_addr(As) + offA[0]), "i"(1024 * i) : "memory");
      asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                   : "=v"(t[1]) : "v"(lds_addr(As) + offA[1]), "i"(1024 * i) : "memory");
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(t[0], t[1], 0, 1, 2, 3, 4, 5, 6, 7));
    } else if constexpr (MODE == GM_STORE) {
      const u32x2 lo = *reinterpret_cast<const u32x2*>(As + offS + 256 * i);
      const u32x2 hi = *reinterpret_cast<const u32x2*>(As + offS + 256 * i + 64);
      return __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
    } else {
      return *reinterpret_cast<const bf16x8*>(As + (wm * WM + i * 16 + fr) * GBK + fk);
    }
  };
  // (GM_ACC: B fragment j at offB + 1024*j bytes from the stage's B rows)
  auto frag_b = [&](const uint16_t* Bs, int j) -> bf16x8 {
    if constexpr (kAT) {
      bf16x8 v;
      asm volatile("ds_read_b128 %0, %1 offset:%2"
                   : "=v"(v) : "v"(lds_addr(Bs) + offB), "i"(1024 * j) : "memory");
      return v;
    } else {
      return *reinterpret_cast<const bf16x8*>(Bs + (wn * WN + j * 16 + fr) * GBK + fk);
    }
  };
  // GM_ACC: every fragment read has landed; the fragments named stay in
  // their registers until here
  // (each empty statement after a wait keeps a fragment's readers below it)
  auto settle_all = [&]() {
    if constexpr (kAT) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int i = 0; i < FM; ++i) asm volatile("" : "+v"(fa[i]));
#pragma unroll
      for (int j = 0; j < FN; ++j) asm volatile("" : "+v"(fb[0][j]), "+v"(fb[1][j]));
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, the other
  // counters left alone): wait until at most n stages of this thread's direct
  // loads are still in flight
  constexpr auto vm_imm = [](int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); };
  static_assert(3 * kDmaPerThread < 64, "vmcnt immediate");
  auto wait_stages = [&](int64_t n) {
    if (n >= 3)
      __builtin_amdgcn_s_waitcnt(vm_imm(3 * kDmaPerThread));
    else if (n == 2)
      __builtin_amdgcn_s_waitcnt(vm_imm(2 * kDmaPerThread));
    else if (n == 1)
      __builtin_amdgcn_s_waitcnt(vm_imm(kDmaPerThread));
    else
      __builtin_amdgcn_s_waitcnt(vm_imm(0));
  };
  // Per-row epilogue tables in the area past the ring.  Their entries are
  // loaded into registers here, before the first stages' loads, and written
  // to LDS after the main loop, whose last wait has seen them land: the
  // loads cost no wait of their own.
  //   GM_LSE, GM_LSE_E: tile-local column of the row's sampled token (-1:
  //           none, or a column of another tile, which never equals a local
  //           column)
  //   GM_LSE_E: the row's reference r_t (rows past M: the last row's, whose
  //           logits they repeat)
  int32_t* const t_yl = reinterpret_cast<int32_t*>(smem + kTableElem);  // [GBM]
  float* const t_mr = reinterpret_cast<float*>(smem + kTableElem) + GBM;  // [GBM]
  constexpr bool kTables = MODE == GM_LSE || MODE == GM_LSE_E;
  constexpr bool kRef = MODE == GM_LSE_E;
  static_assert(!kTables || !kTablesInRing, "the epilogue tables are written while waves may still read the ring");
  static_assert(2 * GBM * 4 <= kTableBytes, "two row tables");
  constexpr int kYPer = (GBM + GT - 1) / GT;
  int32_t ypre[kYPer];
  float mrpre[kYPer];
  if constexpr (kTables) {
#pragma unroll
    for (int k = 0; k < kYPer; ++k) {
      const int r = tid + k * GT;
      const bool ok = r < GBM && m0 + r < M;
      ypre[k] = ok ? g.ycol[m0 + r] : -1;
      if constexpr (kRef) mrpre[k] = r < GBM ? g.mref[ok ? m0 + r : M - 1] : 0.0f;
    }
  }
  if (nk > 0)
    for (int64_t s = 0; s < kStages - 1 && s < nk; ++s) dma(s);
  if (nk > 0) {
    // stage 0 complete; the later prologue stages may still be in flight
    wait_stages(nk - 1 < kStages - 2 ? nk - 1 : kStages - 2);
    ring_barrier();
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[i] = frag_a(smem, i);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[0][j] = frag_b(smem + GBM * GBK, j);
    settle_all();
  }
  // one step: stage kt's operands are in registers (fa, fb[cur]); make stage
  // kt+1 visible, refill the slot stage kt-1 used (its last fragments were
  // consumed in step kt-1), read stage kt+1's operands while stage kt's MFMAs
  // run.  The scheduling groups keep that interleave: after each MFMA row
  // block, the A fragment it freed (and in the first rows one B fragment), so
  // at most 12 LDS reads are in flight and each has most of a step to land.
  auto step = [&](int64_t kt, int cur) {
    // stage kt+1 complete; stages kt+2 .. kt+kStages-2 (those issued) in flight
    const int64_t ahead = nk - 2 - kt;
    wait_stages(ahead < kStages - 3 ? (ahead > 0 ? ahead : 0) : kStages - 3);
    ring_barrier();
    if (kt + kStages - 1 < nk) dma(kt + kStages - 1);
    // unconditional, so the LDS-read count is the same on every path (after
    // the last stage it reads a stale slot, in bounds, never used)
    const uint16_t* As = smem + ((kt + 1) % kStages) * kStageElems;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if constexpr (kAT) {
        // the previous step's (or the prologue's, which waits for all) reads
        // this row block needs, in the order tr_reads describes
        static_assert(FM == 4 && FN == 7, "tr_reads");
        if (i == 0) {
          asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(tr_reads::kWait0) : "memory");
#pragma unroll
          for (int k = 0; k < FM; ++k)
            if (tr_reads::landed0(k)) asm volatile("" : "+v"(fa[k]));
#pragma unroll
          for (int j = 0; j < FN; ++j) asm volatile("" : "+v"(fb[cur][j]));
        } else if (!tr_reads::landed0(i)) {
          asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(tr_reads::wait_a(i)) : "memory");
          asm volatile("" : "+v"(fa[i]));
        }
      }
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[cur][j], acc[i][j], 0, 0, 0);
      if constexpr (kAT) {
#pragma unroll
        for (int jb = tr_reads::b_cum(i); jb < tr_reads::b_cum(i + 1); ++jb)
          fb[cur ^ 1][jb] = frag_b(As + GBM * GBK, jb);
      } else if constexpr (FN <= FM) {
        if (i < FN) fb[cur ^ 1][i] = frag_b(As + GBM * GBK, i);
      } else {  // FN / FM of them after each row block (4 x 7: 1, 2, 2, 2)
#pragma unroll
        for (int jb = i * FN / FM; jb < (i + 1) * FN / FM; ++jb)
          fb[cur ^ 1][jb] = frag_b(As + GBM * GBK, jb);
      }
      fa[i] = frag_a(As, i);
    }
    static_assert((FM == 8 && FN == 4) || (FM == 4 && FN == 7),
                  "scheduling groups below assume 8 x 4 or 4 x 7 MFMA blocks");
    if constexpr (FM == 4) {
      // per row block 7 MFMAs and its 2 or 3 fragment reads
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    } else {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };
  int64_t kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    step(kt, 0);
    step(kt + 1, 1);
  }
  if (kt < nk) step(kt, 0);
  if (nk > 0) settle_all();  // the last step's reads (never used) are no longer in flight
  if constexpr (kTables) {
#pragma unroll
    for (int k = 0; k < kYPer; ++k) {
      const int r = tid + k * GT;
      if (r < GBM) {
        t_yl[r] = ypre[k] < 0 ? -1 : (int32_t)(ypre[k] - (g.col_base + n0));
        if constexpr (kRef) t_mr[r] = mrpre[k];
      }
    }
  }
  // every wavefront is done with the ring before the epilogue reuses it, and
  // the tables are visible
  __syncthreads();

  // accumulator layout: acc[i][j][r] = C[m0 + wm*WM + i*16 + 4*(lane/16) + r]
  //                                    [n0 + wn*WN + j*16 + lane%16]
  // (the LDS stages are free from here on and hold the epilogue's tables)
  const int rq = 4 * (lane >> 4);

  // columns of this tile that exist (the rest of the tile is padding)
  const int ncols = (int)(g.N - n0 < BN ? g.N - n0 : BN);
  const int lc0 = wn * WN + fr;  // tile-local column of acc[.][0]
  if constexpr (MODE == GM_LSE || MODE == GM_LSE_E) {
    float2* red = reinterpret_cast<float2*>(smem + kRedElem);  // [NWN][GBM]
    const int32_t* yl = t_yl;
    // full tiles (the common case) compile without the column checks
    auto body = [&](auto full_tag) {
      constexpr bool kFull = decltype(full_tag)::value;
      // the four rows of a lane run in lockstep so the cross-lane steps of
      // one row fill the others' DPP wait states
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int rt0 = wm * WM + i * 16 + rq;
        const int4 y4 = *reinterpret_cast<const int4*>(yl + rt0);
        // the sampled token's column is held by the lane whose columns
        // lc0 + 16j include it: a rare, divergent store
        const int dy[4] = {y4.x - lc0, y4.y - lc0, y4.z - lc0, y4.w - lc0};
        bool hit[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) hit[r] = (unsigned)dy[r] < (unsigned)WN && (dy[r] & 15) == 0;
        if (hit[0] || hit[1] || hit[2] || hit[3]) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            // a bitwise select (a variable index would send acc to scratch);
            // each element is copied out first, since a bit cast of a vector
            // element expression reads the vector's first element
            uint32_t xb = 0;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
              const float a = acc[i][j][r];
              xb |= __builtin_bit_cast(uint32_t, a) & (dy[r] == 16 * j ? ~0u : 0u);
            }
            if (hit[r]) g.xy[m0 + rt0 + r] = __builtin_bit_cast(float, xb);
          }
        }
        // GM_LSE: the row's maximum over the wavefront's columns (in-lane,
        // then across the 16 lanes of its DPP row); GM_LSE_E needs none
        int mo[4];
        if constexpr (kRef) {
          if constexpr (!kFull) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
              for (int j = 0; j < FN; ++j)
                if (lc0 + j * 16 >= ncols) acc[i][j][r] = -INFINITY;
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float m = -INFINITY;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
              if (!kFull && lc0 + j * 16 >= ncols) acc[i][j][r] = -INFINITY;
              m = fmaxf(m, acc[i][j][r]);
            }
            mo[r] = f32_ord(m);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) mo[r] = max(mo[r], dpp_i32<kDppXor1>(mo[r]));
#pragma unroll
          for (int r = 0; r < 4; ++r) mo[r] = max(mo[r], dpp_i32<kDppXor2>(mo[r]));
#pragma unroll
          for (int r = 0; r < 4; ++r) mo[r] = max(mo[r], dpp_i32<kDppHalfMirror>(mo[r]));
#pragma unroll
          for (int r = 0; r < 4; ++r) mo[r] = max(mo[r], dpp_i32<kDppMirror>(mo[r]));
        }
        float mx[4], sm[4], ref[4];
        if constexpr (kRef) {
          const float4 m4 = *reinterpret_cast<const float4*>(t_mr + rt0);
          ref[0] = m4.x, ref[1] = m4.y, ref[2] = m4.z, ref[3] = m4.w;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (!kRef) mx[r] = ord_f32(mo[r]);
          // exp(x - ref) as exp2(x*log2e - ref*log2e), one fused step per
          // entry (the rounding of ref*log2e scales the whole partial sum by
          // one factor 2^d, |d| <= 2^-24 |ref| log2e).  GM_LSE: ref = the
          // row's maximum over the tile (a quarter tile past the last
          // vocabulary column holds no value at all, only in a partial tile);
          // GM_LSE_E: the row's reference, fixed for the whole call
          if constexpr (!kRef) ref[r] = mx[r];
          const float nb = kRef || kFull || ref[r] != -INFINITY ? -ref[r] * kL2E : 0.0f;
          // the exponentials replace the logits in acc (E below)
          acc[i][0][r] = __builtin_amdgcn_exp2f(fmaf(acc[i][0][r], kL2E, nb));
          sm[r] = acc[i][0][r];
#pragma unroll
          for (int j = 1; j < FN; ++j) {
            acc[i][j][r] = __builtin_amdgcn_exp2f(fmaf(acc[i][j][r], kL2E, nb));
            sm[r] += acc[i][j][r];
          }
        }
        if (kRef && g.E) {
          // bfloat16 (nearest even), the lane's four rows of a column as one
          // 8-byte store (ebk_offset)
          uint16_t* eb = g.E + etile(tm, tn, ntn_t) +
                         (wm * NWN + wn) * (WM * WN) + lane * 4;
#pragma unroll
          for (int j = 0; j < FN; ++j)
            __builtin_nontemporal_store(
                u32x2{bf16x2_bits(acc[i][j][0], acc[i][j][1]), bf16x2_bits(acc[i][j][2], acc[i][j][3])},
                reinterpret_cast<u32x2*>(eb + (i * FN + j) * 256));
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) sm[r] += dpp_f32<kDppXor1>(sm[r]);
#pragma unroll
        for (int r = 0; r < 4; ++r) sm[r] += dpp_f32<kDppXor2>(sm[r]);
#pragma unroll
        for (int r = 0; r < 4; ++r) sm[r] += dpp_f32<kDppHalfMirror>(sm[r]);
#pragma unroll
        for (int r = 0; r < 4; ++r) sm[r] += dpp_f32<kDppMirror>(sm[r]);
        if (fr == 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r) red[wn * GBM + rt0 + r] = make_float2(kRef ? ref[r] : mx[r], sm[r]);
        }
      }
    };
    if (ncols == BN)
      body(BoolC<true>{});
    else
      body(BoolC<false>{});
    __syncthreads();
    for (int r = tid; r < GBM; r += GT) {
      const int64_t row = m0 + r;
      if (row >= M) continue;
      if constexpr (kRef) {
        // the wavefronts' sums share the row's reference
        float sm = 0.0f;
#pragma unroll
        for (int w = 0; w < NWN; ++w) sm += red[w * GBM + r].y;
        g.part[row * g.ntn + tn] = make_float2(t_mr[r], sm);
        // every exponential of the tile's row is at most its sum: a sum
        // beyond e^kRefWindow (or not a number) marks the row and flags the
        // call (rare)
        if (!(sm <= kRefSumMax)) {
          g.rowmark[row] = 1;
          __hip_atomic_store(g.flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        continue;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int w = 0; w < NWN; ++w) mx = fmaxf(mx, red[w * GBM + r].x);
      float sm = 0.0f;
      if (mx != -INFINITY) {
#pragma unroll
        for (int w = 0; w < NWN; ++w) {
          const float2 p = red[w * GBM + r];
          sm += p.y * __builtin_amdgcn_exp2f((p.x - mx) * kL2E);
        }
      }
      g.part[row * g.ntn + tn] = make_float2(mx, sm);
    }
  } else {
    const int nrows = (int)(M - m0 < GBM ? M - m0 : GBM);
    const int ldc = (int)g.ldc;
    // GM_STORE stages its bfloat16 block through LDS like the forward's
    // exponentials
    uint16_t* stg = smem + wave * (WM * WN);
    const int64_t base = (m0 + wm * WM + rq) * g.ldc + n0 + lc0;
    auto body = [&](auto full_tag) {
      constexpr bool kFull = decltype(full_tag)::value;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int rt0 = wm * WM + i * 16 + rq;
        auto ok = [&](int j, int r) { return kFull || (lc0 + j * 16 < ncols && rt0 + r < nrows); };
        if constexpr (MODE == GM_ACC) {
          float* c = g.Cf + base + i * 16 * ldc;
          // the rows' dlogits factors (rscale holds the rows of whole tiles)
          const float4 s4 = *reinterpret_cast<const float4*>(g.rscale + m0 + rt0);
          const float sc[4] = {s4.x, s4.y, s4.z, s4.w};
          float old[FN][4] = {};
          if (g.accumulate) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (ok(j, r)) old[j][r] = c[r * ldc + j * 16];
          }
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (ok(j, r)) c[r * ldc + j * 16] = fmaf(sc[r], acc[i][j][r], old[j][r]);
        } else {
#pragma unroll
          for (int j = 0; j < FN; ++j)
            stage_pair<WM>(stg, lane, i, j, bf16x2_bits(acc[i][j][0], acc[i][j][1]),
                       bf16x2_bits(acc[i][j][2], acc[i][j][3]));
        }
      }
      if constexpr (MODE == GM_STORE) {
        __syncthreads();
        store_staged_rows<kFull, WM, WN>(stg, lane, g.Cb + (m0 + wm * WM) * g.ldc + n0 + wn * WN, g.ldc,
                                 32, nrows - wm * WM, ncols - wn * WN);
      }
    };
    if (ncols == BN && nrows == GBM)
      body(BoolC<true>{});
    else
      body(BoolC<false>{});
  }
}

// One workgroup per output tile; two wavefronts per SIMD (the register
// budget of 8 wavefronts per CU).
template <int MODE>
__global__ void __launch_bounds__(GT) __attribute__((amdgpu_waves_per_eu(2))) k_gemm(GemmArgs g) {
  gemm_tile<MODE>(g, (int)blockIdx.x);
}

// A forward product once more, for a call whose first pass flagged a row
// (GM_LSE: the per-tile maxima the flagged rows' new references come from;
// GM_LSE_E: the exponentials with those references): nothing happens unless
// *run_if != 0, so it is launched on every call with one workgroup per CU,
// and each workgroup walks tiles b, b + gridDim.x, .. below nblocks.
template <int MODE>
__global__ void __launch_bounds__(GT) __attribute__((amdgpu_waves_per_eu(2)))
k_gemm_rerun(GemmArgs g, int nblocks) {
  if (__builtin_amdgcn_readfirstlane(*g.run_if) == 0) return;
  for (int b = (int)blockIdx.x; b < nblocks; b += (int)gridDim.x) {
    gemm_tile<MODE>(g, b);
    __syncthreads();  // the next tile's loads reuse the LDS this one's epilogue reads
  }
}

// ------------------------------------------------------------ small kernels
// Active-token count per completion and exclusive offsets (one workgroup).
// A token is active when counted (t < len_i, token id in range) and
// (A_i != 0 or beta != 0); with adv == NULL every counted token is active
// (the forward-only log-prob pass).  Bad ids are handled separately.
__global__ void __launch_bounds__(1024)
k_lm_offsets(const int32_t* __restrict__ len, const float* __restrict__ adv, int64_t N,
             float beta, int32_t* __restrict__ offs, int32_t* __restrict__ counts) {
  __shared__ int32_t sh[1024];
  const int tid = threadIdx.x;
  int32_t base = 0;
  for (int64_t c0 = 0; c0 < N; c0 += 1024) {
    const int64_t i = c0 + tid;
    const int32_t a =
        (i < N && (adv == nullptr || adv[i] != 0.0f || beta != 0.0f)) ? len[i] : 0;
    sh[tid] = a;
    __syncthreads();
    // inclusive Hillis-Steele scan (fixed order, integers)
    for (int o = 1; o < 1024; o <<= 1) {
      const int32_t v = tid >= o ? sh[tid - o] : 0;
      __syncthreads();
      sh[tid] += v;
      __syncthreads();
    }
    if (i < N) offs[i] = base + sh[tid] - a;
    base += sh[1023];
    __syncthreads();
  }
  if (tid == 0) {
    offs[N] = base;
    counts[0] = base;                // active tokens
    counts[1] = (base + kPad - 1) / kPad * kPad;  // padded for the products over tokens
  }
}

// One workgroup per (completion, block of kGatherTok tokens): list the
// block's active tokens, gather their hidden rows, and zero the loss terms of
// its other tokens (tok_loss == NULL: no loss terms, the forward-only pass).
// The gathered rows are K-paneled: element (k, h) of active token k at
// Ha[(h / 32) * ha_ps + k * 32 + h % 32].  A completion's active tokens are
// its first n_act (all counted tokens, or none).
constexpr int kGatherTok = 32;
__global__ void __launch_bounds__(256)
k_lm_gather(const uint16_t* __restrict__ hidden, int64_t H, const int64_t* __restrict__ tokens,
            int64_t C, int64_t V, const int32_t* __restrict__ len,
            const int32_t* __restrict__ offs, int32_t* __restrict__ act_pos,
            int32_t* __restrict__ ycol, uint16_t* __restrict__ Ha, int64_t ha_ps,
            double* __restrict__ tok_loss, uint8_t* __restrict__ tok_flags) {
  const int64_t nb = (C + kGatherTok - 1) / kGatherTok;
  const int64_t i = blockIdx.x / nb;
  const int64_t t0 = (blockIdx.x - i * nb) * kGatherTok;
  const int64_t t1 = C - t0 < kGatherTok ? C : t0 + kGatherTok;
  const int32_t n_act = offs[i + 1] - offs[i];
  const int32_t k0 = offs[i];
  const int32_t L = len[i];
  for (int64_t t = t0 + threadIdx.x; t < t1; t += blockDim.x) {
    const int64_t pos = i * C + t;
    const int64_t y = tokens[pos];
    const bool bad = t < L && (y < 0 || y >= V);
    if (t < n_act) {
      act_pos[k0 + t] = (int32_t)pos;
      ycol[k0 + t] = bad ? -1 : (int32_t)y;
    }
    if (tok_loss && (t >= n_act || bad)) {
      tok_loss[pos] = bad ? (double)NAN : 0.0;
      tok_flags[pos] = bad ? TF_BADTOK : 0;
    }
  }
  // hidden rows of the block's active tokens: 16-byte copies, four lanes per
  // 64-byte panel record, so a wavefront writes whole records of 16 tokens
  const int64_t nt = (t1 < n_act ? t1 : (int64_t)n_act) - t0;
  const int64_t npan = H / 32;
  for (int64_t q = threadIdx.x; q < nt * npan * 4; q += blockDim.x) {
    const int64_t c4 = q & 3, rest = q >> 2;
    const int64_t t = t0 + rest % nt, pn = rest / nt;
    *reinterpret_cast<u32x4*>(Ha + pn * ha_ps + (k0 + t) * 32 + 8 * c4) =
        *reinterpret_cast<const u32x4*>(hidden + (i * C + t) * H + 32 * pn + 8 * c4);
  }
}

// Transpose into a K-paneled operand: element (c, r) of dst, at
// dst[(r / 32) * d_ps + c * 32 + r % 32], is element (r, c) of src, at
// src[r * s_rs + (c / 32) * s_ps + c % 32] (row-major: s_rs = ld, s_ps = 32),
// for r < rows (or the device count rows_dev) and zero for r up to rows_pad
// (or rows_dev rounded up to kPad); 64 x 64 tiles through LDS with 16-byte
// accesses on both sides (8 columns of a row in, 8 rows of a column out: a
// quarter of a 64-byte panel record), so cols and the row counts are
// multiples of 8 and every offset a multiple of 8 elements.  The grid covers
// ceil(rows_pad / 64) x ceil(cols / 64) tiles.  With rscale, source row r is
// multiplied by rscale[r] (binary32) and rounded to bfloat16 on the way.
__global__ void __launch_bounds__(256)
k_transpose(const uint16_t* __restrict__ src, int64_t s_rs, int64_t s_ps, int64_t rows,
            int64_t rows_pad, int64_t cols, const int32_t* __restrict__ rows_dev,
            const float* __restrict__ rscale, uint16_t* __restrict__ dst, int64_t d_ps) {
  constexpr int TS = 64, TP = TS + 8;  // tile, padded LDS row (16-byte aligned rows)
  __shared__ __attribute__((aligned(16))) uint16_t tile[TS][TP];
  const int64_t R = rows_dev ? (int64_t)*rows_dev : rows;
  const int64_t Rpad = rows_dev ? (R + kPad - 1) / kPad * kPad : rows_pad;
  const int64_t ntr = (rows_pad + TS - 1) / TS;
  const int64_t r0 = (blockIdx.x % ntr) * TS;
  const int64_t c0 = (blockIdx.x / ntr) * TS;
  if (r0 >= Rpad) return;
  for (int e = threadIdx.x; e < TS * (TS / 8); e += blockDim.x) {
    const int k = e >> 3, cc = (e & 7) * 8;  // tile row, first of its 8 columns
    const int64_t r = r0 + k, c = c0 + cc;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (r < R && c < cols) {
      v = *reinterpret_cast<const u32x4*>(src + r * s_rs + (c / 32) * s_ps + c % 32);
      if (rscale) {
        const float sc = rscale[r];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t o[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          o[u] = bf16x2_bits(sc * __builtin_bit_cast(float, w[u] << 16),
                             sc * __builtin_bit_cast(float, w[u] & 0xFFFF0000u));
        v = u32x4{o[0], o[1], o[2], o[3]};
      }
    }
    *reinterpret_cast<u32x4*>(&tile[k][cc]) = v;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < TS * (TS / 8); e += blockDim.x) {
    const int k = e >> 3, rr = (e & 7) * 8;  // tile column, first of its 8 rows
    const int64_t c = c0 + k, r = r0 + rr;
    if (c >= cols || r >= Rpad) continue;
    uint32_t w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      w[u] = (uint32_t)tile[rr + 2 * u][k] | ((uint32_t)tile[rr + 2 * u + 1][k] << 16);
    *reinterpret_cast<u32x4*>(dst + (r / 32) * d_ps + c * 32 + r % 32) =
        u32x4{w[0], w[1], w[2], w[3]};
  }
}

// log-sum-exp of active token k from its per-column-tile (max, sum exp)
// pairs, merged by one wavefront (binary32 per lane, binary64 across lanes):
// lse = M + ln(S); every lane returns (M, S).
struct Lse {
  float M;
  double S;
  __device__ double value() const { return (double)M + log(S); }
};
__device__ inline Lse merge_lse(const float2* __restrict__ part, int64_t ntn, int64_t k,
                                int lane) {
  float m = -INFINITY, s = 0.0f;
  for (int64_t j = lane; j < ntn; j += 64) {
    const float2 p = part[k * ntn + j];
    const float nm = fmaxf(m, p.x);
    if (nm == -INFINITY) continue;
    s = s * __builtin_amdgcn_exp2f((m - nm) * kL2E) + p.y * __builtin_amdgcn_exp2f((p.x - nm) * kL2E);
    m = nm;
  }
  float M = m;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  double term = s != 0.0f ? (double)s * exp2(((double)m - (double)M) * kL2ED) : 0.0;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) term += __shfl_xor(term, o);
  return Lse{M, term};
}

// One wavefront per active token: merge the per-tile (max, sum exp), then
// the per-token loss term and gradient coefficient.
__global__ void __launch_bounds__(256)
k_lm_combine(const float2* __restrict__ part, int64_t ntn, const float* __restrict__ xy,
             const int32_t* __restrict__ counts, const int32_t* __restrict__ act_pos,
             const int32_t* __restrict__ ycol, int64_t C, const float* __restrict__ adv,
             const int32_t* __restrict__ len, const float* __restrict__ logp_old,
             const float* __restrict__ logp_ref, float eps, float beta, double kappa, int agg,
             const int64_t* __restrict__ total_len, const float* __restrict__ mref,
             uint16_t* __restrict__ E, float* __restrict__ rscale, double* __restrict__ tok_loss,
             uint8_t* __restrict__ tok_flags) {
  const int lane = threadIdx.x & 63;
  const int64_t k = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (k >= counts[0]) return;
  const Lse ls = merge_lse(part, ntn, k, lane);
  const double lse = ls.value();
  if (lane != 0) return;
  const int64_t pos = act_pos[k];
  const int64_t i = pos / C;
  const int32_t y = ycol[k];
  if (y < 0) {  // bad token id: excluded from the gradient, poisons the loss
    rscale[k] = 0.0f;
    return;
  }
  const double logp = (double)xy[k] - lse;
  const double div = row_divisor(agg, kappa, len[i], total_len);
  const TokenTerms tt = token_terms(logp, logp_old[pos], beta != 0.0f ? logp_ref[pos] : 0.0f,
                                    adv[i], eps, beta, div);
  tok_loss[pos] = tt.lam / div;
  tok_flags[pos] = tt.flags;
  // dlogits of the row: D[t, v] = coef (p_v - [v = y]) = s E[t, v] with
  // E = exp(x - r) (r the row's reference) and s = coef exp(r - lse), once
  // the sampled entry of E holds exp(x_y - r) - exp(lse - r); coef = 0 (a
  // clip-cut gradient) gives s = 0, exact zero rows
  const double r = (double)mref[k];
  const float cf = (float)tt.coef;
  rscale[k] = (float)((double)cf * exp(r - lse));
  E[ebk_offset(k, y, ntn)] = bf16_bits((float)(exp((double)xy[k] - r) - exp(lse - r)));
}

// Each listed token's reference r_t for a forward product: its sampled
// token's logit hidden_t . W[y_t] (binary32 sum of bfloat16 products, one
// wavefront per token; 0 for a bad token id).  Any value would do as long as
// exp(x - r_t) stays in range: the sampled token's logit is at most the row's
// maximum, and a row whose exponentials sum beyond e^kRefWindow in some tile
// is detected and redone.  Also clears the call's flag and the rows' marks.
__global__ void __launch_bounds__(256)
k_lm_mref(const uint16_t* __restrict__ Ha, int64_t ha_ps, const uint16_t* __restrict__ W, int64_t H,
          const int32_t* __restrict__ counts, const int32_t* __restrict__ ycol,
          float* __restrict__ mref, int32_t* __restrict__ rowmark, int32_t* __restrict__ flag) {
  const int lane = threadIdx.x & 63;
  const int64_t k = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blockIdx.x == 0 && threadIdx.x == 0) *flag = 0;
  if (k >= counts[0]) return;
  const int32_t y = ycol[k];
  float acc = 0.0f;
  if (y >= 0) {
    for (int64_t h = 8 * lane; h < H; h += 8 * 64) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(Ha + (h / 32) * ha_ps + k * 32 + h % 32);
      const u32x4 w = *reinterpret_cast<const u32x4*>(W + (int64_t)y * H + h);
      const uint32_t av[4] = {a.x, a.y, a.z, a.w}, wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        acc = fmaf(__builtin_bit_cast(float, av[u] << 16), __builtin_bit_cast(float, wv[u] << 16), acc);
        acc = fmaf(__builtin_bit_cast(float, av[u] & 0xFFFF0000u),
                   __builtin_bit_cast(float, wv[u] & 0xFFFF0000u), acc);
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) {
    mref[k] = acc;
    rowmark[k] = 0;
  }
}

// After a flagged forward pass and the max-relative pass over the same
// tiles: each marked row takes its maximum over the vocabulary (the largest
// of its per-tile maxima) as the new reference.  Nothing unless flagged.
__global__ void __launch_bounds__(256)
k_lm_mref_fix(const int32_t* __restrict__ counts, const int32_t* __restrict__ flag,
              const int32_t* __restrict__ rowmark, const float2* __restrict__ part, int64_t ntn,
              float* __restrict__ mref) {
  if (*flag == 0) return;
  for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < counts[0];
       k += (int64_t)gridDim.x * blockDim.x) {
    if (rowmark[k] == 0) continue;
    float m = -INFINITY;
    for (int64_t j = 0; j < ntn; ++j) m = fmaxf(m, part[k * ntn + j].x);
    mref[k] = m;
  }
}

// dhidden rows: active tokens get their accumulator, others zero (NaN for a
// bad token id at a counted position).
__global__ void __launch_bounds__(256)
k_lm_dh_out(const float* __restrict__ dHacc, int64_t H, const int32_t* __restrict__ offs,
            const int32_t* __restrict__ len, const int64_t* __restrict__ tokens, int64_t C,
            int64_t V, uint16_t* __restrict__ dhidden) {
  const int64_t pos = blockIdx.x;
  const int64_t i = pos / C, t = pos - i * C;
  const int32_t n_act = offs[i + 1] - offs[i];
  const int64_t y = tokens[pos];
  const bool bad = t < len[i] && (y < 0 || y >= V);
  const int64_t k = offs[i] + t;
  for (int64_t h = threadIdx.x; h < H; h += blockDim.x) {
    float v = 0.0f;
    if (bad) v = NAN;
    else if (t < n_act) v = dHacc[k * H + h];
    dhidden[pos * H + h] = bf16_bits(v);
  }
}

// Forward-only pass: log-prob of active token k (every counted token), one
// wavefront per token; NaN for a token id outside [0, V).
__global__ void __launch_bounds__(256)
k_lm_logp(const float2* __restrict__ part, int64_t ntn, const float* __restrict__ xy,
          const int32_t* __restrict__ counts, const int32_t* __restrict__ act_pos,
          const int32_t* __restrict__ ycol, float* __restrict__ out_logp) {
  const int lane = threadIdx.x & 63;
  const int64_t k = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (k >= counts[0]) return;
  const double lse = merge_lse(part, ntn, k, lane).value();
  if (lane == 0) out_logp[act_pos[k]] = ycol[k] < 0 ? NAN : (float)((double)xy[k] - lse);
}

// Forward-only pass: positions after a completion's first EOS get 0.
__global__ void __launch_bounds__(256)
k_lm_logp_tail(const int32_t* __restrict__ len, int64_t C, float* __restrict__ out_logp) {
  const int64_t i = blockIdx.x;
  for (int64_t t = len[i] + (int64_t)threadIdx.x; t < C; t += blockDim.x) out_logp[i * C + t] = 0.0f;
}

// ------------------------------------------------------------ host side
struct LmWs {
  int32_t* status;
  int32_t* len;
  float* adv;
  uint8_t* row_flags;
  int64_t* total_len;  // [1] counted tokens (token-mean aggregation)
  int32_t* offs;     // [N + 1]
  int32_t* counts;   // [2]: active tokens, that count padded to kPad
  int32_t* act_pos;  // [T]
  int32_t* ycol;     // [T]
  double* tok_loss;  // [T]
  uint8_t* tok_flags;
  float2* part;      // [T, ntn] (reference, sum exp) of each vocabulary tile
  float* xy;         // [T]
  float* mref;       // [round_up(T, GBM)] each active token's reference r_t
  int32_t* rowmark;  // [T] rows beyond their reference (1)
  int32_t* flag;     // [1] some row was beyond its reference
  float* rscale;     // [round_up(T, GBM)] each active token's dlogits factor s_t
  uint16_t* Ha;      // [T, H] K-paneled over H (H/32 panels [T][32])
  uint16_t* Hs;      // [H, Tcap] s_t * hidden_t, K-paneled over tokens (Tcap/32 panels [H][32])
  uint16_t* Wt;      // [H, V rounded up to 32] W transposed, K-paneled over the vocabulary
  float* dH;         // [Tcap, H]
  uint16_t* E;       // bfloat16 exponentials of whole forward tiles (ebk_offset)
};

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

size_t lm_carve(void* base, int64_t N, int64_t T, int64_t V, int64_t H, LmWs* ws) {
  const int64_t Tcap = round_up(T, kPad);
  const int64_t ntn = (V + GBN - 1) / GBN;
  size_t off = 0;
  char* b = static_cast<char*>(base);
  auto take = [&](size_t bytes) {
    char* p = b ? b + off : nullptr;
    off += align256(bytes);
    return p;
  };
  LmWs w;
  w.status = reinterpret_cast<int32_t*>(take(256));
  w.len = reinterpret_cast<int32_t*>(take(4 * N));
  w.adv = reinterpret_cast<float*>(take(4 * N));
  w.row_flags = reinterpret_cast<uint8_t*>(take(N));
  w.total_len = reinterpret_cast<int64_t*>(take(sizeof(int64_t)));
  w.offs = reinterpret_cast<int32_t*>(take(4 * (N + 1)));
  w.counts = reinterpret_cast<int32_t*>(take(16));
  w.act_pos = reinterpret_cast<int32_t*>(take(4 * T));
  w.ycol = reinterpret_cast<int32_t*>(take(4 * T));
  w.tok_loss = reinterpret_cast<double*>(take(8 * T));
  w.tok_flags = reinterpret_cast<uint8_t*>(take(T));
  w.part = reinterpret_cast<float2*>(take(8 * (size_t)T * ntn));
  w.xy = reinterpret_cast<float*>(take(4 * T));
  w.mref = reinterpret_cast<float*>(take(4 * round_up(T, GBM)));
  w.rowmark = reinterpret_cast<int32_t*>(take(4 * T));
  w.flag = reinterpret_cast<int32_t*>(take(4));
  w.rscale = reinterpret_cast<float*>(take(4 * round_up(T, GBM)));
  w.Ha = reinterpret_cast<uint16_t*>(take(2 * (size_t)T * H));
  w.Hs = reinterpret_cast<uint16_t*>(take(2 * (size_t)H * Tcap));
  w.Wt = reinterpret_cast<uint16_t*>(take(2 * (size_t)H * round_up(V, kPad)));
  w.dH = reinterpret_cast<float*>(take(4 * (size_t)Tcap * H));
  // whole forward tiles (ebk_offset)
  w.E = reinterpret_cast<uint16_t*>(take(2 * (size_t)round_up(T, GBM) * ntn * GBN));
  if (ws) *ws = w;
  return off;
}

// Workspace of the forward-only log-prob pass: the loss pass's lists and
// per-tile partials, without the backward buffers.
struct LpWs {
  int32_t* len;      // [N]
  int32_t* offs;     // [N + 1]
  int32_t* counts;   // [2]
  int32_t* act_pos;  // [T]
  int32_t* ycol;     // [T]
  float2* part;      // [T, ntn]
  float* xy;         // [T]
  float* mref;       // [T] each counted token's reference
  int32_t* rowmark;  // [T] rows beyond their reference (1)
  int32_t* flag;     // [1]
  uint16_t* Ha;      // [T, H] K-paneled over H (H/32 panels [T][32])
};

size_t lp_carve(void* base, int64_t N, int64_t T, int64_t V, int64_t H, LpWs* ws) {
  const int64_t ntn = (V + GBN - 1) / GBN;
  size_t off = 0;
  char* b = static_cast<char*>(base);
  auto take = [&](size_t bytes) {
    char* p = b ? b + off : nullptr;
    off += align256(bytes);
    return p;
  };
  LpWs w;
  w.len = reinterpret_cast<int32_t*>(take(4 * N));
  w.offs = reinterpret_cast<int32_t*>(take(4 * (N + 1)));
  w.counts = reinterpret_cast<int32_t*>(take(16));
  w.act_pos = reinterpret_cast<int32_t*>(take(4 * T));
  w.ycol = reinterpret_cast<int32_t*>(take(4 * T));
  w.part = reinterpret_cast<float2*>(take(8 * (size_t)T * ntn));
  w.xy = reinterpret_cast<float*>(take(4 * T));
  w.mref = reinterpret_cast<float*>(take(4 * T));
  w.rowmark = reinterpret_cast<int32_t*>(take(4 * T));
  w.flag = reinterpret_cast<int32_t*>(take(4));
  w.Ha = reinterpret_cast<uint16_t*>(take(2 * (size_t)T * H));
  if (ws) *ws = w;
  return off;
}

int lm_check_shape(int64_t N, int64_t C, int64_t V, int64_t H, int64_t G, int64_t* T) {
  if (N <= 0 || C <= 0 || V <= 0 || H <= 0 || G <= 0 || N % G != 0) return DRGRPO_ERR_SHAPE;
  if (V % 8 != 0 || H % kPad != 0 || V > (int64_t(1) << 30) || H > 65536) return DRGRPO_ERR_SHAPE;
  // token rows up to 2^24 keep every in-tile offset of the epilogues in 32 bits
  if (!mul_ok(N, C, T) || *T > (int64_t(1) << 24)) return DRGRPO_ERR_SHAPE;
  int64_t tmp;
  if (!mul_ok(*T, (V + GBN - 1) / GBN * 16, &tmp) || !mul_ok(*T, H * 4, &tmp) ||
      !mul_ok(V, H * 2, &tmp) || !mul_ok(*T + GBM, (V + GBN) * 2, &tmp))
    return DRGRPO_ERR_SHAPE;
  return DRGRPO_OK;
}

// ev_begin / ev_end (optional) are stamped by the dispatch itself, to time it alone
template <int MODE>
int launch_gemm(const GemmArgs& g, hipStream_t st, hipEvent_t ev_begin = nullptr,
                hipEvent_t ev_end = nullptr) {
  const int64_t ntm = (g.M + GBM - 1) / GBM;
  const int64_t ntn = (g.N + TileShape<MODE>::BN - 1) / TileShape<MODE>::BN;
  const int64_t blocks = ntm * ntn;
  if (blocks <= 0) return DRGRPO_OK;
  if (blocks > INT32_MAX) return DRGRPO_ERR_SHAPE;
  // 132 KB of LDS per workgroup, 140 KB for the forward product (gfx950 has
  // 160 KB per CU)
  const size_t lds = TileShape<MODE>::kFwd ? kGemmLdsLse : kGemmLds;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm<MODE>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return DRGRPO_ERR_HIP;
  if (ev_begin || ev_end)
    hipExtLaunchKernelGGL(k_gemm<MODE>, dim3((unsigned)blocks), dim3(GT), lds, st, ev_begin,
                          ev_end, 0, g);
  else
    hipLaunchKernelGGL(k_gemm<MODE>, dim3((unsigned)blocks), dim3(GT), lds, st, g);
  return launch_status();
}

// The loss's forward product again when *g.run_if is set: one workgroup per
// CU (256 on gfx950) over the same tiles.
constexpr int kRerunGrid = 256;
template <int MODE>
int launch_rerun(const GemmArgs& g, hipStream_t st) {
  static_assert(TileShape<MODE>::kFwd, "forward products only");
  const int64_t blocks = ((g.M + GBM - 1) / GBM) * ((g.N + GBN - 1) / GBN);
  if (blocks <= 0) return DRGRPO_OK;
  if (blocks > INT32_MAX) return DRGRPO_ERR_SHAPE;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_rerun<MODE>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)kGemmLdsLse) != hipSuccess)
    return DRGRPO_ERR_HIP;
  hipLaunchKernelGGL(k_gemm_rerun<MODE>, dim3(kRerunGrid), dim3(GT), kGemmLdsLse, st, g, (int)blocks);
  return launch_status();
}

}  // namespace

// ====================================================================== C ABI
extern "C" size_t drgrpo_lmhead_workspace_bytes(int64_t N, int64_t C, int64_t V, int64_t H,
                                                int64_t G) {
  int64_t T;
  if (lm_check_shape(N, C, V, H, G, &T) != DRGRPO_OK) return 0;
  return lm_carve(nullptr, N, T, V, H, nullptr);
}

extern "C" int drgrpo_lmhead_loss_fwd_bwd_ex(const void* hidden, const void* W,
                                             const int64_t* tokens, int64_t eos_id,
                                             const float* rewards, const float* logp_old,
                                             const float* logp_ref, int64_t G, float eps,
                                             float beta, float norm_const, float* out_loss,
                                             void* out_dhidden, void* out_dW, int64_t N,
                                             int64_t C, int64_t V, int64_t H, void* workspace,
                                             size_t workspace_bytes, void* stream,
                                             const drgrpo_variant_t* variant,
                                             const drgrpo_lmhead_aux_t* aux) {
  if (!hidden || !W || !tokens || !rewards || !logp_old || !out_loss || !out_dhidden || !out_dW)
    return DRGRPO_ERR_NULL;
  int64_t T;
  const int sh = lm_check_shape(N, C, V, H, G, &T);
  if (sh != DRGRPO_OK) return sh;
  if (!finite_f(eps) || eps < 0.0f || !finite_f(beta) || beta < 0.0f || !finite_f(norm_const) ||
      norm_const <= 0.0f)
    return DRGRPO_ERR_PARAM;
  if (beta > 0.0f && !logp_ref) return DRGRPO_ERR_NULL;
  int adv_mode, agg;
  if (!read_variant(variant, &adv_mode, &agg)) return DRGRPO_ERR_PARAM;
  const uintptr_t al = reinterpret_cast<uintptr_t>(hidden) | reinterpret_cast<uintptr_t>(W) |
                       reinterpret_cast<uintptr_t>(out_dhidden) |
                       reinterpret_cast<uintptr_t>(out_dW);
  if (al % 16 != 0) return DRGRPO_ERR_ALIGN;
  if (!workspace || reinterpret_cast<uintptr_t>(workspace) % 256 != 0 ||
      workspace_bytes < lm_carve(nullptr, N, T, V, H, nullptr))
    return DRGRPO_ERR_WORKSPACE;
  LmWs w;
  lm_carve(workspace, N, T, V, H, &w);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t Tcap = round_up(T, kPad);
  const int64_t ntn = (V + GBN - 1) / GBN;
  const uint16_t* hid = static_cast<const uint16_t*>(hidden);
  const uint16_t* Wb = static_cast<const uint16_t*>(W);
  int rc;

  // mask, advantage, active-token list, gathered hidden rows and transposes
  hipLaunchKernelGGL(k_prep, dim3((unsigned)N), dim3(64), 0, st, tokens, C, eos_id, rewards, G,
                     adv_mode, w.len, w.adv, w.row_flags, (int32_t*)nullptr, (uint8_t*)nullptr,
                     (float*)nullptr, (int32_t*)nullptr, (uint32_t*)nullptr);
  if ((rc = launch_status()) != DRGRPO_OK) return rc;
  if (agg == DRGRPO_AGG_TOKEN_MEAN) {
    hipLaunchKernelGGL(k_total_len, dim3(1), dim3(1024), 0, st, w.len, N, w.total_len);
    if ((rc = launch_status()) != DRGRPO_OK) return rc;
  }
  hipLaunchKernelGGL(k_lm_offsets, dim3(1), dim3(1024), 0, st, w.len, w.adv, N, beta, w.offs,
                     w.counts);
  if ((rc = launch_status()) != DRGRPO_OK) return rc;
  // operand layouts: the gathered hidden rows Ha, K-paneled over H (panel
  // stride T * 32); the scaled transpose Hs [H, Tcap], K-paneled over
  // tokens; W transposed, Wt, over vocabulary; E in the forward
  // product's accumulator order (ebk_offset)
  hipLaunchKernelGGL(k_lm_gather, dim3((unsigned)(N * ((C + kGatherTok - 1) / kGatherTok))),
                     dim3(256), 0, st, hid, H, tokens, C, V, w.len,
                     w.offs, w.act_pos, w.ycol, w.Ha, T * 32, w.tok_loss, w.tok_flags);
  if ((rc = launch_status()) != DRGRPO_OK) return rc;
  hipLaunchKernelGGL(k_lm_mref, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, st, w.Ha, T * 32, Wb,
                     H, w.counts, w.ycol, w.mref, w.rowmark, w.flag);
  if ((rc = launch_status()) != DRGRPO_OK) return rc;

  // forward: per-token sums of exp(x - r_t) over the vocabulary and E; the
  // logits are never stored
  GemmArgs g = {};
  g.A = w.Ha;
  g.ar = 32;
  g.ak = T * 32;
  g.B = Wb;
  g.br = H;
  g.bk = 32;
  g.M = T;
  g.N = V;
  g.K = H;
  g.M_dev = w.counts;
  g.part = w.part;
  g.ntn = ntn;
  g.xy = w.xy;
  g.ycol = w.ycol;
  g.col_base = 0;
  g.E = w.E;
  g.mref = w.mref;
  g.rowmark = w.rowmark;
  g.flag = w.flag;
  g.run_if = w.flag;
  if ((rc = launch_gemm<GM_LSE_E>(g, st, aux ? static_cast<hipEvent_t>(aux->fwd_event_begin) : nullptr,
                                  aux ? static_cast<hipEvent_t>(aux->fwd_event_end) : nullptr)) !=
      DRGRPO_OK)
    return rc;
  // rows beyond their reference (if any): their maxima from a max-relative
  // pass, those as new references, the product again
  if ((rc = launch_rerun<GM_LSE>(g, st)) != DRGRPO_OK) return rc;
  hipLaunchKernelGGL(k_lm_mref_fix, dim3(64), dim3(256), 0, st, w.counts, w.flag, w.rowmark,
                     w.part, ntn, w.mref);
  if ((rc = launch_status()) != DRGRPO_OK) return rc;
  if ((rc = launch_rerun<GM_LSE_E>(g, st)) != DRGRPO_OK) return rc;
  hipLaunchKernelGGL(k_lm_combine, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, st, w.part, ntn,
                     w.xy, w.counts, w.act_pos, w.ycol, C, w.adv, w.len, logp_old, logp_ref, eps,
                     beta, (double)norm_const, agg, w.total_len, w.mref, w.E, w.rscale, w.tok_loss,
                     w.tok_flags);
  if ((rc = launch_status()) != DRGRPO_OK) return rc;
  {
    // Hs = s_t * hidden_t, transposed (zero rows past the active count)
    const int64_t blocks2 = ((Tcap + 63) / 64) * ((H + 63) / 64);
    hipLaunchKernelGGL(k_transpose, dim3((unsigned)blocks2), dim3(256), 0, st, w.Ha, (int64_t)32,
                       T * 32, T, Tcap, H, w.counts, (const float*)w.rscale, w.Hs, H * 32);
    if ((rc = launch_status()) != DRGRPO_OK) return rc;
  }

  // dhidden = s . (E . W) over the whole vocabulary in one product: W
  // transposed, [H, V rounded up to 32] with zero columns past V
  const int64_t Vpad = round_up(V, kPad);
  {
    const int64_t tblocks = ((Vpad + 63) / 64) * ((H + 63) / 64);
    hipLaunchKernelGGL(k_transpose, dim3((unsigned)tblocks), dim3(256), 0, st, Wb, H,
                       (int64_t)32, V, Vpad, H, (const int32_t*)nullptr, (const float*)nullptr,
                       w.Wt, H * 32);
    if ((rc = launch_status()) != DRGRPO_OK) return rc;
  }
  GemmArgs a = {};
  a.A = w.E;
  a.ntn = ntn;
  a.col_base = 0;
  a.B = w.Wt;
  a.br = 32;
  a.bk = H * 32;
  a.M = T;
  a.N = H;
  a.K = Vpad;
  a.M_dev = w.counts;
  a.Cf = w.dH;
  a.ldc = H;
  a.accumulate = 0;
  a.rscale = w.rscale;
  if ((rc = launch_gemm<GM_ACC>(a, st)) != DRGRPO_OK) return rc;

  // dW = E^T . Hs, one vocabulary chunk of 32,768 rows at a time (128 row
  // tiles: two full rounds on 256 CUs)
  for (int64_t v0 = 0; v0 < V; v0 += kChunkV) {
    const int64_t wv = V - v0 < kChunkV ? V - v0 : kChunkV;
    GemmArgs s = {};
    s.A = w.E;
    s.ntn = ntn;
    s.col_base = v0;
    s.B = w.Hs;
    s.br = 32;
    s.bk = H * 32;
    s.M = wv;
    s.N = H;
    s.K = Tcap;
    s.K_dev = w.counts + 1;
    s.Cb = static_cast<uint16_t*>(out_dW) + v0 * H;
    s.ldc = H;
    if ((rc = launch_gemm<GM_STORE>(s, st)) != DRGRPO_OK) return rc;
  }

  hipLaunchKernelGGL(k_lm_dh_out, dim3((unsigned)T), dim3(256), 0, st, w.dH, H, w.offs, w.len,
                     tokens, C, V, static_cast<uint16_t*>(out_dhidden));
  if ((rc = launch_status()) != DRGRPO_OK) return rc;
  hipLaunchKernelGGL(k_finish, dim3(1), dim3(1024), 0, st, w.tok_loss, w.tok_flags, T,
                     w.row_flags, w.len, w.adv, beta, N, out_loss, w.status, (int32_t*)nullptr,
                     (int64_t*)nullptr);
  return launch_status();
}

extern "C" int drgrpo_lmhead_loss_fwd_bwd(const void* hidden, const void* W, const int64_t* tokens,
                                          int64_t eos_id, const float* rewards,
                                          const float* logp_old, const float* logp_ref, int64_t G,
                                          float eps, float beta, float norm_const,
                                          float* out_loss, void* out_dhidden, void* out_dW,
                                          int64_t N, int64_t C, int64_t V, int64_t H,
                                          void* workspace, size_t workspace_bytes,
                                          void* stream) {
  return drgrpo_lmhead_loss_fwd_bwd_ex(hidden, W, tokens, eos_id, rewards, logp_old, logp_ref, G,
                                       eps, beta, norm_const, out_loss, out_dhidden, out_dW, N, C,
                                       V, H, workspace, workspace_bytes, stream, nullptr,
                                       nullptr);
}

extern "C" size_t drgrpo_lmhead_logprobs_workspace_bytes(int64_t N, int64_t C, int64_t V,
                                                         int64_t H) {
  int64_t T;
  if (lm_check_shape(N, C, V, H, 1, &T) != DRGRPO_OK) return 0;
  return lp_carve(nullptr, N, T, V, H, nullptr);
}

extern "C" int drgrpo_lmhead_logprobs(const void* hidden, const void* W, const int64_t* tokens,
                                      int64_t eos_id, int64_t N, int64_t C, int64_t V, int64_t H,
                                      float* out_logp, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  if (!hidden || !W || !tokens || !out_logp) return DRGRPO_ERR_NULL;
  int64_t T;
  const int sh = lm_check_shape(N, C, V, H, 1, &T);
  if (sh != DRGRPO_OK) return sh;
  if ((reinterpret_cast<uintptr_t>(hidden) | reinterpret_cast<uintptr_t>(W)) % 16 != 0)
    return DRGRPO_ERR_ALIGN;
  if (!workspace || reinterpret_cast<uintptr_t>(workspace) % 256 != 0 ||
      workspace_bytes < lp_carve(nullptr, N, T, V, H, nullptr))
    return DRGRPO_ERR_WORKSPACE;
  LpWs w;
  lp_carve(workspace, N, T, V, H, &w);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t ntn = (V + GBN - 1) / GBN;
  int rc;
  // counted tokens (first EOS inclusive), listed and gathered like the loss pass
  hipLaunchKernelGGL(k_prep, dim3((unsigned)N), dim3(64), 0, st, tokens, C, eos_id,
                     (const float*)nullptr, (int64_t)1, 0, w.len, (float*)nullptr, (uint8_t*)nullptr,
                     (int32_t*)nullptr, (uint8_t*)nullptr, (float*)nullptr, (int32_t*)nullptr,
                     (uint32_t*)nullptr);
  if ((rc = launch_status()) != DRGRPO_OK) return rc;
  hipLaunchKernelGGL(k_lm_offsets, dim3(1), dim3(1024), 0, st, w.len, (const float*)nullptr, N,
                     0.0f, w.offs, w.counts);
  if ((rc = launch_status()) != DRGRPO_OK) return rc;
  hipLaunchKernelGGL(k_lm_gather, dim3((unsigned)(N * ((C + kGatherTok - 1) / kGatherTok))),
                     dim3(256), 0, st, static_cast<const uint16_t*>(hidden), H, tokens, C, V,
                     w.len, w.offs,
                     w.act_pos, w.ycol, w.Ha, T * 32, (double*)nullptr, (uint8_t*)nullptr);
  if ((rc = launch_status()) != DRGRPO_OK) return rc;
  hipLaunchKernelGGL(k_lm_logp_tail, dim3((unsigned)N), dim3(256), 0, st, w.len, C, out_logp);
  if ((rc = launch_status()) != DRGRPO_OK) return rc;
  GemmArgs g = {};
  g.A = w.Ha;
  g.ar = 32;
  g.ak = T * 32;
  g.B = static_cast<const uint16_t*>(W);
  g.br = H;
  g.bk = 32;
  g.M = T;
  g.N = V;
  g.K = H;
  g.M_dev = w.counts;
  g.part = w.part;
  g.ntn = ntn;
  g.xy = w.xy;
  g.ycol = w.ycol;
  g.col_base = 0;
  // sums relative to each token's sampled logit (no exponentials kept); a
  // call with a row beyond that reference's window redoes every tile
  // relative to its maxima
  hipLaunchKernelGGL(k_lm_mref, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, st, w.Ha, T * 32,
                     static_cast<const uint16_t*>(W), H, w.counts, w.ycol, w.mref, w.rowmark,
                     w.flag);
  if ((rc = launch_status()) != DRGRPO_OK) return rc;
  g.mref = w.mref;
  g.rowmark = w.rowmark;
  g.flag = w.flag;
  g.run_if = w.flag;
  if ((rc = launch_gemm<GM_LSE_E>(g, st)) != DRGRPO_OK) return rc;
  if ((rc = launch_rerun<GM_LSE>(g, st)) != DRGRPO_OK) return rc;
  hipLaunchKernelGGL(k_lm_logp, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, st, w.part, ntn,
                     w.xy, w.counts, w.act_pos, w.ycol, out_logp);
  return launch_status();
}
