/*
 * drgrpo.h - C ABI of the fused Dr. GRPO update loss for AMD Instinct MI355X
 * (gfx950).
 *
 * The library computes, for a rollout batch of N = B*G completions of C
 * tokens each (G completions per prompt, stored as G consecutive rows), the
 * Dr. GRPO loss and its gradient with respect to the policy logits, in one
 * stream-ordered call, without materialising log_softmax.
 *
 * Definitions ("Making Dr GRPO go brrr", sections named per call below):
 *   len_i   = index of the first EOS in row i, plus one; C if the row has no
 *             EOS ("The completion mask": first EOS inclusive, a row without
 *             EOS counts every token).  mask[i,t] = t < len_i.
 *   A_i     = R_i - mean of R over row i's group, no division by the group
 *             standard deviation ("Dr. GRPO"); binary32, sequential group sum.
 *   logp    = x[y] - logsumexp(x), where x = logits[i,t,:] and y = tokens[i,t]
 *             ("compute_logprobs"): the logits passed in are the completion
 *             slice, so logits row t scores token t.
 *   r       = exp(logp - logp_old)                                  ("PPO")
 *   s       = min(r*A, clip(r, 1-eps, 1+eps)*A)        ("PPO", "The loss")
 *   k3      = exp(d) - d - 1 with d = logp_ref - logp   (KL term, beta > 0)
 *   lambda  = -s + beta*k3 per token; the mask multiplies lambda ("The loss")
 *   L       = (sum over mask=1 tokens of lambda) / norm_const  ("Dr. GRPO":
 *             token sum divided by a fixed constant)
 *   dlogits = dL/dlogits = coef*(softmax(x) - onehot(y)), coef = -g/norm_const
 *             with g = dlambda/dlogp = -A*r*chi + beta*(1 - exp(d)), chi = 0
 *             when the clip cuts the surrogate ((A>0 and r>1+eps) or (A<0 and
 *             r<1-eps)), 1 otherwise.
 * A token is "active" when mask = 1 and (A != 0 or beta != 0).  Inactive
 * tokens contribute exactly 0 to L and to dlogits; their logits are not read.
 *
 * Conventions for every call:
 *   - Pointers are device pointers owned by the caller unless stated.  The
 *     library allocates no device memory and keeps no global state, except
 *     the static scratch array of drgrpo_loss_fwd_bwd_noalloc.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued on it; no call synchronises except
 *     drgrpo_device_status.  Results are valid once the stream has reached
 *     the end of the call.  Every call except drgrpo_device_status only
 *     enqueues kernels (no memset, no host synchronisation, no host read of
 *     device data), so it can be captured into a HIP graph and replayed; the
 *     workspace is re-initialised by the captured kernels themselves.
 *   - Host-side argument errors are returned before anything is enqueued.
 *   - Layouts are dense row-major: logits/dlogits [N, C, V]; tokens, logp_old,
 *     logp_ref [N, C]; rewards [N].
 */
#ifndef DRGRPO_H
#define DRGRPO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of logits and dlogits.  The two range markers are no element
 * type: they make every 32-bit value a value of the type, so a C caller's
 * out-of-range value reaches the C++ implementation as a defined value and is
 * rejected with DRGRPO_ERR_DTYPE (without them C++ only defines the values 0
 * and 1 for this enumeration). */
typedef enum {
  DRGRPO_F32 = 0,
  DRGRPO_BF16 = 1,
  DRGRPO_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  DRGRPO_DTYPE_RANGE_MAX_ = 2147483647
} drgrpo_dtype_t;

/* Status codes (0 = success, negative = error). */
enum {
  DRGRPO_OK = 0,
  DRGRPO_ERR_NULL = -1,        /* a required pointer is NULL */
  DRGRPO_ERR_SHAPE = -2,       /* N, C, V, G <= 0, N % G != 0, or a size overflows */
  DRGRPO_ERR_PARAM = -3,       /* eps, beta or norm_const invalid (see each call) */
  DRGRPO_ERR_DTYPE = -4,       /* unknown drgrpo_dtype_t */
  DRGRPO_ERR_WORKSPACE = -5,   /* workspace NULL, too small or not 256-byte aligned */
  DRGRPO_ERR_ALIGN = -6,       /* a pointer lacks the alignment the call requires */
  DRGRPO_ERR_HIP = -7,         /* a HIP launch failed */
  DRGRPO_ERR_TOKEN_RANGE = -8, /* device-side: a token at a mask=1 position is outside [0, V) */
  DRGRPO_ERR_ALIAS = -9,       /* out_dlogits partially overlaps logits */
  DRGRPO_ERR_SCRATCH_LIMIT = -10 /* sizes exceed the static scratch of
                                    drgrpo_loss_fwd_bwd_noalloc */
};

/* Bytes of device workspace drgrpo_loss_fwd_bwd needs for these sizes (0 if
 * the sizes are invalid).  The workspace is caller-owned, 256-byte aligned,
 * needs no initialisation, and holds the device status word read by
 * drgrpo_device_status.  One workspace must not be used by two calls that
 * can run concurrently. */
size_t drgrpo_workspace_bytes(int64_t N, int64_t C, int64_t V, int64_t G);

/* Dr. GRPO loss forward and backward over raw logits.
 *
 *   logits      [N, C, V] of `dtype`; row t scores tokens[:, t].
 *   tokens      [N, C] int64 completion ids; positions after the first EOS
 *               are never read as vocabulary indices.
 *   eos_id      EOS id; a value outside [0, V) means no row ends early.
 *   rewards     [N] float; group b is rows [b*G, (b+1)*G).
 *   logp_old    [N, C] float log-probs of the policy that sampled the batch.
 *   logp_ref    [N, C] float reference-policy log-probs; may be NULL iff
 *               beta == 0.
 *   G           completions per prompt (N % G == 0).
 *   eps         clip half-width, finite and >= 0.
 *   beta        KL weight, finite and >= 0.
 *   norm_const  the aggregation constant, finite and > 0 (G*C reproduces a
 *               per-group token sum divided by C; B*G a mean over completions).
 *   out_loss    [1] float on the device: L rounded to binary32 (NaN when a
 *               device-side error occurred).
 *   out_dlogits [N, C, V] of `dtype`, fully overwritten; may be exactly
 *               `logits` (in place), any other overlap is DRGRPO_ERR_ALIAS.
 *               bfloat16 results are rounded to nearest even from binary32.
 *   workspace   device buffer of drgrpo_workspace_bytes(N, C, V, G) bytes.
 *
 * The logits may have any V up to 2^28; rows whose byte size is a multiple of
 * 16 with 16-byte aligned bases take the vector path, others the element
 * path.  One workgroup runs per token row, so N*C is limited to 2^24 - 1
 * rows for V <= 4864 and to 2^22 - 1 rows above (DRGRPO_ERR_SHAPE).
 * Device-side errors (a token outside [0, V) at a mask=1 position) make the
 * loss and that token's dlogits row NaN and set the status word. */
int drgrpo_loss_fwd_bwd(const void* logits, const int64_t* tokens, int64_t eos_id,
                        const float* rewards, const float* logp_old, const float* logp_ref,
                        int64_t G, float eps, float beta, float norm_const, float* out_loss,
                        void* out_dlogits, int64_t N, int64_t C, int64_t V,
                        drgrpo_dtype_t dtype, void* workspace, size_t workspace_bytes,
                        void* stream);

/* drgrpo_loss_fwd_bwd for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops, harnesses that forbid hipMalloc):
 * the same arguments and results without the workspace, which comes from a
 * static device array of DRGRPO_NOALLOC_SCRATCH_BYTES per GPU instead.
 *
 *   - The call allocates nothing (no hipMalloc, hipFree or allocating library
 *     routine).  The first call on a device looks up that device's array
 *     (hipGetSymbolAddress); the array stays allocated until the process
 *     ends.  The current device (hipGetDevice) is used; `stream` must belong
 *     to it.
 *   - Sizes whose workspace (drgrpo_workspace_bytes) exceeds the array are
 *     rejected with DRGRPO_ERR_SCRATCH_LIMIT before anything is enqueued;
 *     every batch of at most 655,360 token rows (N*C) fits.
 *   - Every call on one GPU shares that GPU's array: calls that can run
 *     concurrently on one GPU (other streams, other threads) race and must
 *     not overlap.  No field needs clearing between calls.
 *   - A device-side error (a token outside [0, V) at a mask=1 position)
 *     makes the loss NaN; the status word lives in the static array, so
 *     drgrpo_device_status does not apply to this call. */
#define DRGRPO_NOALLOC_SCRATCH_BYTES (16u << 20)

int drgrpo_loss_fwd_bwd_noalloc(const void* logits, const int64_t* tokens, int64_t eos_id,
                                const float* rewards, const float* logp_old,
                                const float* logp_ref, int64_t G, float eps, float beta,
                                float norm_const, float* out_loss, void* out_dlogits, int64_t N,
                                int64_t C, int64_t V, drgrpo_dtype_t dtype, void* stream);

/* Normalisation variants ("Making Dr GRPO go brrr", sections "GRPO" and
 * "Dr. GRPO": Dr. GRPO deletes GRPO's division by the group standard
 * deviation and its per-response 1/|o_i| average).  NULL = Dr. GRPO. */
typedef enum {
  DRGRPO_ADV_CENTER = 0,  /* A_i = R_i - mean of the group                 (Dr. GRPO) */
  DRGRPO_ADV_ZSCORE = 1   /* A_i = (R_i - mean) / sample std of the group, divisor G-1;
                             0 for a group whose rewards are all equal     (GRPO) */
} drgrpo_adv_mode_t;
typedef enum {
  DRGRPO_AGG_TOKEN_SUM = 0,  /* L = sum_i sum_t lambda / norm_const                (Dr. GRPO) */
  DRGRPO_AGG_SEQ_MEAN = 1,   /* L = sum_i (sum_t lambda / |o_i|) / norm_const      (GRPO;
                                norm_const = N is the mean over completions) */
  DRGRPO_AGG_TOKEN_MEAN = 2  /* L = sum_i sum_t lambda / (norm_const * sum_i |o_i|)
                                (norm_const = 1 is the mean over counted tokens) */
} drgrpo_agg_mode_t;
typedef struct drgrpo_variant {
  int32_t adv_mode;  /* drgrpo_adv_mode_t */
  int32_t agg_mode;  /* drgrpo_agg_mode_t; |o_i| = len_i, the counted tokens of row i */
} drgrpo_variant_t;

/* Optional per-call diagnostics; every field may be NULL. */
typedef struct drgrpo_aux {
  int32_t* len;     /* [N] completion lengths */
  uint8_t* mask;    /* [N, C] completion mask (1 = counted) */
  float* adv;       /* [N] advantages */
  float* logp;      /* [N, C] log-probs of active tokens, 0 elsewhere */
  float* tok_loss;  /* [N, C] per-token lambda, 0 for inactive tokens */
  int32_t* stats;   /* [4] groups without reward contrast, rows without EOS,
                       active tokens with r outside [1-eps, 1+eps], active
                       tokens whose surrogate gradient the clip cuts */
} drgrpo_aux_t;

/* drgrpo_loss_fwd_bwd plus the diagnostics `aux` asks for (aux may be NULL). */
int drgrpo_loss_fwd_bwd_ex(const void* logits, const int64_t* tokens, int64_t eos_id,
                           const float* rewards, const float* logp_old, const float* logp_ref,
                           int64_t G, float eps, float beta, float norm_const, float* out_loss,
                           void* out_dlogits, int64_t N, int64_t C, int64_t V,
                           drgrpo_dtype_t dtype, void* workspace, size_t workspace_bytes,
                           void* stream, const drgrpo_aux_t* aux);

/* Further options of the loss call; every field may be NULL / 0. */
typedef struct drgrpo_loss_opts {
  const drgrpo_variant_t* variant; /* normalisation variant (NULL: Dr. GRPO; an unknown
                                      mode is DRGRPO_ERR_PARAM).  With a variant,
                                      coef = -g / div_i where div_i is row i's divisor
                                      above (norm_const, norm_const*len_i or
                                      norm_const*sum len) */
  int64_t* token_counts;  /* [2] on the device: counted tokens (sum of len), active
                             tokens (counted tokens of rows with A != 0, or all counted
                             tokens if beta > 0) */
  void* rows_event_begin; /* hipEvent_t stamped when the per-row kernel's dispatch
                             starts, to time it alone */
  void* rows_event_end;   /* hipEvent_t stamped when it ends */
  int32_t require_vector_path; /* nonzero: operands that would take the element path
                                  (row bytes not a multiple of 16, or logits / dlogits
                                  not 16-byte aligned) return DRGRPO_ERR_ALIGN
                                  before anything is enqueued */
} drgrpo_loss_opts_t;

/* drgrpo_loss_fwd_bwd_ex plus the options `opts` holds (opts may be NULL). */
int drgrpo_loss_fwd_bwd_opts(const void* logits, const int64_t* tokens, int64_t eos_id,
                             const float* rewards, const float* logp_old,
                             const float* logp_ref, int64_t G, float eps, float beta,
                             float norm_const, float* out_loss, void* out_dlogits, int64_t N,
                             int64_t C, int64_t V, drgrpo_dtype_t dtype, void* workspace,
                             size_t workspace_bytes, void* stream, const drgrpo_aux_t* aux,
                             const drgrpo_loss_opts_t* opts);

/* Completion mask alone ("The completion mask"): out_len [N] int32 (required),
 * out_mask [N, C] uint8 (may be NULL). */
int drgrpo_completion_mask(const int64_t* tokens, int64_t N, int64_t C, int64_t eos_id,
                           int32_t* out_len, uint8_t* out_mask, void* stream);

/* Group advantages alone ("Dr. GRPO": A_i = R_i - group mean): out_adv [N]
 * float (required); out_nocontrast [1] int32 (may be NULL) receives the
 * number of groups whose rewards are all equal ("The sparse-reward
 * bottleneck" of "The Quiet Library"). */
int drgrpo_group_advantage(const float* rewards, int64_t N, int64_t G, float* out_adv,
                           int32_t* out_nocontrast, void* stream);

/* drgrpo_group_advantage with an advantage mode: DRGRPO_ADV_CENTER (the
 * same result) or DRGRPO_ADV_ZSCORE ("GRPO": divided by the group's sample
 * standard deviation); another value is DRGRPO_ERR_PARAM. */
int drgrpo_group_advantage_ex(const float* rewards, int64_t N, int64_t G, int32_t adv_mode,
                              float* out_adv, int32_t* out_nocontrast, void* stream);

/* Forward-only log-probs of every token ("compute_logprobs"), the no-gradient
 * pass that produces logp_old / logp_ref: out_logp [N, C] float.  A token
 * outside [0, V) gives NaN. */
int drgrpo_logprobs(const void* logits, const int64_t* tokens, int64_t N, int64_t C, int64_t V,
                    drgrpo_dtype_t dtype, float* out_logp, void* stream);

/* Fused lm_head variant: the same loss with logits = hidden . W^T computed
 * on the fly ("compute_logprobs" of "Making Dr GRPO go brrr": the model's
 * final projection feeds the log-softmax), never stored as a [N*C, V] tensor.
 *
 *   hidden      [N*C, H] bfloat16: the policy's final hidden state at the
 *               position that scores completion token t (row i*C + t).
 *   W           [V, H] bfloat16 unembedding (lm_head weight).
 *   out_dhidden [N*C, H] bfloat16 = dL/dhidden = dlogits . W (zero rows for
 *               tokens without gradient; NaN rows for a bad token id).
 *   out_dW      [V, H] bfloat16 = dL/dW = dlogits^T . hidden.
 *   H must be a multiple of 32 and at most 65536, V a multiple of 8 and
 *   N*C at most 2^24 (else DRGRPO_ERR_SHAPE); hidden, W and the outputs
 *   16-byte aligned (else DRGRPO_ERR_ALIGN).  Other arguments as for
 *   drgrpo_loss_fwd_bwd.  Logits accumulate in binary32 on the matrix cores;
 *   the forward keeps E = exp(logit - r) of every active token's logits in
 *   bfloat16 (relative rounding 2^-8), r one reference per token (its sampled
 *   token's logit; its largest logit when that lies more than 48 above, found
 *   by a second pass of the forward product for such calls).  Each token's
 *   dlogits are a factor s = coef exp(r - lse) times E (the sampled entry
 *   adjusted), so the dhidden product reads E and scales its result rows by
 *   s, and the dW product reads E against the hidden rows scaled by s and
 *   rounded to bfloat16, one vocabulary chunk at a time.
 * The workspace (drgrpo_lmhead_workspace_bytes) holds the active tokens'
 * hidden rows (and their scaled transpose), those exponentials (2 bytes per
 * token row and vocabulary entry: 10 GB at N*C = 32768, V = 151936) and one
 * vocabulary chunk of W transposed. */
size_t drgrpo_lmhead_workspace_bytes(int64_t N, int64_t C, int64_t V, int64_t H, int64_t G);

int drgrpo_lmhead_loss_fwd_bwd(const void* hidden, const void* W, const int64_t* tokens,
                               int64_t eos_id, const float* rewards, const float* logp_old,
                               const float* logp_ref, int64_t G, float eps, float beta,
                               float norm_const, float* out_loss, void* out_dhidden,
                               void* out_dW, int64_t N, int64_t C, int64_t V, int64_t H,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Optional timing hooks of the fused lm_head call; every field may be NULL. */
typedef struct drgrpo_lmhead_aux {
  void* fwd_event_begin;  /* hipEvent_t stamped when the dispatch of the forward
                             (log-sum-exp over the whole vocabulary) product starts */
  void* fwd_event_end;    /* hipEvent_t stamped when it ends */
} drgrpo_lmhead_aux_t;

/* drgrpo_lmhead_loss_fwd_bwd with a normalisation variant (NULL: Dr. GRPO),
 * as in drgrpo_loss_opts_t, and optional timing hooks (aux may be NULL). */
int drgrpo_lmhead_loss_fwd_bwd_ex(const void* hidden, const void* W, const int64_t* tokens,
                                  int64_t eos_id, const float* rewards, const float* logp_old,
                                  const float* logp_ref, int64_t G, float eps, float beta,
                                  float norm_const, float* out_loss, void* out_dhidden,
                                  void* out_dW, int64_t N, int64_t C, int64_t V, int64_t H,
                                  void* workspace, size_t workspace_bytes, void* stream,
                                  const drgrpo_variant_t* variant,
                                  const drgrpo_lmhead_aux_t* aux);

/* Forward-only log-probs through the fused lm_head, for the no-gradient
 * old-policy and reference-policy passes of the "Dr. GRPO" pseudo-code
 * ("compute_logprobs": log_softmax of the final projection, gathered at the
 * sampled token), without storing the [N*C, V] logits.
 *
 *   hidden   [N*C, H] bfloat16 (row i*C + t scores tokens[i, t]); W [V, H]
 *            bfloat16; both 16-byte aligned (else DRGRPO_ERR_ALIGN).
 *   tokens   [N, C] int64; eos_id as for drgrpo_loss_fwd_bwd: log-probs are
 *            computed for the counted tokens (up to and including the first
 *            EOS; every token when eos_id is outside [0, V)).
 *   out_logp [N, C] float: x[y] - logsumexp(x) with x = hidden_row . W^T in
 *            binary32 MFMA accumulation; 0 at positions after the first EOS;
 *            NaN for a counted token outside [0, V).
 *   Shape limits as for drgrpo_lmhead_loss_fwd_bwd.  The workspace
 *   (drgrpo_lmhead_logprobs_workspace_bytes, 256-byte aligned, no
 *   initialisation) holds the counted tokens' hidden rows and per-tile
 *   partial sums. */
size_t drgrpo_lmhead_logprobs_workspace_bytes(int64_t N, int64_t C, int64_t V, int64_t H);

int drgrpo_lmhead_logprobs(const void* hidden, const void* W, const int64_t* tokens,
                           int64_t eos_id, int64_t N, int64_t C, int64_t V, int64_t H,
                           float* out_logp, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Decode attention of the rollout step ("Making Dr GRPO go brrr", section
 * "What is RL post-training, and why is it slow": one forward pass per
 * generated token on a (B*G, 1, hidden) input plus a growing KV cache; this
 * is that step's scaled dot-product attention).  For sequence s and query
 * head h, with key/value head g = h / (Hq / Hkv) and len_s cached positions:
 *   out[s,h] = sum_{j < len_s} softmax_j(scale * <q[s,h], K[s,g,j]>) V[s,g,j]
 *
 *   q        [S, Hq, D] bfloat16 (the new token's queries).
 *   k_cache  [S, Hkv, Lmax, D] bfloat16; v_cache likewise.  Positions
 *            j >= len_s are never read.
 *   lens     [S] int32 on the device: cached positions per sequence; values
 *            above Lmax count as Lmax, and len_s < 1 gives a NaN output (an
 *            empty softmax).
 *   scale    finite and > 0 (1/sqrt(D) for standard attention).
 *   out      [S, Hq, D] bfloat16 (binary32 accumulation, rounded to nearest
 *            even); out_lse [S, Hq] float log-sum-exp of the scores, may be
 *            NULL.
 *   D is 64 or 128, Hq a multiple of Hkv with Hq / Hkv <= 16, and one
 *   (sequence, key/value head) cache region Lmax * D * 2 bytes below 2^31
 *   (else DRGRPO_ERR_SHAPE); q, the caches and out 16-byte aligned (else
 *   DRGRPO_ERR_ALIGN).  The workspace (drgrpo_decode_attention_workspace_bytes,
 *   256-byte aligned, no initialisation) holds the per-split partial
 *   results; calls that share a workspace must not overlap.  The call only
 *   enqueues kernels (no memset, no host synchronisation), so it can be
 *   captured into a graph. */
size_t drgrpo_decode_attention_workspace_bytes(int64_t S, int64_t Hq, int64_t Hkv, int64_t Lmax,
                                               int64_t D);

int drgrpo_decode_attention(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* lens, int64_t S, int64_t Hq, int64_t Hkv, int64_t Lmax,
                            int64_t D, float scale, void* out, float* out_lse, void* workspace,
                            size_t workspace_bytes, void* stream);

/* The attention block of the same decode step with the rotary position
 * embedding and the cache append folded in (the step between the q/k/v
 * projection and the output projection: the new token's keys and values are
 * appended to the cache before it is read).  For sequence s with position
 * p = pos[s] in [0, Lmax):
 *   qkv      [S, (Hq + 2 Hkv) * D] bfloat16: the projection output, per
 *            sequence Hq query heads, then Hkv key heads, then Hkv value
 *            heads, each D contiguous (2-byte aligned).
 *   rope_cos, rope_sin  [Lmax, D/2] float: cosine and sine of the angle of
 *            pair i at each position (the caller's frequencies; Qwen2.5
 *            uses p * base^(-2i/D), base 10^6).
 *   pos      [S] int32 on the device.
 *   Each head vector x is rotated in the rotate-half form: for i < D/2,
 *     x'_i = x_i c - x_{i+D/2} s,  x'_{i+D/2} = x_{i+D/2} c + x_i s
 *   with (c, s) = (rope_cos[p, i], rope_sin[p, i]), in binary32 with each
 *   product and the sum rounded separately, then rounded to bfloat16 (nearest
 *   even).  The rotated key heads and the value heads are written to
 *   k_cache / v_cache at [s, g, p] (nothing else in the caches changes), and
 *   out[s] is drgrpo_decode_attention of the rotated queries over p + 1
 *   cached positions (same layouts, scale, out_lse and accuracy).  A
 *   position outside [0, Lmax) writes nothing and gives a NaN output row.
 * Errors as drgrpo_decode_attention (caches and out 16-byte aligned); the
 * workspace (drgrpo_decode_attention_rope_workspace_bytes, 256-byte aligned)
 * also holds the rotated queries and the lengths.  Only enqueues kernels;
 * calls that share a workspace or a cache must not overlap. */
size_t drgrpo_decode_attention_rope_workspace_bytes(int64_t S, int64_t Hq, int64_t Hkv,
                                                    int64_t Lmax, int64_t D);

int drgrpo_decode_attention_rope(const void* qkv, const float* rope_cos, const float* rope_sin,
                                 const int32_t* pos, int64_t S, int64_t Hq, int64_t Hkv,
                                 int64_t Lmax, int64_t D, float scale, void* k_cache,
                                 void* v_cache, void* out, float* out_lse, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Synchronises `stream`, then reads the status word the last
 * drgrpo_loss_fwd_bwd call on `workspace` left: DRGRPO_OK or
 * DRGRPO_ERR_TOKEN_RANGE (DRGRPO_ERR_HIP if the read fails). */
int drgrpo_device_status(const void* workspace, void* stream);

/* Static, human-readable text of a status code. */
const char* drgrpo_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* DRGRPO_H */
