/*
 * dsa.h -- C ABI of the dynamic sparse GQA attention library (libdsa.so).
 *
 * Dynamic sparse attention runs in three stages: an indexer scores every
 * cached token against each query token, a per-query top-k selects keys, and
 * softmax attention runs over the selected keys only ("selected only"
 * attention with grouped query heads: ORT PR #33997 "Support FP16 KV cache
 * and FP16 query/key in DynamicSparseAttention<BFloat16> ...", Description
 * item 2 and its test list; ORT PR #33802 "Optimize Qwen3.8-Flash-Next DSA,
 * Indexer, HC, and QMoE kernels for SM12x and 256K context", Summary
 * items 1-2).
 *
 * Conventions shared by every entry point
 *  - Every tensor pointer is DEVICE memory owned by the caller, dense and
 *    row-major in the layout stated, with a 16-byte-aligned base address.
 *  - The library never allocates, frees or synchronises.  Calls validate
 *    their arguments on the host, enqueue kernels on `stream` (a hipStream_t
 *    passed as void*; NULL is the null stream) and return.  Enqueued work is
 *    ordered on that stream only.
 *  - Validation happens before any launch: a non-OK status means nothing was
 *    enqueued and nothing was written.  dsa_last_error() then describes it.
 *  - The library keeps no state between calls.  Workspace contents on entry
 *    are never trusted (each call initialises what it reads).
 *  - Per-sequence live length kv_len[b] lives on the device; the host passes
 *    an upper bound max_kv_len (<= L_cap) that sizes the launch grids.
 *    Query token s of sequence b sits at position pos(b,s) = kv_len[b]-S+s
 *    and may attend to keys 0..pos(b,s) (its own key included).
 *    Device preconditions (not checkable on the host):
 *    S <= kv_len[b] <= max_kv_len.  Rows with pos < 0 select no key.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 2

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARGUMENT = 1,    /* null pointer, bad size or shape        */
  DSA_ERR_UNSUPPORTED = 2,         /* valid but unimplemented combination    */
  DSA_ERR_MISALIGNED = 3,          /* a base pointer is not 16-byte aligned  */
  DSA_ERR_WORKSPACE_TOO_SMALL = 4, /* workspace smaller than the query says  */
  DSA_ERR_HIP = 5                  /* a HIP runtime call or launch failed    */
} dsa_status;

typedef enum { DSA_F32 = 0, DSA_F16 = 1, DSA_BF16 = 2, DSA_I8 = 3 } dsa_dtype;

/* DSA_ABI_VERSION of the built library. */
int dsa_abi_version(void);

/* Text of the last non-OK status returned on the calling thread ("" if none).
 * The pointer stays valid until the next call on that thread. */
const char* dsa_last_error(void);

/*
 * Indexer score (ORT PR #33802, Summary item 2: per-head scoring of the
 * key-state cache reduced over the indexer heads).
 *
 *   scores[b,s,j] = sum_h w_idx[b,s,h] * sum_d q_idx[b,s,h,d] * key_state[b,j,d]
 *
 * for 0 <= j <= pos(b,s).  Accumulation is FP32; with integer-valued inputs
 * whose partial sums stay below 2^24 the result is exact.
 *   q_idx      [B, S, H_idx, D_idx]  idx_dtype (DSA_BF16 or DSA_F16)
 *   w_idx      [B, S, H_idx]         FP32
 *   key_state  [B, L_cap, D_idx]     idx_dtype
 *   kv_len     [B]                   int32, device
 *   scores     [B, S, L_cap]         FP32, written for j < kv_len[b];
 *              entries pos < j < kv_len[b] hold finite values that mean
 *              nothing, entries j >= kv_len[b] are left untouched.
 * Supported: 1 <= H_idx <= 16, D_idx in {32, 64, 128}, L_cap <= 2^27
 * (DSA_ERR_UNSUPPORTED otherwise).
 */
dsa_status dsa_indexer_score(const void* q_idx, const float* w_idx,
                             const void* key_state, dsa_dtype idx_dtype,
                             const int32_t* kv_len, int B, int S, int H_idx,
                             int D_idx, int L_cap, int max_kv_len,
                             float* scores, void* stream);

/*
 * Per-query top-k (ORT PR #33802, Summary item 2: chunked radix histograms
 * merged across up to 64+ chunks, then emitted).
 *
 * For row (b,s) the candidates are j = 0..pos(b,s).  The k highest scores
 * are kept, equal scores broken toward the LOWER index; the kept indices are
 * written in ascending order, and slots beyond the number of candidates hold
 * -1.  -0.0 ranks equal to +0.0; -inf is allowed; NaN is not supported.
 *   scores   [B, S, L_cap]  FP32 (only j <= pos(b,s) is read)
 *   indices  [B, S, k]      int32 output
 *   workspace: at least dsa_topk_workspace_bytes(B, S, L_cap, k) bytes of
 *   device memory (may be NULL when that is 0); contents on entry are
 *   ignored, contents on return are unspecified.
 * Supported: k >= 1 (k may exceed L_cap: the tail is -1), L_cap <= 2^24.
 */
size_t dsa_topk_workspace_bytes(int B, int S, int L_cap, int k);
dsa_status dsa_topk(const float* scores, const int32_t* kv_len, int B, int S,
                    int L_cap, int max_kv_len, int k, int32_t* indices,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Sparse GQA attention over selected keys (ORT PR #33997, Description item 2;
 * ORT PR #33802, Summary item 1 and follow-up #33847 on the rising running
 * maximum).  For query head h of row (b,s), with g = h / (H_q / H_kv):
 *
 *   logit_j = softmax_scale * sum_d q[b,s,h,d] * K[b,j,g,d]
 *   out[b,s,h,:] = sum_j p_j V[b,j,g,:] / sum_j p_j,  p_j = exp(logit_j - max)
 *
 * over the valid entries j of indices[b,s,:]: 0 <= j <= pos(b,s) and
 * j < L_cap.  Invalid entries (-1 padding included) are skipped.  Entries
 * must be unique.  A row with no valid entry is written as zeros.
 * INT8 cache: K = code * k_scale[b,j,g], V = code * v_scale[b,j,g]
 * (symmetric, no zero point).
 *
 *   q        [B, S, H_q, D]      q_dtype
 *   k_cache  [B, L_cap, H_kv, D] kv_dtype
 *   v_cache  [B, L_cap, H_kv, D] kv_dtype
 *   k_scale, v_scale [B, L_cap, H_kv] FP32 for DSA_I8, NULL otherwise
 *   indices  [B, S, k]           int32
 *   kv_len   [B]                 int32, device
 *   out      [B, S, H_q, D]      out_dtype, rounded to nearest-even
 * Supported combinations: q/kv/out all DSA_F32; or q in {F16, BF16} with
 * kv in {F16, BF16, I8} and out in {F32, F16, BF16}.  D in {64, 128};
 * H_q % H_kv == 0 and H_q / H_kv <= 16.  With an F16 cache (or F16 query
 * against a BF16 cache) both operands are multiplied as FP16: query values
 * must lie within FP16 range.
 * softmax_scale <= 0 selects 1/sqrt(D).
 *
 * Auxiliary K/V (ORT PR #33997 review and follow-up: fresh keys and values
 * kept in their own floating type next to the main cache, taking part in the
 * same softmax): aux_k, aux_v [B, aux_len, H_kv, D] in aux_dtype (F32, F16 or
 * BF16; F32 when q is F32) hold the tokens at positions
 * kv_len[b] - aux_len + t, which the cache does not hold yet.  Query (b,s)
 * then attends to (i) its selected cache keys j < kv_len[b] - aux_len (cache
 * entries in the aux range are ignored) and (ii) the aux tokens whose
 * position is <= pos(b,s), in one softmax.  Aux values are never converted
 * to the cache dtype: products run in their 16-bit type when the query has
 * it (a BF16 query against F16 aux multiplies in FP16, as against an F16
 * cache), otherwise in FP32.  Precondition: aux_len <= kv_len[b].  With aux
 * keys both forms need workspace.
 *
 * decode: the selected keys of each row are split over several workgroups
 * whose partial softmax states are merged exactly in a second kernel; it
 * needs dsa_attention_workspace_bytes(args, 1) bytes of workspace.
 * prefill: one workgroup per (row, KV head); no workspace (size 0).
 * Both accept any S and compute the same function.
 */
typedef struct {
  const void* q;        int32_t q_dtype;
  const void* k_cache;  const void* v_cache;  int32_t kv_dtype;
  const float* k_scale; const float* v_scale;
  const int32_t* indices; int32_t k;
  const int32_t* kv_len;
  int32_t B, S, H_q, H_kv, D, L_cap, max_kv_len;
  float softmax_scale;
  void* out;            int32_t out_dtype;
  /* Auxiliary K/V (aux_len = 0: none); see below. */
  const void* aux_k;    const void* aux_v;    int32_t aux_dtype;
  int32_t aux_len;
} dsa_attention_args;

/* Workspace bytes dsa_attention_decode (is_decode != 0) or _prefill needs
 * for these arguments; depends on sizes and dtypes only (the pointers are not
 * read and may be NULL); 0 when none is needed or the arguments are invalid. */
size_t dsa_attention_workspace_bytes(const dsa_attention_args* args, int is_decode);
dsa_status dsa_attention_decode(const dsa_attention_args* args, void* workspace,
                                size_t workspace_bytes, void* stream);
dsa_status dsa_attention_prefill(const dsa_attention_args* args, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * Launch plans (no device work).  Describes, as one line of "key=value"
 * words, the kernels, grids and tiling that the call `op` would launch for
 * these arguments -- the planning the call itself does, so tests and logs
 * can see which plan runs without a profiler.
 *   DSA_PLAN_INDEXER:  B, S, L_cap, max_kv_len, D_idx (as dsa_indexer_score)
 *   DSA_PLAN_TOPK:     B, S, L_cap, max_kv_len, k    (as dsa_topk)
 *   DSA_PLAN_ATTENTION_DECODE / _PREFILL: `attention` (its pointers are not
 *                      read and may be NULL)
 * Arguments an op does not use are ignored.  Writes at most buf_bytes - 1
 * characters and a NUL to buf (NULL with buf_bytes 0 only measures).
 * Returns the description's full length, or 0 for invalid arguments, with
 * dsa_last_error() saying why.  Makes no HIP call.
 */
typedef enum {
  DSA_PLAN_INDEXER = 0,
  DSA_PLAN_TOPK = 1,
  DSA_PLAN_ATTENTION_DECODE = 2,
  DSA_PLAN_ATTENTION_PREFILL = 3
} dsa_plan_op;
size_t dsa_describe_plan(int op, int B, int S, int L_cap, int max_kv_len, int k, int D_idx,
                         const dsa_attention_args* attention, char* buf, size_t buf_bytes);

/*
 * Allocation-free variant of dsa_attention_decode, for callers that cannot
 * allocate device memory or pass a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * function and kernels as dsa_attention_decode; the split partials go to a
 * built-in scratch array of 16 MiB per GPU (held by the library for the life
 * of the process) instead of a caller workspace.  The call allocates and
 * frees nothing.  Calls whose partials (dsa_attention_workspace_bytes(args,
 * 1)) exceed 16 MiB are rejected with DSA_ERR_WORKSPACE_TOO_SMALL before any
 * launch.  Every call on a GPU shares that GPU's scratch: calls that overlap
 * in time on one GPU (several streams or threads) race and must be ordered
 * by the caller.  The scratch holds no state between calls (every partial
 * is written before it is read).
 */
dsa_status dsa_attention_decode_noalloc(const dsa_attention_args* args, void* stream);

/*
 * KV-cache append (ORT PR #33997, file table: cache writes precede the
 * attention kernels; ORT PR #33802, Summary item 1: an INT8 KV cache with one
 * FP32 scale per token per KV head).  Writes the S new tokens of every
 * sequence into the caches: token s of sequence b goes to position
 * pos = kv_len[b] - S + s, where kv_len is the length AFTER the append (the
 * same kv_len the indexer, top-k and attention calls of that step take);
 * tokens with pos outside [0, L_cap) are skipped.
 *   k_new, v_new    [B, S, H_kv, D]      new_dtype (F32, F16 or BF16)
 *   k_cache, v_cache [B, L_cap, H_kv, D] kv_dtype (F32, F16, BF16 or I8)
 *   k_scale, v_scale [B, L_cap, H_kv]    FP32, written for DSA_I8, NULL
 *                                        otherwise
 *   key_state_new   [B, S, D_idx]        idx_dtype (F16 or BF16), copied to
 *   key_state       [B, L_cap, D_idx]    idx_dtype; both NULL to skip
 *   kv_len          [B]                  int32, device
 * Float caches store each value rounded once to nearest-even.  An INT8 cache
 * stores, per (token, KV head) row x of D values, in FP32 arithmetic:
 *   scale = amax / 127 with amax = max_d |x_d|, and
 *   code_d = clamp(rint(x_d / scale), -127, 127)   (ties to even),
 * both quotients correctly rounded; an all-zero row stores scale 0 and zero
 * codes.  Non-finite inputs are not supported.
 * Supported: D in {64, 128}; D_idx in {32, 64, 128}; an F32 cache needs F32
 * new values.  Rows written by one call must not overlap (unique positions).
 */
typedef struct {
  const void* k_new;  const void* v_new;  int32_t new_dtype;
  void* k_cache;      void* v_cache;      int32_t kv_dtype;
  float* k_scale;     float* v_scale;
  const void* key_state_new; void* key_state; int32_t idx_dtype;
  const int32_t* kv_len;
  int32_t B, S, H_kv, D, D_idx, L_cap;
} dsa_cache_append_args;

dsa_status dsa_cache_append(const dsa_cache_append_args* args, void* stream);

/*
 * RMSNorm + rotary position embedding in FP32 (ORT PR #33997, Description
 * item 1: normalisation and rotation computed in FP32 with FP32 rotary
 * tables and no intermediate 16-bit rounding, then rounded once to the
 * FP16 or BF16 output).  For head vector x of token s of sequence b, at
 * position p = kv_len[b] - S + s:
 *   y_d   = gamma_d * x_d / sqrt(mean_d(x_d^2) + eps)
 *   pair i = (i, i + D/2) ("rotate half"), or (2i, 2i+1) when interleaved:
 *   out_a = y_a * cos[p,i] - y_b * sin[p,i]
 *   out_b = y_b * cos[p,i] + y_a * sin[p,i]
 * with correctly rounded FP32 square root and reciprocal.
 *   x                  [B, S, H, D]   x_dtype (F32, F16 or BF16)
 *   gamma              [D]            FP32
 *   cos_cache, sin_cache [max_pos, D/2] FP32
 *   kv_len             [B]            int32, device
 *   out                [B, S, H, D]   out_dtype (F32, F16 or BF16), RNE;
 *                      may alias x.  Rows whose position lies outside
 *                      [0, max_pos) are left untouched.
 * Supported: D in {32, 64, 128}; eps finite and >= 0.  Used on query heads, key
 * heads and indexer query heads alike (H is their head count).
 */
typedef struct {
  const void* x;          int32_t x_dtype;
  const float* gamma;
  const float* cos_cache; const float* sin_cache;
  const int32_t* kv_len;
  int32_t B, S, H, D, max_pos;
  float eps;              int32_t interleaved;
  void* out;              int32_t out_dtype;
} dsa_rmsnorm_rope_args;

dsa_status dsa_rmsnorm_rope(const dsa_rmsnorm_rope_args* args, void* stream);

/*
 * The same operation on up to 4 independent tensors in one kernel launch:
 * args points to `count` (1..4) argument blocks, each with the meaning,
 * limits and results of dsa_rmsnorm_rope.  A decode step rotates its query
 * heads, key heads and indexer query heads (different H and D), and this
 * call gives them a single launch.  Every block is validated before anything
 * is launched; a job with no rows is skipped.  A job's out may alias its own
 * x, but no job may write memory that another job of the call reads or
 * writes (the jobs run concurrently).  Errors: DSA_ERR_INVALID_ARGUMENT for
 * count outside [1, 4] or a NULL args; otherwise as dsa_rmsnorm_rope, the
 * message naming the job.
 */
dsa_status dsa_rmsnorm_rope_multi(const dsa_rmsnorm_rope_args* args, int32_t count, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
