// Internal host interface between the C-ABI layer (dsa_api.cpp) and the
// kernel translation units.  Plans depend only on host-known arguments, so
// workspace queries and launches always agree.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

// ---------------------------------------------------------------- indexer
struct IndexerLaunch {
  const void* q_idx;
  const float* w_idx;
  const void* key_state;
  const int32_t* kv_len;
  float* scores;
  int B, S, H, D_idx, L_cap;
  bool bf16;
  bool prefill;     // S > 8: 8-wave workgroups streaming key runs
  bool stream_decode;  // long decode context: 4-wave workgroups streaming key runs
  bool fold;        // prefill: head weights folded into the query (indexer_fold_kernel)
  int pairs;        // token pairs per wave (1 or 2)
  int waves;        // waves per workgroup
  int tile;         // keys per LDS buffer
  int tok_blocks;   // grid.x
  int keys_per_wg;  // keys per workgroup
  int key_blocks;   // grid.y
};
// Largest L_cap the indexer supports (32-bit byte offsets of score stores).
constexpr int kIndexerMaxLcap = 1 << 27;
IndexerLaunch plan_indexer(int B, int S, int D_idx, int L_cap, int max_kv_len);
void launch_indexer(const IndexerLaunch& a, hipStream_t st);

// ---------------------------------------------------------------- top-k
struct TopkPlan {
  int kind;            // streaming / resident / split / small
  int rows;            // B*S
  int chunk;           // keys per chunk workgroup (split)
  int chunks;          // chunks per row of L_cap keys (split; the workspace's layout)
  int sample;          // sampled keys per row (split)
  int cap;             // candidate slots per chunk (split)
  int spec;            // slots per chunk the select kernel loads up front (split; 0: none)
  int entries;         // candidates per lane of the select kernel's fast path (split)
  int exact_only;      // k beyond the candidate list: exact selection over whole rows
  int lane_keys;       // keys per thread (small)
  size_t ws_bytes;     // workspace the plan needs
};
TopkPlan plan_topk(int B, int S, int L_cap, int max_kv_len, int k);
void launch_topk(const TopkPlan& p, const float* scores, const int32_t* kv_len, int S,
                 int L_cap, int max_kv_len, int k, int32_t* indices, void* ws, hipStream_t st);

// ---------------------------------------------------------------- attention
enum DType { kF32 = 0, kF16 = 1, kBF16 = 2, kI8 = 3 };

struct AttnLaunch {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* indices;
  const int32_t* kv_len;
  void* out;
  float* part;        // decode partials (nsplit > 1), else null
  int q_dtype, kv_dtype, out_dtype;
  int B, S, H_q, H_kv, D, L_cap, k;
  float scale;
  int nsplit;         // key splits per (row, KV head)
  int keys_per_split;
  const void* aux_k;  // auxiliary (not yet cached) K/V [B, aux_len, H_kv, D], or null
  const void* aux_v;
  int aux_dtype, aux_len;
  int wave_rows;      // prefill: each wave owns a whole (row, KV head)
};
// nsplit/keys_per_split for the decode form; prefill uses nsplit = 1.  Set
// aux_len first: auxiliary keys take one merge slot.
void plan_attention(AttnLaunch& a, bool decode);
size_t attention_partials_bytes(const AttnLaunch& a);
void launch_attention(const AttnLaunch& a, hipStream_t st);
// Built-in scratch of the allocation-free decode entry point: its size, and
// the current device's copy (device address; null with *err set on failure).
constexpr size_t kAttnScratchBytes = (size_t)16 << 20;
float* attention_scratch(hipError_t* err);

// ---------------------------------------------------------------- cache append
struct CacheAppendLaunch {
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  float* k_scale;
  float* v_scale;
  const void* key_state_new;
  void* key_state;          // null: no key-state rows
  const int32_t* kv_len;
  int new_dtype, kv_dtype;
  int B, S, H_kv, D, D_idx, L_cap;
};
void launch_cache_append(const CacheAppendLaunch& a, hipStream_t st);

// ---------------------------------------------------------------- RMSNorm + rotary
struct RopeLaunch {
  const void* x;
  const float* gamma;
  const float* cos_cache;
  const float* sin_cache;
  const int32_t* kv_len;
  void* out;
  int x_dtype, out_dtype;
  int B, S, H, D, max_pos;
  float eps;
  int interleaved;
};
// Up to kRopeMaxJobs independent jobs in one launch (jobs without rows are
// skipped).
constexpr int kRopeMaxJobs = 4;
void launch_rmsnorm_rope(const RopeLaunch* jobs, int n, hipStream_t st);

}  // namespace dsa
