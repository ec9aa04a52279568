// C ABI of libdsa: argument validation, launch planning and error reporting.
// Declarations and the contract of every entry point live in include/dsa.h.
// Validation touches no HIP API, so every rejected call returns before any
// device work is enqueued.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/dsa.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

dsa_status fail(dsa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

dsa_status ok() {
  g_last_error.clear();
  return DSA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

const char* dtype_name(int d) {
  switch (d) {
    case DSA_F32: return "F32";
    case DSA_F16: return "F16";
    case DSA_BF16: return "BF16";
    case DSA_I8: return "I8";
    default: return "unknown";
  }
}

dsa_status check_ptr(const void* p, const char* name) {
  if (!p) return fail(DSA_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (!aligned16(p)) return fail(DSA_ERR_MISALIGNED, "%s is not 16-byte aligned", name);
  return DSA_OK;
}

#define CHECK(expr)                    \
  do {                                 \
    dsa_status _s = (expr);            \
    if (_s != DSA_OK) return _s;       \
  } while (0)

dsa_status hip_result(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// ------------------------------------------------------------------ attention
// Shapes, dtypes and sizes (no pointers).
dsa_status validate_attention_shape(const dsa_attention_args* a) {
  if (!a) return fail(DSA_ERR_INVALID_ARGUMENT, "args is NULL");
  if (a->B < 0 || a->S < 0) return fail(DSA_ERR_INVALID_ARGUMENT, "B=%d S=%d must be >= 0", a->B, a->S);
  if (a->k < 0) return fail(DSA_ERR_INVALID_ARGUMENT, "k=%d must be >= 0", a->k);
  if (a->L_cap < 1) return fail(DSA_ERR_INVALID_ARGUMENT, "L_cap=%d must be >= 1", a->L_cap);
  if (a->max_kv_len < 0 || a->max_kv_len > a->L_cap)
    return fail(DSA_ERR_INVALID_ARGUMENT, "max_kv_len=%d outside [0, L_cap=%d]", a->max_kv_len, a->L_cap);
  if (a->H_q < 1 || a->H_kv < 1 || a->H_q % a->H_kv != 0)
    return fail(DSA_ERR_INVALID_ARGUMENT, "H_q=%d must be a positive multiple of H_kv=%d", a->H_q, a->H_kv);
  if (a->H_q / a->H_kv > 16)
    return fail(DSA_ERR_UNSUPPORTED, "group ratio H_q/H_kv=%d exceeds 16", a->H_q / a->H_kv);
  if (a->D != 64 && a->D != 128) return fail(DSA_ERR_UNSUPPORTED, "head dim D=%d not in {64, 128}", a->D);
  const int qd = a->q_dtype, kd = a->kv_dtype, od = a->out_dtype;
  const bool f32_combo = qd == DSA_F32 && kd == DSA_F32 && od == DSA_F32;
  const bool half_combo = (qd == DSA_F16 || qd == DSA_BF16) &&
                          (kd == DSA_F16 || kd == DSA_BF16 || kd == DSA_I8) &&
                          (od == DSA_F32 || od == DSA_F16 || od == DSA_BF16);
  if (!f32_combo && !half_combo)
    return fail(DSA_ERR_UNSUPPORTED, "dtype combination q=%s kv=%s out=%s is not supported",
                dtype_name(qd), dtype_name(kd), dtype_name(od));
  if (!std::isfinite(a->softmax_scale))
    return fail(DSA_ERR_INVALID_ARGUMENT, "softmax_scale is not finite");
  if ((long long)a->L_cap * a->H_kv * a->D >= (1LL << 40))
    return fail(DSA_ERR_UNSUPPORTED, "cache too large");
  if (a->aux_len < 0) return fail(DSA_ERR_INVALID_ARGUMENT, "aux_len=%d must be >= 0", a->aux_len);
  if (a->aux_len > 0) {
    const int ad = a->aux_dtype;
    if (qd == DSA_F32 ? ad != DSA_F32 : (ad != DSA_F32 && ad != DSA_F16 && ad != DSA_BF16))
      return fail(DSA_ERR_UNSUPPORTED, "auxiliary K/V dtype %s with q=%s is not supported",
                  dtype_name(ad), dtype_name(qd));
    if (a->aux_len > a->L_cap)
      return fail(DSA_ERR_INVALID_ARGUMENT, "aux_len=%d exceeds L_cap=%d", a->aux_len, a->L_cap);
  }
  return DSA_OK;
}

dsa_status validate_attention(const dsa_attention_args* a) {
  CHECK(validate_attention_shape(a));
  if ((long long)a->B * a->S == 0) return DSA_OK;
  const int kd = a->kv_dtype;
  if (a->aux_len > 0) {
    CHECK(check_ptr(a->aux_k, "aux_k"));
    CHECK(check_ptr(a->aux_v, "aux_v"));
  }
  CHECK(check_ptr(a->q, "q"));
  CHECK(check_ptr(a->k_cache, "k_cache"));
  CHECK(check_ptr(a->v_cache, "v_cache"));
  CHECK(check_ptr(a->kv_len, "kv_len"));
  CHECK(check_ptr(a->out, "out"));
  if (a->k > 0) CHECK(check_ptr(a->indices, "indices"));
  if (kd == DSA_I8) {
    CHECK(check_ptr(a->k_scale, "k_scale"));
    CHECK(check_ptr(a->v_scale, "v_scale"));
  } else if (a->k_scale || a->v_scale) {
    return fail(DSA_ERR_INVALID_ARGUMENT, "k_scale/v_scale must be NULL unless kv_dtype is I8");
  }
  return DSA_OK;
}

dsa::AttnLaunch make_attn(const dsa_attention_args* a, bool decode) {
  dsa::AttnLaunch l{};
  l.q = a->q; l.k_cache = a->k_cache; l.v_cache = a->v_cache;
  l.k_scale = a->k_scale; l.v_scale = a->v_scale;
  l.indices = a->indices; l.kv_len = a->kv_len; l.out = a->out;
  l.q_dtype = a->q_dtype; l.kv_dtype = a->kv_dtype; l.out_dtype = a->out_dtype;
  l.B = a->B; l.S = a->S; l.H_q = a->H_q; l.H_kv = a->H_kv; l.D = a->D;
  l.L_cap = a->L_cap; l.k = a->k;
  l.scale = a->softmax_scale > 0.0f ? a->softmax_scale : 1.0f / std::sqrt((float)a->D);
  l.aux_k = a->aux_len > 0 ? a->aux_k : nullptr;
  l.aux_v = a->aux_len > 0 ? a->aux_v : nullptr;
  l.aux_dtype = a->aux_dtype; l.aux_len = a->aux_len;
  dsa::plan_attention(l, decode);
  return l;
}

dsa_status run_attention(const dsa_attention_args* a, void* ws, size_t ws_bytes, void* stream,
                         bool decode) {
  CHECK(validate_attention(a));
  if ((long long)a->B * a->S == 0) return ok();
  dsa::AttnLaunch l = make_attn(a, decode);
  const size_t need = dsa::attention_partials_bytes(l);
  if (need > 0) {
    if (ws_bytes < need)
      return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, %zu needed", ws_bytes, need);
    CHECK(check_ptr(ws, "workspace"));
    l.part = (float*)ws;
  }
  (void)hipGetLastError();
  dsa::launch_attention(l, (hipStream_t)stream);
  return hip_result(decode ? "dsa_attention_decode" : "dsa_attention_prefill");
}

dsa_status validate_indexer_shape(int idx_dtype, int B, int S, int H_idx, int D_idx, int L_cap,
                                  int max_kv_len) {
  if (B < 0 || S < 0) return fail(DSA_ERR_INVALID_ARGUMENT, "B=%d S=%d must be >= 0", B, S);
  if (L_cap < 1) return fail(DSA_ERR_INVALID_ARGUMENT, "L_cap=%d must be >= 1", L_cap);
  if (L_cap > dsa::kIndexerMaxLcap)
    return fail(DSA_ERR_UNSUPPORTED, "L_cap=%d exceeds 2^27", L_cap);
  if (max_kv_len < 0 || max_kv_len > L_cap)
    return fail(DSA_ERR_INVALID_ARGUMENT, "max_kv_len=%d outside [0, L_cap=%d]", max_kv_len, L_cap);
  if (idx_dtype != DSA_BF16 && idx_dtype != DSA_F16)
    return fail(DSA_ERR_UNSUPPORTED, "indexer dtype %s not in {BF16, F16}", dtype_name(idx_dtype));
  if (H_idx < 1 || H_idx > 16) return fail(DSA_ERR_UNSUPPORTED, "H_idx=%d not in [1, 16]", H_idx);
  if (D_idx != 32 && D_idx != 64 && D_idx != 128)
    return fail(DSA_ERR_UNSUPPORTED, "D_idx=%d not in {32, 64, 128}", D_idx);
  return DSA_OK;
}

dsa_status validate_topk_shape(int B, int S, int L_cap, int max_kv_len, int k) {
  if (B < 0 || S < 0) return fail(DSA_ERR_INVALID_ARGUMENT, "B=%d S=%d must be >= 0", B, S);
  if (L_cap < 1 || L_cap > (1 << 24))
    return fail(DSA_ERR_UNSUPPORTED, "L_cap=%d not in [1, 2^24]", L_cap);
  if (k < 1) return fail(DSA_ERR_INVALID_ARGUMENT, "k=%d must be >= 1", k);
  if (max_kv_len < 0 || max_kv_len > L_cap)
    return fail(DSA_ERR_INVALID_ARGUMENT, "max_kv_len=%d outside [0, L_cap=%d]", max_kv_len, L_cap);
  return DSA_OK;
}

// Appends printf-formatted text to out.
void appendf(std::string& out, const char* fmt, ...) {
  char buf[256];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  out += buf;
}

}  // namespace

extern "C" {

int dsa_abi_version(void) { return DSA_ABI_VERSION; }

const char* dsa_last_error(void) { return g_last_error.c_str(); }

dsa_status dsa_indexer_score(const void* q_idx, const float* w_idx, const void* key_state,
                             dsa_dtype idx_dtype, const int32_t* kv_len, int B, int S, int H_idx,
                             int D_idx, int L_cap, int max_kv_len, float* scores, void* stream) {
  CHECK(validate_indexer_shape(idx_dtype, B, S, H_idx, D_idx, L_cap, max_kv_len));
  if ((long long)B * S == 0 || max_kv_len == 0) return ok();
  CHECK(check_ptr(q_idx, "q_idx"));
  CHECK(check_ptr(w_idx, "w_idx"));
  CHECK(check_ptr(key_state, "key_state"));
  CHECK(check_ptr(kv_len, "kv_len"));
  CHECK(check_ptr(scores, "scores"));
  dsa::IndexerLaunch l = dsa::plan_indexer(B, S, D_idx, L_cap, max_kv_len);
  l.q_idx = q_idx; l.w_idx = w_idx; l.key_state = key_state; l.kv_len = kv_len;
  l.scores = scores; l.H = H_idx; l.L_cap = L_cap; l.bf16 = idx_dtype == DSA_BF16;
  (void)hipGetLastError();
  dsa::launch_indexer(l, (hipStream_t)stream);
  return hip_result("dsa_indexer_score");
}

size_t dsa_topk_workspace_bytes(int B, int S, int L_cap, int k) {
  if (B <= 0 || S <= 0 || L_cap < 1 || k < 1 || L_cap > (1 << 24)) return 0;
  // the plan of the largest runtime bound, max_kv_len = L_cap (no shorter bound needs more)
  return dsa::plan_topk(B, S, L_cap, L_cap, k).ws_bytes;
}

dsa_status dsa_topk(const float* scores, const int32_t* kv_len, int B, int S, int L_cap,
                    int max_kv_len, int k, int32_t* indices, void* workspace,
                    size_t workspace_bytes, void* stream) {
  CHECK(validate_topk_shape(B, S, L_cap, max_kv_len, k));
  if ((long long)B * S == 0) return ok();
  CHECK(check_ptr(scores, "scores"));
  CHECK(check_ptr(kv_len, "kv_len"));
  CHECK(check_ptr(indices, "indices"));
  dsa::TopkPlan p = dsa::plan_topk(B, S, L_cap, max_kv_len, k);
  if (p.ws_bytes > 0) {
    if (workspace_bytes < p.ws_bytes)
      return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, %zu needed",
                  workspace_bytes, p.ws_bytes);
    CHECK(check_ptr(workspace, "workspace"));
  }
  (void)hipGetLastError();
  dsa::launch_topk(p, scores, kv_len, S, L_cap, max_kv_len, k, indices, workspace,
                   (hipStream_t)stream);
  return hip_result("dsa_topk");
}

size_t dsa_attention_workspace_bytes(const dsa_attention_args* args, int is_decode) {
  if (validate_attention_shape(args) != DSA_OK) return 0;     // pointers are not needed
  if ((long long)args->B * args->S == 0) return 0;
  return dsa::attention_partials_bytes(make_attn(args, is_decode != 0));
}

dsa_status dsa_attention_decode(const dsa_attention_args* args, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return run_attention(args, workspace, workspace_bytes, stream, true);
}

dsa_status dsa_attention_prefill(const dsa_attention_args* args, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return run_attention(args, workspace, workspace_bytes, stream, false);
}

size_t dsa_describe_plan(int op, int B, int S, int L_cap, int max_kv_len, int k, int D_idx,
                         const dsa_attention_args* attention, char* buf, size_t buf_bytes) {
  std::string d;
  if (op == DSA_PLAN_INDEXER) {
    if (validate_indexer_shape(DSA_BF16, B, S, 1, D_idx, L_cap, max_kv_len) != DSA_OK) return 0;
    if ((long long)B * S == 0 || max_kv_len == 0) {
      d = "op=indexer kernels=none";
    } else {
      const dsa::IndexerLaunch l = dsa::plan_indexer(B, S, D_idx, L_cap, max_kv_len);
      const bool stream = l.prefill || l.stream_decode;
      if (l.fold)
        appendf(d, "op=indexer kernel=indexer_fold_kernel grid=%dx%dx%d threads=%d waves=%d "
                   "tokens_per_workgroup=32 keys_per_workgroup=%d",
                l.tok_blocks, l.key_blocks, B, 64 * l.waves, l.waves, l.keys_per_wg);
      else
        appendf(d, "op=indexer kernel=%s grid=%dx%dx%d threads=%d waves=%d token_pairs_per_wave=%d "
                   "keys_per_buffer=%d keys_per_workgroup=%d",
                stream ? "indexer_stream_kernel" : "indexer_score_kernel", l.tok_blocks,
                l.key_blocks, B, 64 * l.waves, l.waves, l.pairs, l.tile, l.keys_per_wg);
    }
  } else if (op == DSA_PLAN_TOPK) {
    if (validate_topk_shape(B, S, L_cap, max_kv_len, k) != DSA_OK) return 0;
    const dsa::TopkPlan p = dsa::plan_topk(B, S, L_cap, max_kv_len, k);
    if (p.rows == 0) {
      d = "op=topk kernels=none";
    } else if (p.kind == 3) {
      appendf(d, "op=topk plan=small kernel=topk_small_kernel grid=%d threads=256 "
                 "keys_per_thread=%d workspace=0", p.rows, p.lane_keys);
    } else if (p.kind == 0) {
      appendf(d, "op=topk plan=stream kernel=topk_stream_kernel grid=%d threads=1024 workspace=0",
              p.rows);
    } else if (p.kind == 1) {
      appendf(d, "op=topk plan=resident kernel=topk_resident_kernel grid=%d threads=1024 "
                 "workspace=0", p.rows);
    } else {
      const int nch = (max_kv_len + p.chunk - 1) / p.chunk;
      appendf(d, "op=topk plan=split kernels=topk_chunk_kernel,topk_select_kernel "
                 "chunk_grid=%dx%d chunk_threads=512 select_grid=%d select_threads=512 "
                 "chunk=%d chunks=%d sample=%d slots=%d spec=%d entries=%d mode=%s workspace=%zu",
              p.exact_only ? 0 : nch, p.rows, p.rows, p.chunk, p.chunks, p.sample, p.cap, p.spec,
              p.entries, p.exact_only ? "exact" : (p.spec > 0 ? "fast" : "general"), p.ws_bytes);
    }
  } else if (op == DSA_PLAN_ATTENTION_DECODE || op == DSA_PLAN_ATTENTION_PREFILL) {
    if (validate_attention_shape(attention) != DSA_OK) return 0;
    const bool decode = op == DSA_PLAN_ATTENTION_DECODE;
    if ((long long)attention->B * attention->S == 0) {
      d = decode ? "op=attention_decode kernels=none" : "op=attention_prefill kernels=none";
    } else {
      const dsa::AttnLaunch l = make_attn(attention, decode);
      const int rows = l.B * l.S;
      const int splits = l.nsplit + (l.aux_len > 0 ? 1 : 0);
      if (l.wave_rows)
        appendf(d, "op=%s kernel=attn_kernel schedule=wave_rows grid=%d threads=256 "
                   "rows_per_workgroup=4 keys_per_split=%d",
                decode ? "attention_decode" : "attention_prefill", l.H_kv * ((rows + 3) / 4),
                l.keys_per_split);
      else
        appendf(d, "op=%s kernel=attn_kernel schedule=split grid=%dx%dx%d threads=256 "
                   "keys_per_split=%d",
                decode ? "attention_decode" : "attention_prefill", l.nsplit, l.H_kv, rows,
                l.keys_per_split);
      if (l.aux_len > 0) appendf(d, " aux_grid=1x%dx%d", l.H_kv, rows);
      if (splits > 1) appendf(d, " merge_kernel=attn_merge_kernel merge_grid=%d", rows * l.H_q);
      appendf(d, " workspace=%zu", dsa::attention_partials_bytes(l));
    }
  } else {
    fail(DSA_ERR_INVALID_ARGUMENT, "op=%d is not a dsa_plan_op", op);
    return 0;
  }
  if (buf && buf_bytes > 0) {
    const size_t n = d.size() < buf_bytes - 1 ? d.size() : buf_bytes - 1;
    memcpy(buf, d.data(), n);
    buf[n] = '\0';
  }
  ok();
  return d.size();
}

dsa_status dsa_attention_decode_noalloc(const dsa_attention_args* args, void* stream) {
  CHECK(validate_attention(args));
  if ((long long)args->B * args->S == 0) return ok();
  dsa::AttnLaunch l = make_attn(args, true);
  const size_t need = dsa::attention_partials_bytes(l);
  if (need > dsa::kAttnScratchBytes)
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL,
                "decode partials need %zu bytes; the built-in scratch holds %zu", need,
                dsa::kAttnScratchBytes);
  if (need > 0) {
    hipError_t e = hipSuccess;
    l.part = dsa::attention_scratch(&e);
    if (!l.part) return fail(DSA_ERR_HIP, "built-in scratch address: %s", hipGetErrorString(e));
  }
  (void)hipGetLastError();
  dsa::launch_attention(l, (hipStream_t)stream);
  return hip_result("dsa_attention_decode_noalloc");
}

dsa_status dsa_cache_append(const dsa_cache_append_args* a, void* stream) {
  if (!a) return fail(DSA_ERR_INVALID_ARGUMENT, "args is NULL");
  if (a->B < 0 || a->S < 0) return fail(DSA_ERR_INVALID_ARGUMENT, "B=%d S=%d must be >= 0", a->B, a->S);
  if (a->L_cap < 1) return fail(DSA_ERR_INVALID_ARGUMENT, "L_cap=%d must be >= 1", a->L_cap);
  if (a->H_kv < 1) return fail(DSA_ERR_INVALID_ARGUMENT, "H_kv=%d must be >= 1", a->H_kv);
  if (a->D != 64 && a->D != 128) return fail(DSA_ERR_UNSUPPORTED, "head dim D=%d not in {64, 128}", a->D);
  const int nd = a->new_dtype, kd = a->kv_dtype;
  if (nd != DSA_F32 && nd != DSA_F16 && nd != DSA_BF16)
    return fail(DSA_ERR_UNSUPPORTED, "new K/V dtype %s not in {F32, F16, BF16}", dtype_name(nd));
  if (kd != DSA_F32 && kd != DSA_F16 && kd != DSA_BF16 && kd != DSA_I8)
    return fail(DSA_ERR_UNSUPPORTED, "cache dtype %s unsupported", dtype_name(kd));
  if (kd == DSA_F32 && nd != DSA_F32)
    return fail(DSA_ERR_UNSUPPORTED, "an F32 cache needs F32 new values, got %s", dtype_name(nd));
  const bool has_ks = a->key_state != nullptr || a->key_state_new != nullptr;
  if (has_ks) {
    if (a->D_idx != 32 && a->D_idx != 64 && a->D_idx != 128)
      return fail(DSA_ERR_UNSUPPORTED, "indexer dim D_idx=%d not in {32, 64, 128}", a->D_idx);
    if (a->idx_dtype != DSA_F16 && a->idx_dtype != DSA_BF16)
      return fail(DSA_ERR_UNSUPPORTED, "key-state dtype %s not in {F16, BF16}", dtype_name(a->idx_dtype));
  }
  if ((long long)a->B * a->S == 0) return ok();
  CHECK(check_ptr(a->k_new, "k_new"));
  CHECK(check_ptr(a->v_new, "v_new"));
  CHECK(check_ptr(a->k_cache, "k_cache"));
  CHECK(check_ptr(a->v_cache, "v_cache"));
  CHECK(check_ptr(a->kv_len, "kv_len"));
  if (kd == DSA_I8) {
    CHECK(check_ptr(a->k_scale, "k_scale"));
    CHECK(check_ptr(a->v_scale, "v_scale"));
  } else if (a->k_scale || a->v_scale) {
    return fail(DSA_ERR_INVALID_ARGUMENT, "k_scale/v_scale must be NULL for a %s cache", dtype_name(kd));
  }
  if (has_ks) {
    CHECK(check_ptr(a->key_state_new, "key_state_new"));
    CHECK(check_ptr(a->key_state, "key_state"));
  }
  dsa::CacheAppendLaunch l{};
  l.k_new = a->k_new; l.v_new = a->v_new; l.k_cache = a->k_cache; l.v_cache = a->v_cache;
  l.k_scale = a->k_scale; l.v_scale = a->v_scale;
  l.key_state_new = has_ks ? a->key_state_new : nullptr;
  l.key_state = has_ks ? a->key_state : nullptr;
  l.kv_len = a->kv_len; l.new_dtype = nd; l.kv_dtype = kd;
  l.B = a->B; l.S = a->S; l.H_kv = a->H_kv; l.D = a->D; l.D_idx = a->D_idx; l.L_cap = a->L_cap;
  (void)hipGetLastError();
  dsa::launch_cache_append(l, (hipStream_t)stream);
  return hip_result("dsa_cache_append");
}

dsa_status dsa_rmsnorm_rope_multi(const dsa_rmsnorm_rope_args* args, int32_t count, void* stream) {
  if (!args) return fail(DSA_ERR_INVALID_ARGUMENT, "args is NULL");
  if (count < 1 || count > dsa::kRopeMaxJobs)
    return fail(DSA_ERR_INVALID_ARGUMENT, "count=%d not in [1, %d]", count, dsa::kRopeMaxJobs);
  dsa::RopeLaunch jobs[dsa::kRopeMaxJobs] = {};
  long long blocks = 0;
  for (int q = 0; q < count; ++q) {
    const dsa_rmsnorm_rope_args* a = &args[q];
    if (a->B < 0 || a->S < 0 || a->H < 0)
      return fail(DSA_ERR_INVALID_ARGUMENT, "job %d: B=%d S=%d H=%d must be >= 0", q, a->B, a->S,
                  a->H);
    if (a->D != 32 && a->D != 64 && a->D != 128)
      return fail(DSA_ERR_UNSUPPORTED, "job %d: head dim D=%d not in {32, 64, 128}", q, a->D);
    if (a->max_pos < 1)
      return fail(DSA_ERR_INVALID_ARGUMENT, "job %d: max_pos=%d must be >= 1", q, a->max_pos);
    if (!(a->eps >= 0.0f) || !std::isfinite(a->eps))
      return fail(DSA_ERR_INVALID_ARGUMENT, "job %d: eps must be finite and >= 0", q);
    for (int d : {a->x_dtype, a->out_dtype})
      if (d != DSA_F32 && d != DSA_F16 && d != DSA_BF16)
        return fail(DSA_ERR_UNSUPPORTED, "job %d: dtype %s not in {F32, F16, BF16}", q,
                    dtype_name(d));
    const long long rows = (long long)a->B * a->S * a->H;
    if (rows == 0) continue;
    CHECK(check_ptr(a->x, "x"));
    CHECK(check_ptr(a->gamma, "gamma"));
    CHECK(check_ptr(a->cos_cache, "cos_cache"));
    CHECK(check_ptr(a->sin_cache, "sin_cache"));
    CHECK(check_ptr(a->kv_len, "kv_len"));
    CHECK(check_ptr(a->out, "out"));
    blocks += (rows * (a->D / 2) + 255) / 256;
    if (blocks > INT32_MAX)
      return fail(DSA_ERR_UNSUPPORTED, "the jobs need more than 2^31 - 1 workgroups");
    dsa::RopeLaunch& l = jobs[q];
    l.x = a->x; l.gamma = a->gamma; l.cos_cache = a->cos_cache; l.sin_cache = a->sin_cache;
    l.kv_len = a->kv_len; l.out = a->out; l.x_dtype = a->x_dtype; l.out_dtype = a->out_dtype;
    l.B = a->B; l.S = a->S; l.H = a->H; l.D = a->D; l.max_pos = a->max_pos;
    l.eps = a->eps; l.interleaved = a->interleaved != 0;
  }
  if (blocks == 0) return ok();
  (void)hipGetLastError();
  dsa::launch_rmsnorm_rope(jobs, count, (hipStream_t)stream);
  return hip_result("dsa_rmsnorm_rope_multi");
}

dsa_status dsa_rmsnorm_rope(const dsa_rmsnorm_rope_args* a, void* stream) {
  return dsa_rmsnorm_rope_multi(a, 1, stream);
}

}  // extern "C"
