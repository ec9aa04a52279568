// KV-cache append (ORT PR #33997 "Support FP16 KV cache and FP16 query/key
// in DynamicSparseAttention<BFloat16> ...", file table: the implementation
// writes the caches before the attention kernels; ORT PR #33802 Summary
// item 1: an INT8 KV cache with one FP32 scale per token per KV head).
//
// New token s of sequence b is written at position kv_len[b] - S + s (kv_len
// is the post-append length); positions outside [0, L_cap) are skipped.
//   * FP32 / FP16 / BF16 caches: each value rounded once (RNE) to the cache
//     dtype;
//   * INT8 cache, per (token, KV head) row x of D values, in FP32:
//       scale = amax / 127 (correctly rounded), code = rint(x / scale)
//       (correctly rounded quotient, ties to even) clamped to [-127, 127];
//       an all-zero row stores scale 0 and zero codes;
//   * the indexer key-state row of the token is copied as is.
//
// gfx950 design: the op moves (B*S*H_kv*2 rows of D values) + key-state rows,
// a few hundred KB per decode step, so it is latency-bound; one wave owns a
// row, each lane holds D/64 consecutive values (coalesced 2- to 8-byte
// accesses), the absmax is a 6-step wave butterfly, and lane 0 writes the
// scale.  One launch covers K, V and key-state rows.
#include <type_traits>

#include "dsa_device.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kAppendThreads = 256;
constexpr int kAppendWaves = kAppendThreads / kWave;

template <typename T>
__device__ __forceinline__ float load_f32(const void* p, size_t i) {
  return to_f32(((const T*)p)[i]);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// E values per lane (E = D / 64).  InT: dtype of the new K/V; CT: cache dtype
// (int8_t for the INT8 cache).
template <int E, typename InT, typename CT>
__global__ __launch_bounds__(kAppendThreads) void cache_append_kernel(CacheAppendLaunch a) {
  const int wave = threadIdx.x / kWave;
  const int l = lane_id();
  const long long row = (long long)blockIdx.x * kAppendWaves + wave;
  const long long kv_rows = (long long)a.B * a.S * a.H_kv * 2;
  if (row < kv_rows) {
    const int which = (int)(row & 1);                // 0: K, 1: V
    const long long r = row >> 1;                    // (b, s, h)
    const int h = (int)(r % a.H_kv);
    const long long bs = r / a.H_kv;
    const int s = (int)(bs % a.S), b = (int)(bs / a.S);
    const int pos = a.kv_len[b] - a.S + s;
    if (pos < 0 || pos >= a.L_cap) return;           // wave-uniform
    const int D = E * kWave;
    const void* src = which ? a.v_new : a.k_new;
    const size_t in0 = (size_t)r * D + (size_t)l * E;
    float x[E];
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = load_f32<InT>(src, in0 + e);
    const size_t trow = ((size_t)b * a.L_cap + pos) * a.H_kv + h;   // (b, pos, h)
    void* dst = which ? a.v_cache : a.k_cache;
    if constexpr (std::is_same<CT, int8_t>::value) {
      float m = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) m = fmaxf(m, fabsf(x[e]));
      const float amax = wave_max(m);
      const float scale = amax > 0.0f ? __fdiv_rn(amax, 127.0f) : 0.0f;
      int8_t c[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float q = amax > 0.0f ? rintf(__fdiv_rn(x[e], scale)) : 0.0f;
        q = fminf(fmaxf(q, -127.0f), 127.0f);
        c[e] = (int8_t)q;
      }
      int8_t* d = (int8_t*)dst + trow * D + (size_t)l * E;
      if constexpr (E == 2) {
        *(uint16_t*)d = (uint16_t)((uint8_t)c[0] | ((uint16_t)(uint8_t)c[1] << 8));
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) d[e] = c[e];
      }
      if (l == 0) (which ? a.v_scale : a.k_scale)[trow] = scale;
    } else {
      CT* d = (CT*)dst + trow * D + (size_t)l * E;
#pragma unroll
      for (int e = 0; e < E; ++e) d[e] = from_f32<CT>(x[e]);
    }
    return;
  }
  // ---- indexer key-state rows: (b, s) -> (b, pos), D_idx 16-bit values
  const long long kr = row - kv_rows;
  if (a.key_state == nullptr || kr >= (long long)a.B * a.S) return;
  const int s = (int)(kr % a.S), b = (int)(kr / a.S);
  const int pos = a.kv_len[b] - a.S + s;
  if (pos < 0 || pos >= a.L_cap) return;
  const int words = a.D_idx / 2;                     // 32-bit words per row
  const uint32_t* src = (const uint32_t*)a.key_state_new + (size_t)kr * words;
  uint32_t* dst = (uint32_t*)a.key_state + ((size_t)b * a.L_cap + pos) * words;
  for (int i = l; i < words; i += kWave) dst[i] = src[i];
}

template <int E, typename InT>
void launch_in(const CacheAppendLaunch& a, hipStream_t st, dim3 grid) {
  switch (a.kv_dtype) {
    case kF32: hipLaunchKernelGGL((cache_append_kernel<E, InT, float>), grid, dim3(kAppendThreads), 0, st, a); break;
    case kF16: hipLaunchKernelGGL((cache_append_kernel<E, InT, _Float16>), grid, dim3(kAppendThreads), 0, st, a); break;
    case kBF16: hipLaunchKernelGGL((cache_append_kernel<E, InT, __bf16>), grid, dim3(kAppendThreads), 0, st, a); break;
    default: hipLaunchKernelGGL((cache_append_kernel<E, InT, int8_t>), grid, dim3(kAppendThreads), 0, st, a); break;
  }
}

template <int E>
void launch_e(const CacheAppendLaunch& a, hipStream_t st, dim3 grid) {
  switch (a.new_dtype) {
    case kF32: launch_in<E, float>(a, st, grid); break;
    case kF16: launch_in<E, _Float16>(a, st, grid); break;
    default: launch_in<E, __bf16>(a, st, grid); break;
  }
}

}  // namespace

void launch_cache_append(const CacheAppendLaunch& a, hipStream_t st) {
  const long long rows = (long long)a.B * a.S * (a.H_kv * 2 + (a.key_state ? 1 : 0));
  if (rows == 0) return;
  const dim3 grid((unsigned)((rows + kAppendWaves - 1) / kAppendWaves));
  if (a.D == 64) launch_e<1>(a, st, grid);
  else launch_e<2>(a, st, grid);
}

}  // namespace dsa
