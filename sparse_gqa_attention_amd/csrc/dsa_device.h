// Device-side building blocks shared by the gfx950 kernels of libdsa.
//
// Wave64 everywhere.  MFMA operand/result lane layouts used below (CDNA3/4):
//   v_mfma_f32_16x16x32_{f16,bf16}: A[m][k] in lane (m + 16*(k/8)), element k%8;
//       B[k][n] in lane (n + 16*(k/8)), element k%8;
//       C[m][n] in lane (n + 16*(m/4)), element m%4.
//   v_mfma_f32_32x32x16_{f16,bf16}: A[m][k] in lane (m + 32*(k/8)), element k%8;
//       B[k][n] in lane (n + 32*(k/8)), element k%8;
//       C[m][n] in lane (n + 32*((m/4)%2)), element 4*(m/8) + m%4.
//   v_mfma_f32_16x16x4f32: A[m][k] in lane (m + 16*k); B[k][n] in lane (n + 16*k);
//       C as for 16x16x32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kWave = 64;

// ------------------------------------------------------------------ loads
template <typename T>
__device__ __forceinline__ T ld_vec(const void* p) {
  return *reinterpret_cast<const T*>(p);
}

// Wait until every vector memory operation of this wave has completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ------------------------------------------------------------------ conversions
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(_Float16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(int8_t x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ _Float16 from_f32<_Float16>(float x) { return (_Float16)x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// ------------------------------------------------------------------ MFMA
__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <typename T> struct vec8;
template <> struct vec8<_Float16> { typedef f16x8 type; };
template <> struct vec8<__bf16> { typedef bf16x8 type; };

// ------------------------------------------------------------------ exp
// e^x for x <= ~88 (and -inf), keeping FP32 subnormal results: a rise of the
// running maximum by ~88 nats must leave e^-88 (~6e-39, subnormal) intact,
// not flush it to zero.  2^y = 2^(y - n) * 2^n with n = floor(y): the
// hardware exp2 only sees y - n in [0, 1) and ldexp produces the subnormal.
__device__ __forceinline__ float exp_keep_subnormal(float x) {
  if (x == -INFINITY) return 0.0f;
  const float y = x * 1.4426950408889634f;
  const float n = floorf(y);
  const float f = __builtin_amdgcn_exp2f(y - n);
  return __builtin_amdgcn_ldexpf(f, (int)n);
}

// ------------------------------------------------------------------ score keys
// Order-preserving map FP32 -> u32 (larger float <=> larger key); -0.0 maps
// to the key of +0.0 so that the two tie.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ------------------------------------------------------------------ wave ops
__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

__device__ __forceinline__ uint32_t wave_prefix_count(uint64_t mask) {
  // number of set bits of mask below this lane
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Inclusive wave scan on DPP lane moves: four row_shr steps scan each
// 16-lane row, then row_bcast:15 and row_bcast:31 carry the row totals.
// Lanes without a source read `old` = 0.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// Running maximum over lanes 0..l (DPP, as wave_inclusive_scan): the last
// lane ends with the wave's maximum.
__device__ __forceinline__ uint32_t wave_inclusive_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));
  return v;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Block-wide exclusive scan of one u32 per thread; *total gets the sum.
// `scratch` holds NT/64 words of LDS.  One barrier: the caller must not let
// any thread reuse the same scratch words before a later barrier (every
// thread reads all of them after the one inside).
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* scratch,
                                                         uint32_t* total) {
  constexpr int NW = NT / kWave;
  const int w = threadIdx.x / kWave, l = lane_id();
  const uint32_t inc = wave_inclusive_scan(v);
  if (l == kWave - 1) scratch[w] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint32_t x = scratch[i];
    before += i < w ? x : 0u;
    tot += x;
  }
  *total = tot;
  return before + inc - v;
}

}  // namespace dsa
