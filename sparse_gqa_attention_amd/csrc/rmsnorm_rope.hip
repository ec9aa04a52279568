// RMSNorm + rotary position embedding in FP32 (ORT PR #33997 "... FP32 rotary
// cache / FP16 output in RMSNormRotary", Description item 1: the
// normalisation and rotation run in FP32 with no intermediate 16-bit
// rounding, the rotary tables are FP32, and the result is rounded once to
// the output dtype).
//
// For head vector x (D values) of token s of sequence b, at position
// p = kv_len[b] - S + s:
//   y_d = g_d * x_d / sqrt(mean(x^2) + eps)
//   pair i = (d_a, d_b) = (i, i + D/2), or (2i, 2i + 1) when interleaved:
//   out_a = y_a cos[p,i] - y_b sin[p,i],  out_b = y_b cos[p,i] + y_a sin[p,i]
// The square root and the reciprocal are correctly rounded FP32 operations.
//
// gfx950 design: the op is a streaming elementwise pass (bytes in = bytes
// out), so it is built for coalescing, not MFMA.  One lane owns one rotated
// pair, so the rotation needs no data exchange; the D/2 lanes of a head
// vector (64 for D = 128; 32 or 16 for D = 64 or 32: 2 or 4 vectors per
// wave) reduce the sum of squares with a segmented xor butterfly.  Rows
// whose position falls outside the tables are not written.
#include "dsa_device.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kRopeThreads = 256;

template <typename T>
__device__ __forceinline__ float ld_f32(const void* p, size_t i) {
  return to_f32(((const T*)p)[i]);
}

// P lanes (pairs) per head vector; InT / OutT: x and out dtypes.
template <int P, typename InT, typename OutT>
__global__ __launch_bounds__(kRopeThreads) void rmsnorm_rope_kernel(RopeLaunch a) {
  constexpr int D = 2 * P;
  constexpr int kRowsPerBlock = kRopeThreads / P;
  const int i = threadIdx.x % P;                          // pair index
  const long long row = (long long)blockIdx.x * kRowsPerBlock + threadIdx.x / P;
  const long long rows = (long long)a.B * a.S * a.H;
  const bool live_row = row < rows;
  const long long r = live_row ? row : 0;
  const int bs = (int)(r / a.H);
  const int s = bs % a.S, b = bs / a.S;
  const int p = a.kv_len[b] - a.S + s;
  const bool in_table = p >= 0 && p < a.max_pos;
  const int da = a.interleaved ? 2 * i : i;
  const int db = a.interleaved ? 2 * i + 1 : i + P;
  const size_t base = (size_t)r * D;
  const float xa = ld_f32<InT>(a.x, base + da);
  const float xb = ld_f32<InT>(a.x, base + db);
  // sum of squares over the row's P lanes (xor offsets stay inside the row)
  float ss = fmaf(xa, xa, xb * xb);
#pragma unroll
  for (int o = P / 2; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, kWave);
  if (!live_row || !in_table) return;
  const float inv = __fdiv_rn(1.0f, __fsqrt_rn(ss * (1.0f / D) + a.eps));
  const float ya = xa * inv * a.gamma[da];
  const float yb = xb * inv * a.gamma[db];
  const float c = a.cos_cache[(size_t)p * P + i];
  const float sn = a.sin_cache[(size_t)p * P + i];
  OutT* out = (OutT*)a.out;
  out[base + da] = from_f32<OutT>(ya * c - yb * sn);
  out[base + db] = from_f32<OutT>(yb * c + ya * sn);
}

template <int P, typename InT>
void launch_out(const RopeLaunch& a, hipStream_t st) {
  const long long rows = (long long)a.B * a.S * a.H;
  const dim3 grid((unsigned)((rows * P + kRopeThreads - 1) / kRopeThreads));
  switch (a.out_dtype) {
    case kF32: hipLaunchKernelGGL((rmsnorm_rope_kernel<P, InT, float>), grid, dim3(kRopeThreads), 0, st, a); break;
    case kF16: hipLaunchKernelGGL((rmsnorm_rope_kernel<P, InT, _Float16>), grid, dim3(kRopeThreads), 0, st, a); break;
    default: hipLaunchKernelGGL((rmsnorm_rope_kernel<P, InT, __bf16>), grid, dim3(kRopeThreads), 0, st, a); break;
  }
}

template <int P>
void launch_in(const RopeLaunch& a, hipStream_t st) {
  switch (a.x_dtype) {
    case kF32: launch_out<P, float>(a, st); break;
    case kF16: launch_out<P, _Float16>(a, st); break;
    default: launch_out<P, __bf16>(a, st); break;
  }
}

}  // namespace

void launch_rmsnorm_rope(const RopeLaunch& a, hipStream_t st) {
  if ((long long)a.B * a.S * a.H == 0) return;
  if (a.D == 32) launch_in<16>(a, st);
  else if (a.D == 64) launch_in<32>(a, st);
  else launch_in<64>(a, st);
}

}  // namespace dsa
