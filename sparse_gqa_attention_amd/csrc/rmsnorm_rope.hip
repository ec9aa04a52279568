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
// whose position falls outside the tables are not written.  A decode step
// rotates several tensors (query, key and indexer query heads, which differ
// in head count and D): one launch takes up to kRopeMaxJobs of them, each a
// contiguous range of workgroups, so a step pays one launch, not three.
#include "dsa_device.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kRopeThreads = 256;

struct RopeBatch {
  RopeLaunch job[kRopeMaxJobs];
  int first[kRopeMaxJobs + 1];   // first workgroup of each job; first[n] = grid size
  int n;
};

// Dtypes are uniform over a workgroup (one job), so these branches do not
// diverge.
__device__ __forceinline__ float ld_any(const void* p, size_t i, int dt) {
  if (dt == kF32) return ((const float*)p)[i];
  if (dt == kF16) return to_f32(((const _Float16*)p)[i]);
  return to_f32(((const __bf16*)p)[i]);
}

__device__ __forceinline__ void st_any(void* p, size_t i, float v, int dt) {
  if (dt == kF32) ((float*)p)[i] = v;
  else if (dt == kF16) ((_Float16*)p)[i] = from_f32<_Float16>(v);
  else ((__bf16*)p)[i] = from_f32<__bf16>(v);
}

// Workgroup `blk` of job a, P lanes (pairs) per head vector.
template <int P>
__device__ __forceinline__ void rope_rows(const RopeLaunch& a, int blk) {
  constexpr int D = 2 * P;
  constexpr int kRowsPerBlock = kRopeThreads / P;
  const int i = threadIdx.x % P;                          // pair index
  const long long row = (long long)blk * kRowsPerBlock + threadIdx.x / P;
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
  const float xa = ld_any(a.x, base + da, a.x_dtype);
  const float xb = ld_any(a.x, base + db, a.x_dtype);
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
  st_any(a.out, base + da, ya * c - yb * sn, a.out_dtype);
  st_any(a.out, base + db, yb * c + ya * sn, a.out_dtype);
}

__global__ __launch_bounds__(kRopeThreads) void rmsnorm_rope_kernel(RopeBatch bt) {
  const int blk = blockIdx.x;
  // the job of this workgroup (a uniform choice among at most 4)
  int j = 0;
#pragma unroll
  for (int q = 1; q < kRopeMaxJobs; ++q) j += (q < bt.n && blk >= bt.first[q]) ? 1 : 0;
  const RopeLaunch& a = bt.job[j];
  const int local = blk - bt.first[j];
  if (a.D == 32) rope_rows<16>(a, local);
  else if (a.D == 64) rope_rows<32>(a, local);
  else rope_rows<64>(a, local);
}

}  // namespace

void launch_rmsnorm_rope(const RopeLaunch* jobs, int n, hipStream_t st) {
  RopeBatch bt{};
  int blocks = 0;
  bt.n = 0;
  for (int q = 0; q < n && q < kRopeMaxJobs; ++q) {
    const RopeLaunch& a = jobs[q];
    const long long rows = (long long)a.B * a.S * a.H;
    if (rows == 0) continue;                      // nothing to rotate: no workgroups
    const int P = a.D / 2;
    bt.job[bt.n] = a;
    bt.first[bt.n] = blocks;
    blocks += (int)((rows * P + kRopeThreads - 1) / kRopeThreads);
    ++bt.n;
  }
  if (bt.n == 0) return;
  for (int q = bt.n; q <= kRopeMaxJobs; ++q) bt.first[q] = blocks;
  hipLaunchKernelGGL(rmsnorm_rope_kernel, dim3(blocks), dim3(kRopeThreads), 0, st, bt);
}

}  // namespace dsa
