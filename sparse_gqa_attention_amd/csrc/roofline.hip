// Ceiling probes for the benchmark (libdsa_roofline.so, include/dsa_roofline.h):
// the rates the hot-path kernels are compared with, measured on the same
// GPU in the same run as the path itself.
//  * streaming read and copy of large buffers (the HBM ceiling);
//  * back-to-back v_mfma_f32_32x32x16_bf16 on register operands (the MFMA
//    ceiling for the BF16/FP16 contractions of the indexer and attention);
//  * a kernel that only reads one word per workgroup (the launch floor of a
//    step's kernels, replayed in a graph like the step);
//  * random 256-byte row gathers from a buffer (the gather ceiling of
//    attention, whose rows are picked by the top-k: a 128 MiB buffer -- one
//    prefill layer's K/V cache -- stays in the Infinity Cache, a larger one
//    does not).
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/dsa_roofline.h"
#include "dsa_device.h"

namespace {

constexpr int kThreads = 256;

// Eight 16-byte loads per lane in flight.
__global__ __launch_bounds__(kThreads) void roof_read_kernel(const uint4* __restrict__ src,
                                                             size_t n16, uint32_t* out) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    uint4 a[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) a[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= a[u].x ^ a[u].y ^ a[u].z ^ a[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) out[0] = acc;         // keeps the loads; practically never stores
}

__global__ __launch_bounds__(kThreads) void roof_copy_kernel(const uint4* __restrict__ src,
                                                             uint4* __restrict__ dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

// Streaming write: every 16-byte chunk of dst stored once, one store per
// thread over a grid that covers dst in order.  (The dispatch order then
// keeps the chip's writes close together in address; a grid-stride loop
// over 4096 workgroups measured 4.0 TB/s against 6.9 TB/s for this form.)
__global__ __launch_bounds__(kThreads) void roof_write_kernel(dsa::u32x4* __restrict__ dst,
                                                              size_t n16) {
  const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const dsa::u32x4 v = {threadIdx.x, blockIdx.x, 0x3F800000u, 0u};
  if (i < n16) __builtin_nontemporal_store(v, dst + i);
}

// Each wave runs `iters` rounds of four independent 32x32x16 BF16 MFMAs.
__global__ __launch_bounds__(kThreads) void roof_mfma_kernel(float* out, int iters) {
  using namespace dsa;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(float)((threadIdx.x + e) & 7);
    b[e] = (__bf16)(float)((threadIdx.x * 3 + e) & 7);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = mfma32x32x16(a, b, c0);
    c1 = mfma32x32x16(a, b, c1);
    c2 = mfma32x32x16(a, b, c2);
    c3 = mfma32x32x16(a, b, c3);
  }
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  if (s == 1.2345f) out[blockIdx.x] = s;         // keeps the products; practically never stores
}

// 16 lanes per 256-byte row: lane l reads bytes 16 (l % 16) of row idx[r];
// eight rows in flight per lane group.
__global__ __launch_bounds__(kThreads) void roof_gather_kernel(const uint4* __restrict__ buf,
                                                               const int32_t* __restrict__ idx,
                                                               int n_rows, uint32_t* out) {
  const int lane16 = threadIdx.x & 15;
  const int groups = gridDim.x * (kThreads / 16);
  uint32_t acc = 0;
  int r = blockIdx.x * (kThreads / 16) + (threadIdx.x >> 4);
  for (; r + 7 * groups < n_rows; r += 8 * groups) {
    int j[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) j[u] = idx[r + u * groups];
    uint4 a[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) a[u] = buf[(size_t)j[u] * 16 + lane16];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= a[u].x ^ a[u].y ^ a[u].z ^ a[u].w;
  }
  for (; r < n_rows; r += groups) {
    const uint4 a = buf[(size_t)idx[r] * 16 + lane16];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) out[0] = acc;
}

// The K/V reads of a sparse-attention launch and nothing else, in either of
// its schedules.  The workgroup holds 64 KB of LDS, so two fit on a CU: the
// residency of the 16-bit D = 128 attention kernel.
//   WAVE_ROWS = false: workgroup (row, KV head); wave w reads tiles w, w + 4,
//     ... of the row (two in flight: the tile and the one four further);
//   WAVE_ROWS = true: workgroup j takes KV head j % H_kv and rows
//     4 (j / H_kv) + wave; each wave reads every tile of its row in order,
//     two in flight.
constexpr int kKvHoldBytes = 64 * 1024;

template <bool WAVE_ROWS>
__global__ __launch_bounds__(kThreads) void roof_kv_gather_kernel(
    const unsigned char* __restrict__ kc, const unsigned char* __restrict__ vc,
    const int32_t* __restrict__ idx, int k, int S, int H_kv, int L_cap, int rows, uint32_t* out) {
  __shared__ uint32_t hold[kKvHoldBytes / 4];
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  int g, row, first, step, ahead;
  if (WAVE_ROWS) {
    g = (int)(blockIdx.x % (unsigned)H_kv);
    row = (int)(blockIdx.x / (unsigned)H_kv) * 4 + wave;
    first = 0; step = 64; ahead = 32;
  } else {
    g = blockIdx.y; row = blockIdx.z;
    first = 32 * wave; step = 256; ahead = 128;
  }
  uint32_t acc = 0;
  if (row < rows) {
    const int b = row / S;
    const size_t tok_bytes = (size_t)H_kv * 256;
    const unsigned char* kb = kc + (size_t)b * L_cap * tok_bytes + (size_t)g * 256;
    const unsigned char* vb = vc + (size_t)b * L_cap * tok_bytes + (size_t)g * 256;
    const int32_t* ir = idx + (size_t)row * k;
    for (int t0 = first; t0 < k; t0 += step) {
      uint4 x[2][16];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int base = t0 + h * ahead;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int e = base + 8 * q + (l >> 3);
          int j = e < k ? ir[e] : -1;
          j = (j >= 0 && j < L_cap) ? j : -1;
          const size_t off = (size_t)(j < 0 ? 0 : j) * tok_bytes + 16 * (l & 7);
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            x[h][4 * q + 2 * half] = j < 0 ? make_uint4(0, 0, 0, 0)
                                           : *reinterpret_cast<const uint4*>(kb + off + 128 * half);
            x[h][4 * q + 2 * half + 1] = j < 0 ? make_uint4(0, 0, 0, 0)
                                               : *reinterpret_cast<const uint4*>(vb + off + 128 * half);
          }
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc ^= x[h][i].x ^ x[h][i].y ^ x[h][i].z ^ x[h][i].w;
    }
  }
  hold[threadIdx.x] = acc;
  __syncthreads();
  if (hold[(threadIdx.x + 1) % kThreads] == 0x9E3779B9u) out[0] = acc;
}

// The least a hot-path kernel does: every workgroup reads one word of its
// arguments' memory (as the kernels read kv_len) and stores nothing.
__global__ void roof_floor_kernel(const int32_t* __restrict__ word, uint32_t* sink) {
  if (word[0] == 0x1234567 && threadIdx.x == 0) sink[blockIdx.x] = 1u;
}

int grid_for(size_t work_items) {
  const size_t g = (work_items + kThreads - 1) / kThreads;
  return (int)(g < 4096 ? (g > 0 ? g : 1) : 4096);
}

int status(const char* what) {
  (void)what;
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace

extern "C" {

int dsa_roofline_read(const void* src, size_t bytes, void* sink, void* stream) {
  if (!src || !sink || ((uintptr_t)src & 15u) || bytes % 16) return 2;
  (void)hipGetLastError();
  const size_t n16 = bytes / 16;
  hipLaunchKernelGGL(roof_read_kernel, dim3(grid_for(n16 / 8)), dim3(kThreads), 0,
                     (hipStream_t)stream, (const uint4*)src, n16, (uint32_t*)sink);
  return status("read");
}

int dsa_roofline_write(void* dst, size_t bytes, void* stream) {
  if (!dst || ((uintptr_t)dst & 15u) || bytes % 16) return 2;
  (void)hipGetLastError();
  const size_t n16 = bytes / 16;
  const size_t wgs = (n16 + kThreads - 1) / kThreads;
  if (wgs > 0x7FFFFFFFu) return 2;
  hipLaunchKernelGGL(roof_write_kernel, dim3((unsigned)wgs), dim3(kThreads), 0,
                     (hipStream_t)stream, (dsa::u32x4*)dst, n16);
  return status("write");
}

int dsa_roofline_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst || ((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u) || bytes % 16) return 2;
  (void)hipGetLastError();
  const size_t n16 = bytes / 16;
  hipLaunchKernelGGL(roof_copy_kernel, dim3(grid_for(n16 / 4)), dim3(kThreads), 0,
                     (hipStream_t)stream, (const uint4*)src, (uint4*)dst, n16);
  return status("copy");
}

double dsa_roofline_mfma_flops(int workgroups, int iters) {
  // 4 MFMAs of 32 x 32 x 16 x 2 flops per round, per wave
  return (double)workgroups * (kThreads / 64) * iters * 4.0 * 32 * 32 * 16 * 2;
}

int dsa_roofline_mfma(void* sink, int workgroups, int iters, void* stream) {
  if (!sink || workgroups < 1 || iters < 1) return 2;
  (void)hipGetLastError();
  hipLaunchKernelGGL(roof_mfma_kernel, dim3(workgroups), dim3(kThreads), 0, (hipStream_t)stream,
                     (float*)sink, iters);
  return status("mfma");
}

int dsa_roofline_gather(const void* buf, size_t buf_bytes, const int32_t* rows, int n_rows,
                        void* sink, void* stream) {
  if (!buf || !rows || !sink || ((uintptr_t)buf & 15u) || n_rows < 0 || buf_bytes < 256) return 2;
  (void)hipGetLastError();
  const int groups_needed = (n_rows + 7) / 8;
  int grid = (groups_needed * 16 + kThreads - 1) / kThreads;
  grid = grid < 1 ? 1 : (grid > 8192 ? 8192 : grid);
  hipLaunchKernelGGL(roof_gather_kernel, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                     (const uint4*)buf, rows, n_rows, (uint32_t*)sink);
  return status("gather");
}

int dsa_roofline_kv_gather(const void* k_cache, const void* v_cache, const int32_t* indices,
                           int rows, int k, int S, int H_kv, int L_cap, int wave_rows, void* sink,
                           void* stream) {
  if (!k_cache || !v_cache || !indices || !sink || rows < 1 || k < 1 || S < 1 || H_kv < 1 ||
      L_cap < 1 || rows > 65535 || H_kv > 65535 || ((uintptr_t)k_cache & 15u) ||
      ((uintptr_t)v_cache & 15u))
    return 2;
  (void)hipGetLastError();
  if (wave_rows)
    hipLaunchKernelGGL(roof_kv_gather_kernel<true>, dim3(H_kv * ((rows + 3) / 4)), dim3(kThreads),
                       0, (hipStream_t)stream, (const unsigned char*)k_cache,
                       (const unsigned char*)v_cache, indices, k, S, H_kv, L_cap, rows,
                       (uint32_t*)sink);
  else
    hipLaunchKernelGGL(roof_kv_gather_kernel<false>, dim3(1, H_kv, rows), dim3(kThreads), 0,
                       (hipStream_t)stream, (const unsigned char*)k_cache,
                       (const unsigned char*)v_cache, indices, k, S, H_kv, L_cap, rows,
                       (uint32_t*)sink);
  return status("kv_gather");
}

int dsa_roofline_floor(const int32_t* word, void* sink, int workgroups, int threads, void* stream) {
  if (!word || !sink || workgroups < 1 || threads < 1 || threads > 1024) return 2;
  (void)hipGetLastError();
  hipLaunchKernelGGL(roof_floor_kernel, dim3(workgroups), dim3(threads), 0, (hipStream_t)stream,
                     word, (uint32_t*)sink);
  return status("floor");
}

}  // extern "C"
