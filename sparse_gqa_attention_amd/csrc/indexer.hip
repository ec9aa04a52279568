// Indexer score kernel (ORT PR #33802 "Optimize ... for SM12x and 256K
// context", Summary item 2: per-head scores of the key-state cache reduced
// over the indexer heads; several query tokens share every key-state load).
//
//   score[b,s,j] = sum_h w[b,s,h] * (q_idx[b,s,h,:] . key_state[b,j,:])
//
// gfx950 design.  One v_mfma_f32_32x32x16 tile has 32 rows = two query
// tokens x 16 indexer heads (fewer heads are zero-padded) and 32 columns =
// 32 keys, so the per-head contraction is a dense MFMA and the weighted head
// reduction reads straight out of the accumulator: each lane holds 8 heads of
// one token for one key, multiplies them by the head weights, and one
// cross-half exchange (lane l <-> l^32) completes the 16-head sum.  Lanes
// 0..31 then hold token t0's scores for 32 consecutive keys and lanes 32..63
// token t1's: one coalesced 128-byte store per half wave.
//
// A workgroup (4 waves) owns a run of keys and 8*PAIRS query tokens; each
// 64-key tile of key_state is staged once in LDS (16-byte chunks XOR-swizzled
// by row so that the B-operand reads of 32 different keys hit different
// banks) and read by all waves.  Query operands stay in registers.
#include "dsa_device.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kIdxThreads = 256;
constexpr int kIdxTile = 64;   // keys staged in LDS per step

template <typename T, int DI>
struct IdxTraits {
  static constexpr int kSteps = DI / 16;        // K-steps of the 32x32x16 MFMA
  static constexpr int kChunks = DI / 8;        // 16-byte chunks per key row
  static constexpr int kSwz = kChunks < 8 ? kChunks - 1 : 7;
};

template <typename T, int DI, int PAIRS>
__global__ __launch_bounds__(kIdxThreads) void indexer_score_kernel(
    const T* __restrict__ q_idx, const float* __restrict__ w_idx,
    const T* __restrict__ key_state, const int32_t* __restrict__ kv_len,
    int S, int H, int L_cap, int keys_per_wg, float* __restrict__ scores) {
  using Tr = IdxTraits<T, DI>;
  using V8 = typename vec8<T>::type;
  constexpr int kTokPerWg = 8 * PAIRS;
  __shared__ __attribute__((aligned(16))) uint4 tile[kIdxTile * Tr::kChunks];

  const int b = blockIdx.z;
  int kvl = kv_len[b];
  kvl = kvl < 0 ? 0 : (kvl > L_cap ? L_cap : kvl);
  const int j_begin = blockIdx.x * keys_per_wg;
  const int j_end = min(j_begin + keys_per_wg, kvl);
  const int s_first = blockIdx.y * kTokPerWg;
  // Keys beyond the last position of this block's tokens are never selected.
  const int last_pos = kvl - S + min(s_first + kTokPerWg, S) - 1;
  if (j_begin >= j_end || j_begin > last_pos) return;

  const int wave = threadIdx.x / kWave;
  const int l = lane_id();
  const int half = l >> 5;     // 0: lanes 0..31, 1: lanes 32..63
  const int col = l & 31;

  // A operands: row m = l%32 -> token (m/16), head m%16; k = 16*step + 8*half.
  V8 a[PAIRS][Tr::kSteps];
  float wv[PAIRS][16];
#pragma unroll
  for (int p = 0; p < PAIRS; ++p) {
    const int s0 = s_first + wave * 2 * PAIRS + 2 * p;
    {
      const int s = s0 + (col >> 4), h = col & 15;
      const bool ok = (s < S) && (h < H);
      const T* src = q_idx + ((size_t)(b * S + (ok ? s : 0)) * H + (ok ? h : 0)) * DI;
#pragma unroll
      for (int st = 0; st < Tr::kSteps; ++st) {
        uint4 raw = ok ? ld_vec<uint4>(src + 16 * st + 8 * half) : make_uint4(0, 0, 0, 0);
        a[p][st] = __builtin_bit_cast(V8, raw);
      }
    }
    // Weights for the 16 accumulator elements of this lane:
    // element v <-> row m = 8*(v/4) + 4*half + v%4.
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = 8 * (v >> 2) + 4 * half + (v & 3);
      const int s = s0 + (m >> 4), h = m & 15;
      wv[p][v] = (s < S && h < H) ? w_idx[(size_t)(b * S + s) * H + h] : 0.0f;
    }
  }

  const T* ks_b = key_state + (size_t)b * L_cap * DI;
  for (int j0 = j_begin; j0 < j_end; j0 += kIdxTile) {
    // Stage key_state[j0 .. j0+63] (zero rows past j_end) into swizzled LDS.
    for (int c = threadIdx.x; c < kIdxTile * Tr::kChunks; c += kIdxThreads) {
      const int r = c / Tr::kChunks, ch = c % Tr::kChunks;
      const int j = j0 + r;
      uint4 v = (j < j_end) ? ld_vec<uint4>(ks_b + (size_t)j * DI + 8 * ch)
                            : make_uint4(0, 0, 0, 0);
      tile[r * Tr::kChunks + (ch ^ (r & Tr::kSwz))] = v;
    }
    __syncthreads();
#pragma unroll
    for (int ct = 0; ct < kIdxTile / 32; ++ct) {
      const int r = ct * 32 + col;     // this lane's key row (B column n = col)
      f32x16 acc[PAIRS];
#pragma unroll
      for (int p = 0; p < PAIRS; ++p) acc[p] = f32x16{};
#pragma unroll
      for (int st = 0; st < Tr::kSteps; ++st) {
        const int ch = 2 * st + half;
        V8 bop = __builtin_bit_cast(V8, tile[r * Tr::kChunks + (ch ^ (r & Tr::kSwz))]);
#pragma unroll
        for (int p = 0; p < PAIRS; ++p) acc[p] = mfma32x32x16(a[p][st], bop, acc[p]);
      }
      const int j = j0 + ct * 32 + col;
#pragma unroll
      for (int p = 0; p < PAIRS; ++p) {
        float part0 = 0.0f, part1 = 0.0f;
#pragma unroll
        for (int v = 0; v < 8; ++v) part0 += wv[p][v] * acc[p][v];
#pragma unroll
        for (int v = 8; v < 16; ++v) part1 += wv[p][v] * acc[p][v];
        // Lane l keeps token (half) and adds the other half's partial of it.
        const float mine = half ? part1 : part0;
        const float give = half ? part0 : part1;
        const float total = mine + __shfl_xor(give, 32, kWave);
        const int s = s_first + wave * 2 * PAIRS + 2 * p + half;
        if (s < S && j < j_end) scores[((size_t)b * S + s) * L_cap + j] = total;
      }
    }
    __syncthreads();
  }
}

template <typename T, int DI, int PAIRS>
void launch_idx(const IndexerLaunch& a, hipStream_t st) {
  dim3 grid(a.key_blocks, a.tok_blocks, a.B);
  hipLaunchKernelGGL((indexer_score_kernel<T, DI, PAIRS>), grid, dim3(kIdxThreads), 0, st,
                     (const T*)a.q_idx, a.w_idx, (const T*)a.key_state, a.kv_len, a.S, a.H,
                     a.L_cap, a.keys_per_wg, a.scores);
}

template <typename T, int PAIRS>
void launch_idx_d(const IndexerLaunch& a, hipStream_t st) {
  switch (a.D_idx) {
    case 32: launch_idx<T, 32, PAIRS>(a, st); break;
    case 64: launch_idx<T, 64, PAIRS>(a, st); break;
    default: launch_idx<T, 128, PAIRS>(a, st); break;
  }
}

}  // namespace

IndexerLaunch plan_indexer(int B, int S, int D_idx, int max_kv_len) {
  IndexerLaunch a{};
  a.B = B;
  a.S = S;
  a.D_idx = D_idx;
  a.pairs = S > 8 ? 2 : 1;
  const int tok_per_wg = 8 * a.pairs;
  a.tok_blocks = (S + tok_per_wg - 1) / tok_per_wg;
  // Aim for ~1024 workgroups (4 per CU), 64..1024 keys each.
  long long want = ((long long)max_kv_len * B * a.tok_blocks + 1023) / 1024;
  int kpw = kIdxTile;
  while (kpw < want && kpw < 1024) kpw *= 2;
  a.keys_per_wg = kpw;
  a.key_blocks = (max_kv_len + kpw - 1) / kpw;
  return a;
}

void launch_indexer(const IndexerLaunch& a, hipStream_t st) {
  if (a.key_blocks == 0 || a.tok_blocks == 0 || a.B == 0) return;
  if (a.bf16) {
    if (a.pairs == 2) launch_idx_d<__bf16, 2>(a, st); else launch_idx_d<__bf16, 1>(a, st);
  } else {
    if (a.pairs == 2) launch_idx_d<_Float16, 2>(a, st); else launch_idx_d<_Float16, 1>(a, st);
  }
}

}  // namespace dsa
