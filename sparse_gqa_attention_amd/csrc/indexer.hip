// Indexer score kernel (ORT PR #33802 "Optimize ... for SM12x and 256K
// context", Summary item 2: per-head scores of the key-state cache reduced
// over the indexer heads; several query tokens share every key-state load).
//
//   score[b,s,j] = sum_h w[b,s,h] * (q_idx[b,s,h,:] . key_state[b,j,:])
//
// gfx950 design.  One v_mfma_f32_32x32x16 tile has 32 rows = two query
// tokens x 16 indexer heads (fewer heads are zero-padded) and 32 columns =
// 32 keys, so the per-head contraction is a dense MFMA and the weighted head
// reduction reads straight out of the accumulator: rows are ordered so that
// each lane holds all 16 heads of one token for one key and multiplies them
// by the head weights in registers.  Lanes 0..31 then hold token t0's scores
// for 32 consecutive keys and lanes 32..63 token t1's: one coalesced
// 128-byte store per half wave.
//
// A workgroup owns a run of up to KR keys and 2*PAIRS*WAVES query tokens (8
// at decode, 32 at prefill).  The whole key run is copied into LDS once, by
// direct global->LDS loads (16-byte chunks XOR-swizzled by row so that the
// B-operand reads of different keys hit different banks), and every wave
// multiplies its token pairs against all of it.  After that copy the
// workgroup issues no vector-memory loads, only score stores: on gfx9 one
// in-order counter tracks loads and stores alike, so a load issued behind
// stores (a prefetch of the next key tile) would wait for those stores to be
// acknowledged.  Query operands and head weights stay in registers.  Token
// blocks are the fastest grid dimension and the XCD-aware renumbering below
// keeps the workgroups sharing a key run on one XCD, so each key-state run is
// fetched from HBM about once.
#include "dsa_device.h"
#include "launch.h"

namespace dsa {

namespace {

template <typename T, int DI>
struct IdxTraits {
  static constexpr int kSteps = DI / 16;        // K-steps of the 32x32x16 MFMA
  static constexpr int kChunks = DI / 8;        // 16-byte chunks per key row
  // Stored position of 16-byte chunk c of run row r is c ^ swz(r).  A
  // 128-bit LDS read by 16 lanes (rows r0..r0+15, one logical chunk) then
  // touches 16 distinct 16-byte bank groups of a 256-byte bank window, and
  // any 8 consecutive lanes touch 8 distinct groups of a 128-byte window.
  static __device__ __forceinline__ int swz(int r) {
    if constexpr (kChunks == 16) return r & 15;
    else if constexpr (kChunks == 8) return (r & 7) ^ ((r >> 3) & 1);
    else return ((r >> 1) & 3) ^ ((r >> 3) & 1);
  }
};

typedef __attribute__((address_space(3))) void lds_void;

template <typename T, int DI, int PAIRS, int WAVES, int KR>
__global__ __launch_bounds__(WAVES * kWave, WAVES == 8 ? 4 : 1) void indexer_score_kernel(
    const T* __restrict__ q_idx, const float* __restrict__ w_idx,
    const T* __restrict__ key_state, const int32_t* __restrict__ kv_len,
    int S, int H, int L_cap, int keys_per_wg, float* __restrict__ scores) {
  using Tr = IdxTraits<T, DI>;
  using V8 = typename vec8<T>::type;
  constexpr int NT = WAVES * kWave;
  constexpr int kTokPerWg = 2 * PAIRS * WAVES;
  __shared__ __attribute__((aligned(16))) uint4 run[KR * Tr::kChunks];

  // Workgroups are handed to the 8 XCDs round-robin by linear id.  Renumber
  // so that each XCD owns a contiguous range of (token block, key run, batch)
  // tiles in token-fastest order: the token blocks that share a key run then
  // run on one XCD and read it through that XCD's L2.
  int tx = blockIdx.x, ty = blockIdx.y, tz = blockIdx.z;
  {
    const int nx = gridDim.x, nxy = gridDim.x * gridDim.y;
    const int total = nxy * gridDim.z;
    if ((total & 7) == 0) {
      const int lin = blockIdx.x + nx * blockIdx.y + nxy * blockIdx.z;
      const int logical = (lin & 7) * (total >> 3) + (lin >> 3);
      tz = logical / nxy;
      ty = (logical - tz * nxy) / nx;
      tx = logical - tz * nxy - ty * nx;
    }
  }
  const int b = tz;
  int kvl = kv_len[b];
  kvl = kvl < 0 ? 0 : (kvl > L_cap ? L_cap : kvl);
  const int j_begin = ty * keys_per_wg;
  const int j_end = min(j_begin + keys_per_wg, kvl);
  const int s_first = tx * kTokPerWg;
  // Keys beyond the last position of this block's tokens are never selected.
  const int last_pos = kvl - S + min(s_first + kTokPerWg, S) - 1;
  if (j_begin >= j_end || j_begin > last_pos) return;

  const int wave = threadIdx.x / kWave;
  const int l = lane_id();
  const int half = l >> 5;     // 0: lanes 0..31, 1: lanes 32..63
  const int col = l & 31;

  // ---- key run -> LDS.  Slot q holds chunk (q % kChunks) ^ swz(r) of
  // run row r = q / kChunks; a wave fills 64 consecutive slots per load.
  // Rows are rounded up to whole 32-key chunks; rows past the run repeat its
  // last row (their scores are never stored).
  {
    const T* ks_b = key_state + (size_t)b * L_cap * DI;
    const int nvec = ((j_end - j_begin + 31) & ~31) * Tr::kChunks;   // multiple of 64
    for (int q0 = wave * kWave; q0 < nvec; q0 += NT) {
      const int q = q0 + l;
      const int r = q / Tr::kChunks, c = q % Tr::kChunks;
      const int j = min(j_begin + r, j_end - 1);
      __builtin_amdgcn_global_load_lds((const void*)(ks_b + (size_t)j * DI + 8 * (c ^ Tr::swz(r))),
                                       (lds_void*)(run + q0), 16, 0, 0);
    }
  }

  // MFMA row m <-> token (m/4)%2 of the pair, head 4*(m/8) + m%4.  With the
  // 32x32 accumulator layout (element v of lane l is row 8*(v/4) + 4*(l/32)
  // + v%4) every lane then holds all 16 heads of one token, token l/32, as
  // elements v = head.  A operand: lane l supplies row l%32, k = 16*step +
  // 8*(l/32).
  V8 a[PAIRS][Tr::kSteps];
  float wv[PAIRS][16];
#pragma unroll
  for (int p = 0; p < PAIRS; ++p) {
    const int s0 = s_first + wave * 2 * PAIRS + 2 * p;
    // Loads are unconditional from clamped addresses (no per-load branch);
    // rows and heads out of range are zeroed afterwards.
    {
      const int s = s0 + ((col >> 2) & 1), h = 4 * (col >> 3) + (col & 3);
      const bool ok = (s < S) && (h < H);
      const T* src = q_idx + ((size_t)(b * S + min(s, S - 1)) * H + min(h, H - 1)) * DI;
#pragma unroll
      for (int st = 0; st < Tr::kSteps; ++st) {
        uint4 raw = ld_vec<uint4>(src + 16 * st + 8 * half);
        if (!ok) raw = make_uint4(0, 0, 0, 0);
        a[p][st] = __builtin_bit_cast(V8, raw);
      }
    }
    const int s = s0 + half;
    const float* wrow = w_idx + (size_t)(b * S + min(s, S - 1)) * H;
    if (H == 16) {                       // 64-byte aligned row: four 16-byte loads
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const f32x4 w4 = ld_vec<f32x4>(wrow + 4 * v4);
#pragma unroll
        for (int e = 0; e < 4; ++e) wv[p][4 * v4 + e] = w4[e];
      }
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) wv[p][v] = wrow[min(v, H - 1)];
    }
#pragma unroll
    for (int v = 0; v < 16; ++v)
      if (s >= S || v >= H) wv[p][v] = 0.0f;
  }
  // Score row of each pair's token for this lane (lanes 0..31: t0, 32..63: t1).
  float* srow[PAIRS];
  bool s_ok[PAIRS];
#pragma unroll
  for (int p = 0; p < PAIRS; ++p) {
    const int s = s_first + wave * 2 * PAIRS + 2 * p + half;
    s_ok[p] = s < S;
    srow[p] = scores + ((size_t)b * S + (s_ok[p] ? s : 0)) * L_cap + col;
  }
  wait_vmem();              // this wave's share of the run has landed in LDS
  __syncthreads();          // ... and every other wave's

#pragma unroll 2
  for (int jc = j_begin; jc < j_end; jc += 32) {
    const int r = jc - j_begin + col;      // this lane's run row (B column n = col)
    f32x16 acc[PAIRS];
#pragma unroll
    for (int p = 0; p < PAIRS; ++p) acc[p] = f32x16{};
#pragma unroll
    for (int st = 0; st < Tr::kSteps; ++st) {
      const int ch = 2 * st + half;
      V8 bop = __builtin_bit_cast(V8, run[r * Tr::kChunks + (ch ^ Tr::swz(r))]);
#pragma unroll
      for (int p = 0; p < PAIRS; ++p) acc[p] = mfma32x32x16(a[p][st], bop, acc[p]);
    }
    const bool key_ok = jc + col < j_end;
#pragma unroll
    for (int p = 0; p < PAIRS; ++p) {
      // sum over the 16 heads (two chains of 8, then one add)
      float part0 = 0.0f, part1 = 0.0f;
#pragma unroll
      for (int v = 0; v < 8; ++v) part0 += wv[p][v] * acc[p][v];
#pragma unroll
      for (int v = 8; v < 16; ++v) part1 += wv[p][v] * acc[p][v];
      const float total = part0 + part1;
      if (s_ok[p] && key_ok) srow[p][jc] = total;
    }
  }
}

template <typename T, int DI, int PAIRS, int WAVES, int KR>
void launch_idx(const IndexerLaunch& a, hipStream_t st) {
  dim3 grid(a.tok_blocks, a.key_blocks, a.B);
  hipLaunchKernelGGL((indexer_score_kernel<T, DI, PAIRS, WAVES, KR>), grid, dim3(WAVES * kWave), 0,
                     st, (const T*)a.q_idx, a.w_idx, (const T*)a.key_state, a.kv_len, a.S, a.H,
                     a.L_cap, a.keys_per_wg, a.scores);
}

// Largest key run a workgroup keeps in LDS: 64 KB at prefill (two
// workgroups per CU), 32 KB at decode.
template <int DI> constexpr int kPrefillRun = 65536 / (2 * DI);
template <int DI> constexpr int kDecodeRun = 32768 / (2 * DI);

template <typename T, bool PREFILL>
void launch_idx_d(const IndexerLaunch& a, hipStream_t st) {
  switch (a.D_idx) {
    case 32:
      if (PREFILL) launch_idx<T, 32, 2, 8, kPrefillRun<32>>(a, st);
      else launch_idx<T, 32, 1, 4, kDecodeRun<32>>(a, st);
      break;
    case 64:
      if (PREFILL) launch_idx<T, 64, 2, 8, kPrefillRun<64>>(a, st);
      else launch_idx<T, 64, 1, 4, kDecodeRun<64>>(a, st);
      break;
    default:   // one token pair per wave keeps the 128-dim operands in registers
      if (PREFILL) launch_idx<T, 128, 1, 8, kPrefillRun<128>>(a, st);
      else launch_idx<T, 128, 1, 4, kDecodeRun<128>>(a, st);
      break;
  }
}

}  // namespace

IndexerLaunch plan_indexer(int B, int S, int D_idx, int max_kv_len) {
  IndexerLaunch a{};
  a.B = B;
  a.S = S;
  a.D_idx = D_idx;
  // Decode (S <= 8): 4 waves x 1 token pair.  Prefill: 8 waves x 2 pairs
  // (1 pair for D_idx = 128), 32 tokens sharing every key run.
  const bool prefill = S > 8;
  a.prefill = prefill;
  a.pairs = prefill && D_idx < 128 ? 2 : 1;
  a.waves = prefill ? 8 : 4;
  a.tile = (prefill ? 65536 : 32768) / (2 * D_idx);   // key-run capacity (LDS)
  const int tok_per_wg = 2 * a.pairs * a.waves;
  a.tok_blocks = (S + tok_per_wg - 1) / tok_per_wg;
  // Aim for ~1024 workgroups (4 per CU); runs are whole 32-key chunks and
  // fit the LDS capacity.
  const long long want = ((long long)max_kv_len * B * a.tok_blocks + 1023) / 1024;
  long long kpw = ((want + 31) / 32) * 32;
  if (kpw < 32) kpw = 32;
  if (kpw > a.tile) kpw = a.tile;
  a.keys_per_wg = (int)kpw;
  a.key_blocks = (int)((max_kv_len + kpw - 1) / kpw);
  return a;
}

void launch_indexer(const IndexerLaunch& a, hipStream_t st) {
  if (a.key_blocks == 0 || a.tok_blocks == 0 || a.B == 0) return;
  const bool prefill = a.prefill;
  if (a.bf16) {
    if (prefill) launch_idx_d<__bf16, true>(a, st); else launch_idx_d<__bf16, false>(a, st);
  } else {
    if (prefill) launch_idx_d<_Float16, true>(a, st); else launch_idx_d<_Float16, false>(a, st);
  }
}

}  // namespace dsa
