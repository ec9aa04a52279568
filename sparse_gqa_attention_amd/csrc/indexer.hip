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
// Prefill (S > 8) folds the head weights into the query first
// (indexer_fold_kernel, below).  The per-head streaming kernel
// (indexer_stream_kernel) serves very long decode contexts, and prefill
// when L_cap >= 2^24: a workgroup holds 32 query tokens (8
// waves x 2 token pairs; 16 tokens, one pair per wave, at D_idx 128) in
// registers and streams a range of keys through two LDS buffers.  Each run of
// keys is copied by direct global->LDS loads (16-byte chunks XOR-swizzled by
// row so that the B-operand reads of different keys hit different banks);
// the copy of the next run is issued before the current run is scored, so it
// lands while the MFMAs run.  On gfx9 one in-order counter tracks loads and
// stores alike, so the wait for that copy would also wait for every score
// store issued after it, unless the count of those stores is known: scores
// are written with buffer stores issued unconditionally (invalid lanes get an
// out-of-range offset, which the hardware drops), so the wait names exactly
// the stores of one run and never waits for their acknowledgement.  Full
// runs are scored by fully unrolled code whose LDS reads, score stores and
// copy addresses are lane constants plus immediate or scalar offsets, so the
// vector ALU work per chunk is the head-weighted sums alone.
//
// Decode (indexer_score_kernel): a workgroup of 4 waves x 1 pair copies one
// run of keys into LDS, then scores it.  Long decode contexts (more key runs
// than two per CU) use the streaming kernel in a decode shape instead, 4
// waves x 1 pair streaming up to four runs: the next run's copy overlaps the
// current run's MFMAs, and the query operands are read once per four runs.
//
// The XCD-aware renumbering dispatches the token blocks that share a key
// range consecutively on one XCD and deals key ranges to the XCDs in turn,
// so key-state runs are read through L2 (for the per-head streaming kernel
// at a 2048-token prefill over 128K keys: 52-74 MB of HBM-side fetch
// against 1 GiB of LDS copies) and every XCD gets an equal share of every
// sequence.
#include <type_traits>

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

// XCD-aware workgroup renumbering.  Workgroups are handed to the 8 XCDs
// round-robin by linear id.  A key group (key block ty of sequence tz) is
// read by all tok_blocks token blocks; renumber so that each key group's
// token blocks are dispatched consecutively on one XCD (they then share the
// run through that XCD's L2) and key groups are dealt to the XCDs in turn,
// so every XCD gets an equal share of every sequence's keys whatever the
// sequence lengths.  Needs a multiple of 8 key groups (the planner rounds
// the key blocks up); otherwise the dispatch order is kept.
__device__ __forceinline__ void xcd_tile(int& tx, int& ty, int& tz) {
  tx = blockIdx.x; ty = blockIdx.y; tz = blockIdx.z;
  const int nx = gridDim.x, ny = gridDim.y;
  const int groups = ny * gridDim.z;
  if ((groups & 7) == 0) {
    const int lin = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
    const int k = lin >> 3;                  // dispatch slot within the XCD
    const int g = (k / nx) * 8 + (lin & 7);  // key group
    tx = k - (k / nx) * nx;
    tz = g / ny;
    ty = g - tz * ny;
  }
}

// An empty use of a register value.  Placed on a kernel's early-exit path
// it keeps loads whose results the other path consumes above the branch
// (the compiler would otherwise sink them past it, adding a memory round
// trip after the branch); the exit path waits for every load anyway.
template <typename V>
__device__ __forceinline__ void keep_loaded(const V& v) {
  asm volatile("" ::"v"(v));
}

typedef __attribute__((address_space(3))) char lds_char;

// global_load_lds_dwordx4 written out, for copies whose completion the
// caller tracks itself: the compiler does not see the LDS write, so it adds
// no wait for it before later LDS reads (its alias analysis cannot tell the
// two stream buffers apart and would wait for every outstanding load and
// store).  Lane l's 16 bytes land at lds_dst + 16 * l.  M0 is saved and
// restored, and one wait state separates its write from the load that
// reads it.
__device__ __forceinline__ void lds_dma16_untracked(const void* g, void* lds_dst) {
  const uint32_t m = (uint32_t)(uintptr_t)(lds_char*)lds_dst;
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0"
      : "=&s"(saved)
      : "v"(g), "s"(m)
      : "memory");
}

// Direct global->LDS copy of key rows [j0, j1) of one sequence into dst.
// Slot q holds chunk (q % kChunks) ^ swz(r) of row r = q / kChunks; a wave
// fills 64 consecutive slots per load.  Rows are rounded up to whole 32-key
// chunks; rows past j1 repeat row j1 - 1 (their scores are never stored).
// UNTRACKED: issue the loads unseen by the compiler (see above).
template <typename T, int DI, int NT, bool UNTRACKED>
__device__ __forceinline__ void copy_key_rows(const T* __restrict__ ks_b, int j0, int j1,
                                              uint4* __restrict__ dst, int wave, int l) {
  using Tr = IdxTraits<T, DI>;
  const int nvec = ((j1 - j0 + 31) & ~31) * Tr::kChunks;   // multiple of 64
  for (int q0 = wave * kWave; q0 < nvec; q0 += NT) {
    const int q = q0 + l;
    const int r = q / Tr::kChunks, c = q % Tr::kChunks;
    const int j = min(j0 + r, j1 - 1);
    const T* src = ks_b + (size_t)j * DI + 8 * (c ^ Tr::swz(r));
    if (UNTRACKED) lds_dma16_untracked(src, dst + q0);
    else __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(dst + q0), 16, 0, 0);
  }
}

// A operands and head weights of one token pair (tokens s0, s0 + 1).
// MFMA row m <-> token (m/4)%2 of the pair, head 4*(m/8) + m%4.  With the
// 32x32 accumulator layout (element v of lane l is row 8*(v/4) + 4*(l/32)
// + v%4) every lane then holds all 16 heads of one token, token l/32, as
// elements v = head.  A operand: lane l supplies row l%32, k = 16*step +
// 8*(l/32).  Loads are unconditional from clamped addresses (no per-load
// branch); rows and heads out of range are zeroed afterwards.
template <typename T, int DI>
__device__ __forceinline__ void load_pair(const T* __restrict__ q_idx,
                                          const float* __restrict__ w_idx, int b, int S, int H,
                                          int s0, int col, int half,
                                          typename vec8<T>::type (&a)[DI / 16], float (&wv)[16]) {
  using V8 = typename vec8<T>::type;
  {
    const int s = s0 + ((col >> 2) & 1), h = 4 * (col >> 3) + (col & 3);
    const bool ok = (s < S) && (h < H);
    const T* src = q_idx + ((size_t)(b * S + min(s, S - 1)) * H + min(h, H - 1)) * DI;
#pragma unroll
    for (int st = 0; st < DI / 16; ++st) {
      uint4 raw = ld_vec<uint4>(src + 16 * st + 8 * half);
      if (!ok) raw = make_uint4(0, 0, 0, 0);
      a[st] = __builtin_bit_cast(V8, raw);
    }
  }
  const int s = s0 + half;
  const float* wrow = w_idx + (size_t)(b * S + min(s, S - 1)) * H;
  if (H == 16) {                       // 64-byte aligned row: four 16-byte loads
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      const f32x4 w4 = ld_vec<f32x4>(wrow + 4 * v4);
#pragma unroll
      for (int e = 0; e < 4; ++e) wv[4 * v4 + e] = w4[e];
    }
  } else {
#pragma unroll
    for (int v = 0; v < 16; ++v) wv[v] = wrow[min(v, H - 1)];
  }
#pragma unroll
  for (int v = 0; v < 16; ++v)
    if (s >= S || v >= H) wv[v] = 0.0f;
}

// Per-head dot products of one token pair with 32 keys: run row r of the
// LDS copy is this lane's key (B column n = col).
template <typename T, int DI, int PAIRS>
__device__ __forceinline__ void score_chunk(const uint4* __restrict__ run, int r, int half,
                                            const typename vec8<T>::type (&a)[PAIRS][DI / 16],
                                            f32x16 (&acc)[PAIRS]) {
  using Tr = IdxTraits<T, DI>;
  using V8 = typename vec8<T>::type;
#pragma unroll
  for (int p = 0; p < PAIRS; ++p) acc[p] = f32x16{};
#pragma unroll
  for (int st = 0; st < Tr::kSteps; ++st) {
    const int ch = 2 * st + half;
    const V8 bop = __builtin_bit_cast(V8, run[r * Tr::kChunks + (ch ^ Tr::swz(r))]);
#pragma unroll
    for (int p = 0; p < PAIRS; ++p) acc[p] = mfma32x32x16(a[p][st], bop, acc[p]);
  }
}

// Sum over the 16 heads (two chains of 8, then one add).
__device__ __forceinline__ float head_sum(const float (&wv)[16], const f32x16& acc) {
  float part0 = 0.0f, part1 = 0.0f;
#pragma unroll
  for (int v = 0; v < 8; ++v) part0 += wv[v] * acc[v];
#pragma unroll
  for (int v = 8; v < 16; ++v) part1 += wv[v] * acc[v];
  return part0 + part1;
}

// ------------------------------------------------------------------ prefill

constexpr uint32_t kDropOffset = 0x80000000u;   // beyond any record count used
// Cache policy of the streamed score stores (SPOL template arguments):
// prefill writes them non-temporal (streaming), so that a gigabyte of scores
// does not push the key-state runs, which every token block of a key group
// reads, out of the caches (prefill_128k layer 1143 -> 1076 us); long decode
// contexts keep ordinary stores, since the top-k reads the scores back at
// once (decode_256k 39.1 -> 38.5 us).
constexpr int kStoreStreaming = 2, kStoreDefault = 0;

// Raw buffer resource (stride 0) over `bytes` bytes at p.  The fields pass
// through readfirstlane so that the descriptor lives in scalar registers:
// computed with vector instructions it would make every buffer store a
// per-lane loop over distinct descriptors.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t nr = __builtin_amdgcn_readfirstlane(bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, (int)nr,
                                           0x00020000);
}

// Wait until at most N vector-memory operations of this wave are
// outstanding, then a workgroup barrier with no memory fence (a fence would
// wait for every outstanding store).  The empty asm statements keep the
// compiler from moving LDS accesses across the barrier.
template <int N>
__device__ __forceinline__ void wait_vm_then_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  // gfx9 s_waitcnt: vmcnt[3:0], expcnt[6:4] (7 = no wait), lgkmcnt[11:8]
  // (15 = no wait), vmcnt[5:4] in bits [15:14].
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// global_load_lds_dwordx4 with a scalar base and a per-lane 32-bit byte
// offset, untracked as above: lane l's 16 bytes from sbase + voff land at
// lds_dst + 16 * l.
__device__ __forceinline__ void lds_dma16_saddr_untracked(const void* sbase, uint32_t voff,
                                                          void* lds_dst) {
  const uint32_t m = (uint32_t)(uintptr_t)(lds_char*)lds_dst;
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(m)
      : "memory");
}

// Per-lane constants of a full run.  The swizzle depends on the low four
// bits of the row only, and both the copy (NT / kChunks rows per load) and
// the chunks (32 rows) advance the row by multiples of 16, so every address
// of a full run is a lane constant plus a compile-time or scalar offset.
template <typename T, int DI, int NT>
struct FullRunLane {
  using Tr = IdxTraits<T, DI>;
  static_assert((NT / Tr::kChunks) % 16 == 0, "copy rows per load must keep the swizzle");
  uint32_t dma_off;              // byte offset of this lane's 16-byte source chunk
  uint32_t b_off[Tr::kSteps];    // uint4 index of this lane's B operand per K-step
  __device__ __forceinline__ FullRunLane(int wave, int l) {
    const int q = wave * kWave + l;
    const int r = q / Tr::kChunks, c = q % Tr::kChunks;
    dma_off = (uint32_t)(r * DI * (int)sizeof(T) + 16 * (c ^ Tr::swz(r)));
    const int half = l >> 5, col = l & 31;
#pragma unroll
    for (int st = 0; st < Tr::kSteps; ++st)
      b_off[st] = (uint32_t)(col * Tr::kChunks + ((2 * st + half) ^ Tr::swz(col)));
  }
};

// Copy of the R rows starting at src (a full run) into dst: the addresses
// are scalar bases plus the lane constant, no per-load vector arithmetic.
template <typename T, int DI, int NT, int R>
__device__ __forceinline__ void copy_full_run(const T* __restrict__ src, uint4* __restrict__ dst,
                                              int wave, const FullRunLane<T, DI, NT>& ln) {
  using Tr = IdxTraits<T, DI>;
  static_assert((R * Tr::kChunks) % NT == 0, "a full run is a whole number of loads per wave");
  constexpr int kRowsPerLoad = NT / Tr::kChunks;
#pragma unroll
  for (int k = 0; k < R * Tr::kChunks / NT; ++k)
    lds_dma16_saddr_untracked(src + (size_t)k * kRowsPerLoad * DI, ln.dma_off,
                              dst + wave * kWave + k * NT);
}

// Scores of a full run [jr, jr + R) held in `cur`, fully unrolled: LDS reads
// and score stores use immediate offsets from lane constants, so the VALU
// work per chunk is the head-weighted sums alone.  Every chunk issues
// exactly PAIRS buffer stores (all lanes in range: a full run has no key
// past its end).
template <typename T, int DI, int PAIRS, int NT, int R, bool PREFETCH, int SPOL>
__device__ __forceinline__ void score_full_run(
    const uint4* __restrict__ cur, int jr, const FullRunLane<T, DI, NT>& ln,
    const typename vec8<T>::type (&a)[PAIRS][DI / 16], const float (&wv)[PAIRS][16],
    __amdgpu_buffer_rsrc_t rs, const uint32_t (&row_off)[PAIRS]) {
  using Tr = IdxTraits<T, DI>;
  using V8 = typename vec8<T>::type;
  uint32_t off[PAIRS];
#pragma unroll
  for (int p = 0; p < PAIRS; ++p) off[p] = row_off[p] + 4u * (uint32_t)jr;
  // PREFETCH: B operands of chunk c + 1 are read before chunk c's epilogue,
  // so the LDS latency hides behind the head sums (16 more registers).
  V8 bop[2][Tr::kSteps];
#pragma unroll
  for (int st = 0; st < Tr::kSteps; ++st)
    bop[0][st] = __builtin_bit_cast(V8, cur[ln.b_off[st]]);
#pragma unroll
  for (int c = 0; c < R / 32; ++c) {
    f32x16 acc[PAIRS];
#pragma unroll
    for (int p = 0; p < PAIRS; ++p) acc[p] = f32x16{};
#pragma unroll
    for (int st = 0; st < Tr::kSteps; ++st) {
#pragma unroll
      for (int p = 0; p < PAIRS; ++p) acc[p] = mfma32x32x16(a[p][st], bop[c & 1][st], acc[p]);
    }
    if (PREFETCH && c + 1 < R / 32) {
#pragma unroll
      for (int st = 0; st < Tr::kSteps; ++st)
        bop[(c + 1) & 1][st] =
            __builtin_bit_cast(V8, cur[ln.b_off[st] + (c + 1) * 32 * Tr::kChunks]);
    }
#pragma unroll
    for (int p = 0; p < PAIRS; ++p)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(head_sum(wv[p], acc[p])), rs,
                                            off[p] + 128u * c, 0, SPOL);
    if (!PREFETCH && c + 1 < R / 32) {
#pragma unroll
      for (int st = 0; st < Tr::kSteps; ++st)
        bop[(c + 1) & 1][st] =
            __builtin_bit_cast(V8, cur[ln.b_off[st] + (c + 1) * 32 * Tr::kChunks]);
    }
  }
}

// One stage of the key stream: issue the copy of the next run [jn, jn_end)
// into `nxt` (none when jn >= jn_end), then score the run [jr, jr_end) held
// in `cur`.  The copy is issued untracked: the wait for it is the caller's.
// Every chunk issues exactly PAIRS buffer stores.  Full runs take the
// unrolled paths; the last, partial run of a range the general ones.
template <typename T, int DI, int PAIRS, int NT, int R, bool PREFETCH, int SPOL>
__device__ __forceinline__ void stream_stage(
    const uint4* __restrict__ cur, uint4* __restrict__ nxt, const T* __restrict__ ks_b,
    int jn, int jn_end, int jr, int jr_end, int wave, int l, const FullRunLane<T, DI, NT>& ln,
    const typename vec8<T>::type (&a)[PAIRS][DI / 16], const float (&wv)[PAIRS][16],
    __amdgpu_buffer_rsrc_t rs, const uint32_t (&row_off)[PAIRS]) {
  if (jn_end - jn == R) copy_full_run<T, DI, NT, R>(ks_b + (size_t)jn * DI, nxt, wave, ln);
  else if (jn < jn_end) copy_key_rows<T, DI, NT, true>(ks_b, jn, jn_end, nxt, wave, l);
  if (jr_end - jr == R) {
    score_full_run<T, DI, PAIRS, NT, R, PREFETCH, SPOL>(cur, jr, ln, a, wv, rs, row_off);
    return;
  }
  const int half = l >> 5, col = l & 31;
  for (int jc = jr; jc < jr_end; jc += 32) {
    f32x16 acc[PAIRS];
    score_chunk<T, DI, PAIRS>(cur, jc - jr + col, half, a, acc);
    const bool key_ok = jc + col < jr_end;
#pragma unroll
    for (int p = 0; p < PAIRS; ++p) {
      const uint32_t off = key_ok ? row_off[p] + 4u * (uint32_t)jc : kDropOffset;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(head_sum(wv[p], acc[p])), rs, off, 0,
                                            SPOL);
    }
  }
}

// The key stream [j_begin, j_end) in runs of R keys, the first already in b0.
// Two stages per trip, the buffers swapping roles.  The wait before a stage
// covers the copy issued at the start of the previous one: after it, that
// stage (a full run of R keys) issued PAIRS * R / 32 stores.
template <typename T, int DI, int PAIRS, int NT, int R, bool PREFETCH, int SPOL>
__device__ __forceinline__ void stream_keys(
    uint4* __restrict__ b0, uint4* __restrict__ b1, const T* __restrict__ ks_b, int j_begin,
    int j_end, int wave, int l, const FullRunLane<T, DI, NT>& ln,
    const typename vec8<T>::type (&a)[PAIRS][DI / 16],
    const float (&wv)[PAIRS][16], __amdgpu_buffer_rsrc_t rs, const uint32_t (&row_off)[PAIRS]) {
  constexpr int kStoresPerRun = PAIRS * R / 32;
  int jr = j_begin;
  while (true) {
    int jr_end = min(jr + R, j_end);
    stream_stage<T, DI, PAIRS, NT, R, PREFETCH, SPOL>(b0, b1, ks_b, jr_end, min(jr_end + R, j_end), jr, jr_end,
                                      wave, l, ln, a, wv, rs, row_off);
    if (jr_end >= j_end) break;
    wait_vm_then_barrier<kStoresPerRun>();
    jr = jr_end;
    jr_end = min(jr + R, j_end);
    stream_stage<T, DI, PAIRS, NT, R, PREFETCH, SPOL>(b1, b0, ks_b, jr_end, min(jr_end + R, j_end), jr, jr_end,
                                      wave, l, ln, a, wv, rs, row_off);
    if (jr_end >= j_end) break;
    wait_vm_then_barrier<kStoresPerRun>();
    jr = jr_end;
  }
}

// R keys per LDS buffer (two buffers, 64 KB per workgroup: two workgroups
// per CU).  Byte offsets within a wave's 4 score rows stay below 2^31 for
// L_cap <= kIndexerMaxLcap.
template <typename T, int DI, int PAIRS, int WAVES, int R, int WPE, bool PREFETCH, int SPOL>
__global__ __launch_bounds__(WAVES * kWave, WPE) void indexer_stream_kernel(
    const T* __restrict__ q_idx, const float* __restrict__ w_idx,
    const T* __restrict__ key_state, const int32_t* __restrict__ kv_len,
    int S, int H, int L_cap, int keys_per_wg, float* __restrict__ scores) {
  using Tr = IdxTraits<T, DI>;
  using V8 = typename vec8<T>::type;
  constexpr int NT = WAVES * kWave;
  constexpr int kTokPerWave = 2 * PAIRS;
  constexpr int kTokPerWg = kTokPerWave * WAVES;
  static_assert(R % 32 == 0, "runs are whole 32-key chunks");
  __shared__ __attribute__((aligned(16))) uint4 buf0[R * Tr::kChunks];
  __shared__ __attribute__((aligned(16))) uint4 buf1[R * Tr::kChunks];

  int tx, ty, tz;
  xcd_tile(tx, ty, tz);
  const int b = tz;
  const int j_begin = ty * keys_per_wg;
  const int s_first = tx * kTokPerWg;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int l = lane_id();
  const int half = l >> 5, col = l & 31;
  const T* ks_b = key_state + (size_t)b * L_cap * DI;

  // The first run's copy and the query operands go out before kv_len is read
  // (the copy covers cache rows that exist whatever the live length:
  // [j_begin, L_cap)), so they share one memory round trip.  A workgroup
  // that then finds no live key waits for its copies before it ends.
  const FullRunLane<T, DI, NT> ln(wave, l);
  const int j_cap = min(j_begin + R, L_cap);
  if (j_cap - j_begin >= R) copy_full_run<T, DI, NT, R>(ks_b + (size_t)j_begin * DI, buf0, wave, ln);
  else if (j_begin < j_cap) copy_key_rows<T, DI, NT, true>(ks_b, j_begin, j_cap, buf0, wave, l);
  V8 a[PAIRS][Tr::kSteps];
  float wv[PAIRS][16];
  const int s_w = s_first + wave * kTokPerWave;        // first token of this wave
#pragma unroll
  for (int p = 0; p < PAIRS; ++p)
    load_pair<T, DI>(q_idx, w_idx, b, S, H, s_w + 2 * p, col, half, a[p], wv[p]);
  int kvl = kv_len[b];
  kvl = kvl < 0 ? 0 : (kvl > L_cap ? L_cap : kvl);
  const int j_end = min(j_begin + keys_per_wg, kvl);
  // Keys beyond the last position of this block's tokens are never selected.
  const int last_pos = kvl - S + min(s_first + kTokPerWg, S) - 1;
  if (j_begin >= j_end || j_begin > last_pos) {
    wait_vmem();            // no copy may land after the workgroup ends
#pragma unroll
    for (int p = 0; p < PAIRS; ++p)
#pragma unroll
      for (int st = 0; st < Tr::kSteps; ++st) keep_loaded(a[p][st]);
    return;
  }

  // Score stores: one buffer resource per wave based at its first token's
  // row; tokens past S fall outside its record count and are dropped.
  const int n_tok = max(0, min(S - s_w, kTokPerWave));
  const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(
      scores + ((size_t)b * S + min(s_w, S - 1)) * L_cap, (uint32_t)n_tok * (uint32_t)L_cap * 4u);
  uint32_t row_off[PAIRS];
#pragma unroll
  for (int p = 0; p < PAIRS; ++p) {
    const int t = 2 * p + half;
    row_off[p] = t < n_tok ? (uint32_t)(t * L_cap + col) * 4u : kDropOffset;
  }

  wait_vmem();              // this wave's share of the first run has landed
  __syncthreads();          // ... and every other wave's
  stream_keys<T, DI, PAIRS, NT, R, PREFETCH, SPOL>(buf0, buf1, ks_b, j_begin, j_end, wave, l, ln, a,
                                                   wv, rs, row_off);
}

// ------------------------------------------------------------------ folded prefill
// The score has no per-head nonlinearity, so
//   sum_h w_h (q_h . k) = (sum_h w_h q_h) . k:
// the prefill kernel folds the head weights into the query once per token
// (q' in FP32; exact for integer inputs while its partial sums stay below
// 2^24) and contracts q' with the keys: one 32-token x 32-key MFMA tile
// instead of sixteen per-head tiles, so the stage is bound by its score
// stores.  q' enters the MFMA in parts of the key's 16-bit type, each
// multiplied by the exact key and accumulated in FP32:
//   BF16: hi + mid + lo hold q's 24-bit significand (BF16 has FP32's range);
//   FP16: hi + lo hold 22 bits; a token whose largest |q'| is 2^14 or more,
//         or below 1, is scaled by a power of two first (into [2^13, 2^14))
//         and its scores scaled back (both exact), so no part overflows or
//         falls into FP16 subnormals.
// A workgroup of 4 waves holds 32 tokens; wave w walks the 32-key chunks w,
// w + 4, ... of the workgroup's key range, its B operands (the key rows)
// loaded from global memory one chunk ahead; the key ranges of the token
// blocks that share them run consecutively on one XCD (xcd_tile), so the
// key rows come from that XCD's L2.
constexpr int kFoldWaves = 4;
constexpr int kFoldTokens = 32;

template <typename T, int DI, int SPOL>
__global__ __launch_bounds__(kFoldWaves * kWave) void indexer_fold_kernel(
    const T* __restrict__ q_idx, const float* __restrict__ w_idx,
    const T* __restrict__ key_state, const int32_t* __restrict__ kv_len,
    int S, int H, int L_cap, int keys_per_wg, float* __restrict__ scores) {
  using V8 = typename vec8<T>::type;
  constexpr bool kBF16 = std::is_same<T, __bf16>::value;
  constexpr int kParts = kBF16 ? 3 : 2;
  constexpr int NT = kFoldWaves * kWave;
  constexpr int kSteps = DI / 16;
  constexpr int kGroup = DI / 8;                 // threads per token in the fold
  __shared__ float qf[kFoldTokens][DI + 4];      // folded queries, FP32
  __shared__ float qexp[kFoldTokens];            // FP16: 2^-e of the token's scale

  int tx, ty, tz;
  xcd_tile(tx, ty, tz);
  const int b = tz;
  const int j_begin = ty * keys_per_wg;
  const int s0 = tx * kFoldTokens;
  const int wave = threadIdx.x / kWave;
  const int l = lane_id();
  int kvl = kv_len[b];
  kvl = kvl < 0 ? 0 : (kvl > L_cap ? L_cap : kvl);
  const int j_end = min(j_begin + keys_per_wg, kvl);
  // keys beyond the last position of this block's tokens are never selected
  const int last_pos = kvl - S + min(s0 + kFoldTokens, S) - 1;
  if (j_begin >= j_end || j_begin > last_pos) return;   // block-uniform

  // ---- q'[token][d] = sum_h w[token][h] q[token][h][d]: a thread per
  // (token, 8 dims), 16-byte query loads; FP16 scales q' by 2^e (e <= 0)
  static_assert(NT % kGroup == 0 && kGroup <= kWave, "a token's threads share a wave");
  for (int e = threadIdx.x; e < kFoldTokens * kGroup; e += NT) {
    const int tok = e / kGroup, d8 = e % kGroup;
    const int s = s0 + tok;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (s < S) {
      const size_t row = (size_t)b * S + s;
      const T* qrow = q_idx + row * H * DI + 8 * d8;
      const float* wrow = w_idx + row * H;
      for (int h = 0; h < H; ++h) {
        const float wh = wrow[h];
        const uint4 raw = ld_vec<uint4>(qrow + (size_t)h * DI);
        T v[8];
        __builtin_memcpy(v, &raw, 16);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(wh, to_f32(v[i]), acc[i]);
      }
    }
    if constexpr (!kBF16) {
      float mx = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf(acc[i]));
#pragma unroll
      for (int o = kGroup / 2; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
      // a largest |q'| of 2^14 or more is scaled below 2^14 (hi + lo stay
      // finite), one below 1 up to [2^13, 2^14) (clear of FP16 subnormals);
      // integer-valued q' (|q'| >= 1, or 0) is never scaled, so the
      // integer-exact case is unchanged; 0 and non-finite keep e = 0
      int ex = 0;
      if (mx > 0.0f && mx <= 3.0e38f && (mx >= 16384.0f || mx < 1.0f)) {
        int m;
        (void)frexpf(mx, &m);                   // mx in [2^(m-1), 2^m)
        ex = 14 - m;                            // mx * 2^ex in [2^13, 2^14)
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = ldexpf(acc[i], ex);
      if (d8 == 0) qexp[tok] = ldexpf(1.0f, -ex);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) qf[tok][8 * d8 + i] = acc[i];
  }
  __syncthreads();

  // ---- A operands: lane l supplies token l % 32, dims 16 st + 8 (l / 32)
  // + [0, 8) of each K-step, as kParts parts of the 16-bit type
  V8 a[kParts][kSteps];
#pragma unroll
  for (int st = 0; st < kSteps; ++st) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float r = qf[l & 31][16 * st + 8 * (l >> 5) + i];
#pragma unroll
      for (int p = 0; p < kParts; ++p) {
        const T part = from_f32<T>(r);
        a[p][st][i] = part;
        r -= to_f32(part);
      }
    }
  }
  // element v of lane l is token 8 (v / 4) + 4 (l / 32) + v % 4 of the tile
  float post[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) post[v] = kBF16 ? 1.0f : qexp[8 * (v >> 2) + 4 * (l >> 5) + (v & 3)];

  // ---- scores, key l % 32 of each chunk.  One buffer resource over the
  // block's token rows: tokens past S fall outside it and are dropped, keys
  // past the live range get an out-of-range offset.
  const int n_tok = max(0, min(S - s0, kFoldTokens));
  const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(
      scores + ((size_t)b * S + min(s0, S - 1)) * L_cap, (uint32_t)n_tok * (uint32_t)L_cap * 4u);
  const uint32_t row_bytes = (uint32_t)__builtin_amdgcn_readfirstlane(L_cap * 4);
  const T* ks_b = key_state + (size_t)b * L_cap * DI + 8 * (l >> 5);
  // B operands of a chunk: lane l supplies key l % 32, dims 16 st + 8 (l / 32)
  // + [0, 8); addresses clamped into the cache, so the loads are
  // unconditional
  auto load_b = [&](int jc, V8 (&bop)[kSteps]) {
    const int key = min(jc + (l & 31), L_cap - 1);
    const T* src = ks_b + (size_t)key * DI;
#pragma unroll
    for (int st = 0; st < kSteps; ++st) bop[st] = __builtin_bit_cast(V8, ld_vec<uint4>(src + 16 * st));
  };
  constexpr int kStride = 32 * kFoldWaves;
  // One chunk: the MFMAs on its B operands, then its 16 score stores.
  auto chunk = [&](int jc, const V8 (&bop)[kSteps]) {
    f32x16 acc = f32x16{};
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
#pragma unroll
      for (int p = 0; p < kParts; ++p) acc = mfma32x32x16(a[p][st], bop[st], acc);
    }
    // Lane part of the offset (token 4 (l / 32), key l % 32) with bit 31
    // set for keys past the live range (beyond the resource: dropped), and
    // the scalar part per element (token 8 (v / 4) + v % 4); no branch, so
    // every chunk issues exactly 16 stores.
    const int key = jc + (l & 31);
    const uint32_t drop = ((uint32_t)(j_end - 1 - key) >> 31) << 31;
    const uint32_t voff = (((uint32_t)(4 * (l >> 5)) * (uint32_t)L_cap + (uint32_t)key) * 4u) | drop;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const uint32_t soff = (uint32_t)(8 * (v >> 2) + (v & 3)) * row_bytes;
      const float sc = kBF16 ? acc[v] : acc[v] * post[v];
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), rs, voff, (int)soff, SPOL);
    }
  };
  // Two chunks per trip, the operand sets swapping roles; each set is
  // reloaded (one chunk ahead, clamped past the end) right after its chunk.
  // The trip has no exit between its chunks (the compiler would sink the
  // loads past it); a second chunk past the range stores nothing.  The
  // scheduling barriers keep each load ahead of the chunk it overlaps.  The
  // compiler's wait before a chunk counts the memory operations issued after
  // that chunk's loads and takes the smaller count of the loop's entry and
  // back edge; 16 dropped stores (distinct addresses, so none is merged away)
  // in the prologue give the entry the same 20
  // (16 stores, 4 loads) as every later trip, so no wait covers a store.
  int jc = j_begin + 32 * wave;
  if (jc >= j_end) return;                      // this wave has no chunk
  // (the prologue sits in one block with the loop, so the compiler keeps
  // its order)
  V8 b0[kSteps], b1[kSteps];
  load_b(jc, b0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int v = 0; v < 16; ++v)
    __builtin_amdgcn_raw_buffer_store_b32(0u, rs, kDropOffset + 4u * v, 0, SPOL);
  load_b(jc + kStride, b1);
  __builtin_amdgcn_sched_barrier(0);
  do {
    chunk(jc, b0);
    load_b(jc + 2 * kStride, b0);
    __builtin_amdgcn_sched_barrier(0);
    chunk(jc + kStride, b1);
    load_b(jc + 3 * kStride, b1);
    __builtin_amdgcn_sched_barrier(0);
    jc += 2 * kStride;
  } while (jc < j_end);
}

// ------------------------------------------------------------------ decode

template <typename T, int DI, int PAIRS, int WAVES, int KR>
__global__ __launch_bounds__(WAVES * kWave, 1) void indexer_score_kernel(
    const T* __restrict__ q_idx, const float* __restrict__ w_idx,
    const T* __restrict__ key_state, const int32_t* __restrict__ kv_len,
    int S, int H, int L_cap, int keys_per_wg, float* __restrict__ scores) {
  using Tr = IdxTraits<T, DI>;
  using V8 = typename vec8<T>::type;
  constexpr int NT = WAVES * kWave;
  constexpr int kTokPerWg = 2 * PAIRS * WAVES;
  __shared__ __attribute__((aligned(16))) uint4 run[KR * Tr::kChunks];

  int tx, ty, tz;
  xcd_tile(tx, ty, tz);
  const int b = tz;
  const int j_begin = ty * keys_per_wg;
  const int s_first = tx * kTokPerWg;
  const int wave = threadIdx.x / kWave;
  const int l = lane_id();
  const int half = l >> 5;     // 0: lanes 0..31, 1: lanes 32..63
  const int col = l & 31;
  const T* ks_b = key_state + (size_t)b * L_cap * DI;
  // The run's copy and the query operands go out before kv_len is read
  // (cache rows [j_begin, L_cap) exist whatever the live length), so they
  // share one memory round trip; rows past the live length are copied but
  // never scored.  A workgroup that finds no live key waits for its copies
  // before it ends.
  const int j_cap = min(j_begin + keys_per_wg, L_cap);
  if (j_begin < j_cap) copy_key_rows<T, DI, NT, false>(ks_b, j_begin, j_cap, run, wave, l);
  V8 a[PAIRS][Tr::kSteps];
  float wv[PAIRS][16];
#pragma unroll
  for (int p = 0; p < PAIRS; ++p)
    load_pair<T, DI>(q_idx, w_idx, b, S, H, s_first + wave * 2 * PAIRS + 2 * p, col, half, a[p],
                     wv[p]);
  int kvl = kv_len[b];
  kvl = kvl < 0 ? 0 : (kvl > L_cap ? L_cap : kvl);
  const int j_end = min(j_begin + keys_per_wg, kvl);
  const int last_pos = kvl - S + min(s_first + kTokPerWg, S) - 1;
  if (j_begin >= j_end || j_begin > last_pos) {
    wait_vmem();
#pragma unroll
    for (int p = 0; p < PAIRS; ++p)
#pragma unroll
      for (int st = 0; st < Tr::kSteps; ++st) keep_loaded(a[p][st]);
    return;
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

  for (int jc = j_begin; jc < j_end; jc += 32) {
    f32x16 acc[PAIRS];
    score_chunk<T, DI, PAIRS>(run, jc - j_begin + col, half, a, acc);
    const bool key_ok = jc + col < j_end;
#pragma unroll
    for (int p = 0; p < PAIRS; ++p) {
      const float total = head_sum(wv[p], acc[p]);
      if (s_ok[p] && key_ok) srow[p][jc] = total;
    }
  }
}

// Prefill workgroup shapes per D_idx: waves, token pairs per wave, keys per
// LDS buffer (two buffers), the launch bound in waves per SIMD, workgroups
// resident per CU (LDS- and register-limited), and whether a full run
// reads the next chunk's B operands ahead.
template <int DI> struct StreamCfg;
template <> struct StreamCfg<32> {
  static constexpr int kWaves = 8, kPairs = 2, kRun = 512, kWpe = 4, kWgPerCu = 2;
  static constexpr bool kPrefetch = false;
};
template <> struct StreamCfg<64> {
  static constexpr int kWaves = 8, kPairs = 2, kRun = 256, kWpe = 4, kWgPerCu = 2;
  static constexpr bool kPrefetch = false;
};
template <> struct StreamCfg<128> {    // one pair keeps the 128-dim operands in registers
  static constexpr int kWaves = 8, kPairs = 1, kRun = 128, kWpe = 4, kWgPerCu = 2;
  static constexpr bool kPrefetch = false;
};

template <typename T, int DI>
void launch_stream(const IndexerLaunch& a, hipStream_t st) {
  using C = StreamCfg<DI>;
  dim3 grid(a.tok_blocks, a.key_blocks, a.B);
  hipLaunchKernelGGL(
      (indexer_stream_kernel<T, DI, C::kPairs, C::kWaves, C::kRun, C::kWpe, C::kPrefetch,
                             kStoreStreaming>),
      grid,
      dim3(C::kWaves * kWave), 0, st, (const T*)a.q_idx, a.w_idx, (const T*)a.key_state,
      a.kv_len, a.S, a.H, a.L_cap, a.keys_per_wg, a.scores);
}

// Long decode contexts: the streaming kernel with 4 waves x 1 token pair
// (the 8 tokens of a decode step) and decode-sized runs, two workgroups per
// CU (64 KB of LDS each).
template <typename T, int DI>
void launch_stream_decode(const IndexerLaunch& a, hipStream_t st) {
  constexpr int R = 32768 / (2 * DI);
  dim3 grid(a.tok_blocks, a.key_blocks, a.B);
  hipLaunchKernelGGL((indexer_stream_kernel<T, DI, 1, 4, R, 2, false, kStoreDefault>), grid,
                     dim3(4 * kWave), 0,
                     st, (const T*)a.q_idx, a.w_idx, (const T*)a.key_state, a.kv_len, a.S, a.H,
                     a.L_cap, a.keys_per_wg, a.scores);
}

template <typename T, int DI, int PAIRS, int WAVES, int KR>
void launch_resident(const IndexerLaunch& a, hipStream_t st) {
  dim3 grid(a.tok_blocks, a.key_blocks, a.B);
  hipLaunchKernelGGL((indexer_score_kernel<T, DI, PAIRS, WAVES, KR>), grid, dim3(WAVES * kWave), 0,
                     st, (const T*)a.q_idx, a.w_idx, (const T*)a.key_state, a.kv_len, a.S, a.H,
                     a.L_cap, a.keys_per_wg, a.scores);
}

// Decode keeps one 32 KB run per workgroup (4 waves x 1 token pair).
template <int DI> constexpr int kDecodeRun = 32768 / (2 * DI);

template <typename T, int DI>
void launch_fold(const IndexerLaunch& a, hipStream_t st) {
  dim3 grid(a.tok_blocks, a.key_blocks, a.B);
  hipLaunchKernelGGL((indexer_fold_kernel<T, DI, kStoreStreaming>), grid, dim3(kFoldWaves * kWave),
                     0, st, (const T*)a.q_idx, a.w_idx, (const T*)a.key_state, a.kv_len, a.S, a.H,
                     a.L_cap, a.keys_per_wg, a.scores);
}

template <typename T>
void launch_idx_d(const IndexerLaunch& a, hipStream_t st) {
  if (a.fold) {
    if (a.D_idx == 32) launch_fold<T, 32>(a, st);
    else if (a.D_idx == 64) launch_fold<T, 64>(a, st);
    else launch_fold<T, 128>(a, st);
    return;
  }
  switch (a.D_idx) {
    case 32:
      if (a.prefill) launch_stream<T, 32>(a, st);
      else if (a.stream_decode) launch_stream_decode<T, 32>(a, st);
      else launch_resident<T, 32, 1, 4, kDecodeRun<32>>(a, st);
      break;
    case 64:
      if (a.prefill) launch_stream<T, 64>(a, st);
      else if (a.stream_decode) launch_stream_decode<T, 64>(a, st);
      else launch_resident<T, 64, 1, 4, kDecodeRun<64>>(a, st);
      break;
    default:
      if (a.prefill) launch_stream<T, 128>(a, st);
      else if (a.stream_decode) launch_stream_decode<T, 128>(a, st);
      else launch_resident<T, 128, 1, 4, kDecodeRun<128>>(a, st);
      break;
  }
}

template <int DI>
void stream_shape(IndexerLaunch& a, int& wg_per_cu) {
  using C = StreamCfg<DI>;
  a.waves = C::kWaves;
  a.pairs = C::kPairs;
  a.tile = C::kRun;
  wg_per_cu = C::kWgPerCu;
}

constexpr int kNumCUs = 256;

}  // namespace

IndexerLaunch plan_indexer(int B, int S, int D_idx, int L_cap, int max_kv_len) {
  IndexerLaunch a{};
  a.B = B;
  a.S = S;
  a.D_idx = D_idx;
  // Prefill (S > 8) folds the head weights into the query.  Its score
  // stores address a 32-token block with 32-bit byte offsets: L_cap < 2^24.
  if (S > 8 && L_cap < (1 << 24)) {
    a.prefill = true;
    a.fold = true;
    a.waves = kFoldWaves;
    a.pairs = 0;
    a.tile = 0;
    a.tok_blocks = (S + kFoldTokens - 1) / kFoldTokens;
    // about 2048 workgroups (8 per CU), whole 128-key strides of the 4 waves
    const long long tiles = (long long)B * a.tok_blocks;
    long long kpw = ((long long)max_kv_len * tiles + 2047) / 2048;
    kpw = ((kpw + 127) / 128) * 128;
    if (kpw < 128) kpw = 128;
    while ((((long long)max_kv_len + kpw - 1) / kpw + 7) / 8 * 8 > 65535) kpw *= 2;
    a.keys_per_wg = (int)kpw;
    a.key_blocks = (int)((((long long)max_kv_len + kpw - 1) / kpw + 7) & ~7LL);
    return a;
  }
  // Decode (S <= 8) keeps one run per workgroup; a context so long that its
  // key blocks would exceed the grid's y limit streams as prefill does.
  const bool prefill = S > 8 || (long long)max_kv_len > 60000LL * (32768 / (2 * D_idx));
  a.prefill = prefill;
  if (prefill) {
    // Streaming workgroups.  Each takes a whole number of runs; pick the
    // runs per workgroup that minimise the modelled time: dispatch rounds
    // of the resident workgroup slots, each as long as one workgroup's runs
    // plus about half a run of prologue (query operands, first copy).
    int wg_per_cu = 1;
    if (D_idx == 32) stream_shape<32>(a, wg_per_cu);
    else if (D_idx == 64) stream_shape<64>(a, wg_per_cu);
    else stream_shape<128>(a, wg_per_cu);
    const int tok_per_wg = 2 * a.pairs * a.waves;
    a.tok_blocks = (S + tok_per_wg - 1) / tok_per_wg;
    const long long runs = ((long long)max_kv_len + a.tile - 1) / a.tile;
    const long long slots = (long long)kNumCUs * wg_per_cu;
    const long long tiles_per_run = (long long)a.tok_blocks * B;
    long long best_rpw = 1;
    double best_time = -1.0;
    const long long max_rpw = runs < 4096 ? runs : 4096;
    for (long long rpw = 1; rpw <= max_rpw; ++rpw) {
      const long long kb = (((runs + rpw - 1) / rpw) + 7) & ~7LL;
      const long long rounds = (tiles_per_run * kb + slots - 1) / slots;
      const double t = (double)rounds * ((double)rpw + 0.5);
      if (best_time < 0.0 || t < best_time - 1e-9) {
        best_time = t;
        best_rpw = rpw;
      }
    }
    a.keys_per_wg = (int)(best_rpw * a.tile);
  } else {
    // Decode (S <= 8): 4 waves x 1 token pair.  Up to two runs per CU: one
    // key run per workgroup, ~512 workgroups (at 8 x 32K keys, 64 keys each
    // measured 4.1 us against 4.9 us for 32 and 5.5 us for a full run of
    // 256), runs of whole 32-key chunks.  More runs: stream them, enough
    // runs per workgroup (at most four) that one dispatch round of two
    // workgroups per CU covers the keys, so each CU has two runs' copies in
    // flight (at 8 x 256K keys, two runs per workgroup, 512 workgroups:
    // stage 12.35 us against 12.53 us for four runs on 256 workgroups).
    a.pairs = 1;
    a.waves = 4;
    a.tile = 32768 / (2 * D_idx);
    a.tok_blocks = (S + 7) / 8;
    const long long runs = ((long long)max_kv_len + a.tile - 1) / a.tile * B * a.tok_blocks;
    if (runs > 2LL * kNumCUs) {
      a.stream_decode = true;
      long long rpw = (runs + 2 * kNumCUs - 1) / (2 * kNumCUs);
      if (rpw > 4) rpw = 4;
      a.keys_per_wg = (int)(rpw * a.tile);
    } else {
      const long long want = ((long long)max_kv_len * B * a.tok_blocks + 511) / 512;
      long long kpw = ((want + 31) / 32) * 32;
      if (kpw < 32) kpw = 32;
      if (kpw > a.tile) kpw = a.tile;
      a.keys_per_wg = (int)kpw;
    }
  }
  // Key blocks rounded up to a multiple of 8 for the XCD renumbering; the
  // extra blocks start past max_kv_len and exit at once.
  a.key_blocks = (int)((((long long)max_kv_len + a.keys_per_wg - 1) / a.keys_per_wg + 7) & ~7LL);
  return a;
}

void launch_indexer(const IndexerLaunch& a, hipStream_t st) {
  if (a.key_blocks == 0 || a.tok_blocks == 0 || a.B == 0) return;
  if (a.bf16) launch_idx_d<__bf16>(a, st);
  else launch_idx_d<_Float16>(a, st);
}

}  // namespace dsa
