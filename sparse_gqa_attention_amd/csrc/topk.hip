// Per-query top-k with lowest-index tie-break (ORT PR #33802 "Optimize ...
// for SM12x and 256K context", Summary item 2: radix histograms per key
// chunk, a merge across up to 64+ chunks and an emit of the indices).
//
// Exact selection, any FP32 input.  Scores map to order-preserving u32 keys
// (score_key).  A radix descent over the key bits -- levels of 11, 11 and 10
// bits -- finds the bin holding the k-th largest key.  Keys above that bin
// are certainly selected and go straight into a selection bitmap; keys in the
// bin are collected as candidates (or, once the bin is a single key value,
// marked in a tie bitmap).  The exact threshold T among the candidates is
// found in LDS.  Finally both bitmaps are scanned in index order: the first
// k - #{key > T} tie bits are kept (lowest indices win the tie) and the set
// bits are written out in ascending order.  Bitmap words are produced with
// wave ballots, one store per word, so ordering needs no sort at all.
//
// Two plans share these routines:
//  * row plan -- one 1024-thread workgroup per row, everything in LDS; for
//    many long rows (prefill: 2048 rows of 131072 keys).
//  * multi plan -- a few long rows (speculative decode: 8 rows of up to
//    262144 keys) spread over many workgroups per row.  K1 builds per-chunk
//    histograms and merges them with device atomics; the last workgroup of a
//    row to arrive picks the bin.  K2 fills the row's bitmaps and candidate
//    list; its last arriver finishes the selection and emits.  No workgroup
//    ever waits for another one.
#include "dsa_device.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kBins = 2048;
constexpr int kRowThreads = 1024;
constexpr int kChunkThreads = 256;
constexpr int kRowCap = 4096;      // candidate capacity of the row plan
constexpr int kMultiCap = 8192;    // candidate capacity per row of the multi plan

// Radix levels: key bits [31:21], [20:10], [9:0].
__device__ __forceinline__ int lvl_shift(int lvl) { return lvl == 0 ? 21 : (lvl == 1 ? 10 : 0); }
__device__ __forceinline__ uint32_t lvl_digit(uint32_t key, int lvl) {
  return lvl == 0 ? (key >> 21) : (lvl == 1 ? ((key >> 10) & 0x7FFu) : (key & 0x3FFu));
}
// Does `key` share the bits already fixed (all bits above level lvl)?
__device__ __forceinline__ bool lvl_match(uint32_t key, uint32_t prefix, int lvl) {
  return lvl == 0 ? true : (((key ^ prefix) >> (lvl == 1 ? 21 : 10)) == 0u);
}

__device__ __forceinline__ int row_count(const int32_t* kv_len, int row, int S, int L_cap) {
  const int b = row / S, s = row % S;
  int n = kv_len[b] - S + s + 1;     // candidates 0..pos
  return n < 0 ? 0 : (n > L_cap ? L_cap : n);
}

// Find the bin holding the need-th largest key of a 2048-bin histogram.
// Writes {bin, count of keys in higher bins} to out[0..1].  Block-wide.
template <int NT>
__device__ void select_bin(const uint32_t* hist, uint32_t need, uint32_t* scratch,
                           uint32_t* out) {
  constexpr int BPT = kBins / NT;
  const int t = threadIdx.x;
  if (t == 0) { out[0] = 0; out[1] = 0; }   // ordered before the finder by the scan's barriers
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) local += hist[kBins - 1 - (t * BPT + i)];
  uint32_t total;
  uint32_t before = block_exclusive_scan<NT>(local, scratch, &total);
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    const int bin = kBins - 1 - (t * BPT + i);
    const uint32_t h = hist[bin];
    if (before < need && need <= before + h) {
      out[0] = (uint32_t)bin;
      out[1] = before;
    }
    before += h;
  }
  __syncthreads();
}

// Keep the `m` lowest set bits of x.
__device__ __forceinline__ uint32_t keep_lowest_bits(uint32_t x, uint32_t m) {
  uint32_t r = 0;
  for (uint32_t i = 0; i < m && x; ++i) {
    const uint32_t lsb = x & (0u - x);
    r |= lsb;
    x ^= lsb;
  }
  return r;
}

// Ordered emission from bitmaps.  Words [0, nw) of sel/tie; the first
// `eq_take` tie bits (by index) join the selection; writes exactly the set
// bits, ascending, to out.  Each thread owns a contiguous run of words and
// reads them only through load_sel/load_tie.  Block-wide.
__device__ __forceinline__ uint32_t kept_ties(uint32_t tw, uint32_t running, uint32_t eq_take) {
  const uint32_t c = __popc(tw);
  if (running >= eq_take) return 0u;
  if (running + c <= eq_take) return tw;
  return keep_lowest_bits(tw, eq_take - running);
}

template <int NT, typename LoadS, typename LoadT>
__device__ void emit_bitmaps(int nw, uint32_t eq_take, LoadS load_sel, LoadT load_tie,
                             int32_t* out, uint32_t k, uint32_t* scratch) {
  const int t = threadIdx.x;
  const int wpt = (nw + NT - 1) / NT;
  const int w0 = min(t * wpt, nw), w1 = min(w0 + wpt, nw);
  uint32_t tcount = 0;
  for (int w = w0; w < w1; ++w) tcount += __popc(load_tie(w));
  uint32_t total;
  const uint32_t tie_start = block_exclusive_scan<NT>(tcount, scratch, &total);
  uint32_t running = tie_start, fcount = 0;
  for (int w = w0; w < w1; ++w) {
    const uint32_t tw = load_tie(w);
    fcount += __popc(load_sel(w) | kept_ties(tw, running, eq_take));
    running += __popc(tw);
  }
  uint32_t pos = block_exclusive_scan<NT>(fcount, scratch, &total);
  running = tie_start;
  for (int w = w0; w < w1; ++w) {
    const uint32_t tw = load_tie(w);
    uint32_t f = load_sel(w) | kept_ties(tw, running, eq_take);
    running += __popc(tw);
    while (f) {
      const int bit = __ffs(f) - 1;
      if (pos < k) out[pos] = w * 32 + bit;   // exactly k bits are set; never write past k
      ++pos;
      f &= f - 1;
    }
  }
}

// ====================================================================== row plan
// Dynamic LDS: hist[2048] | scratch[32] | misc[8] | sel[W] | tie[W] | ckey[cap] | cidx[cap]
__global__ __launch_bounds__(kRowThreads) void topk_row_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ kv_len, int S, int L_cap,
    int k, int words, int32_t* __restrict__ indices) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  uint32_t* hist = lds;
  uint32_t* scratch = hist + kBins;
  uint32_t* misc = scratch + 32;
  uint32_t* sel = misc + 8;
  uint32_t* tie = sel + words;
  uint32_t* ckey = tie + words;
  uint32_t* cidx = ckey + kRowCap;

  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const int n = row_count(kv_len, row, S, L_cap);
  int32_t* out = indices + (size_t)row * k;
  if (n <= k) {
    for (int i = t; i < k; i += kRowThreads) out[i] = i < n ? i : -1;
    return;
  }
  const float* src = scores + (size_t)row * L_cap;

  // ---- radix descent over the row until the bin is small or exact
  uint32_t prefix = 0, need = (uint32_t)k, inbin = 0;
  int lvl = 0;
  bool exact = false;
  while (true) {
    for (int i = t; i < kBins; i += kRowThreads) hist[i] = 0;
    __syncthreads();
    for (int j = t; j < n; j += kRowThreads) {
      const uint32_t key = score_key(src[j]);
      if (lvl_match(key, prefix, lvl)) atomicAdd(&hist[lvl_digit(key, lvl)], 1u);
    }
    __syncthreads();
    select_bin<kRowThreads>(hist, need, scratch, misc);
    const uint32_t bin = misc[0];
    need -= misc[1];
    inbin = hist[bin];
    prefix |= bin << lvl_shift(lvl);
    ++lvl;
    __syncthreads();
    if (lvl == 3) { exact = true; break; }
    if (inbin <= (uint32_t)kRowCap) break;
  }

  // ---- collect: bitmaps for the whole row, candidates of the bin into LDS
  const int hi_shift = lvl_shift(lvl - 1);
  const uint32_t hp = prefix >> hi_shift;
  if (t == 0) misc[2] = 0;
  __syncthreads();
  const int lane = lane_id();
  const int span = ((n + kRowThreads - 1) / kRowThreads) * kRowThreads;
  for (int base = 0; base < span; base += kRowThreads) {
    const int j = base + t;
    const bool valid = j < n;
    const uint32_t key = valid ? score_key(src[j]) : 0u;
    const uint32_t hk = key >> hi_shift;
    const bool def = valid && hk > hp;
    const bool eq = valid && hk == hp;
    const uint64_t mdef = __ballot(def);
    const uint64_t meq = __ballot(eq);
    const int w0 = (j - lane) >> 5;
    if (lane == 0) { sel[w0] = (uint32_t)mdef; tie[w0] = exact ? (uint32_t)meq : 0u; }
    if (lane == 32) { sel[w0 + 1] = (uint32_t)(mdef >> 32); tie[w0 + 1] = exact ? (uint32_t)(meq >> 32) : 0u; }
    if (!exact && meq) {
      uint32_t base_slot = 0;
      if (lane == 0) base_slot = atomicAdd(&misc[2], (uint32_t)__popcll(meq));
      base_slot = __shfl(base_slot, 0, kWave);
      if (eq) {
        const uint32_t slot = base_slot + wave_prefix_count(meq);
        ckey[slot] = key;
        cidx[slot] = (uint32_t)j;
      }
    }
  }
  __syncthreads();

  if (!exact) {
    // ---- finish the descent on the candidates held in LDS
    const uint32_t nc = misc[2];
    while (lvl < 3) {
      for (int i = t; i < kBins; i += kRowThreads) hist[i] = 0;
      __syncthreads();
      for (uint32_t i = t; i < nc; i += kRowThreads) {
        const uint32_t key = ckey[i];
        if (lvl_match(key, prefix, lvl)) atomicAdd(&hist[lvl_digit(key, lvl)], 1u);
      }
      __syncthreads();
      select_bin<kRowThreads>(hist, need, scratch, misc);
      need -= misc[1];
      prefix |= misc[0] << lvl_shift(lvl);
      ++lvl;
      __syncthreads();
    }
    for (uint32_t i = t; i < nc; i += kRowThreads) {
      const uint32_t key = ckey[i], j = cidx[i];
      if (key > prefix) atomicOr(&sel[j >> 5], 1u << (j & 31));
      else if (key == prefix) atomicOr(&tie[j >> 5], 1u << (j & 31));
    }
    __syncthreads();
  }

  // ---- ordered emission
  const int nw = (n + 31) / 32;
  emit_bitmaps<kRowThreads>(
      nw, need, [&](int w) { return sel[w]; }, [&](int w) { return tie[w]; }, out, (uint32_t)k,
      scratch);
}

// ====================================================================== multi plan
struct MultiWs {
  uint32_t* ghist;   // [rows][2048]
  uint32_t* ctr;     // [rows][4]: arrivals K1, arrivals K2, candidates, spare
  uint32_t* state;   // [rows][4]: prefix, need, inbin, mode
  uint32_t* ckey;    // [rows][cap]
  uint32_t* cidx;    // [rows][cap]
  uint32_t* sel;     // [rows][words]
  uint32_t* tie;     // [rows][words]
};

enum { kModeAll = 0, kModeCollect = 1, kModeRefine = 2 };

__host__ __device__ inline MultiWs carve(void* ws, int rows, int words) {
  MultiWs m;
  uint32_t* p = (uint32_t*)ws;
  m.ghist = p; p += (size_t)rows * kBins;
  m.ctr = p; p += (size_t)rows * 4;
  m.state = p; p += (size_t)rows * 4;
  m.ckey = p; p += (size_t)rows * kMultiCap;
  m.cidx = p; p += (size_t)rows * kMultiCap;
  m.sel = p; p += (size_t)rows * words;
  m.tie = p; p += (size_t)rows * words;
  return m;
}
__host__ inline size_t multi_ws_bytes(int rows, int words) {
  return (size_t)rows * (kBins + 8 + 2 * (size_t)kMultiCap + 2 * (size_t)words) * 4;
}

// K0: clear histograms and counters (plain kernel, safe inside captured graphs).
__global__ __launch_bounds__(kChunkThreads) void topk_clear_kernel(MultiWs m) {
  const int row = blockIdx.x;
  for (int i = threadIdx.x; i < kBins; i += kChunkThreads) m.ghist[(size_t)row * kBins + i] = 0;
  if (threadIdx.x < 4) m.ctr[row * 4 + threadIdx.x] = 0;
}

// Arrive at a per-row counter after publishing this workgroup's global
// writes; returns true in the last workgroup of the row (all threads).
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t expected, uint32_t* flag) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) *flag = (atomicAdd(counter, 1u) == expected - 1) ? 1u : 0u;
  __syncthreads();
  const bool last = *flag != 0;
  if (last) __threadfence();
  return last;
}

// K1: chunk histograms of the top level, merged into the row histogram.
__global__ __launch_bounds__(kChunkThreads) void topk_chunk_hist_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ kv_len, int S, int L_cap,
    int k, int chunk, MultiWs m) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t scratch[32];
  __shared__ uint32_t misc[8];
  const int row = blockIdx.y, c = blockIdx.x, t = threadIdx.x;
  const int n = row_count(kv_len, row, S, L_cap);
  for (int i = t; i < kBins; i += kChunkThreads) hist[i] = 0;
  __syncthreads();
  if (n > k) {
    const float* src = scores + (size_t)row * L_cap;
    const int j1 = min((c + 1) * chunk, n);
    for (int j = c * chunk + t; j < j1; j += kChunkThreads)
      atomicAdd(&hist[score_key(src[j]) >> 21], 1u);
  }
  __syncthreads();
  uint32_t* gh = m.ghist + (size_t)row * kBins;
  for (int i = t; i < kBins; i += kChunkThreads)
    if (hist[i]) atomicAdd(&gh[i], hist[i]);
  if (!arrive_last(&m.ctr[row * 4 + 0], gridDim.x, &misc[4])) return;

  uint32_t* st = m.state + row * 4;
  if (n <= k) {
    if (t == 0) { st[0] = 0; st[1] = 0; st[2] = 0; st[3] = kModeAll; }
    return;
  }
  for (int i = t; i < kBins; i += kChunkThreads) hist[i] = ld_coherent(&gh[i]);
  __syncthreads();
  select_bin<kChunkThreads>(hist, (uint32_t)k, scratch, misc);
  if (t == 0) {
    const uint32_t bin = misc[0];
    st[0] = bin << 21;
    st[1] = (uint32_t)k - misc[1];
    st[2] = hist[bin];
    st[3] = hist[bin] <= (uint32_t)kMultiCap ? kModeCollect : kModeRefine;
  }
}

// K2: bitmaps and candidates per chunk; the row's last arriver selects and emits.
__global__ __launch_bounds__(kChunkThreads) void topk_chunk_collect_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ kv_len, int S, int L_cap,
    int k, int chunk, int words, MultiWs m, int32_t* __restrict__ indices) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t scratch[32];
  __shared__ uint32_t misc[8];
  const int row = blockIdx.y, c = blockIdx.x, t = threadIdx.x, lane = lane_id();
  const int n = row_count(kv_len, row, S, L_cap);
  const uint32_t* st = m.state + row * 4;
  const uint32_t mode = st[3];
  uint32_t prefix = st[0];
  uint32_t need = st[1];
  const float* src = scores + (size_t)row * L_cap;
  uint32_t* sel = m.sel + (size_t)row * words;
  uint32_t* tie = m.tie + (size_t)row * words;
  uint32_t* ckey = m.ckey + (size_t)row * kMultiCap;
  uint32_t* cidx = m.cidx + (size_t)row * kMultiCap;
  uint32_t* ncand = &m.ctr[row * 4 + 2];

  if (mode != kModeAll) {
    const uint32_t hp = prefix >> 21;
    const int j_end = (c + 1) * chunk;    // chunk is a multiple of 64
    for (int j = c * chunk + t; j < j_end; j += kChunkThreads) {
      const bool valid = j < n;
      const uint32_t key = valid ? score_key(src[j]) : 0u;
      const uint32_t hk = key >> 21;
      const bool def = valid && hk > hp;
      const bool eq = valid && hk == hp;
      const uint64_t mdef = __ballot(def);
      const uint64_t meq = __ballot(eq);
      const int w0 = (j - lane) >> 5;
      if (lane == 0) { sel[w0] = (uint32_t)mdef; tie[w0] = 0u; }
      if (lane == 32) { sel[w0 + 1] = (uint32_t)(mdef >> 32); tie[w0 + 1] = 0u; }
      if (mode == kModeCollect && meq) {
        uint32_t base_slot = 0;
        if (lane == 0) base_slot = atomicAdd(ncand, (uint32_t)__popcll(meq));
        base_slot = __shfl(base_slot, 0, kWave);
        if (eq) {
          const uint32_t slot = base_slot + wave_prefix_count(meq);
          ckey[slot] = key;
          cidx[slot] = (uint32_t)j;
        }
      }
    }
  }
  if (!arrive_last(&m.ctr[row * 4 + 1], gridDim.x, &misc[4])) return;

  int32_t* out = indices + (size_t)row * k;
  if (mode == kModeAll) {
    for (int i = t; i < k; i += kChunkThreads) out[i] = i < n ? i : -1;
    return;
  }
  int lvl = 1;
  if (mode == kModeCollect) {
    const uint32_t nc = ld_coherent(ncand);
    while (lvl < 3) {
      for (int i = t; i < kBins; i += kChunkThreads) hist[i] = 0;
      __syncthreads();
      for (uint32_t i = t; i < nc; i += kChunkThreads) {
        const uint32_t key = ld_coherent(&ckey[i]);
        if (lvl_match(key, prefix, lvl)) atomicAdd(&hist[lvl_digit(key, lvl)], 1u);
      }
      __syncthreads();
      select_bin<kChunkThreads>(hist, need, scratch, misc);
      need -= misc[1];
      prefix |= misc[0] << lvl_shift(lvl);
      ++lvl;
      __syncthreads();
    }
    for (uint32_t i = t; i < nc; i += kChunkThreads) {
      const uint32_t key = ld_coherent(&ckey[i]), j = ld_coherent(&cidx[i]);
      if (key > prefix) atomicOr(&sel[j >> 5], 1u << (j & 31));
      else if (key == prefix) atomicOr(&tie[j >> 5], 1u << (j & 31));
    }
  } else {
    // Refine: the top bin is too full for the candidate list; descend over
    // the whole row, then rebuild the row's bitmaps from the exact threshold.
    while (lvl < 3) {
      for (int i = t; i < kBins; i += kChunkThreads) hist[i] = 0;
      __syncthreads();
      for (int j = t; j < n; j += kChunkThreads) {
        const uint32_t key = score_key(src[j]);
        if (lvl_match(key, prefix, lvl)) atomicAdd(&hist[lvl_digit(key, lvl)], 1u);
      }
      __syncthreads();
      select_bin<kChunkThreads>(hist, need, scratch, misc);
      need -= misc[1];
      prefix |= misc[0] << lvl_shift(lvl);
      ++lvl;
      __syncthreads();
    }
    const int span = ((n + 63) / 64) * 64;
    for (int j = t; j < span; j += kChunkThreads) {
      const bool valid = j < n;
      const uint32_t key = valid ? score_key(src[j]) : 0u;
      const uint64_t mdef = __ballot(valid && key > prefix);
      const uint64_t meq = __ballot(valid && key == prefix);
      const int w0 = (j - lane) >> 5;
      if (lane == 0) { sel[w0] = (uint32_t)mdef; tie[w0] = (uint32_t)meq; }
      if (lane == 32) { sel[w0 + 1] = (uint32_t)(mdef >> 32); tie[w0 + 1] = (uint32_t)(meq >> 32); }
    }
  }
  __threadfence();
  __syncthreads();
  const int nw = (n + 31) / 32;
  emit_bitmaps<kChunkThreads>(
      nw, need, [&](int w) { return ld_coherent(&sel[w]); },
      [&](int w) { return ld_coherent(&tie[w]); }, out, (uint32_t)k, scratch);
}

}  // namespace

TopkPlan plan_topk(int B, int S, int L_cap, int k) {
  TopkPlan p{};
  p.rows = B * S;
  p.cap = kRowCap;
  const long long rows = p.rows;
  p.multi = (rows < 128 && L_cap > 8192) || L_cap > 262144;
  if (p.multi) {
    long long want = ((long long)L_cap * rows + 1023) / 1024;
    int ch = 1024;
    while (ch < want && ch < 16384) ch *= 2;
    p.chunk = ch;
    p.chunks = (L_cap + ch - 1) / ch;
    p.words = (int)(((long long)p.chunks * ch) / 32);
    p.cap = kMultiCap;
    p.ws_bytes = multi_ws_bytes(p.rows, p.words);
  } else {
    p.words = ((L_cap + kRowThreads - 1) / kRowThreads) * kRowThreads / 32;
    p.lds_bytes = (size_t)(kBins + 32 + 8 + 2 * p.words + 2 * kRowCap) * 4;
    p.ws_bytes = 0;
  }
  return p;
}

void launch_topk(const TopkPlan& p, const float* scores, const int32_t* kv_len, int S,
                 int L_cap, int k, int32_t* indices, void* ws, hipStream_t st) {
  if (p.rows == 0) return;
  if (!p.multi) {
    // The row plan may use more than the default 64 KiB of dynamic LDS.
    static bool lds_opt_in = false;
    if (!lds_opt_in) {
      (void)hipFuncSetAttribute((const void*)topk_row_kernel,
                                hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
      lds_opt_in = true;
    }
    hipLaunchKernelGGL(topk_row_kernel, dim3(p.rows), dim3(kRowThreads), p.lds_bytes, st,
                       scores, kv_len, S, L_cap, k, p.words, indices);
    return;
  }
  MultiWs m = carve(ws, p.rows, p.words);
  hipLaunchKernelGGL(topk_clear_kernel, dim3(p.rows), dim3(kChunkThreads), 0, st, m);
  hipLaunchKernelGGL(topk_chunk_hist_kernel, dim3(p.chunks, p.rows), dim3(kChunkThreads), 0, st,
                     scores, kv_len, S, L_cap, k, p.chunk, m);
  hipLaunchKernelGGL(topk_chunk_collect_kernel, dim3(p.chunks, p.rows), dim3(kChunkThreads), 0,
                     st, scores, kv_len, S, L_cap, k, p.chunk, p.words, m, indices);
}

}  // namespace dsa
