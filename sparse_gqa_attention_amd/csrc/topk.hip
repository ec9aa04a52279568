// Per-query top-k with lowest-index tie-break (ORT PR #33802 "Optimize ...
// for SM12x and 256K context", Summary item 2: radix histograms per key
// chunk, a merge across up to 64+ chunks and a final emit of the indices).
//
// Exact for any FP32 input.  Scores map to order-preserving u32 keys
// (score_key); selection works on keys only.
//
// 1. Threshold estimate.  A sample of the row (all of it when the row is
//    short, else blocks of 256 consecutive keys spread evenly over the row:
//    2048 keys for an LDS-resident row, 8192 when streaming, 4096 in the
//    multi plan) goes through two radix levels (the top 11 + 11 key bits) to the
//    bin of the key of rank r = ceil(1.2e + 4 sqrt(e)) + 8, where e = k *
//    sample / n is the expected sample rank of the k-th largest key.  The
//    bin's lower edge T_lo is at or below that key; every key >= T_lo is a
//    candidate (about 1.2k + 4 sqrt(e) n/sample keys).
// 2. Collection.  One pass over the row lists the candidates; the resident
//    and multi plans keep the list in index order.
// 3. Exact selection on the list, in LDS: radix select of the k-th largest
//    key T (index-ordered lists: 12-bit digits of key - T_lo, two levels
//    for key spans below 2^24).  When only some of the keys equal to T fit,
//    the lowest indices win.  Exactly k entries.
// 4. Ordered emission.  An index-ordered list is compacted by one block scan
//    (a key equal to T is kept while fewer than `take` equal keys precede
//    it).  The streaming plan's unordered list sets the kept indices in an
//    LDS bitmap one index segment at a time, written in ascending order by a
//    block scan, ties cut by a wave ranking (<= 64 tied indices) or a radix
//    select on the complemented index.
// When the list holds fewer than k keys, overflows, or k itself exceeds its
// capacity, an exact fallback selects from the whole row (three radix
// passes) and emits from selection/tie bitmaps, carrying the tie count
// across segments.  Every path computes the same, exact result.
//
// Plans (host-chosen from B*S and L_cap):
//  * resident  -- few rows of <= 32768 keys (speculative decode at 32K): one
//    1024-thread workgroup per row loads the row once into LDS (128 KB of
//    keys) and does everything there.
//  * streaming -- many rows (prefill: 2048 rows of 131072 keys): one
//    1024-thread workgroup per row reading the row ~1.06 times (two
//    workgroups per CU: at most 64 VGPRs, four 16-byte loads per lane in
//    flight).
//  * multi     -- few rows longer than 32768 keys (decode at 256K): KA (one
//    workgroup per row) computes T_lo and resets the row's pool counter, KB
//    (many workgroups per row) lists each chunk's candidates in index order
//    in the chunk's own slots (or a block of the row's pool), KC (one
//    workgroup per row) gathers the chunks in order, selects and emits.
//    Kernel boundaries order the three.
#include "dsa_device.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kBins = 2048;
constexpr int kSample = 8192;          // sampled keys (rows longer than this)
constexpr int kSampleBlock = 256;      // consecutive keys per sample block
constexpr int kSegWords = 2048;        // bitmap segment: 65536 indices
constexpr int kSegBits = kSegWords * 32;
constexpr int kResKeys = 32768;        // longest row the resident plan holds
constexpr int kResCap = 4096;          // candidate list; the select's histogram follows it
constexpr int kResSample = 2048;       // sample of a resident row (already in LDS)
constexpr int kRowCap = 4096;
constexpr int kMultiCap = 8192;
static_assert(kMultiCap < 65536 && kResCap < 65536, "ordered emission packs counts in 16 bits");
static_assert(kResCap + (1 << 12) <= kResKeys, "resident select histogram fits the row area");
constexpr int kMultiSample = 4096;     // sample of the threshold kernel
constexpr int kChunkThreads = 256;
constexpr int kChunkKeysPerThread = 8;
constexpr int kStreamLoads = 4;        // 16-byte loads per lane in flight (streaming plan)
static_assert(4 * kStreamLoads <= 32, "one hit bit per key of a lane's step");

enum PlanKind { kPlanStream = 0, kPlanResident = 1, kPlanMulti = 2 };

// Radix levels: key bits [31:21], [20:10], [9:0].
__device__ __forceinline__ int lvl_shift(int lvl) { return lvl == 0 ? 21 : (lvl == 1 ? 10 : 0); }
__device__ __forceinline__ uint32_t lvl_digit(uint32_t key, int lvl) {
  return lvl == 0 ? (key >> 21) : (lvl == 1 ? ((key >> 10) & 0x7FFu) : (key & 0x3FFu));
}
__device__ __forceinline__ bool lvl_match(uint32_t key, uint32_t prefix, int lvl) {
  return lvl == 0 ? true : (((key ^ prefix) >> (lvl == 1 ? 21 : 10)) == 0u);
}

__device__ __forceinline__ int row_count(const int32_t* kv_len, int row, int S, int L_cap) {
  const int b = row / S, s = row % S;
  int n = kv_len[b] - S + s + 1;     // candidates 0..pos
  return n < 0 ? 0 : (n > L_cap ? L_cap : n);
}

// Sample rank of the threshold and the row position of sample element i,
// for a sample of `ns` keys (ns a multiple of kSampleBlock) of a row of n > ns.
__device__ __forceinline__ int sample_rank(int k, int n, int ns) {
  const float e = (float)k * (float)ns / (float)n;
  const int r = (int)ceilf(1.2f * e + 4.0f * sqrtf(e)) + 8;
  return r < ns ? r : ns;
}
template <int NS>
__device__ __forceinline__ int sample_pos(int i, int n) {
  constexpr int NB = NS / kSampleBlock;             // <= 32 blocks, n < 2^24: no overflow
  const int blk = i / kSampleBlock;
  return (int)((uint32_t)(blk * (n - kSampleBlock)) / (uint32_t)(NB - 1)) + i % kSampleBlock;
}

// Shared-memory scratch of the block-wide helpers.
struct Lds {
  uint32_t* hist;      // [kBins]
  uint32_t* scratch;   // [32]
  uint32_t* misc;      // [16 + kTieSmall]: results, counters, tie indices at +16
};
constexpr int kTieSmall = 64;     // ties resolved by one wave without a radix pass
constexpr int kMiscWords = 16 + kTieSmall;

// The bin holding the need-th largest key of a 2048-bin histogram:
// misc[0] = bin, misc[1] = keys in higher bins.  Block-wide.
template <int NT>
__device__ void select_bin(const uint32_t* hist, uint32_t need, uint32_t* scratch,
                           uint32_t* misc) {
  constexpr int BPT = kBins / NT;
  static_assert(BPT * NT == kBins, "block size must divide the bin count");
  const int t = threadIdx.x;
  if (t == 0) { misc[0] = 0; misc[1] = 0; }   // ordered before the finder by the scan's barriers
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) local += hist[kBins - 1 - (t * BPT + i)];
  uint32_t total;
  uint32_t before = block_exclusive_scan<NT>(local, scratch, &total);
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    const int bin = kBins - 1 - (t * BPT + i);
    const uint32_t h = hist[bin];
    if (before < need && need <= before + h) { misc[0] = (uint32_t)bin; misc[1] = before; }
    before += h;
  }
  __syncthreads();
}

// Radix select over the keys get(i), i in [0, count), for which get returns
// true.  With levels = 3: T = the need-th largest key exactly, take = how
// many keys equal to T belong to the top `need`, eq = how many keys equal T.
// With levels = 2 the low 10 bits of T are zero and T is a lower bound of
// the need-th largest key (conservative threshold); take/eq then count the
// keys sharing T's upper 22 bits.  Block-wide; 1 <= need <= number of keys.
template <int NT, typename Get>
__device__ void radix_select(Get get, int count, uint32_t need, const Lds& s, uint32_t& T,
                             uint32_t& take, uint32_t& eq, int levels = 3) {
  uint32_t prefix = 0;
  for (int lvl = 0; lvl < levels; ++lvl) {
    for (int i = threadIdx.x; i < kBins; i += NT) s.hist[i] = 0;
    __syncthreads();
    for (int i0 = 0; i0 < count; i0 += NT) {
      const int i = i0 + threadIdx.x;
      uint32_t key = 0;
      const bool in = i < count && get(i, key) && lvl_match(key, prefix, lvl);
      if (in) atomicAdd(&s.hist[lvl_digit(key, lvl)], 1u);
    }
    __syncthreads();
    select_bin<NT>(s.hist, need, s.scratch, s.misc);
    need -= s.misc[1];
    eq = s.hist[s.misc[0]];
    prefix |= s.misc[0] << lvl_shift(lvl);
    __syncthreads();
  }
  T = prefix;
  take = need;
}

// Exact selection over keys that all lie in [base, base + range]: radix
// digits of (key - base), 12 bits wide (kRelBins bins), the first level
// taking the top bits of `range`.  Candidate lists span a narrow key range
// above the sample threshold, so absolute top-bit digits would pile them into
// a few bins (LDS atomics on one address serialise) and need three levels;
// relative digits spread them and need two levels for ranges below 2^24.
// Returns T = the need-th largest key, take = how many keys equal to T
// belong to the top `need`.  hist: kRelBins words of LDS.  Block-wide;
// 1 <= need <= count.
constexpr int kRelBits = 12;
constexpr int kRelBins = 1 << kRelBits;

template <int NT>
__device__ void select_bin_rel(const uint32_t* hist, uint32_t need, uint32_t* scratch,
                               uint32_t* misc) {
  constexpr int BPT = kRelBins / NT;
  static_assert(BPT * NT == kRelBins, "block size must divide the bin count");
  const int t = threadIdx.x;
  if (t == 0) { misc[0] = 0; misc[1] = 0; }
  uint32_t h[BPT];
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    h[i] = hist[kRelBins - 1 - (t * BPT + i)];
    local += h[i];
  }
  uint32_t total;
  uint32_t before = block_exclusive_scan<NT>(local, scratch, &total);
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    if (before < need && need <= before + h[i]) {
      misc[0] = (uint32_t)(kRelBins - 1 - (t * BPT + i));
      misc[1] = before;
    }
    before += h[i];
  }
  __syncthreads();
}

template <int NT, typename KeyOf>
__device__ void radix_select_rel(KeyOf key_of, int count, uint32_t need, uint32_t base,
                                 uint32_t range, uint32_t* hist, uint32_t* scratch,
                                 uint32_t* misc, uint32_t& T, uint32_t& take) {
  const int top = range ? 32 - __clz(range) : 0;          // bit length of the range
  int hi = top > kRelBits ? top : kRelBits;               // bits [lo, hi) are this level's
  uint32_t prefix = 0;                                    // digits fixed so far (bits >= hi)
  while (true) {
    const int lo = hi > kRelBits ? hi - kRelBits : 0;
    for (int i = threadIdx.x; i < kRelBins; i += NT) hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < count; i += NT) {
      const uint32_t d = key_of(i) - base;
      if (hi >= 32 || (d >> hi) == (prefix >> hi))
        atomicAdd(&hist[(d >> lo) & (kRelBins - 1)], 1u);
    }
    __syncthreads();
    select_bin_rel<NT>(hist, need, scratch, misc);
    need -= misc[1];
    prefix |= misc[0] << lo;
    __syncthreads();
    if (lo == 0) break;
    hi = lo;
  }
  T = base + prefix;
  take = need;
}

// Ordered emission from a list sorted by index: entry i is kept iff its key
// is above T, or equals T and fewer than `take` keys equal to T come before
// it; its output slot is the number of kept entries before it.  One block
// scan of the two counts packed in 16-bit halves (m < 2^16).
template <int NT>
__device__ void emit_ordered(const uint32_t* lkey, const uint32_t* lidx, int m, uint32_t T,
                             uint32_t take, int32_t* out, uint32_t* scratch) {
  // m <= kMultiCap < 2^16 (multi plan), m <= kResCap (resident plan)
  const int per = (m + NT - 1) / NT;
  const int i0 = min(threadIdx.x * per, m), i1 = min(i0 + per, m);
  uint32_t gt = 0, eq = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = lkey[i];
    gt += key > T ? 1u : 0u;
    eq += key == T ? 1u : 0u;
  }
  uint32_t total;
  const uint32_t before = block_exclusive_scan<NT>(gt | (eq << 16), scratch, &total);
  uint32_t g = before & 0xFFFFu, e = before >> 16;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = lkey[i];
    if (key > T) {
      out[g + (e < take ? e : take)] = (int32_t)lidx[i];
      ++g;
    } else if (key == T) {
      if (e < take) out[g + e] = (int32_t)lidx[i];
      ++e;
    }
  }
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

__device__ __forceinline__ uint32_t kept_ties(uint32_t tw, uint32_t running, uint32_t eq_take) {
  const uint32_t c = __popc(tw);
  if (running >= eq_take) return 0u;
  if (running + c <= eq_take) return tw;
  return keep_lowest_bits(tw, eq_take - running);
}

// Ordered emission of LDS bitmap words [0, nw) covering indices
// word_base*32 + [0, 32*nw).  With a tie bitmap, the first eq_take tie bits
// of the whole row (tie_run counts earlier ones) join the selection.
// tie_run/out_run are block-uniform and advance by this segment's totals.
// Never writes at or past k.  Block-wide.
template <int NT>
__device__ void emit_words(const uint32_t* sel, const uint32_t* tie, int nw, int word_base,
                           uint32_t eq_take, uint32_t& tie_run, uint32_t& out_run, int32_t* out,
                           uint32_t k, uint32_t* scratch) {
  const int t = threadIdx.x;
  const int wpt = (nw + NT - 1) / NT;
  const int w0 = min(t * wpt, nw), w1 = min(w0 + wpt, nw);
  uint32_t tcount = 0;
  if (tie)
    for (int w = w0; w < w1; ++w) tcount += __popc(tie[w]);
  uint32_t tie_total;
  const uint32_t tie_start = tie_run + block_exclusive_scan<NT>(tcount, scratch, &tie_total);
  uint32_t running = tie_start, fcount = 0;
  for (int w = w0; w < w1; ++w) {
    const uint32_t tw = tie ? tie[w] : 0u;
    fcount += __popc(sel[w] | kept_ties(tw, running, eq_take));
    running += __popc(tw);
  }
  uint32_t out_total;
  uint32_t pos = out_run + block_exclusive_scan<NT>(fcount, scratch + 16, &out_total);
  running = tie_start;
  for (int w = w0; w < w1; ++w) {
    const uint32_t tw = tie ? tie[w] : 0u;
    uint32_t f = sel[w] | kept_ties(tw, running, eq_take);
    running += __popc(tw);
    while (f) {
      const int bit = __ffs(f) - 1;
      if (pos < k) out[pos] = (word_base + w) * 32 + bit;
      ++pos;
      f &= f - 1;
    }
  }
  tie_run += tie_total;
  out_run += out_total;
}

template <int NT>
__device__ __forceinline__ void write_all(int32_t* out, int n, int k) {
  for (int i = threadIdx.x; i < k; i += NT) out[i] = i < n ? i : -1;
}

// Reserve `cnt` consecutive list slots per lane with one LDS atomic per
// wave; returns this lane's first slot.
__device__ __forceinline__ uint32_t wave_reserve(uint32_t cnt, uint32_t* counter) {
  const uint32_t inc = wave_inclusive_scan(cnt);
  const uint32_t total = (uint32_t)__shfl((int)inc, kWave - 1, kWave);
  uint32_t base = 0;
  if (lane_id() == kWave - 1 && total) base = atomicAdd(counter, total);
  base = (uint32_t)__shfl((int)base, kWave - 1, kWave);
  return base + inc - cnt;
}

// ---------------------------------------------------------------- steps 3-4
// Exact selection from m candidates (key_of(i), idx_of(i)) that include every
// key >= the k-th largest of the row; `bm` (kSegWords words of LDS, free for
// this call) holds one bitmap segment of the ordered emission.
template <int NT, typename KeyOf, typename IdxOf>
__device__ void select_from_list(KeyOf key_of, IdxOf idx_of, int m, int n, int k, uint32_t* bm,
                                 int32_t* out, const Lds& s) {
  uint32_t T, take, eq;
  radix_select<NT>([&](int i, uint32_t& key) { key = key_of(i); return true; }, m, (uint32_t)k,
                   s, T, take, eq);
  // Among the eq keys equal to T keep the `take` lowest indices.
  uint32_t cut = 0xFFFFFFFFu;
  if (take < eq) {
    if (eq <= (uint32_t)kTieSmall) {
      uint32_t* ties = s.misc + 16;
      if (threadIdx.x == 0) s.misc[9] = 0;
      __syncthreads();
      for (int i = threadIdx.x; i < m; i += NT)
        if (key_of(i) == T) ties[atomicAdd(&s.misc[9], 1u)] = idx_of(i);
      __syncthreads();
      if (threadIdx.x < kWave) {
        const int l = threadIdx.x;
        const uint32_t mine = l < (int)eq ? ties[l] : 0xFFFFFFFFu;
        uint32_t rank = 0;
        for (uint32_t j = 0; j < eq; ++j) rank += ties[j] < mine ? 1u : 0u;
        if (l < (int)eq && rank == take - 1) s.misc[10] = mine;
      }
      __syncthreads();
      cut = s.misc[10];
    } else {
      // the take-th largest complemented index is the cut
      uint32_t C, one, eq2;
      radix_select<NT>([&](int i, uint32_t& key) { key = ~idx_of(i); return key_of(i) == T; }, m,
                       take, s, C, one, eq2);
      cut = ~C;
    }
  }
  uint32_t tie_run = 0, out_run = 0;
  for (int base = 0; base < n; base += kSegBits) {
    const int nw = min(kSegWords, (n - base + 31) / 32);
    for (int i = threadIdx.x; i < nw; i += NT) bm[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < m; i += NT) {
      const uint32_t key = key_of(i), j = idx_of(i);
      const bool keep = key > T || (key == T && j <= cut);
      if (keep && j >= (uint32_t)base && j < (uint32_t)(base + kSegBits)) {
        const uint32_t r = j - base;
        atomicOr(&bm[r >> 5], 1u << (r & 31));
      }
    }
    __syncthreads();
    emit_words<NT>(bm, nullptr, nw, base / 32, 0, tie_run, out_run, out, (uint32_t)k, s.scratch);
    __syncthreads();
  }
}

// ---------------------------------------------------------------- fallback
// Exact top-k of a whole row of n keys key_at(j): three radix passes for T,
// then one pass per index segment building selection/tie bitmaps (sel, tie:
// kSegWords words of LDS each) with the tie count carried across segments.
template <int NT, typename KeyAt>
__device__ void select_exact_row(KeyAt key_at, int n, int k, uint32_t* sel, uint32_t* tie,
                                 int32_t* out, const Lds& s) {
  uint32_t T, take, eq;
  radix_select<NT>([&](int i, uint32_t& key) { key = key_at(i); return true; }, n, (uint32_t)k,
                   s, T, take, eq);
  const int lane = lane_id();
  uint32_t tie_run = 0, out_run = 0;
  for (int base = 0; base < n; base += kSegBits) {
    const int seg_n = min(kSegBits, n - base);
    const int nw = (seg_n + 31) / 32;
    const int span = ((seg_n + 63) / 64) * 64;
    for (int r = threadIdx.x; r < span; r += NT) {
      const bool valid = r < seg_n;
      const uint32_t key = valid ? key_at(base + r) : 0u;
      const uint64_t mg = __ballot(valid && key > T);
      const uint64_t me = __ballot(valid && key == T);
      const int w0 = (r - lane) >> 5;
      if (lane == 0) { sel[w0] = (uint32_t)mg; tie[w0] = (uint32_t)me; }
      if (lane == 32) { sel[w0 + 1] = (uint32_t)(mg >> 32); tie[w0 + 1] = (uint32_t)(me >> 32); }
    }
    __syncthreads();
    emit_words<NT>(sel, tie, nw, base / 32, take, tie_run, out_run, out, (uint32_t)k, s.scratch);
    __syncthreads();
  }
}

// Variants of radix_select (two levels) and radix_select_rel for callers
// that zeroed one histogram per level beforehand and give each level its
// own result words: three barriers per level instead of five.
//
// Lower bound of the need-th largest key: the 22-bit bin edge (low 10 bits
// zero) after levels on bits [31:21] and [20:10].  h0, h1: kBins zeroed
// words each; misc[0..3] receive the levels' results.
template <int NT, typename Get>
__device__ void radix_lower_bound_pre(Get get, int count, uint32_t need, uint32_t* h0,
                                      uint32_t* h1, uint32_t* scratch, uint32_t* misc,
                                      uint32_t& T_lo) {
  for (int i = threadIdx.x; i < count; i += NT) atomicAdd(&h0[get(i) >> 21], 1u);
  __syncthreads();
  select_bin<NT>(h0, need, scratch, misc);
  const uint32_t b0 = misc[0];
  need -= misc[1];
  for (int i = threadIdx.x; i < count; i += NT) {
    const uint32_t key = get(i);
    if ((key >> 21) == b0) atomicAdd(&h1[(key >> 10) & 0x7FFu], 1u);
  }
  __syncthreads();
  select_bin<NT>(h1, need, scratch, misc + 2);
  T_lo = (b0 << 21) | (misc[2] << 10);
}

// radix_select_rel over up to three zeroed histograms (hists + lvl *
// kRelBins); misc[2 lvl], misc[2 lvl + 1] receive level lvl's results.
template <int NT, typename KeyOf>
__device__ void radix_select_rel_pre(KeyOf key_of, int count, uint32_t need, uint32_t base,
                                     uint32_t range, uint32_t* hists, uint32_t* scratch,
                                     uint32_t* misc, uint32_t& T, uint32_t& take) {
  const int top = range ? 32 - __clz(range) : 0;
  int hi = top > kRelBits ? top : kRelBits;
  uint32_t prefix = 0;
  for (int lvl = 0;; ++lvl) {                             // at most 3 levels (hi <= 32)
    const int lo = hi > kRelBits ? hi - kRelBits : 0;
    uint32_t* hist = hists + lvl * kRelBins;
    for (int i = threadIdx.x; i < count; i += NT) {
      const uint32_t d = key_of(i) - base;
      if (hi >= 32 || (d >> hi) == (prefix >> hi))
        atomicAdd(&hist[(d >> lo) & (kRelBins - 1)], 1u);
    }
    __syncthreads();
    select_bin_rel<NT>(hist, need, scratch, misc + 2 * lvl);
    need -= misc[2 * lvl + 1];
    prefix |= misc[2 * lvl] << lo;
    if (lo == 0) break;
    hi = lo;
  }
  T = base + prefix;
  take = need;
}

// ====================================================================== resident plan
// Dynamic LDS: row scores [kResKeys] (later the candidates' keys and the
// select's histogram) | hist | scratch | misc | list indices [kResCap].
// The row stays in LDS as FP32: hits are tested on floats and only the
// sample and the candidates become keys, which keeps the per-key work of
// the one-workgroup row small.
constexpr int kResThreads = 1024;
constexpr size_t kResLds = (size_t)(kResKeys + kBins + 32 + kMiscWords + kResCap) * 4;

template <int NT>
__global__ __launch_bounds__(NT) void topk_resident_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ kv_len, int S, int L_cap,
    int k, int vec4, int32_t* __restrict__ indices) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  float* rowf = reinterpret_cast<float*>(lds);
  uint32_t* rowk = lds;
  Lds s{lds + kResKeys, lds + kResKeys + kBins, lds + kResKeys + kBins + 32};
  uint32_t* lidx = s.misc + kMiscWords;
  const int row = blockIdx.x, t = threadIdx.x;
  const float* src = scores + (size_t)row * L_cap;
  int32_t* out = indices + (size_t)row * k;

  // ---- the whole row into LDS, every load in flight at once.  With
  // 16-byte rows the loads are direct global -> LDS copies that cover the
  // L_cap-long row and go out before the row's length is known (no wait for
  // kv_len).
  if (vec4) {
    // direct global -> LDS copies: a wave's 64 lanes fill 1 KB of the row
    // at a time (lane l's 16 bytes at the wave's base + 16 l)
    constexpr int U = kResKeys / 4 / NT;
    const int L4 = L_cap / 4;                   // L_cap % 4 == 0
    const float4* src4 = reinterpret_cast<const float4*>(src);
    float4* row4 = reinterpret_cast<float4*>(rowf);
    const int wbase = t - lane_id();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i4 = u * NT + t;
      if (i4 < L4)
        __builtin_amdgcn_global_load_lds((const void*)(src4 + i4),
                                         (__attribute__((address_space(3))) void*)(row4 + u * NT + wbase),
                                         16, 0, 0);
    }
    const int n = row_count(kv_len, row, S, L_cap);
    if (n <= k) {
      wait_vmem();                              // no copy may land after the workgroup ends
      write_all<NT>(out, n, k);
      return;
    }
  } else {
    const int n = row_count(kv_len, row, S, L_cap);
    if (n <= k) { write_all<NT>(out, n, k); return; }
    constexpr int U = 8;
    for (int b0 = 0; b0 < n; b0 += U * NT) {
      float v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = b0 + u * NT + t;
        v[u] = j < n ? src[j] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = b0 + u * NT + t;
        if (j < n) rowf[j] = v[u];
      }
    }
  }
  const int n = row_count(kv_len, row, S, L_cap);
  // The sample threshold's two histograms: hist, and the list area, which
  // is free until the candidates are listed.
  uint32_t* h1 = lidx;
  for (int i = t; i < kBins; i += NT) { s.hist[i] = 0; h1[i] = 0; }
  // Every lane reads keys that other waves copied: each wave waits for its
  // own copies (the compiler would only wait before this wave's LDS reads),
  // then the barrier.
  wait_vmem();
  __syncthreads();

  if (k <= kResCap) {
    // ---- threshold from the sample (the row itself when short)
    uint32_t T_lo;
    if (n <= kResSample)
      radix_lower_bound_pre<NT>([&](int i) { return score_key(rowf[i]); }, n, (uint32_t)k,
                                s.hist, h1, s.scratch, s.misc, T_lo);
    else
      radix_lower_bound_pre<NT>(
          [&](int i) { return score_key(rowf[sample_pos<kResSample>(i, n)]); }, kResSample,
          (uint32_t)sample_rank(k, n, kResSample), s.hist, h1, s.scratch, s.misc, T_lo);
    // ---- candidates, in index order.  Lane t owns keys [32 t, 32 t + 32)
    // and tests them on floats: x >= f_lo <=> score_key(x) >= T_lo
    // (score_key is order-preserving and gives -0.0 the key of +0.0;
    // denormals are preserved in comparisons).  A threshold inside the -inf
    // bin has a NaN pattern and no hits; the exact fallback then runs.
    // Eight 16-byte LDS reads, rotated by t so that any 8 consecutive lanes
    // read distinct bank groups: read i covers the lane's chunk
    // g = (i + t) % 8.  Hit bits are shifted in from the last read to the
    // first (bit 4 i + e: element e of read i), and one rotation by
    // 4 (t % 8) moves them to bit 4 g + e, the key's offset in the lane's
    // range.  One block scan of the hit counts ranks every candidate.
    const float f_lo = __uint_as_float((T_lo & 0x80000000u) ? (T_lo & 0x7FFFFFFFu) : ~T_lo);
    constexpr int KPL = kResKeys / NT;          // keys per lane
    static_assert(KPL == 32, "hit mask holds one bit per key of a lane");
    if (t == 0) s.misc[11] = 0;                 // ordered by the scan's barrier
    const float4* row4 = reinterpret_cast<const float4*>(rowf);
    uint32_t mask = 0;
#pragma unroll
    for (int i = KPL / 4 - 1; i >= 0; --i) {
      const float4 q = row4[(KPL / 4) * t + ((i + t) & (KPL / 4 - 1))];
      mask = (mask << 1) | (q.w >= f_lo ? 1u : 0u);
      mask = (mask << 1) | (q.z >= f_lo ? 1u : 0u);
      mask = (mask << 1) | (q.y >= f_lo ? 1u : 0u);
      mask = (mask << 1) | (q.x >= f_lo ? 1u : 0u);
    }
    const uint32_t rot = 4u * (uint32_t)(t & (KPL / 4 - 1));
    mask = (mask << rot) | (mask >> ((32u - rot) & 31u));
    const int nv = n - KPL * t;                 // keys of this lane inside the row
    mask &= nv >= KPL ? 0xFFFFFFFFu : (nv <= 0 ? 0u : (1u << nv) - 1u);
    uint32_t m_total;
    uint32_t slot = block_exclusive_scan<NT>((uint32_t)__popc(mask), s.scratch, &m_total);
    const int m = (int)m_total;
    if (m >= k && m <= kResCap) {               // block-uniform; else the list is not used
      for (uint32_t mm = mask; mm; mm &= mm - 1) lidx[slot++] = (uint32_t)(KPL * t + __ffs(mm) - 1);
    }
    __syncthreads();
    if (m >= k && m <= kResCap) {
      // The row is no longer needed beyond the candidates: their keys go to
      // a compact array at the front of the row area, the select's
      // histogram right after it.  The largest key - T_lo sizes the
      // select's digits.
      constexpr int MU = kResCap / NT;
      uint32_t kk[MU];
      uint32_t span = 0;
#pragma unroll
      for (int u = 0; u < MU; ++u) {
        const int i = u * NT + t;
        kk[u] = i < m ? score_key(rowf[lidx[i]]) : 0u;
        if (i < m) span = max(span, kk[u] - T_lo);
      }
      span = wave_inclusive_max_u32(span);
      if (lane_id() == kWave - 1) atomicMax(&s.misc[11], span);
      __syncthreads();
      // keys to the front of the row area, the select's three level
      // histograms zeroed right after them
      uint32_t* hists = rowk + kResCap;
#pragma unroll
      for (int u = 0; u < MU; ++u) {
        const int i = u * NT + t;
        if (i < m) rowk[i] = kk[u];
      }
      static_assert(kResCap + 3 * kRelBins <= kResKeys, "select histograms fit the row area");
      uint4* h4 = reinterpret_cast<uint4*>(hists);
      for (int i = t; i < 3 * kRelBins / 4; i += NT) h4[i] = make_uint4(0u, 0u, 0u, 0u);
      __syncthreads();
      uint32_t T, take;
      radix_select_rel_pre<NT>([&](int i) { return rowk[i]; }, m, (uint32_t)k, T_lo, s.misc[11],
                               hists, s.scratch, s.misc + 4, T, take);
      emit_ordered<NT>(rowk, lidx, m, T, take, out, s.scratch);
      return;
    }
  }
  // ---- exact fallback over the LDS row; sel/tie bitmaps in the hist area
  // (n <= 32768 keys: 1024 words each).
  uint32_t T, take, eq;
  radix_select<NT>([&](int i, uint32_t& key) { key = score_key(rowf[i]); return true; }, n,
                   (uint32_t)k, s, T, take, eq);
  uint32_t* sel = s.hist;
  uint32_t* tie = s.hist + kBins / 2;
  const int lane = lane_id();
  const int span = ((n + 63) / 64) * 64;
  for (int r = t; r < span; r += NT) {
    const bool valid = r < n;
    const uint32_t key = valid ? score_key(rowf[r]) : 0u;
    const uint64_t mg = __ballot(valid && key > T);
    const uint64_t me = __ballot(valid && key == T);
    const int w0 = (r - lane) >> 5;
    if (lane == 0) { sel[w0] = (uint32_t)mg; tie[w0] = (uint32_t)me; }
    if (lane == 32) { sel[w0 + 1] = (uint32_t)(mg >> 32); tie[w0 + 1] = (uint32_t)(me >> 32); }
  }
  __syncthreads();
  uint32_t tie_run = 0, out_run = 0;
  emit_words<NT>(sel, tie, (n + 31) / 32, 0, take, tie_run, out_run, out, (uint32_t)k, s.scratch);
}

// ====================================================================== streaming plan
// Dynamic LDS: hist | scratch | misc | region A (sample, then the list
// keys+indices, or the fallback's sel/tie segments) | bitmap segment.
template <int NT, int CAP>
struct StreamCfg {
  static constexpr int kRegionA = kSample > 2 * CAP ? kSample : 2 * CAP;
  static constexpr size_t kLds = (size_t)(kBins + 32 + kMiscWords + kRegionA + kSegWords) * 4;
  static_assert(kRegionA >= 2 * kSegWords, "fallback segments must fit region A");
};

// VEC4: rows start 16-byte aligned (L_cap % 4 == 0), read with 16-byte loads.
template <int NT, int CAP, bool VEC4>
__global__ __launch_bounds__(NT) void topk_stream_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ kv_len, int S, int L_cap,
    int k, int32_t* __restrict__ indices) {
  using Cfg = StreamCfg<NT, CAP>;
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  Lds s{lds, lds + kBins, lds + kBins + 32};
  uint32_t* regionA = lds + kBins + 32 + kMiscWords;
  uint32_t* bm = regionA + Cfg::kRegionA;
  const int row = blockIdx.x, t = threadIdx.x;
  const int n = row_count(kv_len, row, S, L_cap);
  int32_t* out = indices + (size_t)row * k;
  if (n <= k) { write_all<NT>(out, n, k); return; }
  const float* src = scores + (size_t)row * L_cap;

  if (k <= CAP) {
    // ---- sample into LDS (every load in flight first), threshold
    uint32_t* sample = regionA;
    const int cnt = n <= kSample ? n : kSample;
    constexpr int U = kSample / NT;
    constexpr int V = kStreamLoads;
    // The row's first stream step goes out with the sample, so that every
    // workgroup's HBM traffic continues while it computes the threshold.
    // All these loads are unconditional (indices clamped into the row), so
    // the sample's wait leaves the stream loads in flight.
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = u * NT + t;
      v[u] = src[i < cnt ? (n <= kSample ? i : sample_pos<kSample>(i, n)) : 0];
    }
    const float4* src4 = reinterpret_cast<const float4*>(src);
    const int n4 = VEC4 ? n / 4 : 0;
    float4 first[V];
    if (VEC4) {
#pragma unroll
      for (int u = 0; u < V; ++u) {
        // beyond the row: index 0 (L_cap >= 4); the stream masks those lanes
        const int i4 = u * NT + t;
        const f32x4 r = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(src4 + (i4 < n4 ? i4 : 0)));
        first[u] = make_float4(r[0], r[1], r[2], r[3]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) sample[u * NT + t] = score_key(v[u]);   // read below cnt only
    for (int i = t; i < kBins; i += NT) { s.hist[i] = 0u; bm[i] = 0u; }   // bm: free until emission
    __syncthreads();
    uint32_t T_lo;
    radix_lower_bound_pre<NT>([&](int i) { return sample[i]; }, cnt,
                              (uint32_t)(n <= kSample ? k : sample_rank(k, n, kSample)), s.hist,
                              bm, s.scratch, s.misc, T_lo);
    // ---- one pass over the row: 16-byte loads, kStreamLoads per lane in flight
    uint32_t* lkey = regionA;
    uint32_t* lidx = regionA + CAP;
    if (t == 0) s.misc[8] = 0;
    __syncthreads();
    // 16 keys per lane per step (4 x 16-byte loads in flight); lanes count
    // their hits and one LDS reservation per wave places them.
    auto place = [&](const uint32_t* kk, const int* jj, int nk) {
      uint32_t hits = 0;
      for (int e = 0; e < nk; ++e) hits += (jj[e] >= 0 && kk[e] >= T_lo) ? 1u : 0u;
      uint32_t slot = wave_reserve(hits, &s.misc[8]);
      for (int e = 0; e < nk; ++e)
        if (jj[e] >= 0 && kk[e] >= T_lo) {
          if (slot < (uint32_t)CAP) { lkey[slot] = kk[e]; lidx[slot] = (uint32_t)jj[e]; }
          ++slot;
        }
    };
    int done = 0;
    if (VEC4) {
      // Hits are tested on floats: x >= f_lo <=> score_key(x) >= T_lo
      // (score_key is order-preserving and gives -0.0 the key of +0.0;
      // denormals are preserved in comparisons).  Only hits become keys.
      const float f_lo = __uint_as_float((T_lo & 0x80000000u) ? (T_lo & 0x7FFFFFFFu) : ~T_lo);
      for (int b4 = 0; b4 < n4; b4 += V * NT) {
        float x[4 * V];
        uint32_t hm = 0;
#pragma unroll
        for (int u = 0; u < V; ++u) {
          const int i4 = b4 + u * NT + t;
          float4 q = first[u];                  // step 0: loaded with the sample
          if (b4 > 0) {
            q = make_float4(0.f, 0.f, 0.f, 0.f);
            if (i4 < n4) {                      // streamed once: non-temporal
              const f32x4 r = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src4 + i4));
              q = make_float4(r[0], r[1], r[2], r[3]);
            }
          }
          x[4 * u + 0] = q.x; x[4 * u + 1] = q.y; x[4 * u + 2] = q.z; x[4 * u + 3] = q.w;
        }
#pragma unroll
        for (int u = 0; u < V; ++u) {
          const bool ok = b4 + u * NT + t < n4;
#pragma unroll
          for (int e = 0; e < 4; ++e) hm |= (uint32_t)(ok && x[4 * u + e] >= f_lo) << (4 * u + e);
        }
        if (__ballot(hm != 0u) == 0) continue;            // wave-uniform
        uint32_t slot = wave_reserve((uint32_t)__popc(hm), &s.misc[8]);
        if (hm) {
#pragma unroll
          for (int e = 0; e < 4 * V; ++e)
            if ((hm >> e) & 1u) {
              if (slot < (uint32_t)CAP) {
                lkey[slot] = score_key(x[e]);
                lidx[slot] = (uint32_t)(4 * (b4 + (e >> 2) * NT + t) + (e & 3));
              }
              ++slot;
            }
        }
      }
      done = 4 * n4;
    }
    for (int b0 = done; b0 < n; b0 += 4 * NT) {
      uint32_t kk[4];
      int jj[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = b0 + u * NT + t;
        kk[u] = j < n ? score_key(src[j]) : 0u;
        jj[u] = j < n ? j : -1;
      }
      place(kk, jj, 4);
    }
    __syncthreads();
    const int m = (int)s.misc[8];
    __syncthreads();
    if (m >= k && m <= CAP) {
      select_from_list<NT>([&](int i) { return lkey[i]; }, [&](int i) { return lidx[i]; }, m, n,
                           k, bm, out, s);
      return;
    }
  }
  select_exact_row<NT>([&](int j) { return score_key(src[j]); }, n, k, regionA,
                       regionA + kSegWords, out, s);
}

// ====================================================================== multi plan
enum { kModeAll = 0, kModeList = 1, kModeExact = 2 };

// Candidates of chunk c of a row are kept in index order: in the chunk's
// own slots when there are at most kSlotCap of them, else in a block of the
// row's pool reserved with one atomic.  Meta[c] = (count, pool offset or
// kNoPool).  A pool that would overflow flags the row for the exact path.
constexpr int kSlotCap = 64;
constexpr uint32_t kNoPool = 0xFFFFFFFFu;
// Chunks of 256..2048 keys: at most 2^24 / 2048 per row (a chunk below 2048
// keys only when the row has at most 1024 of them).
constexpr int kMaxChunks = 8192;
constexpr int kSpecSlots = 16384;      // slots per row the finish kernel loads up front

struct MultiWs {
  uint32_t* state;   // [rows][4]: T_lo, mode, pool count, pool overflow flag
  uint2* meta;       // [rows][chunks]: (candidates, pool offset | kNoPool)
  uint2* slots;      // [rows][chunks][kSlotCap]: (key, index)
  uint2* pool;       // [rows][kMultiCap]: (key, index)
};

__host__ __device__ inline MultiWs carve(void* ws, int rows, int chunks) {
  MultiWs m;
  m.state = (uint32_t*)ws;
  m.meta = (uint2*)(m.state + (size_t)rows * 4);
  m.slots = m.meta + (size_t)rows * chunks;
  m.pool = m.slots + (size_t)rows * chunks * kSlotCap;
  return m;
}
__host__ inline size_t multi_ws_bytes(int rows, int chunks) {
  return (size_t)rows * 4 * 4 +
         (size_t)rows * ((size_t)chunks * (1 + kSlotCap) + kMultiCap) * sizeof(uint2);
}

constexpr int kStateThreads = 1024;
constexpr int kFinishThreads = 1024;

// KA: threshold estimate and list reset, one workgroup per row.
__global__ __launch_bounds__(kStateThreads) void topk_threshold_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ kv_len, int S, int L_cap,
    int k, MultiWs m) {
  constexpr int NT = kStateThreads;
  __shared__ uint32_t h0[kBins], h1[kBins];
  __shared__ uint32_t scratch[32];
  __shared__ uint32_t misc[4];
  __shared__ uint32_t sample[kMultiSample];
  const int row = blockIdx.x, t = threadIdx.x;
  const int n = row_count(kv_len, row, S, L_cap);
  uint32_t* st = m.state + row * 4;
  uint32_t mode = kModeAll, T_lo = 0;
  if (n > k) {
    if (k <= kMultiCap) {
      const float* src = scores + (size_t)row * L_cap;
      const int cnt = n <= kMultiSample ? n : kMultiSample;
      constexpr int U = kMultiSample / NT;
      float v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = u * NT + t;
        v[u] = i < cnt ? src[n <= kMultiSample ? i : sample_pos<kMultiSample>(i, n)] : 0.0f;
      }
      for (int i = t; i < kBins; i += NT) { h0[i] = 0u; h1[i] = 0u; }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = u * NT + t;
        if (i < cnt) sample[i] = score_key(v[u]);
      }
      __syncthreads();
      radix_lower_bound_pre<NT>([&](int i) { return sample[i]; }, cnt,
                                (uint32_t)(n <= kMultiSample ? k : sample_rank(k, n, kMultiSample)),
                                h0, h1, scratch, misc, T_lo);
      mode = kModeList;
    } else {
      mode = kModeExact;
    }
  }
  if (t == 0) { st[0] = T_lo; st[1] = mode; st[2] = 0; st[3] = 0; }
}

// KB: candidates of one chunk, in index order.  Lane t owns the U
// consecutive keys j0 + U t + [0, U), so a block scan of the per-lane counts
// gives every candidate its rank in the chunk.
template <int U, bool VEC>
__global__ __launch_bounds__(kChunkThreads) void topk_collect_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ kv_len, int S, int L_cap,
    int chunk, int chunks, MultiWs m) {
  __shared__ uint32_t scratch[32];
  __shared__ uint32_t pool_base;
  const int row = blockIdx.y, c = blockIdx.x, t = threadIdx.x;
  uint32_t* st = m.state + row * 4;
  if (st[1] != kModeList) return;
  const uint32_t T_lo = st[0];
  const int n = row_count(kv_len, row, S, L_cap);
  const int j0 = c * chunk, j1 = min(j0 + chunk, n);
  if (j0 >= j1) return;
  const float* src = scores + (size_t)row * L_cap + j0 + U * t;
  const int lim = j1 - j0 - U * t;          // keys of this lane inside the row: min(U, lim)
  float v[U];
  if (VEC && lim >= U) {                    // 16-byte aligned: L_cap % 4 == 0, U % 4 == 0
#pragma unroll
    for (int u4 = 0; u4 < U / 4; ++u4) {
      const float4 q = reinterpret_cast<const float4*>(src)[u4];
      v[4 * u4] = q.x; v[4 * u4 + 1] = q.y; v[4 * u4 + 2] = q.z; v[4 * u4 + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = u < lim ? src[u] : 0.0f;
  }
  uint32_t key[U];
  uint32_t hits = 0, cnt = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    key[u] = score_key(v[u]);
    const bool hit = u < lim && key[u] >= T_lo;
    hits |= (uint32_t)hit << u;
    cnt += hit ? 1u : 0u;
  }
  uint32_t total;
  uint32_t pos = block_exclusive_scan<kChunkThreads>(cnt, scratch, &total);
  uint2* dst = m.slots + ((size_t)row * chunks + c) * kSlotCap;
  uint32_t poff = kNoPool;
  if (total > (uint32_t)kSlotCap) {
    if (t == 0) pool_base = atomicAdd(&st[2], total);
    __syncthreads();
    poff = pool_base;
    if (poff + total > (uint32_t)kMultiCap) {      // the row's list is too long
      if (t == 0) st[3] = 1u;
      return;
    }
    dst = m.pool + (size_t)row * kMultiCap + poff;
  }
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (hits >> u & 1u) dst[pos++] = make_uint2(key[u], (uint32_t)(j0 + U * t + u));
  if (t == 0) m.meta[(size_t)row * chunks + c] = make_uint2(total, poff);
}

// KC: exact selection and ordered emission, one workgroup per row.
// Dynamic LDS: keys[kMultiCap] | indices[kMultiCap] | select histograms
// [nh kRelBins] | chunk prefix offsets [chunks + 1] | chunk pool offsets
// [chunks]; the fallback's sel/tie segments reuse the list area and its
// histogram the first select histogram.  Up to kPreHistChunks chunks per row
// there are three select histograms, zeroed while the slot loads are in
// flight (three barriers per select level instead of five); beyond, one,
// zeroed per level.
constexpr int kPreHistChunks = 2048;
__host__ __device__ inline int finish_hists(int chunks) { return chunks <= kPreHistChunks ? 3 : 1; }
__host__ inline size_t finish_lds_bytes(int chunks) {
  return (size_t)(2 * kMultiCap + finish_hists(chunks) * kRelBins + 2 * chunks + 1) * 4;
}
static_assert(kMultiCap >= kSegWords, "fallback segments must fit the list area");
static_assert(kRelBins >= kBins, "the fallback histogram fits a select histogram");

__global__ __launch_bounds__(kFinishThreads) void topk_finish_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ kv_len, int S, int L_cap,
    int k, int chunk, int chunks, MultiWs m, int32_t* __restrict__ indices) {
  constexpr int NT = kFinishThreads;
  __shared__ uint32_t scratch[32];
  __shared__ uint32_t misc[kMiscWords];
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];
  uint32_t* lkey = dyn;
  uint32_t* lidx = dyn + kMultiCap;
  uint32_t* hist = dyn + 2 * kMultiCap;         // [nh * kRelBins]
  const int nh = finish_hists(chunks);          // grid-uniform
  uint32_t* pre = hist + nh * kRelBins;         // [chunks + 1]
  uint32_t* poff = pre + chunks + 1;            // [chunks]
  Lds s{hist, scratch, misc};
  const int row = blockIdx.x, t = threadIdx.x;
  // With at most kSpecSlots slots per row, every slot is loaded first, before
  // the state and the counts are known: slot positions are fixed, so these
  // loads overlap the count scan (slots past a chunk's count are ignored).
  constexpr int SG = kSpecSlots / NT;
  const bool spec = chunks * kSlotCap <= kSpecSlots;      // grid-uniform
  const uint2* slots = m.slots + (size_t)row * chunks * kSlotCap;
  uint2 se[SG];
  if (spec) {
#pragma unroll
    for (int g = 0; g < SG; ++g) {
      const int i = g * NT + t;
      if (i < chunks * kSlotCap) se[g] = slots[i];
    }
  }
  if (nh == 3) {                                // ordered before the select by the scan's barrier
    uint4* h4 = reinterpret_cast<uint4*>(hist);
    for (int i = t; i < 3 * kRelBins / 4; i += NT) h4[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  const int n = row_count(kv_len, row, S, L_cap);
  int32_t* out = indices + (size_t)row * k;
  const uint32_t* st = m.state + row * 4;
  const uint32_t mode = st[1];
  if (mode == kModeAll) { write_all<NT>(out, n, k); return; }
  const float* src = scores + (size_t)row * L_cap;
  if (mode == kModeList && st[3] == 0u) {
    // candidate key span; whether any chunk listed into the pool (both
    // ordered by the scan's barrier)
    if (t == 0) { misc[11] = 0; misc[12] = 0; }
    // chunk counts -> prefix offsets (lane t sums chunks [cpt t, cpt (t+1)))
    const int nch = (n + chunk - 1) / chunk;
    const int cpt = (nch + NT - 1) / NT;
    const int c0 = min(t * cpt, nch), c1 = min(c0 + cpt, nch);
    const uint2* meta = m.meta + (size_t)row * chunks;
    uint32_t local = 0;
    for (int c = c0; c < c1; ++c) local += meta[c].x;
    uint32_t total;
    uint32_t run = block_exclusive_scan<NT>(local, scratch, &total);
    for (int c = c0; c < c1; ++c) {
      const uint2 mc = meta[c];
      pre[c] = run;
      poff[c] = mc.y;
      run += mc.x;
      if (mc.y != kNoPool) misc[12] = 1u;
    }
    if (t == 0) pre[nch] = total;
    __syncthreads();
    if (total >= (uint32_t)k && total <= (uint32_t)kMultiCap) {
      const uint2* pool = m.pool + (size_t)row * kMultiCap;
      const uint32_t T_lo = st[0];
      uint32_t span = 0;                     // largest key - T_lo of this lane
      if (spec) {
        // slot r of chunk c goes to list entry pre[c] + r
#pragma unroll
        for (int g = 0; g < SG; ++g) {
          const int i = g * NT + t;
          const int c = i / kSlotCap, r = i % kSlotCap;
          if (c < nch && poff[c] == kNoPool && (uint32_t)r < pre[c + 1] - pre[c]) {
            lkey[pre[c] + r] = se[g].x;
            lidx[pre[c] + r] = se[g].y;
            span = max(span, se[g].x - T_lo);
          }
        }
      }
      if (!spec || misc[12] != 0u) {
        // gather in index order: entry i belongs to the chunk c with
        // pre[c] <= i < pre[c + 1] (only pooled chunks' entries when the
        // slots are already placed)
        constexpr int G = kMultiCap / NT;    // entries per lane; all loads in flight first
        uint2 e[G];
        uint32_t want = 0;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const int i = g * NT + t;
          if (i < (int)total) {
            int lo = 0, hi = nch - 1;
            while (lo < hi) {
              const int mid = (lo + hi + 1) >> 1;
              if (pre[mid] <= (uint32_t)i) lo = mid; else hi = mid - 1;
            }
            const uint32_t r = (uint32_t)i - pre[lo];
            if (!spec || poff[lo] != kNoPool) {
              e[g] = poff[lo] == kNoPool ? slots[(size_t)lo * kSlotCap + r] : pool[poff[lo] + r];
              want |= 1u << g;
            }
          }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const int i = g * NT + t;
          if (want >> g & 1u) {
            lkey[i] = e[g].x;
            lidx[i] = e[g].y;
            span = max(span, e[g].x - T_lo);
          }
        }
      }
      span = wave_inclusive_max_u32(span);
      if (lane_id() == kWave - 1) atomicMax(&misc[11], span);
      __syncthreads();
      uint32_t T, take;
      if (nh == 3)
        radix_select_rel_pre<NT>([&](int i) { return lkey[i]; }, (int)total, (uint32_t)k, T_lo,
                                 misc[11], hist, scratch, misc + 4, T, take);
      else
        radix_select_rel<NT>([&](int i) { return lkey[i]; }, (int)total, (uint32_t)k, T_lo,
                             misc[11], hist, scratch, misc, T, take);
      emit_ordered<NT>(lkey, lidx, (int)total, T, take, out, scratch);
      return;
    }
  }
  select_exact_row<NT>([&](int j) { return score_key(src[j]); }, n, k, dyn, dyn + kSegWords,
                       out, s);
}

template <typename K>
void opt_in_lds(K kernel, size_t bytes) {
  (void)hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)bytes);
}

constexpr int kStreamThreads = 1024;
using StreamPlan = StreamCfg<kStreamThreads, kRowCap>;

}  // namespace

TopkPlan plan_topk(int B, int S, int L_cap, int k) {
  (void)k;
  TopkPlan p{};
  p.rows = B * S;
  const long long rows = p.rows;
  if (rows >= 128) {
    p.kind = kPlanStream;
  } else if (L_cap <= kResKeys) {
    p.kind = kPlanResident;
  } else {
    p.kind = kPlanMulti;
  }
  if (p.kind == kPlanMulti) {
    // ~1024 chunk workgroups in all, at most 8 keys per thread each.
    long long want = ((long long)L_cap * rows + 1023) / 1024;
    int ch = 256;
    while (ch < want && ch < kChunkKeysPerThread * kChunkThreads) ch *= 2;
    p.chunk = ch;
    p.chunks = (L_cap + ch - 1) / ch;
    if (p.chunks > kMaxChunks) p.chunks = kMaxChunks;     // unreachable for L_cap <= 2^24
    p.ws_bytes = multi_ws_bytes(p.rows, p.chunks);
  }
  return p;
}

void launch_topk(const TopkPlan& p, const float* scores, const int32_t* kv_len, int S,
                 int L_cap, int k, int32_t* indices, void* ws, hipStream_t st) {
  if (p.rows == 0) return;
  static bool lds_opt_in = false;
  if (!lds_opt_in) {
    opt_in_lds(topk_resident_kernel<kResThreads>, kResLds);
    opt_in_lds(topk_stream_kernel<kStreamThreads, kRowCap, true>, StreamPlan::kLds);
    opt_in_lds(topk_stream_kernel<kStreamThreads, kRowCap, false>, StreamPlan::kLds);
    opt_in_lds(topk_finish_kernel, finish_lds_bytes(kMaxChunks));
    lds_opt_in = true;
  }
  const int vec4 = (L_cap & 3) == 0 ? 1 : 0;
  switch (p.kind) {
    case kPlanStream:
      if (vec4)
        hipLaunchKernelGGL((topk_stream_kernel<kStreamThreads, kRowCap, true>), dim3(p.rows),
                           dim3(kStreamThreads), StreamPlan::kLds, st, scores, kv_len, S, L_cap,
                           k, indices);
      else
        hipLaunchKernelGGL((topk_stream_kernel<kStreamThreads, kRowCap, false>), dim3(p.rows),
                           dim3(kStreamThreads), StreamPlan::kLds, st, scores, kv_len, S, L_cap,
                           k, indices);
      return;
    case kPlanResident:
      hipLaunchKernelGGL((topk_resident_kernel<kResThreads>), dim3(p.rows), dim3(kResThreads), kResLds, st,
                         scores, kv_len, S, L_cap, k, vec4, indices);
      return;
    default: {
      MultiWs m = carve(ws, p.rows, p.chunks);
      hipLaunchKernelGGL(topk_threshold_kernel, dim3(p.rows), dim3(kStateThreads), 0, st, scores,
                         kv_len, S, L_cap, k, m);
      const dim3 cg(p.chunks, p.rows);
      switch (p.chunk / kChunkThreads) {
        case 1:
          hipLaunchKernelGGL((topk_collect_kernel<1, false>), cg, dim3(kChunkThreads), 0, st,
                             scores, kv_len, S, L_cap, p.chunk, p.chunks, m);
          break;
        case 2:
          hipLaunchKernelGGL((topk_collect_kernel<2, false>), cg, dim3(kChunkThreads), 0, st,
                             scores, kv_len, S, L_cap, p.chunk, p.chunks, m);
          break;
        case 4:
          if (vec4) hipLaunchKernelGGL((topk_collect_kernel<4, true>), cg, dim3(kChunkThreads), 0,
                                       st, scores, kv_len, S, L_cap, p.chunk, p.chunks, m);
          else hipLaunchKernelGGL((topk_collect_kernel<4, false>), cg, dim3(kChunkThreads), 0, st,
                                  scores, kv_len, S, L_cap, p.chunk, p.chunks, m);
          break;
        default:
          if (vec4) hipLaunchKernelGGL((topk_collect_kernel<8, true>), cg, dim3(kChunkThreads), 0,
                                       st, scores, kv_len, S, L_cap, p.chunk, p.chunks, m);
          else hipLaunchKernelGGL((topk_collect_kernel<8, false>), cg, dim3(kChunkThreads), 0, st,
                                  scores, kv_len, S, L_cap, p.chunk, p.chunks, m);
          break;
      }
      hipLaunchKernelGGL(topk_finish_kernel, dim3(p.rows), dim3(kFinishThreads),
                         finish_lds_bytes(p.chunks), st, scores, kv_len, S, L_cap, k, p.chunk,
                         p.chunks, m, indices);
    }
  }
}

}  // namespace dsa
