// Per-query top-k with lowest-index tie-break (ORT PR #33802 "Optimize ...
// for SM12x and 256K context", Summary item 2: radix histograms per key
// chunk, a merge across up to 64+ chunks and a final emit of the indices).
//
// Exact for any FP32 input.  Scores map to order-preserving u32 keys
// (score_key); selection works on keys only.
//
// 1. Threshold estimate.  A sample of the row (all of it when the row is
//    short, else blocks of 256 consecutive keys spread evenly over the row:
//    2048 keys for an LDS-resident row, 8192 when streaming, 2048 or 4096 in
//    the split plan) goes through two radix levels (the top 11 + 11 key bits;
//    the resident plan: 8 + 8 bits of key - the sample's smallest key) to the
//    bin of the key of rank r = ceil(1.2e + 4 sqrt(e)) + 8, where e = k *
//    sample / n is the expected sample rank of the k-th largest key.  The
//    bin's lower edge T_lo is at or below that key; every key >= T_lo is a
//    candidate (about 1.2k + 4 sqrt(e) n/sample keys).
// 2. Collection.  One pass over the row lists the candidates; the resident
//    and split plans keep the list in index order.
// (The small plan for short rows skips steps 1-2: it selects on the whole row.)
// 3. Exact selection on the list: radix select of the k-th largest key T
//    on digits of key - T_lo (the split plan: 12-bit digits, two levels for
//    key spans below 2^24; the resident plan: the candidates held in
//    registers, 8-bit digits, and a direct rank once a bin holds at most 64
//    keys).  When only some of the keys equal to T fit, the lowest indices
//    win.  Exactly k entries.
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
// Plans (host-chosen from B*S, L_cap and the runtime bound max_kv_len):
//  * small     -- rows of at most 4096 keys (max_kv_len), any number of
//    rows: one 256-thread workgroup per row holds the row in registers and
//    selects exactly on 8-bit digits of key - (the row's smallest key), with
//    no threshold estimate.
//  * resident  -- few rows of <= 32768 keys by max_kv_len, whatever the
//    cache capacity (speculative decode at 32K): one 1024-thread workgroup
//    per row loads the row once into LDS (128 KB of keys) and does
//    everything there.
//  * streaming -- many rows (prefill: 2048 rows of 131072 keys): one
//    1024-thread workgroup per row reading the row ~1.06 times (two
//    workgroups per CU: at most 64 VGPRs, four 16-byte loads per lane in
//    flight).
//  * split     -- few rows longer than 32768 keys (decode at 256K): K1 (one
//    workgroup per chunk of a row) recomputes the row's sample threshold and
//    lists the chunk's candidates in index order in the chunk's own slots;
//    K2 (one workgroup per row) selects exactly on the chunks' lists and
//    emits.  The kernel boundary orders the two.
#include <cmath>

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
constexpr int kResCap = 4096;          // candidate list of a resident row
constexpr int kResSample = 2048;       // sample of a resident row (already in LDS)
constexpr int kRowCap = 4096;
static_assert(kResCap < 65536, "ordered emission packs counts in 16 bits");
constexpr int kStreamLoads = 4;        // 16-byte loads per lane in flight (streaming plan)
static_assert(4 * kStreamLoads <= 32, "one hit bit per key of a lane's step");

enum PlanKind { kPlanStream = 0, kPlanResident = 1, kPlanSplit = 2, kPlanSmall = 3 };

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

// h[i] = hist[nbins - 1 - (t BPT + i)]: thread t's BPT bins, highest first
// (16-byte LDS reads when BPT is a multiple of 4).
template <int BPT>
__device__ __forceinline__ void load_bins_desc(const uint32_t* hist, int nbins, int t,
                                               uint32_t (&h)[BPT]) {
  if constexpr (BPT % 4 == 0) {
    const uint4* q = reinterpret_cast<const uint4*>(hist + nbins - BPT * (t + 1));
#pragma unroll
    for (int j = 0; j < BPT / 4; ++j) {
      const uint4 v = q[BPT / 4 - 1 - j];
      h[4 * j] = v.w; h[4 * j + 1] = v.z; h[4 * j + 2] = v.y; h[4 * j + 3] = v.x;
    }
  } else {
#pragma unroll
    for (int i = 0; i < BPT; ++i) h[i] = hist[nbins - 1 - (t * BPT + i)];
  }
}

// The bin holding the need-th largest key of a 2048-bin histogram:
// misc[0] = bin, misc[1] = keys in higher bins.  Block-wide.  Each thread
// reads its BPT bins once into registers (a second pass of LDS reads behind
// the finder's conditional LDS writes would run as a serial chain).
template <int NT>
__device__ void select_bin(const uint32_t* hist, uint32_t need, uint32_t* scratch,
                           uint32_t* misc) {
  constexpr int BPT = kBins / NT;
  static_assert(BPT * NT == kBins, "block size must divide the bin count");
  const int t = threadIdx.x;
  if (t == 0) { misc[0] = 0; misc[1] = 0; }   // ordered before the finder by the scan's barriers
  uint32_t h[BPT];
  load_bins_desc<BPT>(hist, kBins, t, h);
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) local += h[i];
  uint32_t total;
  uint32_t before = block_exclusive_scan<NT>(local, scratch, &total);
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    if (before < need && need <= before + h[i]) {
      misc[0] = (uint32_t)(kBins - 1 - (t * BPT + i));
      misc[1] = before;
    }
    before += h[i];
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
__device__ uint32_t select_bin_rel(const uint32_t* hist, uint32_t need, uint32_t* scratch,
                                   uint32_t* misc) {
  constexpr int BPT = kRelBins / NT;
  static_assert(BPT * NT == kRelBins, "block size must divide the bin count");
  const int t = threadIdx.x;
  if (t == 0) { misc[0] = 0; misc[1] = 0; }
  uint32_t h[BPT];
  load_bins_desc<BPT>(hist, kRelBins, t, h);
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) local += h[i];
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
  return total;
}

// Exact selection inside one radix bin that holds at most a wave's worth of
// keys: the bin's keys, appended to `list` (LDS, list[kWave] a zeroed append
// counter), are ranked by wave 0, each lane comparing its key with all the
// others (ties counted), instead of one or two more radix levels with their
// histogram, scan and barriers.  res[0] = T, the need-th largest of the bin's
// nb keys; res[1] = how many keys equal to T belong to the top `need`.
// Block-wide: call after the appends, with every thread; 1 <= need <= nb.
template <int NT>
__device__ __forceinline__ void rank_small_bin(const uint32_t* list, uint32_t nb, uint32_t need,
                                               uint32_t* res) {
  __syncthreads();                             // the appends have landed
  if (threadIdx.x < kWave) {
    const int l = threadIdx.x;
    const uint32_t v = l < (int)nb ? list[l] : 0u;
    uint32_t gt = 0, ge = 0;
    for (int j = 0; j < (int)nb; ++j) {
      const uint32_t x = list[j];
      gt += x > v ? 1u : 0u;
      ge += x >= v ? 1u : 0u;
    }
    if (l < (int)nb && gt < need && need <= ge) {   // the lanes holding T agree
      res[0] = v;
      res[1] = need - gt;
    }
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
  // m <= kListCap < 2^16 (split plan), m <= kResCap (resident plan)
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

// A variant of radix_select (two levels) for callers that zeroed one
// histogram per level beforehand and give each level its own result words:
// three barriers per level instead of five.
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

// Hit bits of x[0..N) against a threshold's float image f_lo: bit u is set
// when x[u] >= f_lo.  For a finite f_lo (the caller branches on it,
// block-uniformly) the test is the sign of x - g, g = f_lo but -0.0 for a
// zero threshold (so that -0.0 - g = +0.0): the difference of two distinct
// finite floats is nonzero and keeps its sign (FP32 denormals are not
// flushed), equal ones give +0.0, and x = +-inf gives +-inf.  Two VALU
// operations per key (subtract, shift the sign bit in), with no compare and
// no condition-register hazard.
template <int N>
__device__ __forceinline__ uint32_t hits_finite(const float (&x)[N], float f_lo) {
  static_assert(N <= 32, "one bit per key");
  const float g = f_lo == 0.0f ? -0.0f : f_lo;
  uint32_t miss = 0;
#pragma unroll
  for (int u = N - 1; u >= 0; --u) miss = __builtin_amdgcn_alignbit(miss, __float_as_uint(x[u] - g), 31);
  return N == 32 ? ~miss : (~miss & ((1u << N) - 1u));
}

// ====================================================================== resident plan
// Dynamic LDS: row scores [kResKeys] (later the select's rank list) | hist
// (the sample threshold's, later the select's level histograms) | scratch |
// misc | list indices [kResCap].
// The row stays in LDS as FP32: hits are tested on floats and only the
// sample and the candidates become keys, which keeps the per-key work of
// the one-workgroup row small.
constexpr int kSmallBins = 256;
constexpr int kSmallLevels = 4;          // 8-bit digits of a 32-bit key range
static_assert(kSmallBins == 4 * kWave, "a lane reads four bins");

// Sum over aligned groups of G lanes (G = 4 or 16); every lane of a group
// gets its group's sum.  DPP lane moves: two quad permutations, then (16)
// two rotations of the 16-lane row by 4 and by 8.
template <int G>
__device__ __forceinline__ uint32_t group_sum(uint32_t v) {
  static_assert(G == 4 || G == 16, "quads or DPP rows");
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  if constexpr (G == 16) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false);  // row_ror:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false);  // row_ror:8
  }
  return v;
}

// One radix level over keys held in registers (thread t: KPL keys, valid
// where u < nv, all >= base): the keys whose bits >= hi of key - base match
// prefix count into h (256 zeroed words of LDS) by their digit bits
// [sh, hi); after a barrier every wave scans the bins itself (lane l reads
// four) and finds the bin holding the need-th largest of them, the keys in
// higher bins (above) and in that bin (cnt); all waves agree.  Block-wide.
template <int KPL>
__device__ __forceinline__ void held_keys_level(const uint32_t (&key)[KPL], int nv, uint32_t base,
                                                int hi, int sh, uint32_t prefix, uint32_t need,
                                                uint32_t* h, uint32_t& bin, uint32_t& above,
                                                uint32_t& cnt) {
  const int l = lane_id();
#pragma unroll
  for (int u = 0; u < KPL; ++u) {
    const uint32_t d = key[u] - base;
    if (u < nv && (hi >= 32 || (d >> hi) == (prefix >> hi))) atomicAdd(&h[(d >> sh) & 0xFFu], 1u);
  }
  __syncthreads();
  // lane l holds bins 255 - 4 l - i, i = 0..3 (highest first)
  const uint4 q = reinterpret_cast<const uint4*>(h)[kWave - 1 - l];
  const uint32_t b4[4] = {q.w, q.z, q.y, q.x};
  const uint32_t local = b4[0] + b4[1] + b4[2] + b4[3];
  uint32_t before = wave_inclusive_scan(local) - local;
  int b = -1;
  uint32_t a = 0u, c = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (before < need && need <= before + b4[i]) { b = kSmallBins - 1 - (4 * l + i); a = before; c = b4[i]; }
    before += b4[i];
  }
  const int fl = (int)__builtin_ctzll(__ballot(b >= 0)) & (kWave - 1);   // the one finder
  bin = (uint32_t)__builtin_amdgcn_readlane(b, fl);
  above = (uint32_t)__builtin_amdgcn_readlane((int)a, fl);
  cnt = (uint32_t)__builtin_amdgcn_readlane((int)c, fl);
}

// Lower bound of the need-th largest of keys held in registers (as for
// held_keys_level): two levels of 8-bit digits of key - base, the first on
// the top 8 bits of range; the lower edge of the chosen bin (exact when the
// range has at most 16 bits).  hist: two levels' zeroed bins.  Block-wide.
template <int KPL>
__device__ uint32_t lower_bound_held_keys(const uint32_t (&key)[KPL], int nv, uint32_t base,
                                          uint32_t range, uint32_t need,
                                          uint32_t (*hist)[kSmallBins]) {
  int hi = range ? 32 - __clz(range) : 0;
  uint32_t prefix = 0u;
  for (int lvl = 0; lvl < 2; ++lvl) {
    const int sh = hi > 8 ? hi - 8 : 0;
    uint32_t bin, above, cnt;
    held_keys_level<KPL>(key, nv, base, hi, sh, prefix, need, hist[lvl], bin, above, cnt);
    need -= above;
    prefix |= bin << sh;
    if (sh == 0) break;
    hi = sh;
  }
  return base + prefix;
}

// Exact selection over keys held in registers: thread t holds KPL keys
// (valid where u < nv), all in [base, base + range].  Radix digits of
// key - base, 8 bits per level, the first level on the top 8 bits of range;
// level lvl counts into hist[lvl] (kSmallLevels x 256 words of LDS, zeroed by
// the caller before a barrier).  After each level's barrier every wave scans
// the 256 bins itself and reaches the same bin, so a level needs no second
// barrier.  Once the chosen bin holds at most 64 keys they go to `list` (68
// words of LDS, 16-byte aligned) at block-scanned offsets and are ranked
// (each key compared with all of them, ties counted), the comparisons spread
// over the whole block; res (2 words of LDS) passes the result on.
// T = the need-th largest key, take = how many keys equal to T are kept.
// Block-wide; 1 <= need <= the number of valid keys.  scratch: NT/64 words.
template <int NT, int KPL>
__device__ void select_held_keys(const uint32_t (&key)[KPL], int nv, uint32_t base,
                                 uint32_t range, uint32_t need,
                                 uint32_t (*hist)[kSmallBins], uint32_t* list, uint32_t* scratch,
                                 uint32_t* res, uint32_t& T, uint32_t& take) {
  constexpr int TPK = NT / kWave;              // threads per ranked list entry
  constexpr int EPT = kWave / TPK;             // list entries each of them compares
  static_assert(TPK * EPT == kWave && EPT % 4 == 0, "whole 16-byte list reads");
  const int t = threadIdx.x;
  int hi = range ? 32 - __clz(range) : 0;      // bits [sh, hi) of key - base are this level's
  uint32_t prefix = 0u;                        // digits fixed so far (bits >= hi)
  T = 0u;
  take = 0u;
  for (int lvl = 0; lvl < kSmallLevels; ++lvl) {
    const int sh = hi > 8 ? hi - 8 : 0;
    uint32_t bin, above, cnt;
    held_keys_level<KPL>(key, nv, base, hi, sh, prefix, need, hist[lvl], bin, above, cnt);
    need -= above;
    prefix |= bin << sh;
    if (sh == 0) { T = base + prefix; take = need; return; }
    if (cnt <= (uint32_t)kWave) {
      // the bin's keys into the list (zero-padded to whole 16-byte reads:
      // every key is above 0, the key of no FP32 value but a negative NaN)
      uint32_t mine = 0u;
#pragma unroll
      for (int u = 0; u < KPL; ++u)
        mine += (u < nv && ((key[u] - base) >> sh) == (prefix >> sh)) ? 1u : 0u;
      uint32_t total;
      uint32_t slot = block_exclusive_scan<NT>(mine, scratch, &total);
#pragma unroll
      for (int u = 0; u < KPL; ++u) {
        if (u < nv && ((key[u] - base) >> sh) == (prefix >> sh)) {
          list[slot] = key[u];
          ++slot;
        }
      }
      if (t < 4) list[cnt + t] = 0u;
      __syncthreads();
      // ranks spread over the block: TPK consecutive threads share list
      // entry i = t / TPK, each comparing it with EPT entries, and sum their
      // counts with lane exchanges
      const int i = t / TPK, j0 = (t % TPK) * EPT;
      const uint32_t x = list[i];
      uint32_t gt = 0u, ge = 0u;
#pragma unroll
      for (int j = 0; j < EPT; j += 4) {
        const uint4 y = *reinterpret_cast<const uint4*>(list + j0 + j);
        const bool in0 = j0 + j < (int)cnt, in1 = j0 + j + 1 < (int)cnt;
        const bool in2 = j0 + j + 2 < (int)cnt, in3 = j0 + j + 3 < (int)cnt;
        gt += (in0 && y.x > x) + (in1 && y.y > x) + (in2 && y.z > x) + (in3 && y.w > x);
        ge += (in0 && y.x >= x) + (in1 && y.y >= x) + (in2 && y.z >= x) + (in3 && y.w >= x);
      }
      gt = group_sum<TPK>(gt);
      ge = group_sum<TPK>(ge);
      // the threads holding T agree; they write the same values
      if (t % TPK == 0 && i < (int)cnt && gt < need && need <= ge) { res[0] = x; res[1] = need - gt; }
      __syncthreads();
      T = res[0];
      take = res[1];
      return;
    }
    hi = sh;
  }
}

constexpr int kResThreads = 1024;
constexpr size_t kResLds = (size_t)(kResKeys + kBins + 32 + kMiscWords + kResCap) * 4;

template <int NT>
__global__ __launch_bounds__(NT) void topk_resident_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ kv_len, int S, int L_cap,
    int span, int k, int vec4, int32_t* __restrict__ indices) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  float* rowf = reinterpret_cast<float*>(lds);
  uint32_t* rowk = lds;
  Lds s{lds + kResKeys, lds + kResKeys + kBins, lds + kResKeys + kBins + 32};
  uint32_t* lidx = s.misc + kMiscWords;
  const int row = blockIdx.x, t = threadIdx.x;
  const float* src = scores + (size_t)row * L_cap;
  int32_t* out = indices + (size_t)row * k;

  // ---- the whole row into LDS, every load in flight at once.  Rows hold
  // at most span = min(L_cap, max_kv_len) <= 32768 keys (the runtime bound:
  // a long cache may hold short rows).  With 16-byte rows the loads are
  // direct global -> LDS copies that cover the span and go out before the
  // row's length is known (no wait for kv_len).
  if (vec4) {
    // direct global -> LDS copies: a wave's 64 lanes fill 1 KB of the row
    // at a time (lane l's 16 bytes at the wave's base + 16 l)
    constexpr int U = kResKeys / 4 / NT;
    const int L4 = (span + 3) / 4;              // <= L_cap / 4 (L_cap % 4 == 0)
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
    const int n = min(row_count(kv_len, row, S, L_cap), span);
    if (n <= k) {
      wait_vmem();                              // no copy may land after the workgroup ends
      write_all<NT>(out, n, k);
      return;
    }
  } else {
    const int n = min(row_count(kv_len, row, S, L_cap), span);
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
  const int n = min(row_count(kv_len, row, S, L_cap), span);
  // The sample threshold's two level histograms: the first 512 words of hist.
  if (t < 2 * kSmallBins / 4) reinterpret_cast<uint4*>(s.hist)[t] = make_uint4(0u, 0u, 0u, 0u);
  if (t == 0) { s.misc[12] = 0u; s.misc[13] = 0u; }   // the sample's largest key, ~(its smallest)
  // Every lane reads keys that other waves copied: each wave waits for its
  // own copies (the compiler would only wait before this wave's LDS reads),
  // then the barrier.
  wait_vmem();
  __syncthreads();

  if (k <= kResCap) {
    // ---- threshold from the sample (the row itself when short): two levels
    // of 8-bit digits of key - (the sample's smallest key); T_lo is the
    // lower edge of the bin holding the sample's r-th largest key
    constexpr int SPT = kResSample / NT;        // sample keys per thread
    const int ns = min(n, kResSample);
    const int nvs = ns - SPT * t;
    uint32_t sk[SPT];
    uint32_t smax = 0u, sminc = 0u;
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
      const int i = SPT * t + u;
      sk[u] = u < nvs ? score_key(rowf[n <= kResSample ? i : sample_pos<kResSample>(i, n)]) : 0u;
      if (u < nvs) { smax = max(smax, sk[u]); sminc = max(sminc, ~sk[u]); }
    }
    smax = wave_inclusive_max_u32(smax);
    sminc = wave_inclusive_max_u32(sminc);
    if (lane_id() == kWave - 1) { atomicMax(&s.misc[12], smax); atomicMax(&s.misc[13], sminc); }
    __syncthreads();
    const uint32_t smin = ~s.misc[13];
    const uint32_t need_s = (uint32_t)(n <= kResSample ? k : sample_rank(k, n, kResSample));
    const uint32_t T_lo = lower_bound_held_keys<SPT>(
        sk, nvs, smin, s.misc[12] - smin, need_s, reinterpret_cast<uint32_t (*)[kSmallBins]>(s.hist));
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
    if (__builtin_isfinite(f_lo)) {             // block-uniform
      float x[KPL];                             // read i's keys at 4 i (rotated back below)
#pragma unroll
      for (int i = 0; i < KPL / 4; ++i) {
        const float4 q = row4[(KPL / 4) * t + ((i + t) & (KPL / 4 - 1))];
        x[4 * i] = q.x; x[4 * i + 1] = q.y; x[4 * i + 2] = q.z; x[4 * i + 3] = q.w;
      }
      mask = hits_finite<KPL>(x, f_lo);
    } else {
#pragma unroll
      for (int i = KPL / 4 - 1; i >= 0; --i) {
        const float4 q = row4[(KPL / 4) * t + ((i + t) & (KPL / 4 - 1))];
        mask = (mask << 1) | (q.w >= f_lo ? 1u : 0u);
        mask = (mask << 1) | (q.z >= f_lo ? 1u : 0u);
        mask = (mask << 1) | (q.y >= f_lo ? 1u : 0u);
        mask = (mask << 1) | (q.x >= f_lo ? 1u : 0u);
      }
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
      // Thread t takes list entries [MU t, MU t + MU) (index order across
      // threads) and their keys into registers.  The largest key - T_lo
      // sizes the select's digits; the select's level histograms take the
      // sample threshold's histogram area, its rank list the row area's
      // front (free once every key is in registers).
      constexpr int MU = kResCap / NT;
      static_assert(MU == 4, "one 16-byte read of list entries per thread");
      const uint4 ix = reinterpret_cast<const uint4*>(lidx)[t];
      const uint32_t idx[MU] = {ix.x, ix.y, ix.z, ix.w};
      const int nvl = m - MU * t;               // entries of this thread inside the list
      uint32_t kk[MU];
      uint32_t span = 0;
#pragma unroll
      for (int u = 0; u < MU; ++u) {
        kk[u] = u < nvl ? score_key(rowf[idx[u]]) : 0u;
        if (u < nvl) span = max(span, kk[u] - T_lo);
      }
      span = wave_inclusive_max_u32(span);
      if (lane_id() == kWave - 1) atomicMax(&s.misc[11], span);
      uint32_t (*lh)[kSmallBins] = reinterpret_cast<uint32_t (*)[kSmallBins]>(s.hist);
      static_assert(kSmallLevels * kSmallBins <= kBins, "level histograms fit the sample's");
      if (t < kSmallLevels * kSmallBins / 4) reinterpret_cast<uint4*>(s.hist)[t] = make_uint4(0u, 0u, 0u, 0u);
      __syncthreads();                          // keys read, bins zeroed, span complete
      uint32_t T, take;
      select_held_keys<NT, MU>(kk, nvl, T_lo, s.misc[11], (uint32_t)k, lh, rowk, s.scratch, s.misc + 12,
                               T, take);
      // ---- ordered emission from the registers
      uint32_t gtc = 0u, eqc = 0u;
#pragma unroll
      for (int u = 0; u < MU; ++u) {
        gtc += (u < nvl && kk[u] > T) ? 1u : 0u;
        eqc += (u < nvl && kk[u] == T) ? 1u : 0u;
      }
      uint32_t total;
      const uint32_t ex = block_exclusive_scan<NT>(gtc | (eqc << 16), s.scratch + 16, &total);
      uint32_t g = ex & 0xFFFFu, e = ex >> 16;
#pragma unroll
      for (int u = 0; u < MU; ++u) {
        const bool above = u < nvl && kk[u] > T, tie = u < nvl && kk[u] == T;
        if (above || (tie && e < take)) out[g + min(e, take)] = (int32_t)idx[u];
        g += above ? 1u : 0u;
        e += tie ? 1u : 0u;
      }
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
  const int n64 = ((n + 63) / 64) * 64;
  for (int r = t; r < n64; r += NT) {
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
      const bool fin = __builtin_isfinite(f_lo);
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
        if (fin) {                              // block-uniform
          hm = hits_finite<4 * V>(x, f_lo);
#pragma unroll
          for (int u = 0; u < V; ++u)
            if (b4 + u * NT + t >= n4) hm &= ~(0xFu << (4 * u));
        } else {
#pragma unroll
          for (int u = 0; u < V; ++u) {
            const bool ok = b4 + u * NT + t < n4;
#pragma unroll
            for (int e = 0; e < 4; ++e) hm |= (uint32_t)(ok && x[4 * u + e] >= f_lo) << (4 * u + e);
          }
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

// ====================================================================== small plan
// Short rows: every row at most kSmallKeys keys long (by the runtime bound
// max_kv_len), any number of rows.  One 256-thread workgroup per row; thread
// t holds keys [KPL t, KPL t + KPL) of its row in registers, so the threads
// hold the row in index order.  There is no threshold estimate: exact
// selection runs on 8-bit radix digits of key - kmin (kmin, kmax: the row's
// smallest and largest live keys; the first level takes the top 8 bits of
// kmax - kmin), each level one 256-bin LDS histogram of the keys that share
// the digits chosen so far.  Every wave scans the whole histogram itself
// (the four waves reach the same bin), so a level costs one barrier, and the
// levels' histograms are zeroed up front.  Once the chosen bin holds at most
// 64 keys they are listed and ranked directly (each compared with all of
// them, ties counted; the comparisons spread over the workgroup).  Ordered
// emission: one block scan of the threads' (above, tie) counts.  With four
// waves a thread holds at most 16 keys, so the per-key loops stay short on
// each SIMD (select_held_keys, shared with the resident plan's select).
constexpr int kSmallKeys = 4096;
constexpr int kSmallThreads = 256;
static_assert(kSmallKeys < 65536, "emission packs counts in 16 bits");

template <int KPL, bool VEC>
__global__ __launch_bounds__(kSmallThreads) void topk_small_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ kv_len, int S, int L_cap,
    int k, int32_t* __restrict__ indices) {
  constexpr int NT = kSmallThreads;
  constexpr int NW = NT / kWave;
  static_assert(KPL % 4 == 0 && KPL * NT <= kSmallKeys, "whole 16-byte loads per thread");
  __shared__ __attribute__((aligned(16))) uint32_t hist[kSmallLevels][kSmallBins];
  __shared__ __attribute__((aligned(16))) uint32_t list[kWave + 4];
  __shared__ uint32_t scratch[32];
  __shared__ uint32_t wmm[2 * NW];
  __shared__ uint32_t res[2];
  const int row = blockIdx.x, t = threadIdx.x, l = lane_id(), w = t / kWave;
  const float* src = scores + (size_t)row * L_cap;
  int32_t* out = indices + (size_t)row * k;
  const int j0 = KPL * t;

  // ---- the thread's keys; the loads go out before kv_len is known (they
  // stay inside the L_cap-long row)
  uint32_t key[KPL];
  if (VEC && j0 + KPL <= L_cap) {              // rows 16-byte aligned (L_cap % 4 == 0)
#pragma unroll
    for (int q = 0; q < KPL / 4; ++q) {
      const float4 x = reinterpret_cast<const float4*>(src + j0)[q];
      key[4 * q] = __float_as_uint(x.x); key[4 * q + 1] = __float_as_uint(x.y);
      key[4 * q + 2] = __float_as_uint(x.z); key[4 * q + 3] = __float_as_uint(x.w);
    }
  } else {
#pragma unroll
    for (int u = 0; u < KPL; ++u) key[u] = j0 + u < L_cap ? __float_as_uint(src[j0 + u]) : 0u;
  }
  reinterpret_cast<uint4*>(&hist[0][0])[t] = make_uint4(0u, 0u, 0u, 0u);   // all levels' bins
  // rows are at most max_kv_len <= KPL * NT keys long
  const int n = min(row_count(kv_len, row, S, L_cap), KPL * NT);
  if (n <= k) {                                // block-uniform
    write_all<NT>(out, n, k);
    return;
  }
  const int nv = n - j0;                       // keys of this thread inside the row (may be <= 0)
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int u = 0; u < KPL; ++u) {
    key[u] = score_key(__uint_as_float(key[u]));
    if (u < nv) { kmin = min(kmin, key[u]); kmax = max(kmax, key[u]); }
  }
  kmax = wave_inclusive_max_u32(kmax);
  kmin = wave_inclusive_max_u32(~kmin);
  if (l == kWave - 1) { wmm[w] = kmax; wmm[NW + w] = kmin; }
  __syncthreads();                             // bins zeroed, wave extremes written
  kmax = 0u; kmin = 0u;
#pragma unroll
  for (int i = 0; i < NW; ++i) { kmax = max(kmax, wmm[i]); kmin = max(kmin, wmm[NW + i]); }
  kmin = ~kmin;

  // ---- exact selection: T = the k-th largest key, take = how many keys
  // equal to T are kept
  uint32_t T, take;
  select_held_keys<NT, KPL>(key, nv, kmin, kmax - kmin, (uint32_t)k, hist, list, scratch, res, T, take);

  // ---- ordered emission: the threads hold the row in index order
  uint32_t gtc = 0u, eqc = 0u;
#pragma unroll
  for (int u = 0; u < KPL; ++u) {
    gtc += (u < nv && key[u] > T) ? 1u : 0u;
    eqc += (u < nv && key[u] == T) ? 1u : 0u;
  }
  uint32_t total;
  const uint32_t ex = block_exclusive_scan<NT>(gtc | (eqc << 16), scratch + 16, &total);
  uint32_t g = ex & 0xFFFFu, e = ex >> 16;
#pragma unroll
  for (int u = 0; u < KPL; ++u) {
    const bool above = u < nv && key[u] > T, tie = u < nv && key[u] == T;
    if (above || (tie && e < take)) out[g + min(e, take)] = j0 + u;
    g += above ? 1u : 0u;
    e += tie ? 1u : 0u;
  }
}

// ====================================================================== split plan
// Few rows (B*S < 128) of any length.  Each row is cut into chunks of CH keys.
//
// K1, topk_chunk_kernel: one 512-thread workgroup per (chunk, row).  Every
// workgroup of a row draws the same sample of the row and computes the same
// sample threshold T_lo (a kernel of its own, or a hand-off between
// workgroups, costs more than recomputing it).  The sample is spread over the
// host bound max_kv_len, so its loads go out together with the chunk's own,
// before the row's length is known; a row much shorter than that bound draws
// a second sample over its own length.  The workgroup lists the chunk's keys
// >= T_lo, in index order, in the chunk's slots and writes the chunk's
// record (count, T_lo, largest sampled key).
//
// K2, topk_select_kernel: one workgroup per row.  The first `spec` slots of
// every chunk are stored interleaved so that lane t of K2 loads, coalesced,
// the E consecutive entries it owns (chunk t / (spec / E), entries
// E (t % (spec / E)) + [0, E)); lanes therefore hold the whole candidate list
// in index order in registers, in one memory round with the chunk records.
// The exact selection runs on relative radix digits of key - T_lo
// (histograms in LDS), and one block scan emits the kept indices in order.
// Rows with a chunk of more than `spec` candidates take a general path that
// gathers the list into LDS.
//
// Exactness: the list holds every key >= T_lo.  When it holds at least k keys
// and no chunk overflowed its slots, the row's k-th largest key is >= T_lo,
// so every key that can be selected is listed and the selection on the list
// equals the selection on the row.  Otherwise (a threshold above the k-th
// key, a chunk with more candidates than slots, a list longer than LDS holds)
// K2 selects exactly from the whole row.
constexpr int kChunkThreads = 512;
static_assert(kChunkThreads % kSampleBlock == 0, "whole sample blocks per pass of the lanes");
constexpr int kSelThreads = 512;
constexpr int kListCap = 8192;          // candidates the general path holds in LDS
static_assert(kListCap < 65536, "ordered emission packs counts in 16 bits");
constexpr int kSpecMax = 16384;         // entries the fast path holds (kSelThreads x 32)
static_assert(kSpecMax == kSelThreads * 32, "fast-path entries: 32 per select lane at most");
constexpr int kMaxSplitChunks = 2048;   // chunks per row (L_cap <= 2^24 with CH = 8192)
constexpr int kMinSample = 1024;        // smaller valid samples are drawn again over the row
static_assert(kListCap >= 2 * kSegWords, "fallback segments fit the list area");
static_assert(kRelBins >= kBins, "the fallback histogram fits a select histogram");

struct SplitWs {
  uint4* meta;       // [rows][nch_ws]: (candidates, T_lo, largest sampled key, 0)
  uint2* slots;      // [rows][nch_ws][cap]: (key, index)
};

__host__ __device__ inline SplitWs split_carve(void* ws, int rows, int nch_ws) {
  SplitWs w;
  w.meta = (uint4*)ws;
  w.slots = (uint2*)(w.meta + (size_t)rows * nch_ws);
  return w;
}

// Slot of candidate r of a chunk: the first `spec` interleaved for the fast
// path's lane-contiguous, coalesced loads (pair p = r / 2 at 16-byte position
// (p % (E/2)) (spec / E) + p / (E/2)), the rest in order.
__device__ __forceinline__ int slot_of(int r, int spec, int e_log2, int tpc_log2) {
  if (r >= spec) return r;
  const int p = r >> 1, ph = (1 << (e_log2 - 1)) - 1;
  return 2 * (((p & ph) << tpc_log2) + (p >> (e_log2 - 1))) + (r & 1);
}

// First key of sample block u of a row sampled over [0, span): NS / 256
// blocks of 256 consecutive keys, consecutive when span <= NS, else spread
// evenly over [0, span).
template <int NS>
__device__ __forceinline__ int sample_block_base(int u, int span) {
  constexpr int NB = NS / kSampleBlock;
  return span > NS ? (int)((uint32_t)(u * (span - kSampleBlock)) / (uint32_t)(NB - 1))
                   : u * kSampleBlock;
}
// Sampled keys below n (sampling over [0, span)).
template <int NS>
__device__ __forceinline__ int sample_valid(int n, int span) {
  constexpr int NB = NS / kSampleBlock;
  const int m = min(n, span);
  int v = 0;
#pragma unroll
  for (int u = 0; u < NB; ++u) v += min(max(m - sample_block_base<NS>(u, span), 0), kSampleBlock);
  return v;
}

// K1.  U keys per lane (lane t owns keys jl = c CH + U t + [0, U)).
template <int U, int NS, bool VEC>
__global__ __launch_bounds__(kChunkThreads) void topk_chunk_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ kv_len, int S, int L_cap,
    int span, int k, int nch_ws, int cap, int spec, int e_log2, int tpc_log2, SplitWs w) {
  constexpr int NT = kChunkThreads;
  constexpr int CH = U * NT;
  constexpr int SPL = NS / NT;                 // sample keys per lane
  constexpr int BPP = NT / kSampleBlock;       // sample blocks per pass of the lanes
  __shared__ __attribute__((aligned(16))) uint32_t h0[kBins];
  __shared__ __attribute__((aligned(16))) uint32_t h1[kBins];
  __shared__ uint32_t scratch[32];
  __shared__ uint32_t misc[8];
  __shared__ __attribute__((aligned(16))) float chunk[CH];   // lane t's keys at U t + [0, U)
  const int c = blockIdx.x, row = blockIdx.y, t = threadIdx.x;
  const float* src = scores + (size_t)row * L_cap;
  const int jl = c * CH + U * t;

  // ---- chunk keys and the sample: every load in flight before kv_len is known
  float v[U];
  if (VEC && jl + U <= L_cap) {                // rows 16-byte aligned (L_cap % 4 == 0)
    if constexpr (U % 4 == 0) {
#pragma unroll
      for (int q = 0; q < U / 4; ++q) {
        const float4 x = reinterpret_cast<const float4*>(src + jl)[q];
        v[4 * q] = x.x; v[4 * q + 1] = x.y; v[4 * q + 2] = x.z; v[4 * q + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int q = 0; q < U / 2; ++q) {
        const float2 x = reinterpret_cast<const float2*>(src + jl)[q];
        v[2 * q] = x.x; v[2 * q + 1] = x.y;
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = jl + u < L_cap ? src[jl + u] : 0.0f;
  }
  // lane t takes element t % 256 of sample blocks BPP u + t / 256
  const int se = t % kSampleBlock, sb = t / kSampleBlock;
  float sv[SPL];
#pragma unroll
  for (int u = 0; u < SPL; ++u) {
    const int p = sample_block_base<NS>(BPP * u + sb, span) + se;
    sv[u] = src[p < span ? p : 0];             // span <= L_cap
  }
  for (int i = t; i < kBins; i += NT) { h0[i] = 0u; h1[i] = 0u; }
  if (t == 0) misc[4] = 0u;
  const int b = row / S;
  int n = kv_len[b] - S + row % S + 1;
  n = max(0, min(n, min(L_cap, gridDim.x * CH)));
  if (n <= k || c * CH >= n) return;           // K2 handles the row / nothing to list here
  int sspan = span;
  int nsv = sample_valid<NS>(n, span);
  if (nsv < kMinSample && nsv < n) {
    // a row much shorter than the bound: sample its own length instead
    sspan = n;
    nsv = sample_valid<NS>(n, n);
#pragma unroll
    for (int u = 0; u < SPL; ++u) {
      const int p = sample_block_base<NS>(BPP * u + sb, n) + se;
      sv[u] = src[p < n ? p : 0];
    }
  }
  const int slim = min(n, sspan);

  // ---- sample threshold: two radix levels (key bits [31:21], [20:10]); the
  // largest sampled key sizes the select kernel's digits
  uint32_t sk[SPL];
  uint32_t smax = 0u, sok = 0u;
#pragma unroll
  for (int u = 0; u < SPL; ++u) {
    sk[u] = score_key(sv[u]);
    if (sample_block_base<NS>(BPP * u + sb, sspan) + se < slim) {
      sok |= 1u << u;
      smax = max(smax, sk[u]);
    }
  }
  smax = wave_inclusive_max_u32(smax);
  __syncthreads();                             // histograms zeroed
#pragma unroll
  for (int u = 0; u < SPL; ++u)
    if ((sok >> u) & 1u) atomicAdd(&h0[sk[u] >> 21], 1u);
  if (lane_id() == kWave - 1) atomicMax(&misc[4], smax);
  __syncthreads();
  uint32_t need = (uint32_t)(nsv == n ? k : sample_rank(k, n, nsv));
  select_bin<NT>(h0, need, scratch, misc);
  const uint32_t b0 = misc[0];
  need -= misc[1];
#pragma unroll
  for (int u = 0; u < SPL; ++u)
    if (((sok >> u) & 1u) && (sk[u] >> 21) == b0) atomicAdd(&h1[(sk[u] >> 10) & 0x7FFu], 1u);
  __syncthreads();
  select_bin<NT>(h1, need, scratch, misc + 2);
  const uint32_t T_lo = (b0 << 21) | (misc[2] << 10);

  // ---- candidates of the chunk, in index order.  Tested on floats:
  // x >= f_lo <=> score_key(x) >= T_lo (score_key is order-preserving and
  // gives -0.0 the key of +0.0).  A threshold inside the -inf bin has a NaN
  // pattern and no hits; K2 then selects from the whole row.
  const float f_lo = __uint_as_float((T_lo & 0x80000000u) ? (T_lo & 0x7FFFFFFFu) : ~T_lo);
  uint32_t hits = 0;
  if (__builtin_isfinite(f_lo)) {               // block-uniform
    const int nv = n - jl;                      // keys of this lane inside the row
    hits = hits_finite<U>(v, f_lo) & (nv >= U ? 0xFFFFFFFFu : (nv <= 0 ? 0u : (1u << nv) - 1u));
  } else {
#pragma unroll
    for (int u = 0; u < U; ++u) hits |= (uint32_t)(jl + u < n && v[u] >= f_lo) << u;
  }
  // The lane's keys go to LDS so that the write loop visits its hits only
  // (a key picked by a per-lane bit index cannot be read from registers).
  // Each lane reads back only what it wrote itself: no barrier.
  if constexpr (U % 4 == 0) {
#pragma unroll
    for (int q = 0; q < U / 4; ++q)
      reinterpret_cast<float4*>(chunk + U * t)[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  } else {
#pragma unroll
    for (int q = 0; q < U / 2; ++q)
      reinterpret_cast<float2*>(chunk + U * t)[q] = make_float2(v[2 * q], v[2 * q + 1]);
  }
  uint32_t total;
  uint32_t pos = block_exclusive_scan<NT>((uint32_t)__popc(hits), scratch, &total);
  if (total <= (uint32_t)cap) {
    uint2* dst = w.slots + ((size_t)row * nch_ws + c) * cap;
    for (uint32_t hm = hits; hm; hm &= hm - 1) {
      const int u = __builtin_ctz(hm);
      dst[slot_of((int)pos, spec, e_log2, tpc_log2)] =
          make_uint2(score_key(chunk[U * t + u]), (uint32_t)(jl + u));
      ++pos;
    }
  }
  if (t == 0) w.meta[(size_t)row * nch_ws + c] = make_uint4(total, T_lo, misc[4], 0u);
}

// K2.  Dynamic LDS: keys[kListCap] | indices[kListCap] | three select
// histograms [3 kRelBins] | chunk prefix offsets [kMaxSplitChunks + 1].
// Each select histogram is followed by kWave spare bins: entries that must
// not count add to their lane's spare bin, so the atomics need no branches.
constexpr int kHistStride = kRelBins + kWave;
constexpr size_t kSelLds = (size_t)(2 * kListCap + 3 * kHistStride + kMaxSplitChunks + 1) * 4;

// Exact k-th largest of the keys held by the lanes (E per lane, valid bits
// in `vm`), all >= base: relative radix digits of key - base, the first
// level on the bits below the bit length of `range` (keys beyond base +
// range share the top bin).  Returns false when the k-th key falls in that
// shared top bin or the keys number fewer than `need`; else T and take
// (how many keys equal to T are kept).  hA, hB, hC: zeroed kRelBins each.
template <int NT, int E>
__device__ bool select_regs(const uint32_t (&key)[E], uint32_t vm, uint32_t base, uint32_t range,
                            uint32_t need, uint32_t* hA, uint32_t* hB, uint32_t* hC,
                            uint32_t* scratch, uint32_t* misc, uint32_t& T, uint32_t& take) {
  const int top = range ? 32 - __clz(range) : 0;
  const int shA = top > kRelBits ? top - kRelBits : 0;
  const uint32_t spare = kRelBins + lane_id();
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const uint32_t d = min((key[j] - base) >> shA, (uint32_t)(kRelBins - 1));
    atomicAdd(&hA[((vm >> j) & 1u) ? d : spare], 1u);
  }
  __syncthreads();
  const uint32_t m = select_bin_rel<NT>(hA, need, scratch, misc);
  const uint32_t bA = misc[0];
  if (m < need || bA == kRelBins - 1) return false;
  need -= misc[1];
  uint32_t prefix = base + (bA << shA);
  if (shA > 0) {
    const uint32_t nb = hA[bA];                 // keys in the chosen bin (block-uniform)
    if (nb <= (uint32_t)kWave) {
      // few keys left: rank them in one wave; hB (zeroed, unused) holds the
      // list and, at hB[kWave], its counter
#pragma unroll
      for (int j = 0; j < E; ++j)
        if (((vm >> j) & 1u) && ((key[j] - base) >> shA) == bA) hB[atomicAdd(&hB[kWave], 1u)] = key[j];
      rank_small_bin<NT>(hB, nb, need, misc + 2);
      T = misc[2];
      take = misc[3];
      return true;
    }
    const int shB = shA > kRelBits ? shA - kRelBits : 0;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const bool in = ((vm >> j) & 1u) && ((key[j] - base) >> shA) == bA;
      atomicAdd(&hB[in ? (key[j] - prefix) >> shB : spare], 1u);
    }
    __syncthreads();
    select_bin_rel<NT>(hB, need, scratch, misc + 2);
    need -= misc[3];
    prefix += misc[2] << shB;
    if (shB > 0) {                             // shB <= 8: the last level
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const bool in = ((vm >> j) & 1u) && key[j] >= prefix && key[j] - prefix < (1u << shB);
        atomicAdd(&hC[in ? key[j] - prefix : spare], 1u);
      }
      __syncthreads();
      select_bin_rel<NT>(hC, need, scratch, misc + 4);
      need -= misc[5];
      prefix += misc[4];
    }
  }
  T = prefix;
  take = need;
  return true;
}

template <int E>
__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ kv_len, int S, int L_cap,
    int k, int CH, int nch, int nch_ws, int cap, int spec, int e_log2, int tpc_log2,
    int mode, SplitWs w, int32_t* __restrict__ indices) {
  constexpr int NT = kSelThreads;
  constexpr int P = E / 2;                      // (key, index) pairs per lane, one uint4 each
  __shared__ uint32_t scratch[32];
  __shared__ uint32_t misc[kMiscWords];
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];
  uint32_t* lkey = dyn;
  uint32_t* lidx = dyn + kListCap;
  uint32_t* hA = dyn + 2 * kListCap;
  uint32_t* hB = hA + kHistStride;
  uint32_t* hC = hB + kHistStride;
  uint32_t* pre = hC + kHistStride;             // [kMaxSplitChunks + 1]
  const int row = blockIdx.x, t = threadIdx.x;
  int32_t* out = indices + (size_t)row * k;
  const float* src = scores + (size_t)row * L_cap;
  const uint4* meta = w.meta + (size_t)row * nch_ws;
  const uint2* slots = w.slots + (size_t)row * nch_ws * cap;
  // mode 0: fast path first (lane t owns chunk c's entries E u + [0, E); the
  // host guarantees nch * spec <= NT * E), 1: general path, 2: exact only
  const bool fast = mode == 0;
  const bool exact_only = mode == 2;
  const int c = t >> tpc_log2, u = t & ((1 << tpc_log2) - 1);

  // ---- one memory round: the lane's entries, its chunk's record, chunk 0's
  // record (T_lo and the largest sampled key of the row), kv_len
  uint4 ent[P];
  uint4 mine = make_uint4(0u, 0u, 0u, 0u), m0 = mine;
  if (fast && c < nch) {
    mine = meta[c];
    const uint4* cs = reinterpret_cast<const uint4*>(slots + (size_t)c * cap);
#pragma unroll
    for (int q = 0; q < P; ++q) ent[q] = cs[(q << tpc_log2) + u];
  }
  if (!exact_only && nch > 0) m0 = meta[0];
  {
    uint4* h4 = reinterpret_cast<uint4*>(hA);
    static_assert(kHistStride % 4 == 0, "histograms zeroed in 16-byte stores");
    for (int i = t; i < 3 * kHistStride / 4; i += NT) h4[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  if (t == 0) { misc[8] = 0u; misc[9] = 0u; }
  const int b = row / S;
  int n = kv_len[b] - S + row % S + 1;
  n = max(0, min(n, min(L_cap, nch * CH)));
  if (n <= k) { write_all<NT>(out, n, k); return; }
  const int nch_row = (n + CH - 1) / CH;
  const uint32_t T_lo = m0.y;
  __syncthreads();                              // histograms and flags zeroed

  if (fast) {
    const uint32_t cnt = c < nch_row ? mine.x : 0u;
    const int r0 = E * u;
    uint32_t key[E], vm = 0u;
#pragma unroll
    for (int q = 0; q < P; ++q) { key[2 * q] = ent[q].x; key[2 * q + 1] = ent[q].z; }
    if ((uint32_t)r0 < cnt) vm = cnt - r0 >= (uint32_t)E ? 0xFFFFFFFFu >> (32 - E) : (1u << (cnt - r0)) - 1u;
    // a chunk beyond its speculative slots (or its capacity) leaves the fast path
    if (cnt > (uint32_t)spec && u == 0) atomicOr(&misc[8], 1u);
    const uint32_t range = m0.z > T_lo ? m0.z - T_lo : 0u;
    uint32_t T = 0, take = 0;
    // misc[8] is read after the first level's barrier
    const bool ok = select_regs<NT, E>(key, vm, T_lo, range, (uint32_t)k, hA, hB, hC, scratch,
                                       misc, T, take) && misc[8] == 0u;
    if (ok) {
      // ---- ordered emission: entries are in index order across lanes
      uint32_t gt = 0, eq = 0;
#pragma unroll
      for (int j = 0; j < E; ++j)
        if ((vm >> j) & 1u) { gt += key[j] > T ? 1u : 0u; eq += key[j] == T ? 1u : 0u; }
      uint32_t total;
      const uint32_t before = block_exclusive_scan<NT>(gt | (eq << 16), scratch, &total);
      uint32_t g = before & 0xFFFFu, e = before >> 16;
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const bool v = (vm >> j) & 1u;
        const bool above = v && key[j] > T, tie = v && key[j] == T;
        const uint32_t slot = g + (e < take ? e : take);
        if (above || (tie && e < take)) out[slot] = (int32_t)((j & 1) ? ent[j >> 1].w : ent[j >> 1].y);
        g += above ? 1u : 0u;
        e += tie ? 1u : 0u;
      }
      return;
    }
    __syncthreads();                            // misc, scratch and histograms are reused below
  }

  if (!exact_only) {
    // ---- general path: chunk counts -> prefix offsets, the list gathered
    // into LDS in index order (chunks past the row's end were not written by
    // this call and count 0)
    constexpr int CPT = kMaxSplitChunks / NT;
    uint32_t cl[CPT], local = 0, over = 0;
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int ci = CPT * t + q;
      cl[q] = ci < nch_row ? meta[ci].x : 0u;
      local += cl[q];
      over |= cl[q] > (uint32_t)cap ? 1u : 0u;
    }
    if (t == 0) { misc[10] = 0u; misc[11] = 0u; }
    uint32_t m;
    uint32_t run = block_exclusive_scan<NT>(local, scratch, &m);
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int ci = CPT * t + q;
      if (ci < nch_row) pre[ci] = run;
      run += cl[q];
    }
    if (t == 0) pre[nch_row] = m;
    if (over) misc[10] = 1u;
    __syncthreads();
    if (misc[10] == 0u && m >= (uint32_t)k && m <= (uint32_t)kListCap) {
      constexpr int G = kListCap / NT;           // entries per lane; all loads in flight first
      uint2 x[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int i = g * NT + t;
        if (i < (int)m) {
          int lo = 0, hi = nch_row - 1;          // chunk of entry i: pre[lo] <= i < pre[lo + 1]
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (pre[mid] <= (uint32_t)i) lo = mid; else hi = mid - 1;
          }
          x[g] = slots[(size_t)lo * cap + slot_of(i - (int)pre[lo], spec, e_log2, tpc_log2)];
        }
      }
      uint32_t kmax = 0u;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int i = g * NT + t;
        if (i < (int)m) {
          lkey[i] = x[g].x;
          lidx[i] = x[g].y;
          kmax = max(kmax, x[g].x);
        }
      }
      kmax = wave_inclusive_max_u32(kmax);
      if (lane_id() == kWave - 1) atomicMax(&misc[11], kmax);
      __syncthreads();
      uint32_t T, take;
      radix_select_rel<NT>([&](int i) { return lkey[i]; }, (int)m, (uint32_t)k, T_lo,
                           misc[11] - T_lo, hA, scratch, misc, T, take);
      emit_ordered<NT>(lkey, lidx, (int)m, T, take, out, scratch);
      return;
    }
    __syncthreads();                            // misc and the list area are reused below
  }
  Lds s{hA, scratch, misc};
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

TopkPlan plan_topk(int B, int S, int L_cap, int max_kv_len, int k) {
  TopkPlan p{};
  p.rows = B * S;
  const long long rows = p.rows;
  if (max_kv_len <= kSmallKeys) {
    p.kind = kPlanSmall;
    int kpl = 4;
    while (kpl * kSmallThreads < max_kv_len) kpl *= 2;
    p.lane_keys = kpl;
    return p;
  }
  if (rows >= 128) {
    p.kind = kPlanStream;
    return p;
  }
  if (max_kv_len <= kResKeys) {
    p.kind = kPlanResident;
    return p;
  }
  p.kind = kPlanSplit;
  // About one chunk workgroup per CU over all rows, 1024..8192 keys each
  // (8192-key chunks keep L_cap <= 2^24 within kMaxSplitChunks per row).
  const long long want = (rows * L_cap + 255) / 256;
  int ch = 1024;
  while (ch < want && ch < 8192) ch *= 2;
  p.chunk = ch;
  p.chunks = (L_cap + ch - 1) / ch;
  p.sample = L_cap <= 65536 ? 2048 : 4096;
  p.exact_only = k > kListCap ? 1 : 0;
  // Expected candidates per chunk of a full row: the sample threshold sits
  // at sample rank r = ceil(1.2 e + 4 sqrt(e)) + 8, e = k * sample / L_cap.
  double per_chunk;
  if (L_cap <= p.sample) {
    per_chunk = (double)ch * k / L_cap;
  } else {
    const double e = (double)k * p.sample / L_cap;
    double r = std::ceil(1.2 * e + 4.0 * std::sqrt(e)) + 8.0;
    if (r > p.sample) r = p.sample;
    per_chunk = (double)ch * r / p.sample;
  }
  // Slots: a whole chunk's worth while that stays within 256 MiB (no chunk
  // can overflow), else four times the expectation (an overflowing chunk
  // sends its row to the exact selection over the whole row).
  const size_t full = (size_t)rows * p.chunks * ch * sizeof(uint2);
  if (full <= ((size_t)256 << 20)) {
    p.cap = ch;
  } else {
    int cap = (int)((4.0 * per_chunk + 64.0 + 63.0) / 64.0) * 64;
    p.cap = cap < ch ? cap : ch;
  }
  // Speculative slots per chunk: a power of two >= 1.5 times the expectation,
  // E = spec * chunks / kSelThreads entries per lane (8, 16 or 32; a lane's
  // entries lie in one chunk).  Beyond kSpecMax entries per row there is no
  // fast path (spec = 0).
  int spec = 32;
  while (spec < 1.5 * per_chunk + 32.0 && spec < p.cap) spec *= 2;
  if (spec > p.cap) spec = p.cap;
  int e = 8;
  while ((long long)e * kSelThreads < (long long)spec * p.chunks && e < 32) e *= 2;
  if ((long long)spec * p.chunks > (long long)e * kSelThreads || spec < e) spec = 0;
  p.spec = spec;
  p.entries = e;
  p.ws_bytes = (size_t)p.rows * p.chunks * (sizeof(uint4) + (size_t)p.cap * sizeof(uint2));
  return p;
}

namespace {
int ilog2(int x) { int l = 0; while ((1 << (l + 1)) <= x) ++l; return l; }

template <int U, int NS>
void launch_chunk(bool vec, dim3 grid, hipStream_t st, const float* scores, const int32_t* kv_len,
                  int S, int L_cap, int span, int k, int nch_ws, int cap, int spec, int el,
                  int tl, SplitWs w) {
  if (vec)
    hipLaunchKernelGGL((topk_chunk_kernel<U, NS, true>), grid, dim3(kChunkThreads), 0, st, scores,
                       kv_len, S, L_cap, span, k, nch_ws, cap, spec, el, tl, w);
  else
    hipLaunchKernelGGL((topk_chunk_kernel<U, NS, false>), grid, dim3(kChunkThreads), 0, st, scores,
                       kv_len, S, L_cap, span, k, nch_ws, cap, spec, el, tl, w);
}
template <int NS>
void launch_chunk_ns(int U, bool vec, dim3 grid, hipStream_t st, const float* scores,
                     const int32_t* kv_len, int S, int L_cap, int span, int k, int nch_ws, int cap,
                     int spec, int el, int tl, SplitWs w) {
  switch (U) {
    case 2: launch_chunk<2, NS>(vec, grid, st, scores, kv_len, S, L_cap, span, k, nch_ws, cap, spec, el, tl, w); break;
    case 4: launch_chunk<4, NS>(vec, grid, st, scores, kv_len, S, L_cap, span, k, nch_ws, cap, spec, el, tl, w); break;
    case 8: launch_chunk<8, NS>(vec, grid, st, scores, kv_len, S, L_cap, span, k, nch_ws, cap, spec, el, tl, w); break;
    default: launch_chunk<16, NS>(vec, grid, st, scores, kv_len, S, L_cap, span, k, nch_ws, cap, spec, el, tl, w); break;
  }
}
template <int KPL>
void launch_small(bool vec, int rows, hipStream_t st, const float* scores, const int32_t* kv_len,
                  int S, int L_cap, int k, int32_t* indices) {
  if (vec)
    hipLaunchKernelGGL((topk_small_kernel<KPL, true>), dim3(rows), dim3(kSmallThreads), 0, st,
                       scores, kv_len, S, L_cap, k, indices);
  else
    hipLaunchKernelGGL((topk_small_kernel<KPL, false>), dim3(rows), dim3(kSmallThreads), 0, st,
                       scores, kv_len, S, L_cap, k, indices);
}
}  // namespace

void launch_topk(const TopkPlan& p, const float* scores, const int32_t* kv_len, int S,
                 int L_cap, int max_kv_len, int k, int32_t* indices, void* ws, hipStream_t st) {
  if (p.rows == 0) return;
  static bool lds_opt_in = false;
  if (!lds_opt_in) {
    opt_in_lds(topk_resident_kernel<kResThreads>, kResLds);
    opt_in_lds(topk_stream_kernel<kStreamThreads, kRowCap, true>, StreamPlan::kLds);
    opt_in_lds(topk_stream_kernel<kStreamThreads, kRowCap, false>, StreamPlan::kLds);
    opt_in_lds(topk_select_kernel<8>, kSelLds);
    opt_in_lds(topk_select_kernel<16>, kSelLds);
    opt_in_lds(topk_select_kernel<32>, kSelLds);
    lds_opt_in = true;
  }
  const int vec4 = (L_cap & 3) == 0 ? 1 : 0;
  switch (p.kind) {
    case kPlanSmall:
      switch (p.lane_keys) {
        case 4: launch_small<4>(vec4, p.rows, st, scores, kv_len, S, L_cap, k, indices); break;
        case 8: launch_small<8>(vec4, p.rows, st, scores, kv_len, S, L_cap, k, indices); break;
        default: launch_small<16>(vec4, p.rows, st, scores, kv_len, S, L_cap, k, indices); break;
      }
      return;
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
                         scores, kv_len, S, L_cap, min(L_cap, max_kv_len), k, vec4, indices);
      return;
    default: {
      SplitWs w = split_carve(ws, p.rows, p.chunks);
      // chunks covering the runtime bound; K2 treats rows as at most this long
      const int nch = (max_kv_len + p.chunk - 1) / p.chunk;
      // slot interleave of the fast path (spec = 0: none; the general path
      // then reads every slot in order)
      const int spec = p.spec > 0 ? p.spec : 1 << 30;
      const int el = p.spec > 0 ? ilog2(p.entries) : 1;
      const int tl = p.spec > 0 ? ilog2(p.spec / p.entries) : 0;
      if (nch > 0 && !p.exact_only) {
        const dim3 grid(nch, p.rows);
        if (p.sample == 2048)
          launch_chunk_ns<2048>(p.chunk / kChunkThreads, vec4, grid, st, scores, kv_len, S, L_cap,
                                max_kv_len, k, p.chunks, p.cap, spec, el, tl, w);
        else
          launch_chunk_ns<4096>(p.chunk / kChunkThreads, vec4, grid, st, scores, kv_len, S, L_cap,
                                max_kv_len, k, p.chunks, p.cap, spec, el, tl, w);
      }
      const int ex = p.exact_only ? 2 : (p.spec > 0 ? 0 : 1);
      switch (p.entries) {
        case 8:
          hipLaunchKernelGGL((topk_select_kernel<8>), dim3(p.rows), dim3(kSelThreads), kSelLds, st,
                             scores, kv_len, S, L_cap, k, p.chunk, nch, p.chunks, p.cap, spec, el,
                             tl, ex, w, indices);
          break;
        case 16:
          hipLaunchKernelGGL((topk_select_kernel<16>), dim3(p.rows), dim3(kSelThreads), kSelLds, st,
                             scores, kv_len, S, L_cap, k, p.chunk, nch, p.chunks, p.cap, spec, el,
                             tl, ex, w, indices);
          break;
        default:
          hipLaunchKernelGGL((topk_select_kernel<32>), dim3(p.rows), dim3(kSelThreads), kSelLds, st,
                             scores, kv_len, S, L_cap, k, p.chunk, nch, p.chunks, p.cap, spec, el,
                             tl, ex, w, indices);
      }
    }
  }
}

}  // namespace dsa
