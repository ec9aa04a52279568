// Sparse GQA attention over the selected keys (ORT PR #33997 "Support FP16 KV
// cache and FP16 query/key in DynamicSparseAttention<BFloat16> ...",
// Description item 2: selected-only attention, grouped decode, FP16 cache
// with BF16 activations, query read without a separate conversion kernel;
// ORT PR #33802, Summary item 1: INT8 cache with per-token scales, split-K
// decode, and follow-up #33847: a rising running maximum rescales the
// accumulator by exp(old_max - new_max) and must not flush it to zero).
//
// gfx950 design.  A workgroup (4 waves) owns one (row, KV head g, key split).
// Each wave walks 32-key tiles of the split's selected-index list.  The
// logits are formed transposed, S^T = K . Q^T, with v_mfma_f32_16x16x32:
//   * A operand = K rows: lane c16 + 16 g4 holds quarter g4 (in a d <-> k-slot
//     permutation that is free because Q uses the same one) of the row of
//     key c16; the rows arrive by line-wide 16-byte loads staged through the
//     wave's LDS tile (or, for rows shorter than a line, by lane permutes);
//   * B operand = Q^T: the R <= 16 query heads of group g (zero-padded),
//     converted once to the MFMA type and kept in registers.
// S^T leaves each lane with 4 keys of one head, which is exactly the B
// operand layout of the next product, O^T = V^T . P^T: P never moves between
// lanes.  V^T needs keys along the k-slot, so the wave stages its 32 V rows
// in LDS and reads them back transposed.
// Numerics: FP32 accumulation everywhere; P enters the PV product as a
// hi/lo pair of 16-bit values (two MFMAs), keeping ~16 bits of each weight;
// INT8 codes enter the MFMAs exactly and their per-token scales are applied
// in FP32 (logit * k_scale, p * v_scale).  The online-softmax rescale keeps
// FP32 subnormals (exp_keep_subnormal).
// The 4 waves' (max, sum, O) states merge in LDS; with several key splits
// the workgroup writes an unnormalised partial and attn_merge_kernel
// combines the splits in a fixed order (deterministic).
#include <mutex>
#include <type_traits>

#include "dsa_device.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / kWave;
constexpr int kTile = 32;
// Running-maximum slack of the online softmax, in nats (see the tile loop).
constexpr float kLazyNats = 8.0f;

struct AttnParams {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* indices;
  const int32_t* kv_len;
  void* out;
  float* part;
  int S, H_q, H_kv, L_cap, k, ratio, out_dtype, nsplit, kps;
  float scale;
  int aux_tokens;     // cache keys at positions >= kv_len - aux_tokens are not attended
  int kvl_const;      // >= 0: use this live length for every sequence (aux keys)
  int write_partial;  // write (m, l, O) partials instead of the output
  int part_stride;    // splits per (row, head) in the partial buffer
  int part_offset;    // first split index of this launch
  int rows;           // B * S
};

// out[i .. i+3] = O / L (0 where L == 0), rounded to the output dtype.
__device__ __forceinline__ void store_out4(void* out, size_t i, f32x4 O, float L, int dt) {
  f32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = L > 0.0f ? O[e] / L : 0.0f;
  if (dt == kF32) {
    *reinterpret_cast<f32x4*>((float*)out + i) = r;
  } else if (dt == kF16) {
    typedef __attribute__((ext_vector_type(4))) _Float16 h4;
    h4 v = {(_Float16)r[0], (_Float16)r[1], (_Float16)r[2], (_Float16)r[3]};
    *reinterpret_cast<h4*>((_Float16*)out + i) = v;
  } else {
    typedef __attribute__((ext_vector_type(4))) __bf16 b4;
    b4 v = {(__bf16)r[0], (__bf16)r[1], (__bf16)r[2], (__bf16)r[3]};
    *reinterpret_cast<b4*>((__bf16*)out + i) = v;
  }
}

// Interleaved row load.  Quarter q (0..3) of a row is taken in chunks of E
// elements: element j = c*E + e of the result is row element (4c + q)*E + e.
// With E elements of the KV type per 16 bytes and the four quarters of a
// row in four consecutive lanes, one load instruction covers 64 contiguous
// bytes of each row it touches.  The QK dot product is unchanged by the
// permutation as long as query and key use the same one; values are
// written to LDS at their true positions.
template <typename T, int E, int N>
__device__ __forceinline__ void load_perm(const T* row, int q, T (&dst)[N]) {
  constexpr int CB = E * (int)sizeof(T);          // bytes per chunk: 8, 16 or 32
  static_assert(N % E == 0 && CB % 8 == 0, "whole chunks of 8-byte multiples");
#pragma unroll
  for (int c = 0; c < N / E; ++c) {
    const char* src = (const char*)(row + (4 * c + q) * E);
    if constexpr (CB == 8) {
      const uint2 v = ld_vec<uint2>(src);
      __builtin_memcpy(&dst[c * E], &v, 8);
    } else {
#pragma unroll
      for (int b = 0; b < CB / 16; ++b) {
        const uint4 v = ld_vec<uint4>(src + 16 * b);
        __builtin_memcpy(&dst[c * E + b * (16 / (int)sizeof(T))], &v, 16);
      }
    }
  }
}

// dst = src of lane `from` (per 32-bit word, through ds_bpermute).
template <typename T, int N>
__device__ __forceinline__ void lane_gather(const T (&src)[N], int from, T (&dst)[N]) {
  constexpr int NW = N * (int)sizeof(T) / 4;
  static_assert(NW * 4 == N * (int)sizeof(T), "whole 32-bit words");
  uint32_t w[NW];
  __builtin_memcpy(w, src, sizeof(w));
#pragma unroll
  for (int i = 0; i < NW; ++i) w[i] = (uint32_t)__builtin_amdgcn_ds_bpermute(from * 4, (int)w[i]);
  __builtin_memcpy(dst, w, sizeof(w));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// (i % 4) of the 8-byte chunks addressed by lanes i/4, 4 + i/4, 8 + i/4 and
// 12 + i/4 (in that order).  p must be 8-byte aligned.
template <typename T>
__device__ __forceinline__ s16x4 ds_read_tr16x4(const T* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(__attribute__((address_space(3))) void*)(p));
}

template <typename To, typename From>
__device__ __forceinline__ To cvt(From x) {
  if constexpr (std::is_same<To, From>::value) return x;
  else return from_f32<To>(to_f32(x));
}

template <int D, typename QT, typename KVT, typename MQK, typename MPV>
struct AttnCfg {
  // FP32 operands (v_mfma_f32_16x16x4_f32): the FP32 cache, and query /
  // auxiliary dtype pairs that no 16-bit type holds exactly.
  static constexpr bool kF32Path = std::is_same<MQK, float>::value;
  static constexpr bool kInt8 = std::is_same<KVT, int8_t>::value;
  static constexpr int kQuarter = D / 4;             // elements of a row per lane
  // Loads of K/V rows: coalesced (four consecutive lanes per row) with
  // 16-byte chunks, or, for INT8, a 32-byte quarter per lane in the MFMA
  // layout.  Elements per chunk of a lane (load_perm).
  static constexpr bool kCoalesced = !kInt8;
  static constexpr int kChunkElems = kInt8 ? kQuarter : 16 / (int)sizeof(KVT);
  static constexpr int kSteps = D / 32;              // QK K-steps (16-bit path)
  static constexpr int kDTiles = D / 16;             // O^T tiles of 16 dims
  // LDS row padding (elements).  16-bit rows are padded by 32 bytes so that
  // the 16 lanes of a transposing read (4 keys x 4 eight-byte chunks) hit
  // distinct banks.
  static constexpr int kVPad = kF32Path ? 4 : 16;
  static constexpr int kVStride = D + kVPad;
  static constexpr size_t kVBytes = (size_t)kAttnWaves * kTile * kVStride * sizeof(MPV);
  static constexpr size_t kSclBytes = kInt8 ? (size_t)kAttnWaves * 64 * sizeof(float) : 0;
  static constexpr int kOStride = D + 4;              // padded O^T row (floats) in the merge
  static constexpr size_t kMergeBytes =
      ((size_t)kAttnWaves * 16 * kOStride + 4 * kAttnWaves * 16 + 2 * 16) * sizeof(float);
  static constexpr size_t kLds =
      kVBytes + kSclBytes > kMergeBytes ? kVBytes + kSclBytes : kMergeBytes;
};

// DENSE: key slot j is key j (the auxiliary keys), no index list.
// INT8 caches run three waves per SIMD (at most 168 registers): measured
// faster there than two waves with wider prefetch.
// WAVE_ROWS (prefill with many rows, one key split): each wave owns a whole
// (row, KV head) and walks all of its tiles; workgroup j takes KV head
// j % H_kv and rows 4 (j / H_kv) + wave.  Consecutive workgroups land on
// consecutive XCDs, so with H_kv dividing 8 an XCD serves one KV head, and
// its rows, all started together and walking their index-ordered lists at
// one tile per step, read the same key region at the same time: the K/V
// rows that several query rows selected are reused from that XCD's L2.
// (With four waves sharing a row, a workgroup sweeps its list four times
// faster, the dispatch rounds start at different times, and the region read
// at once is larger than the L2.)  The waves never synchronise.
template <int D, typename QT, typename KVT, typename MQK, typename MPV, bool DENSE,
          bool WAVE_ROWS = false>
__global__ __launch_bounds__(kAttnThreads)
__attribute__((amdgpu_waves_per_eu(std::is_same<KVT, int8_t>::value ? 3 : 1)))
void attn_kernel(AttnParams p) {
  using Cfg = AttnCfg<D, QT, KVT, MQK, MPV>;
  constexpr int Q4 = Cfg::kQuarter;
  __shared__ __attribute__((aligned(16))) unsigned char smem[Cfg::kLds];
  static_assert(!(WAVE_ROWS && DENSE), "whole-row waves walk an index list");

  const int wave = threadIdx.x / kWave;
  int split, g, row;
  if constexpr (WAVE_ROWS) {
    split = 0;
    g = (int)(blockIdx.x % (unsigned)p.H_kv);
    row = (int)(blockIdx.x / (unsigned)p.H_kv) * kAttnWaves + wave;
    if (row >= p.rows) return;                 // no barrier follows in this form
  } else {
    split = blockIdx.x; g = blockIdx.y; row = blockIdx.z;
  }
  const int b = row / p.S, s = row % p.S;
  int kvl = p.kvl_const >= 0 ? p.kvl_const : p.kv_len[b];
  kvl = kvl < 0 ? 0 : (kvl > p.L_cap ? p.L_cap : kvl);
  const int pos = kvl - p.S + s;
  const int live = min(kvl - p.aux_tokens, pos + 1);   // valid key indices are [0, live)
  const int32_t* idx_row = DENSE ? nullptr : p.indices + (size_t)row * p.k;
  const int k0 = split * p.kps;
  const int k1 = min(p.k, k0 + p.kps);

  const int l = lane_id();
  const int g4 = l >> 4;        // lane group 0..3
  const int c16 = l & 15;       // head column / key row within a half tile
  // This lane's key-list entries of the wave's first tile, fetched right
  // away so that their latency overlaps the kv_len and query loads.
  // Tiles of the wave: every kAttnWaves-th of the split, or all of the row.
  constexpr int kStep = WAVE_ROWS ? kTile : kTile * kAttnWaves;   // keys between a wave's tiles
  const int t_first = WAVE_ROWS ? k0 : k0 + kTile * wave;
  int next_a = -1, next_b = -1;
  {
    const int ja = t_first + c16, jb = ja + 16;
    if (ja < k1) next_a = DENSE ? ja : idx_row[ja];
    if (jb < k1) next_b = DENSE ? jb : idx_row[jb];
  }
  const int R = p.ratio;
  const bool head_ok = c16 < R;
  const int h = g * R + (head_ok ? c16 : 0);

  const size_t kv_row_stride = (size_t)p.H_kv * D;                  // elements per token
  const KVT* kbase = (const KVT*)p.k_cache + (size_t)b * p.L_cap * kv_row_stride + (size_t)g * D;
  const KVT* vbase = (const KVT*)p.v_cache + (size_t)b * p.L_cap * kv_row_stride + (size_t)g * D;
  const float* ksc = Cfg::kInt8 ? p.k_scale + (size_t)b * p.L_cap * p.H_kv + g : nullptr;
  const float* vsc = Cfg::kInt8 ? p.v_scale + (size_t)b * p.L_cap * p.H_kv + g : nullptr;

  // ---- Q^T operand: lane holds head c16, dims [Q4*g4, Q4*g4 + Q4)
  QT qraw[Q4];
  {
    const QT* qrow = (const QT*)p.q + ((size_t)row * p.H_q + h) * D;
    load_perm<QT, Cfg::kChunkElems, Q4>(qrow, g4, qraw);
    if (!head_ok) {
#pragma unroll
      for (int i = 0; i < Q4; ++i) qraw[i] = cvt<QT>(0.0f);
    }
  }

  MPV* vt = (MPV*)smem + (size_t)wave * kTile * Cfg::kVStride;
  // INT8: per-key (softmax_scale * k_scale) for the 32 keys, then v_scale.
  float* scl = (float*)(smem + Cfg::kVBytes) + wave * 64;
  float m_run = -INFINITY;
  float l_run = 0.0f;
  f32x4 o[Cfg::kDTiles];
#pragma unroll
  for (int dt = 0; dt < Cfg::kDTiles; ++dt) o[dt] = f32x4{};

  // K rows of a tile are loaded one tile ahead of their use: the K rows
  // (and INT8 scales) of the wave's next tile are requested before the
  // current tile is computed, and the index-list entries two tiles ahead.
  // V rows are requested when their tile starts; they are first needed
  // after the QK product and the softmax, which cover their latency.
  // Rows whose length is a whole number of 128-byte lines (16-bit and
  // INT8 at D 128, 16-bit at D 64) are read a line per eight lanes (see
  // below).  Otherwise K and V rows are loaded coalesced: lane l reads row
  // l/4 of each half tile, chunks 4c + l%4, so four consecutive lanes cover
  // 64 contiguous bytes of one row (rows themselves are scattered), and K
  // moves into the MFMA layout -- lane c16 + 16 g4 holds chunks 4c + g4 of
  // row c16, which load lane 4 c16 + g4 read -- by lane permutes; INT8 rows
  // of 64 bytes keep the MFMA layout for the loads: lane c16 + 16 g4 reads
  // the quarter g4 of row c16.
  constexpr bool kCoal = Cfg::kCoalesced;
  constexpr int E = Cfg::kChunkElems;
  const int lrow = kCoal ? l >> 2 : c16, lq = kCoal ? l & 3 : g4;
  // 16-bit V rows that go to LDS unconverted are read whole cache lines at a
  // time: eight consecutive lanes cover 128 contiguous bytes of one row, so
  // an instruction touches 8 lines instead of 16 half lines.  Instruction k
  // of a half tile covers rows 8 (k / LPR) + l / 8, bytes 128 (k % LPR) +
  // 16 (l % 8) (LPR: 128-byte lines per row).
  // INT8 rows of 128 bytes are read the same way and converted on the way
  // to LDS.  16-bit K rows are read the same way too and pass through the
  // wave's LDS tile into the MFMA layout (instead of lane permutes), and so
  // are INT8 K rows of 128 bytes.
  constexpr int kRowBytes = D * (int)sizeof(KVT);
  constexpr bool kVLines = kRowBytes % 128 == 0 &&
      ((kCoal && sizeof(KVT) == 2 && std::is_same<MPV, KVT>::value) || Cfg::kInt8);
  constexpr bool kKLines = kRowBytes % 128 == 0 &&
      ((kCoal && sizeof(KVT) == 2 && !Cfg::kF32Path) || Cfg::kInt8);
  constexpr int kLPR = kRowBytes / 128 > 0 ? kRowBytes / 128 : 1;
  constexpr int kVI = 16 * kRowBytes / 1024;    // 16-byte loads per lane per half tile
  // Row (of half tile h) and byte offset within it of this lane's load k.
  auto line_row = [&](int h, int k) { return 16 * h + 8 * (k / kLPR) + (l >> 3); };
  auto line_off = [&](int k) { return 128 * (k % kLPR) + 16 * (l & 7); };
  struct TileRegs {
    KVT k0[Q4], k1[Q4];                   // K rows of half tiles a and b, as loaded
    int ra, rb;                           // the rows this lane loads (-1: none)
    float sc;                             // INT8: this lane's k or v scale
  };
  // Row of entry e as loaded by this lane, clamped to a valid row.
  auto load_row = [&](int e) { return kCoal ? __shfl(e, lrow, kWave) : e; };
  // Request the K rows of the tile whose entries (this lane's rows c16 and
  // c16 + 16) are ia, ib.
  auto issue = [&](int ia, int ib, TileRegs& r) {
    const int ia_l = load_row(ia), ib_l = load_row(ib);
    r.ra = ia_l >= 0 && ia_l < live ? ia_l : 0;
    r.rb = ib_l >= 0 && ib_l < live ? ib_l : 0;
    if constexpr (kKLines) {
      static_assert(kVI * 16 == Q4 * (int)sizeof(KVT), "a half tile's lines fill k0 / k1");
      u32x4 kl[2 * kVI];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int k = 0; k < kVI; ++k) {
          const int e = __shfl(h == 0 ? ia : ib, line_row(0, k), kWave);
          const int row = e >= 0 && e < live ? e : 0;
          kl[h * kVI + k] = ld_vec<u32x4>((const char*)(kbase + (size_t)row * kv_row_stride) +
                                          line_off(k));
        }
      }
      __builtin_memcpy(r.k0, &kl[0], sizeof(r.k0));
      __builtin_memcpy(r.k1, &kl[kVI], sizeof(r.k1));
    } else {
      load_perm<KVT, E, Q4>(kbase + (size_t)r.ra * kv_row_stride, lq, r.k0);
      load_perm<KVT, E, Q4>(kbase + (size_t)r.rb * kv_row_stride, lq, r.k1);
    }
    // INT8: lane l fetches one scale of key (l % 32): k_scale for l < 32,
    // v_scale above (lane l holds that key's index as ia or ib).
    r.sc = 0.0f;
    if constexpr (Cfg::kInt8) {
      const int si = (l & 16) ? ib : ia;
      const bool sok = si >= 0 && si < live;
      const float* sp = (l < 32) ? ksc : vsc;
      if (sok) r.sc = sp[(size_t)si * p.H_kv];
    }
  };
  // Compute one tile from its entries and loaded rows.
  auto compute = [&](int ia, int ib, const TileRegs& r) {
    const bool va = ia >= 0 && ia < live;
    const bool vb = ib >= 0 && ib < live;
    KVT vra[kVLines ? 1 : Q4], vrb[kVLines ? 1 : Q4];
    u32x4 vline[kVLines ? 2 * kVI : 1];
    if constexpr (kVLines) {
      static_assert(kRowBytes % 128 == 0 && kVI * 1024 == 16 * kRowBytes, "whole lines per row");
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int k = 0; k < kVI; ++k) {
          const int e = __shfl(h == 0 ? ia : ib, 8 * (k / kLPR) + (l >> 3), kWave);
          const int row = e >= 0 && e < live ? e : 0;
          vline[h * kVI + k] = ld_vec<u32x4>((const char*)(vbase + (size_t)row * kv_row_stride) +
                                             128 * (k % kLPR) + 16 * (l & 7));
        }
      }
    } else {
      load_perm<KVT, E, Q4>(vbase + (size_t)r.ra * kv_row_stride, lq, vra);
      load_perm<KVT, E, Q4>(vbase + (size_t)r.rb * kv_row_stride, lq, vrb);
    }
    KVT kra[Q4], krb[Q4];
    if constexpr (kKLines) {
      // lines -> rows of the wave's LDS tile -> lane c16 + 16 g4 reads the
      // chunks c of E elements at dims (4 c + g4) E of row c16 (half a) and
      // 16 + c16 (half b): the MFMA A layout, in the D order the query was
      // loaded in
      char* tile = reinterpret_cast<char*>(vt);
      constexpr int kRS = Cfg::kVStride * (int)sizeof(MPV);     // tile row stride, bytes
      static_assert(kRS >= kRowBytes, "K rows fit the tile's rows");
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int k = 0; k < kVI; ++k) {
          u32x4 w;
          __builtin_memcpy(&w, (h == 0 ? (const char*)r.k0 : (const char*)r.k1) + 16 * k, 16);
          *reinterpret_cast<u32x4*>(tile + line_row(h, k) * kRS + line_off(k)) = w;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      constexpr int kCB = E * (int)sizeof(KVT);             // chunk bytes: 16 or 32
      static_assert(kCB % 16 == 0, "chunks of whole 16-byte reads");
#pragma unroll
      for (int c = 0; c < Q4 / E; ++c) {
#pragma unroll
        for (int b = 0; b < kCB / 16; ++b) {
          const int off = (4 * c + g4) * kCB + 16 * b;
          const u32x4 wa = *reinterpret_cast<const u32x4*>(tile + c16 * kRS + off);
          const u32x4 wb = *reinterpret_cast<const u32x4*>(tile + (16 + c16) * kRS + off);
          __builtin_memcpy(&kra[c * E + b * (16 / (int)sizeof(KVT))], &wa, 16);
          __builtin_memcpy(&krb[c * E + b * (16 / (int)sizeof(KVT))], &wb, 16);
        }
      }
      // the V rows reuse the tile: every K read of this wave is done first
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else if constexpr (kCoal) {
      lane_gather(r.k0, 4 * c16 + g4, kra);
      lane_gather(r.k1, 4 * c16 + g4, krb);
    } else {
#pragma unroll
      for (int i = 0; i < Q4; ++i) { kra[i] = r.k0[i]; krb[i] = r.k1[i]; }
    }
    const float my_scale = r.sc;
    // Validity of keys 4*g4 + i (half a) and 16 + 4*g4 + i (half b): lanes
    // 0..15 hold rows 0..15 of each half.
    const uint32_t bits_a = ((uint32_t)__ballot(va) >> (4 * g4)) & 0xFu;
    const uint32_t bits_b = ((uint32_t)__ballot(vb) >> (4 * g4)) & 0xFu;

    // ---- S^T = K . Q^T for both halves
    f32x4 sa = f32x4{}, sb = f32x4{};
    if constexpr (Cfg::kF32Path) {
#pragma unroll
      for (int j = 0; j < Q4; ++j) {
        sa = mfma16x16x4((float)kra[j], (float)qraw[j], sa);
        sb = mfma16x16x4((float)krb[j], (float)qraw[j], sb);
      }
    } else {
      using V8 = typename vec8<MQK>::type;
#pragma unroll
      for (int st = 0; st < Cfg::kSteps; ++st) {
        V8 qa, ka, kb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          qa[e] = cvt<MQK>(qraw[8 * st + e]);
          ka[e] = cvt<MQK>(kra[8 * st + e]);
          kb[e] = cvt<MQK>(krb[8 * st + e]);
        }
        sa = mfma16x16x32(ka, qa, sa);
        sb = mfma16x16x32(kb, qa, sb);
      }
    }

    // ---- V rows into this wave's LDS tile (converted to the PV operand type)
    if constexpr (kVLines) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int k = 0; k < kVI; ++k) {
          constexpr int kEl = 16 / (int)sizeof(KVT);   // elements per 16-byte load
          MPV* dst = vt + (size_t)(16 * h + 8 * (k / kLPR) + (l >> 3)) * Cfg::kVStride +
                     (128 * (k % kLPR) + 16 * (l & 7)) / (int)sizeof(KVT);
          if constexpr (std::is_same<MPV, KVT>::value) {
            *reinterpret_cast<u32x4*>(dst) = vline[h * kVI + k];
          } else {
            KVT raw[kEl];
            __builtin_memcpy(raw, &vline[h * kVI + k], 16);
            MPV cv[kEl];
#pragma unroll
            for (int i = 0; i < kEl; ++i) cv[i] = cvt<MPV>(raw[i]);
#pragma unroll
            for (int i = 0; i < kEl * (int)sizeof(MPV) / 16; ++i) {
              u32x4 w;
              __builtin_memcpy(&w, &cv[i * 16 / (int)sizeof(MPV)], 16);
              reinterpret_cast<u32x4*>(dst)[i] = w;
            }
          }
        }
      }
    } else {
      MPV va_c[Q4], vb_c[Q4];
#pragma unroll
      for (int i = 0; i < Q4; ++i) { va_c[i] = cvt<MPV>(vra[i]); vb_c[i] = cvt<MPV>(vrb[i]); }
      // chunk c of this lane goes to dims (4c + lq)*E .. +E of its key rows
      constexpr int NV = E * (int)sizeof(MPV) / 16;   // 16-byte stores per chunk
      static_assert(NV * 16 == E * (int)sizeof(MPV), "chunks of whole 16-byte stores");
      MPV* ra = vt + (size_t)lrow * Cfg::kVStride + lq * E;
      MPV* rb = vt + (size_t)(16 + lrow) * Cfg::kVStride + lq * E;
#pragma unroll
      for (int c = 0; c < Q4 / E; ++c) {
        uint4 ta[NV], tb[NV];
        __builtin_memcpy(ta, &va_c[c * E], sizeof(ta));
        __builtin_memcpy(tb, &vb_c[c * E], sizeof(tb));
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          reinterpret_cast<uint4*>(ra + 4 * c * E)[i] = ta[i];
          reinterpret_cast<uint4*>(rb + 4 * c * E)[i] = tb[i];
        }
      }
    }
    if constexpr (Cfg::kInt8) scl[l] = (l < 32) ? my_scale * p.scale : my_scale;
    // This wave's LDS writes must land before its reads below.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- logits of keys 4*g4+i (half a) and 16+4*g4+i (half b), head c16
    float x[8];
    f32x4 vs_a, vs_b;
    if constexpr (Cfg::kInt8) {
      const f32x4 ks_a = *reinterpret_cast<const f32x4*>(scl + 4 * g4);
      const f32x4 ks_b = *reinterpret_cast<const f32x4*>(scl + 16 + 4 * g4);
      vs_a = *reinterpret_cast<const f32x4*>(scl + 32 + 4 * g4);
      vs_b = *reinterpret_cast<const f32x4*>(scl + 48 + 4 * g4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = ((bits_a >> i) & 1u) ? sa[i] * ks_a[i] : -INFINITY;
        x[4 + i] = ((bits_b >> i) & 1u) ? sb[i] * ks_b[i] : -INFINITY;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = ((bits_a >> i) & 1u) ? sa[i] * p.scale : -INFINITY;
        x[4 + i] = ((bits_b >> i) & 1u) ? sb[i] * p.scale : -INFINITY;
      }
    }

    // ---- online softmax per head column (lanes c16, c16+16, c16+32, c16+48).
    // The reference maximum only moves when a tile's maximum exceeds it by
    // more than kLazyNats, so most tiles skip the O rescale; weights are
    // then at most e^kLazyNats, and the final O / L is unchanged.
    float tmax = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                       fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    const bool grow = tmax > m_run + kLazyNats;      // also the first valid key (m_run = -inf)
    if (__ballot(grow) != 0) {                       // wave-uniform branch
      const float m_new = grow ? tmax : m_run;
      const float alpha = (m_run == -INFINITY) ? 0.0f : exp_keep_subnormal(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < Cfg::kDTiles; ++dt) o[dt] *= alpha;
      m_run = m_new;
    }
    float pv[8];
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pv[i] = (x[i] == -INFINITY) ? 0.0f : exp_keep_subnormal(x[i] - m_run);
      psum += pv[i];
    }
    l_run += psum;
    if constexpr (Cfg::kInt8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) { pv[i] *= vs_a[i]; pv[4 + i] *= vs_b[i]; }
    }

    // ---- O^T += V^T . P^T
    if constexpr (Cfg::kF32Path) {
#pragma unroll
      for (int dt = 0; dt < Cfg::kDTiles; ++dt) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int key = (j < 4) ? (4 * g4 + j) : (16 + 4 * g4 + j - 4);
          const float a = (float)vt[(size_t)key * Cfg::kVStride + 16 * dt + c16];
          o[dt] = mfma16x16x4(a, pv[j], o[dt]);
        }
      }
    } else {
      using V8 = typename vec8<MPV>::type;
      V8 phi, plo;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const MPV hi = from_f32<MPV>(pv[j]);
        phi[j] = hi;
        plo[j] = from_f32<MPV>(pv[j] - to_f32(hi));
      }
      // A operand (V^T, dims x keys) by transposing LDS reads: lane
      // 16*g4 + 4*e + c addresses dims [4c, 4c+4) of key 4*g4 + e, and the
      // read hands lane 16*g4 + n the dim-n element of keys 4*g4 + 0..3.
      const MPV* tr_a = vt + (size_t)(4 * g4 + (c16 >> 2)) * Cfg::kVStride + 4 * (c16 & 3);
      const MPV* tr_b = tr_a + 16 * Cfg::kVStride;
#pragma unroll
      for (int dt = 0; dt < Cfg::kDTiles; ++dt) {
        const s16x4 lo = ds_read_tr16x4(tr_a + 16 * dt);
        const s16x4 hi = ds_read_tr16x4(tr_b + 16 * dt);
        const V8 a = __builtin_bit_cast(V8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[dt] = mfma16x16x32(a, phi, o[dt]);
        o[dt] = mfma16x16x32(a, plo, o[dt]);
      }
    }
    // Reads of this tile must finish before the next tile overwrites the LDS.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  auto entry = [&](int j) { return j < k1 ? (DENSE ? j : idx_row[j]) : -1; };
  int ia = next_a, ib = next_b;                 // this tile's entries
  int na = entry(t_first + kStep + c16), nb = entry(t_first + kStep + 16 + c16);
  TileRegs ra, rb;
  if constexpr (Cfg::kF32Path || Cfg::kInt8) {
    // One register set, loaded right before use: FP32 rows are twice as
    // wide, and a second set would cost INT8 a wave per SIMD (3 -> 2),
    // measured 7% slower on the batched INT8 decode.
    for (int t0 = t_first; t0 < k1; t0 += kStep) {
      issue(ia, ib, ra);
      const int fa = entry(t0 + 2 * kStep + c16), fb = entry(t0 + 2 * kStep + 16 + c16);
      compute(ia, ib, ra);
      ia = na; ib = nb; na = fa; nb = fb;
    }
  } else {
  if (t_first < k1) issue(ia, ib, ra);
  // Two tiles per trip, the register sets swapping roles.
  for (int t0 = t_first; t0 < k1; t0 += 2 * kStep) {
    if (t0 + kStep < k1) issue(na, nb, rb);
    int fa = entry(t0 + 2 * kStep + c16), fb = entry(t0 + 2 * kStep + 16 + c16);
    compute(ia, ib, ra);
    ia = na; ib = nb; na = fa; nb = fb;
    if (t0 + kStep >= k1) break;
    if (t0 + 2 * kStep < k1) issue(na, nb, ra);
    fa = entry(t0 + 3 * kStep + c16); fb = entry(t0 + 3 * kStep + 16 + c16);
    compute(ia, ib, rb);
    ia = na; ib = nb; na = fa; nb = fb;
  }
  }

  float l_col = l_run + __shfl_xor(l_run, 16, kWave);
  l_col += __shfl_xor(l_col, 32, kWave);
  if constexpr (WAVE_ROWS) {
    // The wave's state is the row's: lane c16 + 16 g4 holds dims
    // 16 dt + 4 g4 + [0, 4) of head c16 (the O^T accumulator layout).
    if (c16 < R) {
      const size_t hrow = (size_t)row * p.H_q + g * R + c16;
      if (!p.write_partial) {
#pragma unroll
        for (int dt = 0; dt < Cfg::kDTiles; ++dt)
          store_out4(p.out, hrow * D + 16 * dt + 4 * g4, o[dt], l_col, p.out_dtype);
      } else {
        const size_t slot = hrow * p.part_stride + p.part_offset + split;
        float* po = p.part + (size_t)2 * p.rows * p.H_q * p.part_stride;
#pragma unroll
        for (int dt = 0; dt < Cfg::kDTiles; ++dt)
          *reinterpret_cast<f32x4*>(&po[slot * D + 16 * dt + 4 * g4]) = o[dt];
        if (g4 == 0) {
          p.part[slot * 2 + 0] = m_run;
          p.part[slot * 2 + 1] = l_col;
        }
      }
    }
    return;
  }
  // ---- merge the 4 waves' states in LDS
  __syncthreads();
  constexpr int OS = Cfg::kOStride;
  float* ob = (float*)smem;                                  // [waves][16][OS]
  float* mb = ob + kAttnWaves * 16 * OS;                     // [waves][16]
  float* lb = mb + kAttnWaves * 16;                          // [waves][16]
  float* fb = lb + kAttnWaves * 16;                          // [waves][16] rescale factors
  float* hb = fb + kAttnWaves * 16;                          // [16] L, [16] M
  if (g4 == 0) {
    mb[wave * 16 + c16] = m_run;
    lb[wave * 16 + c16] = l_col;
  }
#pragma unroll
  for (int dt = 0; dt < Cfg::kDTiles; ++dt)
    *reinterpret_cast<f32x4*>(&ob[((size_t)wave * 16 + c16) * OS + 16 * dt + 4 * g4]) = o[dt];
  __syncthreads();
  if (threadIdx.x < 16) {
    const int n = threadIdx.x;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, mb[w * 16 + n]);
    float L = 0.0f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      const float mw = mb[w * 16 + n];
      const float f = (mw == -INFINITY) ? 0.0f : exp_keep_subnormal(mw - M);
      fb[w * 16 + n] = f;
      L += f * lb[w * 16 + n];
    }
    hb[n] = L;
    hb[16 + n] = M;
  }
  __syncthreads();
  constexpr int C4 = D / 4;
  for (int e = threadIdx.x; e < R * C4; e += kAttnThreads) {
    const int n = e / C4, c = e % C4;
    f32x4 O = f32x4{};
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w)
      O += fb[w * 16 + n] * *reinterpret_cast<const f32x4*>(&ob[((size_t)w * 16 + n) * OS + 4 * c]);
    const float L = hb[n];
    const size_t hrow = (size_t)row * p.H_q + g * R + n;
    if (!p.write_partial) {
      store_out4(p.out, hrow * D + 4 * c, O, L, p.out_dtype);
    } else {
      const size_t slot = hrow * p.part_stride + p.part_offset + split;
      float* pml = p.part;
      float* po = p.part + (size_t)2 * p.rows * p.H_q * p.part_stride;
      *reinterpret_cast<f32x4*>(&po[slot * D + 4 * c]) = O;
      if (c == 0) {
        pml[slot * 2 + 0] = hb[16 + n];
        pml[slot * 2 + 1] = L;
      }
    }
  }
}

// Combine the key splits of one (row, head) in a fixed order (deterministic).
// Thread t owns a float4 column chunk (t % (D/4)) and the splits
// t / (D/4), + G, + 2G, ... (G = 256 / (D/4)).  Lane i of every wave also
// reads split i's (m, l) (at most 64 splits: one per lane), so all loads go
// out together and the kernel waits on one round of memory latency.  Each
// wave forms the maximum, the factors and L with lane shuffles (no LDS),
// and the G partial sums meet in LDS behind a single barrier.  The sums run
// in the same order in every wave, so the result does not depend on timing.
constexpr int kMergeThreads = 256;
constexpr int kMaxSplits = 64;
constexpr long long kWaveRowsMinPairs = 2LL * 256 * kAttnWaves;
static_assert(kMaxSplits <= kWave, "one split per lane");

template <int D>
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(
    const float* __restrict__ part, int rows_h, int nsplit, void* out, int out_dtype) {
  constexpr int C4 = D / 4;                 // float4 chunks per row
  constexpr int G = kMergeThreads / C4;     // split groups
  constexpr int Q = kMaxSplits / G;         // splits per thread at most
  __shared__ __attribute__((aligned(16))) float4 acc[G][C4];
  const int hrow = blockIdx.x, t = threadIdx.x, lane = lane_id();
  const float2* pml = reinterpret_cast<const float2*>(part) + (size_t)hrow * nsplit;
  const float4* po = (const float4*)(part + (size_t)2 * rows_h * nsplit) + (size_t)hrow * nsplit * C4;
  const int c = t % C4, g = t / C4;
  float4 ov[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int sp = g + q * G;
    ov[q] = sp < nsplit ? po[(size_t)sp * C4 + c] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const float2 ml = lane < nsplit ? pml[lane] : make_float2(-INFINITY, 0.0f);
  float M = ml.x;
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, kWave));
  const float f = (ml.x == -INFINITY) ? 0.0f : exp_keep_subnormal(ml.x - M);
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const float fq = __shfl(f, g + q * G, kWave);   // 0 for splits >= nsplit
    o.x += fq * ov[q].x; o.y += fq * ov[q].y; o.z += fq * ov[q].z; o.w += fq * ov[q].w;
  }
  // L = sum of f * l over the splits (a fixed butterfly, all lanes active)
  float L = f * ml.y;
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) L += __shfl_xor(L, off, kWave);
  acc[g][c] = o;
  __syncthreads();
  if (t < C4) {
    float4 r = acc[0][t];
#pragma unroll
    for (int q = 1; q < G; ++q) {
      const float4 v = acc[q][t];
      r.x += v.x; r.y += v.y; r.z += v.z; r.w += v.w;
    }
    store_out4(out, (size_t)hrow * D + 4 * t, f32x4{r.x, r.y, r.z, r.w}, L, out_dtype);
  }
}

AttnParams base_params(const AttnLaunch& a) {
  AttnParams p;
  p.q = a.q; p.k_cache = a.k_cache; p.v_cache = a.v_cache;
  p.k_scale = a.k_scale; p.v_scale = a.v_scale;
  p.indices = a.indices; p.kv_len = a.kv_len; p.out = a.out; p.part = a.part;
  p.S = a.S; p.H_q = a.H_q; p.H_kv = a.H_kv; p.L_cap = a.L_cap; p.k = a.k;
  p.ratio = a.H_q / a.H_kv; p.out_dtype = a.out_dtype;
  p.nsplit = a.nsplit; p.kps = a.keys_per_split; p.scale = a.scale;
  p.aux_tokens = a.aux_len; p.kvl_const = -1;
  p.write_partial = a.nsplit > 1 || a.aux_len > 0;
  p.part_stride = a.nsplit + (a.aux_len > 0 ? 1 : 0);
  p.part_offset = 0;
  p.rows = a.B * a.S;
  return p;
}

template <int D, typename QT, typename KVT, typename MQK, typename MPV, bool DENSE = false>
void launch_kernel(const AttnParams& p, int nsplit, int H_kv, int rows, hipStream_t st,
                   bool wave_rows = false) {
  if constexpr (!DENSE) {
    if (wave_rows) {
      const dim3 grid((unsigned)(H_kv * ((rows + kAttnWaves - 1) / kAttnWaves)));
      hipLaunchKernelGGL((attn_kernel<D, QT, KVT, MQK, MPV, false, true>), grid,
                         dim3(kAttnThreads), 0, st, p);
      return;
    }
  }
  dim3 grid(nsplit, H_kv, rows);
  hipLaunchKernelGGL((attn_kernel<D, QT, KVT, MQK, MPV, DENSE>), grid, dim3(kAttnThreads), 0, st,
                     p);
}

// Main launch over the selected cache keys.
template <int D>
void launch_main(const AttnLaunch& a, const AttnParams& p, hipStream_t st) {
  typedef _Float16 H;
  typedef __bf16 BH;
  const int rows = a.B * a.S;
  const bool wr = a.wave_rows != 0;
  if (a.kv_dtype == kF32) { launch_kernel<D, float, float, float, float>(p, a.nsplit, a.H_kv, rows, st, wr); return; }
  if (a.q_dtype == kBF16) {
    if (a.kv_dtype == kF16) launch_kernel<D, BH, H, H, H>(p, a.nsplit, a.H_kv, rows, st, wr);
    else if (a.kv_dtype == kBF16) launch_kernel<D, BH, BH, BH, BH>(p, a.nsplit, a.H_kv, rows, st, wr);
    else launch_kernel<D, BH, int8_t, BH, BH>(p, a.nsplit, a.H_kv, rows, st, wr);
  } else {
    if (a.kv_dtype == kF16) launch_kernel<D, H, H, H, H>(p, a.nsplit, a.H_kv, rows, st, wr);
    else if (a.kv_dtype == kBF16) launch_kernel<D, H, BH, H, BH>(p, a.nsplit, a.H_kv, rows, st, wr);
    else launch_kernel<D, H, int8_t, H, BH>(p, a.nsplit, a.H_kv, rows, st, wr);
  }
}

// Auxiliary keys: every (row, KV head) attends its causal prefix of the S_aux
// fresh keys, one workgroup each, writing the last partial split.  The aux
// values keep their dtype: the products run in that 16-bit type when the
// query has it too (a BF16 query is taken to FP16 against FP16 aux, as
// against an FP16 cache), and in FP32 otherwise.
template <int D>
void launch_aux(const AttnLaunch& a, AttnParams p, hipStream_t st) {
  typedef _Float16 H;
  typedef __bf16 BH;
  p.k_cache = a.aux_k; p.v_cache = a.aux_v; p.k_scale = p.v_scale = nullptr;
  p.indices = nullptr; p.k = a.aux_len; p.kps = a.aux_len;
  p.L_cap = a.aux_len; p.kvl_const = a.aux_len; p.aux_tokens = 0;
  p.write_partial = 1; p.part_offset = a.nsplit;
  const int rows = a.B * a.S;
  if (a.q_dtype == kF32) { launch_kernel<D, float, float, float, float, true>(p, 1, a.H_kv, rows, st); return; }
  if (a.q_dtype == kBF16) {
    if (a.aux_dtype == kBF16) launch_kernel<D, BH, BH, BH, BH, true>(p, 1, a.H_kv, rows, st);
    else if (a.aux_dtype == kF16) launch_kernel<D, BH, H, H, H, true>(p, 1, a.H_kv, rows, st);
    else launch_kernel<D, BH, float, float, float, true>(p, 1, a.H_kv, rows, st);
  } else {
    if (a.aux_dtype == kF16) launch_kernel<D, H, H, H, H, true>(p, 1, a.H_kv, rows, st);
    else if (a.aux_dtype == kBF16) launch_kernel<D, H, BH, float, float, true>(p, 1, a.H_kv, rows, st);
    else launch_kernel<D, H, float, float, float, true>(p, 1, a.H_kv, rows, st);
  }
}

template <int D>
void launch_d(const AttnLaunch& a, hipStream_t st) {
  const AttnParams p = base_params(a);
  launch_main<D>(a, p, st);
  if (a.aux_len > 0) launch_aux<D>(a, p, st);
  if (p.write_partial) {
    hipLaunchKernelGGL((attn_merge_kernel<D>), dim3(a.B * a.S * a.H_q), dim3(kMergeThreads), 0, st,
                       (const float*)a.part, a.B * a.S * a.H_q, p.part_stride, a.out, a.out_dtype);
  }
}

}  // namespace

void plan_attention(AttnLaunch& a, bool decode) {
  // The merge combines at most 64 splits; auxiliary keys take one of them.
  const int max_split = a.aux_len > 0 ? 63 : 64;
  a.wave_rows = 0;
  if (!decode || a.k <= 0) {
    a.nsplit = 1;
    a.keys_per_split = a.k > 0 ? a.k : 1;
    // Whole-row waves once they fill a dispatch round (512 workgroups of 4
    // rows at two per CU); fewer rows keep four waves per row for latency.
    a.wave_rows = !decode && (long long)a.B * a.S * a.H_kv >= kWaveRowsMinPairs ? 1 : 0;
    return;
  }
  // Aim for ~3072 workgroups: a whole number of dispatch rounds whether the
  // kernel fits 2, 3 or 4 workgroups per CU (3072 = 256 CUs x 12), so no
  // round runs partly empty.  At least 128 keys (one tile per wave) per
  // split, whole 32-key tiles, at most 64 splits (one merge lane per split).
  const long long rows_kv = (long long)a.B * a.S * a.H_kv;
  long long kps = (a.k * rows_kv + 3071) / 3072;
  kps = ((kps + kTile - 1) / kTile) * kTile;
  if (kps < 128) kps = 128;
  long long ns = (a.k + kps - 1) / kps;
  // 16-bit caches at D = 128 fit two workgroups per CU and load each tile's
  // K rows one tile ahead (two register sets).  With one tile per wave, a
  // grid beyond two workgroups per CU runs a second dispatch round of
  // latency-bound workgroups; two tiles per wave (the second tile's loads
  // overlap the first's compute) in one round are faster there.  INT8 and
  // FP32 caches load each tile just before use and D = 64 fits more
  // workgroups per CU, so the rule is kept to the case it was measured on.
  constexpr long long kOneRound = 2LL * 256;      // 256 CUs
  const bool two_sets_d128 = (a.kv_dtype == kF16 || a.kv_dtype == kBF16) && a.D == 128;
  if (two_sets_d128 && kps == 128 && rows_kv * ns > kOneRound) {
    kps = 256;
    ns = (a.k + kps - 1) / kps;
  }
  if (ns > max_split) {
    ns = max_split;
    kps = (a.k + max_split - 1) / max_split;
    kps = ((kps + kTile - 1) / kTile) * kTile;
    ns = (a.k + kps - 1) / kps;
  }
  a.nsplit = (int)ns;
  a.keys_per_split = (int)kps;
}

// ---------------------------------------------------------------- built-in scratch
// Split partials of the allocation-free decode entry point: a file-scope
// device array (each GPU the library runs on holds its own copy, at its own
// address, until the process ends).  Host code never passes the array's
// name to a kernel: the device address comes from hipGetSymbolAddress, taken
// once per device with that device current.
static __device__ __align__(256) float scratch[kAttnScratchBytes / sizeof(float)];

float* attention_scratch(hipError_t* err) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess && (dev < 0 || dev >= kMaxDevices)) e = hipErrorInvalidDevice;
  if (e != hipSuccess) { *err = e; return nullptr; }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) { *err = e != hipSuccess ? e : hipErrorInvalidSymbol; return nullptr; }
    addr[dev] = p;
  }
  *err = hipSuccess;
  return static_cast<float*>(addr[dev]);
}

size_t attention_partials_bytes(const AttnLaunch& a) {
  const int splits = a.nsplit + (a.aux_len > 0 ? 1 : 0);
  if (splits <= 1) return 0;
  return (size_t)a.B * a.S * a.H_q * splits * (a.D + 2) * sizeof(float);
}

void launch_attention(const AttnLaunch& a, hipStream_t st) {
  if (a.B * a.S == 0) return;
  if (a.D == 64) launch_d<64>(a, st);
  else launch_d<128>(a, st);
}

}  // namespace dsa
