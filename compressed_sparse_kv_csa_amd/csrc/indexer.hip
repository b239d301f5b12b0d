// Lightning-indexer scoring and top-k selection for CSA decode.
//
// What is computed ("DeepSeek-V4 KV Cache 深度分析", section 四 "索引器（Indexer）机制" and
// the section 十一 forward-flow diagram): the query token's indexer query is scored
// against the indexer key of every compressed entry, and the top-k entries are kept.
// Score s_j = sum_h w_h * ReLU(q_h . k_j); ties are broken toward the smaller index.
//
// Two launches per call:
//   1. scan kernel, one persistent workgroup per CU.  A workgroup owns a run of
//      consecutive 2048-row slices of one query.  Its 8 waves stream 16-row key tiles
//      from HBM straight into registers through a 4-deep prefetch ring that runs on
//      across slice boundaries, so the next slice's loads are in flight while the
//      current slice is being selected.  Each tile is one [H_I x 128] x [128 x 16]
//      contraction on 16x16x32 MFMA with fp32 accumulation; ReLU, the head weights and
//      the head sum are applied to the accumulators and the scores stay in LDS.  Per
//      slice a radix select in LDS keeps the top-k, with the slice's top-P placed first.
//   2. merge kernel, one workgroup per query: selects the k-th largest key among the
//      top-P prefixes of all slices, and reads further into any slice whose whole
//      prefix lies above it (exact for any input).
// Selection keys are 64-bit: (order-preserving score bits << 32) | ~index, so a larger
// key means a higher score, then a lower index; all keys of a query are distinct.
//
// Precision.  bf16 keys meet bf16 queries on bf16 MFMA.  FP4 keys (E2M1 value times an
// E4M3 scale: at most 6 significant bits, within [2^-10, 2688]) are decoded exactly to
// fp16 and meet fp16 queries on fp16 MFMA.  Each query's indexer query is first scaled
// by a power of two that puts its largest magnitude in [2^14, 2^15); the scaling is
// exact and only multiplies every score of that query by the same positive factor.
// Elements below 2^-24 of that maximum lose bits in fp16; their effect is far below
// the fp32 accumulation error of the score.  Products are exact in fp32 either way.
#include "csakv_device.h"
#include "csakv_launch.h"

namespace csakv {

namespace {

constexpr int kIdxDim = 128;
constexpr int kScanWaves = 8;
constexpr int kScanThreads = kScanWaves * kWave;
constexpr int kRing = 4;   // tiles in flight per wave; divides slice_rows / (16 * kScanWaves)
constexpr int kMergeThreads = 1024;

// ------------------------------------------------------------------ block primitives

constexpr int kHistBins = 2048;  // 11-bit digits
constexpr int kListCap = 256;    // boundary-bin keys resolved by direct ranking

struct SelectSmem {
  uint32_t hist[kHistBins];
  uint64_t red[2 * 16];
  uint32_t wsum[16];
  uint32_t bc[8];
  uint64_t list[2][kListCap];
  uint32_t nlist[2];
  uint64_t res[2];
};

// Exclusive prefix sum of one value per thread over the block; *total gets the sum.
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  const uint32_t x = wave_incl_scan_add(v);
  if (lane == kWave - 1) wsum[w] = x;
  lds_barrier();
  uint32_t base = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    const uint32_t s = wsum[i];
    if (i < w) base += s;
    tot += s;
  }
  lds_barrier();
  *total = tot;
  return base + x - v;
}

// Minimum and maximum of the nonzero keys of the block (0 = absent).
template <class KeyAt>
__device__ void block_minmax(KeyAt key_at, int n, SelectSmem& sm, uint64_t* mn_out,
                             uint64_t* mx_out) {
  uint64_t mn = ~0ull, mx = 0ull;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const uint64_t k = key_at(i);
    if (k != 0ull) {
      mn = k < mn ? k : mn;
      mx = k > mx ? k : mx;
    }
  }
  wave_minmax_u64(mn, mx);
  const int w = threadIdx.x / kWave, nw = blockDim.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    sm.red[w] = mn;
    sm.red[16 + w] = mx;
  }
  lds_barrier();
  mn = ~0ull;
  mx = 0ull;
  for (int i = 0; i < nw; ++i) {
    mn = sm.red[i] < mn ? sm.red[i] : mn;
    mx = sm.red[16 + i] > mx ? sm.red[16 + i] : mx;
  }
  lds_barrier();
  *mn_out = mn;
  *mx_out = mx;
}

// Wave 0: digit holding the `remaining`-th largest key of a 256-bin histogram.
// bc = {digit, keys in higher digits, keys in the digit}.
__device__ void radix_pick_digit(const uint32_t* hist, uint32_t remaining, uint32_t* bc) {
  const int lane = threadIdx.x;
  uint32_t h[4];
  uint32_t tot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = hist[4 * lane + i];
    tot += h[i];
  }
  const uint32_t incl = wave_incl_scan_add(tot);
  const uint32_t all = (uint32_t)__builtin_amdgcn_readlane(incl, kWave - 1);
  uint32_t above = all - incl;  // keys in lanes above this one
#pragma unroll
  for (int i = 3; i >= 0; --i) {
    if (above < remaining && remaining <= above + h[i]) {
      bc[0] = 4 * lane + i;
      bc[1] = above;
      bc[2] = h[i];
    }
    above += h[i];
  }
}

// Threshold T such that exactly k of the nonzero keys are >= T (keys distinct apart
// from zeros, which are absent entries; 1 <= k <= number of nonzero keys).  General
// 8-bit radix passes from the common prefix of min and max, stopping as soon as a
// whole bin is needed.  Used for bins that hold too many keys to rank directly.
template <class KeyAt>
__device__ uint64_t block_kth_largest(KeyAt key_at, int n, int k, SelectSmem& sm, uint64_t mn,
                                      uint64_t mx) {
  if (mn == mx) return mn;
  const int hb = 63 - __builtin_clzll(mn ^ mx);
  int shift = hb + 1;
  uint64_t prefix = shift >= 64 ? 0ull : (mx & (~0ull << shift));
  uint32_t remaining = (uint32_t)k;
  while (true) {
    const int lo = shift > 8 ? shift - 8 : 0;
    const uint32_t dmask = (1u << (shift - lo)) - 1u;
    const uint64_t hi_mask = shift >= 64 ? 0ull : (~0ull << shift);
    for (int i = threadIdx.x; i < 256; i += blockDim.x) sm.hist[i] = 0;
    lds_barrier();
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const uint64_t key = key_at(i);
      if (key != 0ull && (key & hi_mask) == prefix)
        atomicAdd(&sm.hist[(uint32_t)(key >> lo) & dmask], 1u);
    }
    lds_barrier();
    if (threadIdx.x < kWave) radix_pick_digit(sm.hist, remaining, sm.bc);
    lds_barrier();
    const uint32_t d = sm.bc[0], above = sm.bc[1], cnt = sm.bc[2];
    lds_barrier();
    prefix |= (uint64_t)d << lo;
    remaining -= above;
    shift = lo;
    if (cnt == remaining || shift == 0) return prefix > 0 ? prefix : 1ull;
  }
}

// Thresholds for two ranks at once: *ta (*tb) is such that exactly ra (rb) of the
// nonzero keys are >= it.  Keys are distinct apart from zeros (absent); 1 <= ra, rb <=
// number of nonzero keys.  One histogram of the 11 bits below the common prefix of the
// keys' min and max places both ranks in a bin; a bin only partly needed is resolved by
// ranking its few keys directly (or by radix passes if it holds many).
template <class KeyAt>
__device__ void block_select2(KeyAt key_at, int n, int ra, int rb, SelectSmem& sm, uint64_t* ta,
                              uint64_t* tb) {
  uint64_t mn, mx;
  block_minmax(key_at, n, sm, &mn, &mx);
  if (mn == mx) {
    *ta = *tb = mn;
    return;
  }
  const int hb = 63 - __builtin_clzll(mn ^ mx);
  const int lo = hb + 1 > 11 ? hb + 1 - 11 : 0;
  const uint32_t dmask = (1u << (hb + 1 - lo)) - 1u;
  const uint64_t prefix = hb >= 63 ? 0ull : (mx & (~0ull << (hb + 1)));
  auto digit = [&](uint64_t key) -> uint32_t { return (uint32_t)(key >> lo) & dmask; };

  for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) sm.hist[i] = 0;
  if (threadIdx.x < 2) sm.nlist[threadIdx.x] = 0;
  lds_barrier();
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const uint64_t key = key_at(i);
    if (key != 0ull) atomicAdd(&sm.hist[digit(key)], 1u);
  }
  lds_barrier();
  const int bpt = kHistBins / blockDim.x;  // blockDim divides kHistBins
  const int b0 = threadIdx.x * bpt;
  uint32_t own = 0;
  for (int j = 0; j < bpt; ++j) own += sm.hist[b0 + j];
  uint32_t total;
  const uint32_t below = block_exclusive_scan(own, sm.wsum, &total);
  const uint32_t above = total - below - own;  // keys in bins >= b0 + bpt
  const uint32_t rr[2] = {(uint32_t)ra, (uint32_t)rb};
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    uint32_t a = above;
    if (a < rr[q] && rr[q] <= a + own) {
      for (int j = bpt - 1; j >= 0; --j) {
        const uint32_t h = sm.hist[b0 + j];
        if (a < rr[q] && rr[q] <= a + h) {
          sm.bc[2 * q] = b0 + j;
          sm.bc[2 * q + 1] = a;
        }
        a += h;
      }
    }
  }
  lds_barrier();
  uint64_t t[2];
  uint32_t bin[2], rem[2], cnt[2];
  bool need[2], small[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    bin[q] = sm.bc[2 * q];
    rem[q] = rr[q] - sm.bc[2 * q + 1];
    cnt[q] = sm.hist[bin[q]];
    t[q] = prefix | ((uint64_t)bin[q] << lo);
    if (t[q] == 0ull) t[q] = 1ull;  // never admit the absent (zero) keys
    need[q] = cnt[q] != rem[q];
    small[q] = cnt[q] <= (uint32_t)kListCap;
  }
  if (need[0] || need[1]) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const uint64_t key = key_at(i);
      if (key == 0ull) continue;
      const uint32_t d = digit(key);
#pragma unroll
      for (int q = 0; q < 2; ++q)
        if (need[q] && small[q] && d == bin[q]) sm.list[q][atomicAdd(&sm.nlist[q], 1u)] = key;
    }
    lds_barrier();
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (need[q] && small[q] && wave == q) {
        for (uint32_t i = lane; i < cnt[q]; i += kWave) {
          const uint64_t k = sm.list[q][i];
          uint32_t greater = 0;
          for (uint32_t j = 0; j < cnt[q]; ++j) greater += sm.list[q][j] > k;
          if (greater == rem[q] - 1) sm.res[q] = k;
        }
      }
    }
    lds_barrier();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (need[q] && small[q]) t[q] = sm.res[q];
    }
    lds_barrier();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (need[q] && !small[q]) {
        const uint32_t bq = bin[q];
        auto in_bin = [&](int i) -> uint64_t {
          const uint64_t key = key_at(i);
          return (key != 0ull && digit(key) == bq) ? key : 0ull;
        };
        uint64_t bmn, bmx;
        block_minmax(in_bin, n, sm, &bmn, &bmx);
        t[q] = block_kth_largest(in_bin, n, (int)rem[q], sm, bmn, bmx);
      }
    }
  }
  *ta = t[0];
  *tb = t[1];
}

__device__ __forceinline__ uint64_t compose_key(uint32_t score_key, uint32_t idx) {
  return ((uint64_t)score_key << 32) | (uint32_t)(~idx);
}
__device__ __forceinline__ int32_t key_index(uint64_t key) { return (int32_t)(~(uint32_t)key); }

// ------------------------------------------------------------------ key tiles

// Lane (g, n) owns row n of a 16-row tile and 32 of its 128 channels.

// bf16 rows: in K-step t the lane supplies channels 32t + 8g .. 32t + 8g + 7.
struct KeyTileBf16 {
  typedef bf16x8 Op;
  u32x4 c[4];
  static constexpr int kRowBytes = kIdxDim * 2;
  __device__ __forceinline__ void load(const uint8_t* codes, const uint8_t*, int row, int g) {
    const uint8_t* p = codes + row * kRowBytes + 16 * g;
#pragma unroll
    for (int t = 0; t < 4; ++t) c[t] = *reinterpret_cast<const u32x4*>(p + 64 * t);
  }
  __device__ __forceinline__ void decode(Op* op) const {
#pragma unroll
    for (int t = 0; t < 4; ++t) op[t] = as_bf16x8(c[t]);
  }
  static __device__ __forceinline__ int q_channel(int g, int t) { return 32 * t + 8 * g; }
  static __device__ __forceinline__ f32x4 mma(Op a, Op b, f32x4 c) { return mfma16x16x32(a, b, c); }
};

// FP4 rows: the lane loads channels 32g .. 32g + 31 (16 code bytes) and their two
// scales; in K-step t it supplies channels 32g + 8t .. 32g + 8t + 7 as exact fp16.
struct KeyTileFp4 {
  typedef f16x8 Op;
  u32x4 c;
  uint32_t s;  // the dword of scale bytes holding blocks 2g and 2g + 1
  int hi;      // 1 when those two bytes are the dword's upper half (odd g)
  static constexpr int kRowBytes = kIdxDim / 2;
  __device__ __forceinline__ void load(const uint8_t* codes, const uint8_t* scales, int row,
                                       int g) {
    c = *reinterpret_cast<const u32x4*>(codes + row * kRowBytes + 16 * g);
    s = *reinterpret_cast<const uint32_t*>(scales + row * (kIdxDim / 16) + 4 * (g >> 1));
    hi = g & 1;
  }
  __device__ __forceinline__ void decode(Op* op) const {
    // Both E4M3 scales as an fp16 pair (exact), then each broadcast to a pair.
    const uint32_t sp = __builtin_bit_cast(
        uint32_t, hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s, 1.0f, true)
                     : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s, 1.0f, false));
    const uint32_t s0 = __builtin_amdgcn_perm(sp, sp, 0x01000100u);
    const uint32_t s1 = __builtin_amdgcn_perm(sp, sp, 0x03020302u);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const f16x2 sc = __builtin_bit_cast(f16x2, t < 2 ? s0 : s1);
      u32x4 r;
      r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[t], 1.0f, 0) * sc);
      r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[t], 1.0f, 1) * sc);
      r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[t], 1.0f, 2) * sc);
      r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[t], 1.0f, 3) * sc);
      op[t] = as_f16x8(r);
    }
  }
  static __device__ __forceinline__ int q_channel(int g, int t) { return 32 * g + 8 * t; }
  static __device__ __forceinline__ f32x4 mma(Op a, Op b, f32x4 c) { return mfma16x16x32_f16(a, b, c); }
};

// Query fragment in the MMA operand type: 8 bf16 values as loaded, or as fp16 after
// scaling by 2^p.
__device__ __forceinline__ bf16x8 q_operand(u32x4 v, float, bf16x8*) { return as_bf16x8(v); }
__device__ __forceinline__ f16x8 q_operand(u32x4 v, float scale, f16x8*) {
  f16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[2 * i] = (_Float16)(bf16_to_f32(v[i] & 0xFFFFu) * scale);
    r[2 * i + 1] = (_Float16)(bf16_to_f32(v[i] >> 16) * scale);
  }
  return r;
}

// ------------------------------------------------------------------ scan kernel

template <class KT, int HT, int PS>
__global__ __launch_bounds__(kScanThreads) void indexer_scan_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t seq_stride,
    int64_t n_c, const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx, int n_heads,
    int top_k, int slice_rows, int n_slices, int slices_per_wg, int wg_per_query, int prefix,
    int cand_stride, uint64_t* __restrict__ cand) {
  typedef typename KT::Op Op;
  __shared__ uint32_t s_score[kMaxSliceRows];
  __shared__ SelectSmem sm;

  const int b = blockIdx.x / wg_per_query;
  const int slice0 = (blockIdx.x - b * wg_per_query) * slices_per_wg;
  const int n_sl = min(slices_per_wg, n_slices - slice0);
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int g = lane >> 4;
  const int n = lane & 15;
  const int64_t row_base = (int64_t)slice0 * slice_rows;              // compressed row index
  const int64_t rows_total = min((int64_t)n_sl * slice_rows, n_c - row_base);
  const int64_t seq_row0 = (int64_t)b * seq_stride + row_base;

  // Indexer query fragments (A operand, head n of each 16-head tile) and the weights of
  // the accumulator rows this lane holds (heads 16*ht + 4g + i).
  u32x4 qraw[HT][4];
  float qmax = 0.0f;
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int head = 16 * ht + n;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (head < n_heads)
        v = *reinterpret_cast<const u32x4*>(q_idx + ((int64_t)b * n_heads + head) * kIdxDim +
                                            KT::q_channel(g, t));
      qraw[ht][t] = v;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        qmax = fmaxf(qmax, fmaxf(fabsf(bf16_to_f32(v[i] & 0xFFFFu)), fabsf(bf16_to_f32(v[i] >> 16))));
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) qmax = fmaxf(qmax, __shfl_xor(qmax, off));
  // Power of two putting max|q| in [2^14, 2^15) (used by the fp16 path only).
  int p = 0;
  if (qmax > 0.0f) p = 14 - ((int)((__float_as_uint(qmax) >> 23) & 0xFF) - 127);
  p = max(-100, min(p, 100));
  const float qscale = __builtin_ldexpf(1.0f, p);
  Op qa[HT][4];
  float wv[HT][4];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
    for (int t = 0; t < 4; ++t) qa[ht][t] = q_operand(qraw[ht][t], qscale, (Op*)nullptr);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 16 * ht + 4 * g + i;
      wv[ht][i] = h < n_heads ? w_idx[(int64_t)b * n_heads + h] : 0.0f;
    }
  }

  // The wave's tile sequence: slot k -> slice k / per_slice, tile w + 8m of that slice.
  // Every slot loads (rows clamped into range) and computes, so the loads are straight-
  // line code and the ring keeps kRing tiles in flight; only valid rows store a score.
  // PS = tiles per wave per slice (slice_rows / (16 * kScanWaves)), a multiple of kRing;
  // the slice's tile loop is unrolled whole so the ring's waits are counted exactly.
  const int tiles_per_slice = PS * kScanWaves;
  const int per_slice = PS;
  const int total = n_sl * per_slice;
  auto slot_tile = [&](int k) -> int {
    const int j = k / per_slice, m = k - j * per_slice;
    return j * tiles_per_slice + wave + kScanWaves * m;
  };
  const int rows_last = (int)rows_total - 1;
  const uint8_t* kcodes = codes + seq_row0 * KT::kRowBytes;
  const uint8_t* kscales = scales ? scales + seq_row0 * (kIdxDim / 16) : nullptr;
  auto load_slot = [&](KT& kt, int k) {
    kt.load(kcodes, kscales, min(slot_tile(k) * 16 + n, rows_last), g);
  };

  KT ring[kRing];
#pragma unroll
  for (int d = 0; d < kRing; ++d) load_slot(ring[d], min(d, total - 1));

  for (int j = 0; j < n_sl; ++j) {
#pragma unroll
    for (int m = 0; m < PS; ++m) {
      {
        const int d = m % kRing;
        const int k = j * per_slice + m;
        Op kb[4];
        ring[d].decode(kb);
        load_slot(ring[d], min(k + kRing, total - 1));
        f32x4 acc[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int ht = 0; ht < HT; ++ht) acc[ht] = KT::mma(qa[ht][t], kb[t], acc[ht]);
        float sc = 0.0f;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
          for (int i = 0; i < 4; ++i) sc += wv[ht][i] * fmaxf(acc[ht][i], 0.0f);
        sc = wave_sum_rows(sc);
        const int tile = slot_tile(k);
        if (g == 0 && (int64_t)tile * 16 + n < rows_total)
          s_score[(tile - j * tiles_per_slice) * 16 + n] = f32_order_key(sc);
      }
    }

    // ---- slice j complete: keep its top-k1 with its top-P first
    const int64_t srow0 = row_base + (int64_t)j * slice_rows;
    const int rows = (int)min((int64_t)slice_rows, n_c - srow0);
    const int k1 = min(top_k, rows);
    const int pk = min(prefix, k1);
    lds_barrier();
    auto key_at = [&](int i) -> uint64_t { return compose_key(s_score[i], (uint32_t)(srow0 + i)); };
    uint64_t t_k, t_p;
    block_select2(key_at, rows, k1, pk, sm, &t_k, &t_p);
    const int chunk = (rows + kScanThreads - 1) / kScanThreads;
    const int p0 = threadIdx.x * chunk, p1 = min(p0 + chunk, rows);
    uint32_t ca = 0, cb = 0;
    for (int i = p0; i < p1; ++i) {
      const uint64_t key = key_at(i);
      ca += key >= t_p;
      cb += key >= t_k && key < t_p;
    }
    uint32_t tot;
    const uint32_t base = block_exclusive_scan((ca << 16) | cb, sm.wsum, &tot);
    uint32_t pa = base >> 16, pb = pk + (base & 0xFFFFu);
    uint64_t* dst = cand + ((int64_t)b * n_slices + slice0 + j) * cand_stride;
    for (int i = p0; i < p1; ++i) {
      const uint64_t key = key_at(i);
      if (key >= t_p) dst[pa++] = key;
      else if (key >= t_k) dst[pb++] = key;
    }
    lds_barrier();
  }
}

// ------------------------------------------------------------------ merge kernel

__global__ __launch_bounds__(kMergeThreads) void indexer_merge_kernel(
    const uint64_t* __restrict__ cand, int64_t n_c, int top_k, int slice_rows, int n_slices,
    int cand_stride, int prefix, int32_t* __restrict__ topk) {
  __shared__ uint64_t s_buf[kMergeCap];
  __shared__ uint64_t s_tmp[kMaxTopK];
  __shared__ SelectSmem sm;
  __shared__ int s_sat[kMaxMergeSlices];
  __shared__ int s_nsat;

  const int b = blockIdx.x;
  const int k1 = (int)min((int64_t)top_k, n_c);
  const uint64_t* cb = cand + (int64_t)b * n_slices * cand_stride;
  int32_t* out = topk + (int64_t)b * top_k;
  for (int i = k1 + threadIdx.x; i < top_k; i += blockDim.x) out[i] = -1;
  if (k1 == 0) return;

  auto slice_count = [&](int s) -> int {
    const int64_t r = min((int64_t)slice_rows, n_c - (int64_t)s * slice_rows);
    return (int)min((int64_t)top_k, r);
  };

  if (n_slices == 1) {  // the single slice holds exactly the top-k1
    for (int i = threadIdx.x; i < k1; i += blockDim.x) out[i] = key_index(cb[i]);
    return;
  }

  // Top-P prefix of every slice at stride `prefix`; missing entries are 0.
  int n_buf = n_slices * prefix;
  for (int i = threadIdx.x; i < n_buf; i += blockDim.x) {
    const int s = i / prefix, j = i - s * prefix;
    s_buf[i] = j < slice_count(s) ? cb[(int64_t)s * cand_stride + j] : 0ull;
  }
  if (threadIdx.x == 0) s_nsat = 0;
  lds_barrier();

  auto buf_at = [&](int i) -> uint64_t { return s_buf[i]; };
  uint64_t kth, unused;
  block_select2(buf_at, n_buf, k1, k1, sm, &kth, &unused);

  // A slice whose whole prefix is >= the k1-th key may hold more winners below it.
  for (int s = threadIdx.x; s < n_slices; s += blockDim.x) {
    const int cnt = slice_count(s);
    if (cnt <= prefix) continue;
    int ge = 0;
    for (int j = 0; j < prefix; ++j) ge += s_buf[s * prefix + j] >= kth;
    if (ge == prefix) s_sat[atomicAdd(&s_nsat, 1)] = s;
  }
  lds_barrier();
  const int n_sat = s_nsat;

  // Keep the k1 largest of s_buf[0..n) in s_buf[0..k1).
  auto compact_topk = [&](int n, uint64_t t) {
    const int chunk = (n + kMergeThreads - 1) / kMergeThreads;
    const int p0 = threadIdx.x * chunk, p1 = min(p0 + chunk, n);
    uint32_t c = 0;
    for (int p = p0; p < p1; ++p) c += s_buf[p] >= t;
    uint32_t total;
    uint32_t pos = block_exclusive_scan(c, sm.wsum, &total);
    for (int p = p0; p < p1; ++p)
      if (s_buf[p] >= t) s_tmp[pos++] = s_buf[p];
    lds_barrier();
    for (int i = threadIdx.x; i < k1; i += blockDim.x) s_buf[i] = s_tmp[i];
    lds_barrier();
  };

  if (n_sat > 0) {  // rare: stream the rest of each saturated slice, keeping keys > kth
    compact_topk(n_buf, kth);
    n_buf = k1;
    for (int si = 0; si < n_sat; ++si) {
      const int s = s_sat[si];
      const int cnt = slice_count(s);
      for (int j0 = prefix; j0 < cnt; j0 += kMergeCap - k1) {
        const int m = min(kMergeCap - k1, cnt - j0);
        for (int i = threadIdx.x; i < m; i += blockDim.x) {
          const uint64_t key = cb[(int64_t)s * cand_stride + j0 + i];
          s_buf[k1 + i] = key > kth ? key : 0ull;
        }
        lds_barrier();
        block_select2(buf_at, k1 + m, k1, k1, sm, &kth, &unused);
        compact_topk(k1 + m, kth);
      }
    }
  }

  // Write the selected indices in buffer order (deterministic).
  const int chunk = (n_buf + kMergeThreads - 1) / kMergeThreads;
  const int p0 = threadIdx.x * chunk, p1 = min(p0 + chunk, n_buf);
  uint32_t c = 0;
  for (int p = p0; p < p1; ++p) c += s_buf[p] >= kth;
  uint32_t total;
  uint32_t pos = block_exclusive_scan(c, sm.wsum, &total);
  for (int p = p0; p < p1; ++p)
    if (s_buf[p] >= kth) out[pos++] = key_index(s_buf[p]);
}

template <class KT, int HT>
void launch_scan(hipStream_t stream, const uint8_t* codes, const uint8_t* scales,
                 int64_t seq_stride, int64_t n_c, const uint16_t* q_idx, const float* w_idx,
                 int batch, int n_heads, int top_k, const IndexerPlan& plan, uint64_t* cand) {
#define CSAKV_SCAN_PS(PS)                                                                         \
  hipLaunchKernelGGL((indexer_scan_kernel<KT, HT, PS>), dim3(batch * plan.wg_per_query),          \
                     dim3(kScanThreads), 0, stream, codes, scales, seq_stride, n_c, q_idx, w_idx, \
                     n_heads, top_k, plan.slice_rows, plan.n_slices, plan.slices_per_wg,          \
                     plan.wg_per_query, plan.prefix, plan.cand_stride, cand)
  if (plan.slice_rows == 16 * kScanWaves * 16) CSAKV_SCAN_PS(16);
  else CSAKV_SCAN_PS(32);
#undef CSAKV_SCAN_PS
}

template <class KT>
void launch_scan_ht(int ht, hipStream_t stream, const uint8_t* codes, const uint8_t* scales,
                    int64_t seq_stride, int64_t n_c, const uint16_t* q_idx, const float* w_idx,
                    int batch, int n_heads, int top_k, const IndexerPlan& plan, uint64_t* cand) {
#define CSAKV_SCAN(H) \
  launch_scan<KT, H>(stream, codes, scales, seq_stride, n_c, q_idx, w_idx, batch, n_heads, top_k, plan, cand)
  switch (ht) {
    case 1: CSAKV_SCAN(1); break;
    case 2: CSAKV_SCAN(2); break;
    case 3: CSAKV_SCAN(3); break;
    default: CSAKV_SCAN(4); break;
  }
#undef CSAKV_SCAN
}

}  // namespace

IndexerPlan plan_indexer(int batch, int64_t n_c, int top_k) {
  IndexerPlan p{};
  // 2048-row slices (4096 for very long contexts, so the merge input stays bounded);
  // about one workgroup per CU (256), each owning a run of slices of one query.
  int64_t rows = 2048;
  if ((n_c + rows - 1) / rows > kMaxMergeSlices / 2) rows = kMaxSliceRows;
  p.slice_rows = (int)rows;
  p.n_slices = n_c > 0 ? (int)((n_c + rows - 1) / rows) : 0;
  p.cand_stride = (int)(top_k < rows ? top_k : rows);
  if (p.n_slices > 0) {
    int64_t wg = (256 + batch - 1) / batch;
    if (wg > p.n_slices) wg = p.n_slices;
    p.slices_per_wg = (int)((p.n_slices + wg - 1) / wg);
    p.wg_per_query = (p.n_slices + p.slices_per_wg - 1) / p.slices_per_wg;
  }
  const int per_slice = p.n_slices > 0 ? (top_k + p.n_slices - 1) / p.n_slices : top_k;
  int pre = 32;
  while (pre < 4 * per_slice) pre <<= 1;
  p.prefix = pre < p.cand_stride ? pre : p.cand_stride;
  return p;
}

size_t indexer_workspace_bytes(int batch, const IndexerPlan& plan) {
  return (size_t)batch * plan.n_slices * plan.cand_stride * sizeof(uint64_t);
}

bool indexer_supported(const IndexerPlan& plan) {
  return plan.n_slices <= kMaxMergeSlices && (int64_t)plan.n_slices * plan.prefix <= kMergeCap;
}

hipError_t launch_indexer(int key_fmt, const uint8_t* codes, const uint8_t* scales,
                          int64_t seq_stride, int64_t n_c, const uint16_t* q_idx,
                          const float* w_idx, int batch, int n_heads, int top_k,
                          const IndexerPlan& plan, void* workspace, int32_t* topk,
                          hipStream_t stream) {
  uint64_t* cand = static_cast<uint64_t*>(workspace);
  if (plan.n_slices > 0) {
    const int ht = (n_heads + 15) / 16;
    if (key_fmt == 0)
      launch_scan_ht<KeyTileBf16>(ht, stream, codes, scales, seq_stride, n_c, q_idx, w_idx, batch,
                                  n_heads, top_k, plan, cand);
    else
      launch_scan_ht<KeyTileFp4>(ht, stream, codes, scales, seq_stride, n_c, q_idx, w_idx, batch,
                                 n_heads, top_k, plan, cand);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(indexer_merge_kernel, dim3(batch), dim3(kMergeThreads), 0, stream, cand, n_c,
                     top_k, plan.slice_rows, plan.n_slices, plan.cand_stride, plan.prefix, topk);
  return hipGetLastError();
}

}  // namespace csakv
