// Block-wide top-k selection primitives of the indexer (histogram thresholds, exact k-th
// largest key, block scans) and the per-query merge of its slice candidates, as device
// functions templated on the block size.  Device code only; every definition lives in
// an unnamed namespace of the including translation unit.
#pragma once

#include "csakv_device.h"
#include "csakv_launch.h"

namespace csakv {

namespace {

// ------------------------------------------------------------------ block primitives

constexpr int kHistBins = 2048;  // 11-bit digits
constexpr int kListCap = 256;    // boundary-bin keys resolved by direct ranking (scan)
constexpr int kMergeListCap = 1024;  // the same in the merge

struct SelectSmem {
  uint32_t hist[kHistBins];
  uint64_t red[2 * 16];    // per-wave 64-bit minima / maxima
  uint32_t red32[2 * 16];  // per-wave 32-bit minima / maxima
  uint64_t res64[16];
  uint32_t wsum[16];
  uint32_t bc[8];
  uint64_t list[2][kListCap];
  uint32_t nlist[2];
  uint64_t res[2];
};

// Block primitives take the block size NT as a compile-time constant: reading blockDim
// would load it from the dispatch packet and wait for every outstanding memory load.

// Exclusive prefix sum of one value per thread over the block; *total gets the sum.
template <int NT>
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  constexpr int nw = NT / kWave;
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
template <int NT, class KeyAt>
__device__ void block_minmax(KeyAt key_at, int n, SelectSmem& sm, uint64_t* mn_out,
                             uint64_t* mx_out) {
  uint64_t mn = ~0ull, mx = 0ull;
  for (int i = threadIdx.x; i < n; i += NT) {
    const uint64_t k = key_at(i);
    if (k != 0ull) {
      mn = k < mn ? k : mn;
      mx = k > mx ? k : mx;
    }
  }
  wave_minmax_u64(mn, mx);
  const int w = threadIdx.x / kWave;
  constexpr int nw = NT / kWave;
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
template <int NT, class KeyAt>
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
    for (int i = threadIdx.x; i < 256; i += NT) sm.hist[i] = 0;
    lds_barrier();
    for (int i = threadIdx.x; i < n; i += NT) {
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
template <int NT, class KeyAt>
__device__ void block_select2(KeyAt key_at, int n, int ra, int rb, SelectSmem& sm, uint64_t* ta,
                              uint64_t* tb) {
  uint64_t mn, mx;
  block_minmax<NT>(key_at, n, sm, &mn, &mx);
  if (mn == mx) {
    *ta = *tb = mn;
    return;
  }
  const int hb = 63 - __builtin_clzll(mn ^ mx);
  const int lo = hb + 1 > 11 ? hb + 1 - 11 : 0;
  const uint32_t dmask = (1u << (hb + 1 - lo)) - 1u;
  const uint64_t prefix = hb >= 63 ? 0ull : (mx & (~0ull << (hb + 1)));
  auto digit = [&](uint64_t key) -> uint32_t { return (uint32_t)(key >> lo) & dmask; };

  for (int i = threadIdx.x; i < kHistBins; i += NT) sm.hist[i] = 0;
  if (threadIdx.x < 2) sm.nlist[threadIdx.x] = 0;
  lds_barrier();
  for (int i = threadIdx.x; i < n; i += NT) {
    const uint64_t key = key_at(i);
    if (key != 0ull) atomicAdd(&sm.hist[digit(key)], 1u);
  }
  lds_barrier();
  constexpr int bpt = kHistBins / NT;  // NT divides kHistBins
  const int b0 = threadIdx.x * bpt;
  uint32_t own = 0;
  for (int j = 0; j < bpt; ++j) own += sm.hist[b0 + j];
  uint32_t total;
  const uint32_t below = block_exclusive_scan<NT>(own, sm.wsum, &total);
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
    for (int i = threadIdx.x; i < n; i += NT) {
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
        block_minmax<NT>(in_bin, n, sm, &bmn, &bmx);
        t[q] = block_kth_largest<NT>(in_bin, n, (int)rem[q], sm, bmn, bmx);
      }
    }
  }
  *ta = t[0];
  *tb = t[1];
}

// Lower edge *t of the histogram bin that holds the P-th largest of the block's valid
// 32-bit keys (thread t holds key[r] of row t + NT*r, valid when that row is below n;
// 1 <= P <= n), and *cnt = how many keys are >= *t.  mn and mx are the keys' minimum
// and maximum; sm.hist must be zero.  The 2048 bins split [mn, mx] evenly (by a power
// of two), so one pass places P; no ranking inside the bin.
template <int NT, int R>
__device__ void slice_threshold(const uint32_t (&key)[R], int n, int P, uint32_t mn, uint32_t mx,
                                SelectSmem& sm, uint32_t* t, uint32_t* cnt) {
  constexpr int bpt = kHistBins / NT;
  const uint32_t range = mx - mn;
  const int sh = range == 0 ? 0 : max(0, 32 - __builtin_clz(range) - 11);
#pragma unroll
  for (int r = 0; r < R; ++r)
    if ((int)threadIdx.x + NT * r < n) atomicAdd(&sm.hist[(key[r] - mn) >> sh], 1u);
  lds_barrier();
  const int b0 = threadIdx.x * bpt;
  uint32_t own = 0;
#pragma unroll
  for (int j = 0; j < bpt; ++j) own += sm.hist[b0 + j];
  uint32_t total;
  const uint32_t below = block_exclusive_scan<NT>(own, sm.wsum, &total);
  const uint32_t above = total - below - own;  // values in bins >= b0 + bpt
  const uint32_t p = (uint32_t)P;
  if (above < p && p <= above + own) {
    uint32_t a = above;
#pragma unroll
    for (int j = bpt - 1; j >= 0; --j) {
      const uint32_t h = sm.hist[b0 + j];
      if (a < p && p <= a + h) {
        sm.bc[0] = b0 + j;
        sm.bc[1] = a + h;
      }
      a += h;
    }
  }
  lds_barrier();
  *t = mn + (sm.bc[0] << sh);
  *cnt = sm.bc[1];
}

// The k-th largest of n distinct nonzero 64-bit keys held in LDS (1 <= k <= n), given
// the minimum mn and maximum mx of their high words, with sm.hist zeroed and sm.bc[4] = 0
// before the caller's last barrier.  A histogram of the high words (2048 bins between mn
// and mx) locates the bin holding it; if that whole bin is needed the answer is its
// smallest key, otherwise the bin's keys are ranked directly (general radix passes if the
// bin is very full).
template <int NT>
__device__ uint64_t block_kth_in_range(const uint64_t* keys, int n, int k, SelectSmem& sm,
                                       uint64_t* list, uint32_t mn, uint32_t mx) {
  constexpr int nw = NT / kWave;
  const int w = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  auto at = [&](int i) -> uint64_t { return keys[i]; };
  if (mn == mx) {  // one high word: rank by the low words
    uint64_t kmn, kmx;
    block_minmax<NT>(at, n, sm, &kmn, &kmx);
    return block_kth_largest<NT>(at, n, k, sm, kmn, kmx);
  }
  const int sh = max(0, 32 - __builtin_clz(mx - mn) - 11);
  auto bin_of = [&](uint64_t key) -> uint32_t { return ((uint32_t)(key >> 32) - mn) >> sh; };
  for (int i = threadIdx.x; i < n; i += NT) atomicAdd(&sm.hist[bin_of(keys[i])], 1u);
  lds_barrier();
  const uint32_t kk = (uint32_t)k;
  constexpr int bpt = kHistBins / NT;
  const int b0 = threadIdx.x * bpt;
  uint32_t own = 0;
#pragma unroll
  for (int j = 0; j < bpt; ++j) own += sm.hist[b0 + j];
  uint32_t total;
  const uint32_t below = block_exclusive_scan<NT>(own, sm.wsum, &total);
  const uint32_t above = total - below - own;  // keys in bins >= b0 + bpt
  if (above < kk && kk <= above + own) {
    uint32_t a = above;
#pragma unroll
    for (int j = bpt - 1; j >= 0; --j) {
      const uint32_t h = sm.hist[b0 + j];
      if (a < kk && kk <= a + h) {
        sm.bc[0] = b0 + j;
        sm.bc[1] = a;
      }
      a += h;
    }
  }
  lds_barrier();
  const uint32_t tb = sm.bc[0];
  const uint32_t need = kk - sm.bc[1];  // rank of the answer inside bin tb
  const uint32_t cnt = sm.hist[tb];
  if (cnt == need) {  // every key of the bin is in: the answer is the bin's smallest
    uint64_t m = ~0ull, unused = 0ull;
    for (int i = threadIdx.x; i < n; i += NT) {
      const uint64_t key = keys[i];
      if (bin_of(key) == tb && key < m) m = key;
    }
    wave_minmax_u64(m, unused);
    if (lane == 0) sm.res64[w] = m;
    lds_barrier();
    uint64_t r = sm.res64[0];
#pragma unroll
    for (int i = 1; i < nw; ++i) r = sm.res64[i] < r ? sm.res64[i] : r;
    lds_barrier();
    return r;
  }
  if (cnt <= (uint32_t)kMergeListCap && cnt <= (uint32_t)NT) {
    for (int i = threadIdx.x; i < n; i += NT) {
      const uint64_t key = keys[i];
      if (bin_of(key) == tb) list[atomicAdd(&sm.bc[4], 1u)] = key;
    }
    lds_barrier();
    if (threadIdx.x < cnt) {
      const uint64_t x = list[threadIdx.x];
      uint32_t greater = 0;
      for (uint32_t j = 0; j < cnt; ++j) greater += list[j] > x;
      if (greater == need - 1) sm.res64[0] = x;
    }
    lds_barrier();
    const uint64_t r = sm.res64[0];
    lds_barrier();
    return r;
  }
  auto bin_at = [&](int i) -> uint64_t {
    const uint64_t key = keys[i];
    return bin_of(key) == tb ? key : 0ull;
  };
  uint64_t bmn, bmx;
  block_minmax<NT>(bin_at, n, sm, &bmn, &bmx);
  return block_kth_largest<NT>(bin_at, n, (int)need, sm, bmn, bmx);
}

// The k-th largest of n distinct nonzero 64-bit keys held in LDS (1 <= k <= n): the
// high words' range, then block_kth_in_range.
template <int NT>
__device__ uint64_t block_kth_exact(const uint64_t* keys, int n, int k, SelectSmem& sm,
                                    uint64_t* list) {
  constexpr int nw = NT / kWave;
  const int w = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  uint32_t mn = ~0u, mx = 0u;
  for (int i = threadIdx.x; i < n; i += NT) {
    const uint32_t h = (uint32_t)(keys[i] >> 32);
    mn = h < mn ? h : mn;
    mx = h > mx ? h : mx;
  }
  for (int i = threadIdx.x; i < kHistBins; i += NT) sm.hist[i] = 0;
  if (threadIdx.x == 0) sm.bc[4] = 0;
  wave_minmax_u32(mn, mx);
  if (lane == 0) {
    sm.red32[w] = mn;
    sm.red32[16 + w] = mx;
  }
  lds_barrier();
  mn = sm.red32[0];
  mx = sm.red32[16];
#pragma unroll
  for (int i = 1; i < nw; ++i) {
    mn = sm.red32[i] < mn ? sm.red32[i] : mn;
    mx = sm.red32[16 + i] > mx ? sm.red32[16 + i] : mx;
  }
  return block_kth_in_range<NT>(keys, n, k, sm, list, mn, mx);
}

__device__ __forceinline__ uint64_t compose_key(uint32_t score_key, uint32_t idx) {
  return ((uint64_t)score_key << 32) | (uint32_t)(~idx);
}
__device__ __forceinline__ int32_t key_index(uint64_t key) { return (int32_t)(~(uint32_t)key); }

struct IndexerWs {
  uint64_t* cand;    // [B][n_slices][cap] candidate selection keys of each slice
  uint64_t* bound;   // [B][n_slices] every key of the slice not in cand is below this
  uint32_t* count;   // [B][n_slices] candidates of each slice
  uint32_t* scores;  // [B][n_c] score key of every row
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

IndexerWs carve_indexer_ws(void* base, int batch, const IndexerPlan& plan) {
  uint8_t* p = static_cast<uint8_t*>(base);
  const size_t ns = (size_t)batch * plan.n_slices;
  IndexerWs ws;
  ws.cand = reinterpret_cast<uint64_t*>(p);
  p += align256(ns * plan.cap * sizeof(uint64_t));
  ws.bound = reinterpret_cast<uint64_t*>(p);
  p += align256(ns * sizeof(uint64_t));
  ws.count = reinterpret_cast<uint32_t*>(p);
  p += align256(ns * sizeof(uint32_t));
  ws.scores = reinterpret_cast<uint32_t*>(p);
  return ws;
}


// ------------------------------------------------------------------ merge

// LDS of one query's merge.
struct MergeSmem {
  uint64_t buf[kMergeCap];
  // The boundary bin's keys (block_kth_exact), and the current winners (up to top_k).
  uint64_t list[kMaxTopK > kMergeListCap ? kMaxTopK : kMergeListCap];
  uint64_t bound[kMaxMergeSlices];
  uint32_t off[kMaxMergeSlices + 1];
  int sat[kMaxMergeSlices];
  SelectSmem sm;
};

// The top-k of query b from the scan's per-slice candidates: the exact k-th largest
// candidate key, by a histogram of the candidates and a direct ranking of the one bin
// that holds it; a slice whose bound lies above that key may hide further winners, so its
// stored scores are re-read and the selection repeated.  The selected indices are written
// in candidate-buffer order to out_g and/or out_l (either may be null); positions past
// the sequence's rows get -1.  Called by every thread of an NT-thread block.
template <int NT, int FPT>
__device__ void merge_query(const IndexerWs& ws, int64_t n_c, const int32_t* __restrict__ seq_rows,
                            int top_k, int n_slices, int cap, int first, int b, MergeSmem& ms,
                            int32_t* out_g, int32_t* out_l) {
  uint64_t* const s_buf = ms.buf;
  uint64_t* const s_list = ms.list;
  uint64_t* const s_bound = ms.bound;
  uint32_t* const s_off = ms.off;
  int* const s_sat = ms.sat;
  SelectSmem& sm = ms.sm;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int64_t n_cb = seq_len(seq_rows, b, n_c);  // this sequence's rows
  const int k1 = (int)min((int64_t)top_k, n_cb);
  for (int i = k1 + threadIdx.x; i < top_k; i += NT) {
    if (out_g) out_g[i] = -1;
    if (out_l) out_l[i] = -1;
  }
  if (k1 == 0) return;
  const int64_t s0 = (int64_t)b * n_slices;

  // Slots j < first of every slice (first a power of two, n_slices * first <= FPT * NT)
  // are read in the same round of loads as the counts; slots past a slice's count are
  // dropped once the counts are known.
  constexpr int kFirstPerThread = FPT;
  const int f_shift = __builtin_ctz((unsigned)first);
  const int n_first = n_slices << f_shift;
  uint64_t slot[kFirstPerThread];
#pragma unroll
  for (int r = 0; r < kFirstPerThread; ++r) {
    const int i = (int)threadIdx.x + NT * r;
    slot[r] = i < n_first ? ws.cand[(s0 + (i >> f_shift)) * cap + (i & (first - 1))] : 0ull;
  }
  // Candidate counts -> offsets in the buffer (n_slices <= NT); on the way, the histogram
  // of the k-th key search is cleared, and the high words' range of the placed keys taken.
  for (int i = threadIdx.x; i < kHistBins; i += NT) sm.hist[i] = 0;
  if (threadIdx.x == 0) {
    sm.bc[4] = 0;
    sm.bc[5] = 0;  // set below when a slice saturates
  }
  uint32_t hmn = ~0u, hmx = 0u;
  const uint32_t c = threadIdx.x < n_slices ? ws.count[s0 + threadIdx.x] : 0u;
  if (threadIdx.x < n_slices) s_bound[threadIdx.x] = ws.bound[s0 + threadIdx.x];
  uint32_t n_buf;
  const uint32_t off = block_exclusive_scan<NT>(c, sm.wsum, &n_buf);
  if (threadIdx.x < n_slices) s_off[threadIdx.x] = off;
  if (threadIdx.x == 0) s_off[n_slices] = n_buf;
  lds_barrier();
#pragma unroll
  for (int r = 0; r < kFirstPerThread; ++r) {
    const int i = (int)threadIdx.x + NT * r;
    if (i < n_first) {
      const int s = i >> f_shift, j = i & (first - 1);
      const uint32_t o = s_off[s];
      if ((uint32_t)j < s_off[s + 1] - o) {
        s_buf[o + j] = slot[r];
        const uint32_t h = (uint32_t)(slot[r] >> 32);
        hmn = h < hmn ? h : hmn;
        hmx = h > hmx ? h : hmx;
      }
    }
  }
  // The rest of the slices that sent more than `first` keys, one wave per slice.
  for (int s = wave; s < n_slices; s += NT / kWave) {
    const uint32_t o = s_off[s], m = s_off[s + 1] - o;
    if (m <= (uint32_t)first) continue;
    const uint64_t* src = ws.cand + (s0 + s) * cap;
    for (uint32_t j = (uint32_t)first + lane; j < m; j += kWave) {
      const uint64_t key = src[j];
      s_buf[o + j] = key;
      const uint32_t h = (uint32_t)(key >> 32);
      hmn = h < hmn ? h : hmn;
      hmx = h > hmx ? h : hmx;
    }
  }
  wave_minmax_u32(hmn, hmx);
  if (lane == 0) {
    sm.red32[wave] = hmn;
    sm.red32[16 + wave] = hmx;
  }
  lds_barrier();
  hmn = sm.red32[0];
  hmx = sm.red32[16];
#pragma unroll
  for (int i = 1; i < NT / kWave; ++i) {
    hmn = sm.red32[i] < hmn ? sm.red32[i] : hmn;
    hmx = sm.red32[16 + i] > hmx ? sm.red32[16 + i] : hmx;
  }

  // The k1-th largest candidate; 1 (accept all) while there are fewer than k1.
  uint64_t kth = (int)n_buf >= k1 ? block_kth_in_range<NT>(s_buf, (int)n_buf, k1, sm, s_list, hmn, hmx) : 1ull;

  // Slices whose bound lies above kth may hold winners among the keys they did not send.
  // Usually none does: a flag and one barrier settle that before any scan.
  const uint32_t sat = threadIdx.x < n_slices && s_bound[threadIdx.x] > kth;
  if (sat) sm.bc[5] = 1u;
  lds_barrier();
  if (sm.bc[5] != 0u) {
    uint32_t n_sat;
    const uint32_t pos = block_exclusive_scan<NT>(sat, sm.wsum, &n_sat);
    if (sat) s_sat[pos] = threadIdx.x;
    lds_barrier();
    for (uint32_t q = 0; q < n_sat; ++q) {
      const int s = s_sat[q];
      if (!(s_bound[s] > kth)) continue;  // kth has risen past this slice's bound
      // Keep only the current winners (>= kth), in buffer order, to make room.
      {
        const int chunk = ((int)n_buf + NT - 1) / NT;
        const int p0 = threadIdx.x * chunk, p1 = min(p0 + chunk, (int)n_buf);
        uint32_t cw = 0;
        for (int p = p0; p < p1; ++p) cw += s_buf[p] >= kth;
        uint32_t kept;
        uint32_t w = block_exclusive_scan<NT>(cw, sm.wsum, &kept);
        for (int p = p0; p < p1; ++p)
          if (s_buf[p] >= kth) s_list[w++] = s_buf[p];
        lds_barrier();
        for (uint32_t i = threadIdx.x; i < kept; i += NT) s_buf[i] = s_list[i];
        n_buf = kept;
        lds_barrier();
      }
      // Append the slice's unsent keys >= kth, read back from its stored scores.
      {
        const int64_t srow0 = (int64_t)s * kSliceRows;
        const int rows = (int)min((int64_t)kSliceRows, n_cb - srow0);
        const uint32_t* sc = ws.scores + (int64_t)b * n_c + srow0;
        const uint64_t bnd = s_bound[s];
        const int chunk = (rows + NT - 1) / NT;
        const int p0 = threadIdx.x * chunk, p1 = min(p0 + chunk, rows);
        uint32_t ca = 0;
        for (int i = p0; i < p1; ++i) {
          const uint64_t key = compose_key(sc[i], (uint32_t)(srow0 + i));
          ca += key >= kth && key < bnd;
        }
        uint32_t added;
        uint32_t w = n_buf + block_exclusive_scan<NT>(ca, sm.wsum, &added);
        for (int i = p0; i < p1; ++i) {
          const uint64_t key = compose_key(sc[i], (uint32_t)(srow0 + i));
          if (key >= kth && key < bnd) s_buf[w++] = key;
        }
        n_buf += added;
        lds_barrier();
        if (threadIdx.x == 0) s_bound[s] = 0ull;
      }
      kth = (int)n_buf >= k1 ? block_kth_exact<NT>(s_buf, (int)n_buf, k1, sm, s_list) : 1ull;
    }
  }

  // Write the selected indices in buffer order (deterministic).
  const int chunk = ((int)n_buf + NT - 1) / NT;
  const int p0 = threadIdx.x * chunk, p1 = min(p0 + chunk, (int)n_buf);
  uint32_t cw = 0;
  for (int p = p0; p < p1; ++p) cw += s_buf[p] >= kth;
  uint32_t total;
  uint32_t pos = block_exclusive_scan<NT>(cw, sm.wsum, &total);
  for (int p = p0; p < p1; ++p)
    if (s_buf[p] >= kth) {
      const int32_t idx = key_index(s_buf[p]);
      if (out_g) out_g[pos] = idx;
      if (out_l) out_l[pos] = idx;
      ++pos;
    }
}

}  // namespace

}  // namespace csakv
