// Lightning-indexer scoring and top-k selection for CSA decode.
//
// What is computed ("DeepSeek-V4 KV Cache 深度分析", section 四 "索引器（Indexer）机制" and
// the section 十一 forward-flow diagram): the query token's indexer query is scored
// against the indexer key of every compressed entry, and the top-k entries are kept.
// Score s_j = sum_h w_h * ReLU(q_h . k_j); ties are broken toward the smaller index.
//
// Structure (two launches per call):
//   1. slice kernel, grid (slices, B): each workgroup streams one slice of indexer-key
//      rows straight from HBM into registers, dequantises FP4 rows to bf16 in
//      registers (exact: an E2M1 value times an E4M3 scale has at most 6 significant
//      bits), and runs the [H_I x 128] x [128 x 16] contraction on 16x16x32 bf16 MFMA
//      with fp32 accumulation.  ReLU, the head weights and the head sum are applied to
//      the accumulators, and the slice's scores stay in LDS.  A radix select in LDS
//      then keeps the slice's top-k, which is bitonic-sorted and written out.
//   2. merge kernel, grid (B): reads a sorted prefix of every slice, selects the
//      k-th largest key, and reads further into any slice whose prefix does not yet
//      fall below it; the result is exact for any input.
// Selection keys are 64-bit: (order-preserving score bits << 32) | ~index, so
// "larger key" means higher score, then lower index.
#include "csakv_device.h"
#include "csakv_launch.h"

namespace csakv {

namespace {

constexpr int kIdxDim = 128;
constexpr int kSliceThreads = 512;
constexpr int kSliceWaves = kSliceThreads / kWave;
constexpr int kMergeThreads = 512;

__device__ __forceinline__ uint64_t compose_key(uint32_t score_key, uint32_t idx) {
  return ((uint64_t)score_key << 32) | (uint32_t)(~idx);
}
__device__ __forceinline__ int32_t key_index(uint64_t key) { return (int32_t)(~(uint32_t)key); }

// ------------------------------------------------------------------ block primitives

// Exclusive prefix sum of one value per thread over the whole block.
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) wsum[w] = x;
  __syncthreads();
  uint32_t base = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    uint32_t s = wsum[i];
    if (i < w) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// Finds the digit of the k-th largest element given a 256-bin histogram of the
// elements that share the current prefix.  Wave 0 only; writes (digit, count above).
__device__ void radix_pick_digit(const uint32_t* hist, uint32_t remaining, uint32_t* bcast) {
  const int lane = threadIdx.x;
  uint32_t h[4];
  uint32_t tot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = hist[4 * lane + i];
    tot += h[i];
  }
  uint32_t x = tot;  // inclusive suffix sum over lanes
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    uint32_t y = __shfl_down(x, off);
    if (lane + off < kWave) x += y;
  }
  uint32_t above = x - tot;
#pragma unroll
  for (int i = 3; i >= 0; --i) {
    if (above < remaining && remaining <= above + h[i]) {
      bcast[0] = 4 * lane + i;
      bcast[1] = above;
    }
    above += h[i];
  }
}

// k-th largest of n 32-bit keys in LDS (1 <= k <= n).  Returns it and how many keys
// are strictly larger.
__device__ void block_select32(const uint32_t* keys, int n, int k, uint32_t* hist,
                               uint32_t* bcast, uint32_t* kth, int* n_greater) {
  uint32_t prefix = 0, mask = 0;
  uint32_t remaining = (uint32_t)k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      uint32_t key = keys[i];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x < kWave) radix_pick_digit(hist, remaining, bcast);
    __syncthreads();
    prefix |= bcast[0] << shift;
    mask |= 255u << shift;
    remaining -= bcast[1];
  }
  *kth = prefix;
  *n_greater = k - (int)remaining;
}

// k-th largest of n distinct 64-bit keys in LDS (1 <= k <= n).
__device__ uint64_t block_select64(const uint64_t* keys, int n, int k, uint32_t* hist,
                                   uint32_t* bcast) {
  uint64_t prefix = 0, mask = 0;
  uint32_t remaining = (uint32_t)k;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      uint64_t key = keys[i];
      if ((key & mask) == prefix) atomicAdd(&hist[(uint32_t)(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x < kWave) radix_pick_digit(hist, remaining, bcast);
    __syncthreads();
    prefix |= (uint64_t)bcast[0] << shift;
    mask |= (uint64_t)255u << shift;
    remaining -= bcast[1];
  }
  return prefix;
}

// Descending bitonic sort of s[0..p), p a power of two.
__device__ void block_sort_desc(uint64_t* s, int p) {
  for (int k = 2; k <= p; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < p; i += blockDim.x) {
        int ixj = i ^ j;
        if (ixj > i) {
          uint64_t a = s[i], b = s[ixj];
          bool desc = (i & k) == 0;
          if (desc ? (a < b) : (a > b)) {
            s[i] = b;
            s[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// ------------------------------------------------------------------ key tiles

// Raw indexer-key data of one lane for a 16-row tile.  Lane (g, n) owns row n of the
// tile and 32 of its 128 channels.
template <int KFMT>
struct KeyTile;

// bf16 rows: in K-step t the lane supplies channels 32t + 8g .. 32t + 8g + 7.
template <>
struct KeyTile<0> {
  u32x4 c[4];
  __device__ __forceinline__ void load(const uint8_t* codes, const uint8_t*, int64_t row, int g) {
    const uint8_t* p = codes + row * (kIdxDim * 2) + 16 * g;
#pragma unroll
    for (int t = 0; t < 4; ++t) c[t] = *reinterpret_cast<const u32x4*>(p + 64 * t);
  }
  __device__ __forceinline__ bf16x8 operand(int t) const { return as_bf16x8(c[t]); }
  static __device__ __forceinline__ int q_channel(int g, int t) { return 32 * t + 8 * g; }
};

// FP4 rows: the lane loads channels 32g .. 32g + 31 (16 code bytes, 2 scales); in
// K-step t it supplies channels 32g + 8t .. 32g + 8t + 7.
template <>
struct KeyTile<1> {
  u32x4 c;
  uint32_t s;  // two E4M3 scale bytes: blocks 2g (low) and 2g + 1
  __device__ __forceinline__ void load(const uint8_t* codes, const uint8_t* scales, int64_t row,
                                       int g) {
    c = *reinterpret_cast<const u32x4*>(codes + row * (kIdxDim / 2) + 16 * g);
    s = *reinterpret_cast<const uint16_t*>(scales + row * (kIdxDim / 16) + 2 * g);
  }
  __device__ __forceinline__ bf16x8 operand(int t) const {
    const float sc = e4m3_to_f32(t < 2 ? (s & 0xFFu) : (s >> 8));
    return as_bf16x8(fp4x8_to_bf16(c[t], sc));
  }
  static __device__ __forceinline__ int q_channel(int g, int t) { return 32 * g + 8 * t; }
};

// ------------------------------------------------------------------ slice kernel

template <int KFMT, int HT>
__global__ __launch_bounds__(kSliceThreads) void indexer_slice_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t seq_stride,
    int64_t n_c, const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx, int n_heads,
    int top_k, int slice_rows, int n_slices, int cand_stride, uint64_t* __restrict__ cand) {
  __shared__ uint32_t s_score[kMaxSliceRows];
  __shared__ uint64_t s_cand[kMaxTopK];
  __shared__ uint32_t s_hist[256];
  __shared__ uint32_t s_bcast[2];
  __shared__ uint32_t s_wsum[kSliceWaves];

  const int slice = blockIdx.x;
  const int b = blockIdx.y;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int g = lane >> 4;
  const int n = lane & 15;

  const int64_t row0 = (int64_t)slice * slice_rows;
  const int rows = (int)min((int64_t)slice_rows, n_c - row0);
  const int n_tiles = (rows + 15) >> 4;

  // Indexer query fragments (A operand: head n of each 16-head tile) and head weights
  // of the accumulator rows this lane holds (heads 16*ht + 4g + i).
  bf16x8 qa[HT][4];
  float wv[HT][4];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int head = 16 * ht + n;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (head < n_heads)
        v = *reinterpret_cast<const u32x4*>(q_idx + ((int64_t)b * n_heads + head) * kIdxDim +
                                            KeyTile<KFMT>::q_channel(g, t));
      qa[ht][t] = as_bf16x8(v);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 16 * ht + 4 * g + i;
      wv[ht][i] = h < n_heads ? w_idx[(int64_t)b * n_heads + h] : 0.0f;
    }
  }

  const int64_t seq_row0 = (int64_t)b * seq_stride + row0;
  KeyTile<KFMT> cur, nxt;
  int tile = wave;
  if (tile < n_tiles) cur.load(codes, scales, seq_row0 + min(tile * 16 + n, rows - 1), g);
  for (; tile < n_tiles; tile += kSliceWaves) {
    const int next = tile + kSliceWaves;
    if (next < n_tiles) nxt.load(codes, scales, seq_row0 + min(next * 16 + n, rows - 1), g);
    f32x4 acc[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      bf16x8 kb = cur.operand(t);
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) acc[ht] = mfma16x16x32(qa[ht][t], kb, acc[ht]);
    }
    float s = 0.0f;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int i = 0; i < 4; ++i) s += wv[ht][i] * fmaxf(acc[ht][i], 0.0f);
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    const int p = tile * 16 + n;
    if (g == 0 && p < rows) s_score[p] = f32_order_key(s);
    cur = nxt;
  }
  __syncthreads();

  // ---- slice top-k1, ties toward the lower index (= lower position)
  const int k1 = min(top_k, rows);
  uint32_t kth;
  int n_gt;
  block_select32(s_score, rows, k1, s_hist, s_bcast, &kth, &n_gt);
  const int ties = k1 - n_gt;

  const int chunk = (rows + kSliceThreads - 1) / kSliceThreads;
  const int p0 = threadIdx.x * chunk;
  const int p1 = min(p0 + chunk, rows);
  uint32_t cnt_gt = 0, cnt_eq = 0;
  for (int p = p0; p < p1; ++p) {
    uint32_t key = s_score[p];
    cnt_gt += key > kth;
    cnt_eq += key == kth;
  }
  uint32_t total;
  uint32_t base = block_exclusive_scan((cnt_gt << 16) | cnt_eq, s_wsum, &total);
  uint32_t pos_gt = base >> 16, pos_eq = base & 0xFFFFu;
  for (int p = p0; p < p1; ++p) {
    uint32_t key = s_score[p];
    if (key > kth) {
      s_cand[pos_gt++] = compose_key(key, (uint32_t)(row0 + p));
    } else if (key == kth) {
      if ((int)pos_eq < ties) s_cand[n_gt + pos_eq] = compose_key(key, (uint32_t)(row0 + p));
      ++pos_eq;
    }
  }
  const int psort = next_pow2(k1);
  for (int i = k1 + threadIdx.x; i < psort; i += blockDim.x) s_cand[i] = 0;
  __syncthreads();
  block_sort_desc(s_cand, psort);

  uint64_t* dst = cand + ((int64_t)b * n_slices + slice) * cand_stride;
  for (int i = threadIdx.x; i < k1; i += blockDim.x) dst[i] = s_cand[i];
}

// ------------------------------------------------------------------ merge kernel

__global__ __launch_bounds__(kMergeThreads) void indexer_merge_kernel(
    const uint64_t* __restrict__ cand, int64_t n_c, int top_k, int slice_rows, int n_slices,
    int cand_stride, int prefix, int32_t* __restrict__ topk) {
  __shared__ uint64_t s_buf[kMergeCap];
  __shared__ uint64_t s_tmp[kMaxTopK];
  __shared__ uint32_t s_hist[256];
  __shared__ uint32_t s_bcast[2];
  __shared__ uint32_t s_wsum[kMergeThreads / kWave];

  const int b = blockIdx.x;
  const int k1 = (int)min((int64_t)top_k, n_c);
  const uint64_t* cb = cand + (int64_t)b * n_slices * cand_stride;
  int32_t* out = topk + (int64_t)b * top_k;

  for (int i = k1 + threadIdx.x; i < top_k; i += blockDim.x) out[i] = -1;
  if (k1 == 0) return;

  auto slice_count = [&](int s) -> int {
    int64_t r = min((int64_t)slice_rows, n_c - (int64_t)s * slice_rows);
    return (int)min((int64_t)top_k, r);
  };

  if (n_slices == 1) {  // the single slice's sorted list is the answer
    for (int i = threadIdx.x; i < k1; i += blockDim.x) out[i] = key_index(cb[i]);
    return;
  }

  // Sorted prefix of every slice, at stride `prefix`; short slices pad with key 0,
  // which is below every real key.
  const int n_load = n_slices * prefix;
  for (int i = threadIdx.x; i < n_load; i += blockDim.x) {
    const int s = i / prefix, j = i - s * prefix;
    s_buf[i] = j < slice_count(s) ? cb[(int64_t)s * cand_stride + j] : 0ull;
  }
  __syncthreads();

  // Keep the k1 largest of s_buf[0..n) in s_buf[0..k1); returns the k1-th key.
  auto reduce_to_topk = [&](int n) -> uint64_t {
    uint64_t kth = block_select64(s_buf, n, k1, s_hist, s_bcast);
    const int chunk = (n + kMergeThreads - 1) / kMergeThreads;
    const int p0 = threadIdx.x * chunk, p1 = min(p0 + chunk, n);
    uint32_t c = 0;
    for (int p = p0; p < p1; ++p) c += s_buf[p] >= kth;
    uint32_t total;
    uint32_t pos = block_exclusive_scan(c, s_wsum, &total);
    for (int p = p0; p < p1; ++p)
      if (s_buf[p] >= kth) s_tmp[pos++] = s_buf[p];
    __syncthreads();
    for (int i = threadIdx.x; i < k1; i += blockDim.x) s_buf[i] = s_tmp[i];
    __syncthreads();
    return kth;
  };

  uint64_t kth = reduce_to_topk(n_load);

  // A slice whose last loaded key still beats the k1-th may hold more winners:
  // stream the rest of it (keys below the current k1-th cannot win) and reselect.
  for (int s = 0; s < n_slices; ++s) {
    const int cnt = slice_count(s);
    if (prefix >= cnt) continue;
    if (cb[(int64_t)s * cand_stride + prefix - 1] <= kth) continue;  // uniform branch
    int fill = k1;
    for (int j0 = prefix; j0 < cnt; j0 += kMergeCap - k1) {
      const int m = min(kMergeCap - k1, cnt - j0);
      for (int i = threadIdx.x; i < m; i += blockDim.x) {
        uint64_t key = cb[(int64_t)s * cand_stride + j0 + i];
        s_buf[k1 + i] = key > kth ? key : 0ull;
      }
      __syncthreads();
      fill = k1 + m;
      kth = reduce_to_topk(fill);
    }
  }

  const int psort = next_pow2(k1);
  for (int i = k1 + threadIdx.x; i < psort; i += blockDim.x) s_buf[i] = 0;
  __syncthreads();
  block_sort_desc(s_buf, psort);
  for (int i = threadIdx.x; i < k1; i += blockDim.x) out[i] = key_index(s_buf[i]);
}

template <int KFMT, int HT>
void launch_slice(dim3 grid, hipStream_t stream, const uint8_t* codes, const uint8_t* scales,
                  int64_t seq_stride, int64_t n_c, const uint16_t* q_idx, const float* w_idx,
                  int n_heads, int top_k, const IndexerPlan& plan, uint64_t* cand) {
  hipLaunchKernelGGL((indexer_slice_kernel<KFMT, HT>), grid, dim3(kSliceThreads), 0, stream, codes,
                     scales, seq_stride, n_c, q_idx, w_idx, n_heads, top_k, plan.slice_rows,
                     plan.n_slices, plan.cand_stride, cand);
}

template <int KFMT>
void launch_slice_ht(int ht, dim3 grid, hipStream_t stream, const uint8_t* codes,
                     const uint8_t* scales, int64_t seq_stride, int64_t n_c,
                     const uint16_t* q_idx, const float* w_idx, int n_heads, int top_k,
                     const IndexerPlan& plan, uint64_t* cand) {
  switch (ht) {
    case 1: launch_slice<KFMT, 1>(grid, stream, codes, scales, seq_stride, n_c, q_idx, w_idx, n_heads, top_k, plan, cand); break;
    case 2: launch_slice<KFMT, 2>(grid, stream, codes, scales, seq_stride, n_c, q_idx, w_idx, n_heads, top_k, plan, cand); break;
    case 3: launch_slice<KFMT, 3>(grid, stream, codes, scales, seq_stride, n_c, q_idx, w_idx, n_heads, top_k, plan, cand); break;
    default: launch_slice<KFMT, 4>(grid, stream, codes, scales, seq_stride, n_c, q_idx, w_idx, n_heads, top_k, plan, cand); break;
  }
}

}  // namespace

IndexerPlan plan_indexer(int batch, int64_t n_c, int top_k) {
  IndexerPlan p{};
  // Aim for at least two workgroups per CU (256 CUs) while keeping slices large
  // enough that the merge reads few candidates.
  int64_t want_slices = (512 + batch - 1) / batch;
  int64_t rows = (n_c + want_slices - 1) / want_slices;
  rows = ((rows + 15) / 16) * 16;
  int64_t min_rows = top_k > 1024 ? top_k : 1024;
  if (rows < min_rows) rows = min_rows;
  if (rows > kMaxSliceRows) rows = kMaxSliceRows;
  p.slice_rows = (int)rows;
  p.n_slices = n_c > 0 ? (int)((n_c + rows - 1) / rows) : 0;
  p.cand_stride = (int)(top_k < rows ? top_k : rows);
  int per_slice = p.n_slices > 0 ? (top_k + p.n_slices - 1) / p.n_slices : top_k;
  int pre = 32;
  while (pre < 4 * per_slice) pre <<= 1;
  if (pre > p.cand_stride) pre = p.cand_stride;
  p.prefix = pre;
  return p;
}

size_t indexer_workspace_bytes(int batch, const IndexerPlan& plan) {
  return (size_t)batch * plan.n_slices * plan.cand_stride * sizeof(uint64_t);
}

hipError_t launch_indexer(int key_fmt, const uint8_t* codes, const uint8_t* scales,
                          int64_t seq_stride, int64_t n_c, const uint16_t* q_idx,
                          const float* w_idx, int batch, int n_heads, int top_k,
                          const IndexerPlan& plan, void* workspace, int32_t* topk,
                          hipStream_t stream) {
  uint64_t* cand = static_cast<uint64_t*>(workspace);
  if (plan.n_slices > 0) {
    dim3 grid(plan.n_slices, batch);
    const int ht = (n_heads + 15) / 16;
    if (key_fmt == 0)
      launch_slice_ht<0>(ht, grid, stream, codes, scales, seq_stride, n_c, q_idx, w_idx, n_heads,
                         top_k, plan, cand);
    else
      launch_slice_ht<1>(ht, grid, stream, codes, scales, seq_stride, n_c, q_idx, w_idx, n_heads,
                         top_k, plan, cand);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(indexer_merge_kernel, dim3(batch), dim3(kMergeThreads), 0, stream, cand, n_c,
                     top_k, plan.slice_rows, plan.n_slices, plan.cand_stride, plan.prefix, topk);
  return hipGetLastError();
}

}  // namespace csakv
