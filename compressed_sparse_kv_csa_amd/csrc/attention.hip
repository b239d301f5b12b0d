// Multi-query softmax attention over gathered shared-KV rows (CSA sparse, HCA dense).
//
// What is computed ("DeepSeek-V4 KV Cache 深度分析", section 三 for the CSA/HCA row sets,
// section 五 for one entry serving as both key and value, and the section 十一 diagram):
//   o[h] = sum_r softmax_r(scale * q[h] . e_r) * e_r
// over the rows r of one query: CSA = the window rows plus the selected compressed
// rows (one softmax over their union), HCA = every row of the sequence.
//
// Structure: grid (chunks, B).  A workgroup owns one chunk of a query's row list and
// all heads (one wave per 16 heads).  It first resolves the chunk's row indices into
// LDS, then per 32-row step gathers whole rows (coalesced 16-byte loads, the next
// step's rows in flight while the current one computes), decodes them to fp16 into
// one of two row-major LDS tiles, and runs
//   S^T[32 rows x 16 heads] = K[32 x 512] . Q^T            (16x16x32 f16 MFMA)
//   O^T[512 x 16 heads]    += V^T[512 x 32] . P^T[32 x 16]  (16x16x32 f16 MFMA)
// with an online softmax in fp32 (exp2 domain).  The same tile serves both products:
// K fragments are plain 16-byte LDS reads, V^T fragments come from transposing LDS
// reads (ds_read_b64_tr_b16), so no transposed copy is ever written.
//
// Precision: FP8 (E4M3) and FP4 (E2M1 x E4M3) values are exact in fp16; bf16 values
// are exact in fp16 from 2^-14 to 65504 (smaller magnitudes keep an absolute error
// below 2^-25).  q is rounded to fp16 the same way.  Products are exact in fp32 and
// accumulate in fp32; the probabilities (in [0, 1]) keep 11 significant bits.
// Each chunk writes (max, sum, unnormalised O) per head; a combine kernel merges the
// chunks and rounds to bf16.
#include "csakv_device.h"
#include "csakv_launch.h"

namespace csakv {

namespace {

constexpr int kDim = 512;
constexpr int kNope = 448;
constexpr int kStepRows = 32;
constexpr int kPitch = kDim + 16;     // fp16 elements per LDS row (32-byte pad)
constexpr int kOutPitch = kDim + 4;   // floats per LDS row when staging the output
constexpr float kLog2e = 1.4426950408889634f;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef v4i16 __attribute__((address_space(3))) lds_v4i16;

// Two floats exactly representable in fp16 (or to be rounded toward zero) -> packed bits.
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}
// bf16 pair (one dword) -> fp16 pair.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  return pack_f16(__uint_as_float(w << 16), __uint_as_float(w & 0xFFFF0000u));
}

// Raw bytes of one (row, 64-dim segment) work item, and their decode to 32 dwords of
// fp16 pairs (dims seg*64 .. seg*64+63).  Raw data is kept in scalar arrays so that it
// stays in registers.
__device__ __forceinline__ void load16(uint32_t* w, const uint8_t* p) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(p);
  w[0] = v[0];
  w[1] = v[1];
  w[2] = v[2];
  w[3] = v[3];
}

template <int KVFMT>
struct SegRaw;

template <>
struct SegRaw<0> {  // bf16: 128 bytes per item; rows split into 8 equal segments
  static constexpr int kRowItems = 8;
  uint32_t w[32];
  static __device__ __forceinline__ void item_rs(int item, int* r, int* seg) {
    *r = item >> 3;
    *seg = item & 7;
  }
  __device__ __forceinline__ void load(const uint8_t* codes, const uint8_t*, int64_t row, int seg) {
    const uint8_t* p = codes + row * (kDim * 2) + seg * 128;
#pragma unroll
    for (int i = 0; i < 8; ++i) load16(w + 4 * i, p + 16 * i);
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 32; ++i) w[i] = 0u;
  }
  __device__ __forceinline__ void decode(int, u32x4* out) const {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) out[i][j] = bf16x2_to_f16x2(w[4 * i + j]);
  }
};

// Mixed rows: items 0 .. 7*32-1 are the E4M3 segments (row = item / 7, 64 bytes each),
// items 7*32 .. 8*32-1 the bf16 RoPE segments (128 bytes), so that only the one wave
// holding both kinds diverges.
template <>
struct SegRaw<1> {
  static constexpr int kRowItems = 8;
  uint32_t w[32];
  static __device__ __forceinline__ void item_rs(int item, int* r, int* seg) {
    if (item < 7 * kStepRows) {
      *r = item / 7;
      *seg = item - 7 * (item / 7);
    } else {
      *r = item - 7 * kStepRows;
      *seg = 7;
    }
  }
  // Every item loads 128 contiguous bytes of its row (an E4M3 item also reads the next
  // 64 bytes, which stay unused), so the load shape does not depend on the segment.
  __device__ __forceinline__ void load(const uint8_t* codes, const uint8_t*, int64_t row, int seg) {
    const uint8_t* p = codes + row * (kNope + 2 * (kDim - kNope)) + (seg < 7 ? seg * 64 : kNope);
#pragma unroll
    for (int i = 0; i < 8; ++i) load16(w + 4 * i, p + 16 * i);
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 32; ++i) w[i] = 0u;
  }
  __device__ __forceinline__ void decode(int seg, u32x4* out) const {
    if (seg < 7) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {  // 4 E4M3 codes -> 4 fp16 (exact)
        out[i >> 1][2 * (i & 1)] = __builtin_bit_cast(
            uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[i], 1.0f, false));
        out[i >> 1][2 * (i & 1) + 1] = __builtin_bit_cast(
            uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[i], 1.0f, true));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) out[i][j] = bf16x2_to_f16x2(w[4 * i + j]);
    }
  }
};

template <>
struct SegRaw<2> {  // FP4: 32 code bytes + 4 E4M3 scale bytes (one per 16 dims)
  static constexpr int kRowItems = 8;
  uint32_t c[8];
  uint32_t s;
  static __device__ __forceinline__ void item_rs(int item, int* r, int* seg) {
    *r = item >> 3;
    *seg = item & 7;
  }
  __device__ __forceinline__ void load(const uint8_t* codes, const uint8_t* scales, int64_t row,
                                       int seg) {
    const uint8_t* p = codes + row * (kDim / 2) + seg * 32;
    load16(c, p);
    load16(c + 4, p + 16);
    s = *reinterpret_cast<const uint32_t*>(scales + row * (kDim / 16) + seg * 4);
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = 0u;
    s = 0u;
  }
  __device__ __forceinline__ void decode(int, u32x4* out) const {
    // The four scales as fp16 (exact), each broadcast to both halves of a pair.
    const uint32_t s01 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s, 1.0f, false));
    const uint32_t s23 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s, 1.0f, true));
    const uint32_t sc[4] = {__builtin_amdgcn_perm(s01, s01, 0x01000100u),
                            __builtin_amdgcn_perm(s01, s01, 0x03020302u),
                            __builtin_amdgcn_perm(s23, s23, 0x01000100u),
                            __builtin_amdgcn_perm(s23, s23, 0x03020302u)};
#pragma unroll
    for (int w = 0; w < 8; ++w) {  // code dword w holds dims 8w .. 8w+7 (block w / 2)
      const uint32_t cw = c[w];
      const f16x2 scv = __builtin_bit_cast(f16x2, sc[w >> 1]);
      out[w][0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 0) * scv);
      out[w][1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 1) * scv);
      out[w][2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 2) * scv);
      out[w][3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 3) * scv);
    }
  }
};

// V^T fragment of dims 16*dt .. 16*dt+15 for the K-slots of lane group g (rows 4g..4g+3
// and 16+4g..16+4g+3 of the tile): two transposing reads.  Within each 16-lane group
// the hardware hands lane i, slot j, element i%4 of the 8 bytes addressed by lane
// 4j + i/4; lane k therefore addresses row base + k/4, dims 16*dt + 4*(k%4).
__device__ __forceinline__ f16x8 v_fragment(const uint16_t* tile, int g, int k, int dt) {
  const uint16_t* p = tile + (4 * g + (k >> 2)) * kPitch + 16 * dt + 4 * (k & 3);
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 16 * kPitch));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  return as_f16x8(u32x4{l2[0], l2[1], h2[0], h2[1]});
}

constexpr int kAttnThreads = 256;  // 4 waves
constexpr int kDimsPerWave = kDim / 4;

// Workgroup -> (query b, chunk, head group).  Workgroups are dispatched round-robin over
// the 8 XCDs by index, so the head groups of one (query, chunk) pair are given indices
// that are equal modulo 8: they run on one XCD and share its L2 for the gathered rows.
__device__ __forceinline__ bool attn_block(int n_pairs, int n_groups, int n_chunks, int* b,
                                           int* chunk, int* hg) {
  const int x = blockIdx.x & 7, k = blockIdx.x >> 3;
  *hg = k % n_groups;
  const int pair = x + 8 * (k / n_groups);
  if (pair >= n_pairs) return false;
  *b = pair / n_chunks;
  *chunk = pair - *b * n_chunks;
  return true;
}

// One workgroup: 16 heads, one chunk of a query's row list.  All 4 waves gather and
// decode; each wave then computes the logits of all 16 heads (the K tile and the query
// rows are shared in LDS) and the output for its own 128 dims.  NB = decode tiles (2
// when the chunk has several steps, so that one barrier per step suffices).
template <int KVFMT, bool CSA, int NB>
__global__ __launch_bounds__(kAttnThreads) void attention_chunk_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t seq_stride,
    int64_t n_rows, const uint16_t* __restrict__ q, int n_heads, float scale_log2,
    const int32_t* __restrict__ topk, int top_k, int window, int64_t n_list, int rows_per_chunk,
    int n_chunks, int n_pairs, float* __restrict__ part_o, float* __restrict__ part_ml) {
  constexpr int kTileElems = kStepRows * kPitch;
  constexpr int kTileBytes = NB * kTileElems * 2;
  constexpr int kQBytes = 16 * kPitch * 2;
  constexpr int kOutBytes = 16 * kOutPitch * 4;
  constexpr int kSmem = kTileBytes + kQBytes > kOutBytes ? kTileBytes + kQBytes : kOutBytes;
  __shared__ __attribute__((aligned(16))) uint8_t s_mem[kSmem];
  __shared__ int s_rows[kMaxChunkRows];
  uint16_t* const s_kv0 = reinterpret_cast<uint16_t*>(s_mem);
  uint16_t* const s_q = reinterpret_cast<uint16_t*>(s_mem + kTileBytes);
  float* const s_out = reinterpret_cast<float*>(s_mem);

  int b, chunk, hg;
  if (!attn_block(n_pairs, n_heads / 16, n_chunks, &b, &chunk, &hg)) return;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int g = lane >> 4;
  const int n = lane & 15;

  const int64_t p_begin = (int64_t)chunk * rows_per_chunk;
  const int64_t p_end = min(p_begin + rows_per_chunk, n_list);
  const int n_steps = (int)((p_end - p_begin + kStepRows - 1) / kStepRows);
  const int64_t n_c = n_rows - window;

  // Sequence row of every list position of the chunk (-1: absent or out of range).
  for (int i = threadIdx.x; i < n_steps * kStepRows; i += kAttnThreads) {
    const int64_t p = p_begin + i;
    int row = -1;
    if (p < p_end) {
      if (!CSA || p < window) {
        row = (int)p;
      } else {
        const int32_t j = topk[(int64_t)b * top_k + (p - window)];
        row = (j >= 0 && j < n_c) ? window + j : -1;
      }
    }
    s_rows[i] = row;
  }
  // The group's 16 query rows as fp16 in LDS (B operand of the logits).
  {
    constexpr int kQIters = 16 * (kDim / 8) / kAttnThreads;
    u32x4 qv[kQIters];
    const uint16_t* qb = q + ((int64_t)b * n_heads + 16 * hg) * kDim;
#pragma unroll
    for (int k = 0; k < kQIters; ++k)
      qv[k] = *reinterpret_cast<const u32x4*>(qb + 8 * (threadIdx.x + k * kAttnThreads));
#pragma unroll
    for (int k = 0; k < kQIters; ++k) {
      const int i = threadIdx.x + k * kAttnThreads;
      const int h = i / (kDim / 8), c8 = i - h * (kDim / 8);
      *reinterpret_cast<u32x4*>(s_q + h * kPitch + 8 * c8) =
          u32x4{bf16x2_to_f16x2(qv[k][0]), bf16x2_to_f16x2(qv[k][1]), bf16x2_to_f16x2(qv[k][2]),
                bf16x2_to_f16x2(qv[k][3])};
    }
  }
  lds_barrier();

  f32x4 o[kDimsPerWave / 16];
#pragma unroll
  for (int i = 0; i < kDimsPerWave / 16; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;

  // This thread's work item inside a step: row r, segment seg (one item per thread).
  // Two steps are fetched ahead (raw0 / raw1 alternate), so both steps of a 64-row chunk
  // are in flight as soon as the row indices are known.
  int item_r, item_seg;
  SegRaw<KVFMT>::item_rs(threadIdx.x, &item_r, &item_seg);
  SegRaw<KVFMT> raw0, raw1;
  auto fetch = [&](SegRaw<KVFMT>& raw, int step) {
    const int row = s_rows[step * kStepRows + item_r];
    if (row >= 0) raw.load(codes, scales, (int64_t)b * seq_stride + row, item_seg);
    else raw.zero();
  };

  auto run_step = [&](SegRaw<KVFMT>& raw, int step) {
    uint16_t* tile = s_kv0 + (NB == 2 ? (step & 1) * kTileElems : 0);
    if (NB == 1 && step > 0) lds_barrier();  // the previous step's tile is consumed
    // ---- decode the fetched rows into the tile (fp16, row-major)
    {
      u32x4 d[8];
      raw.decode(item_seg, d);
      u32x4* dst = reinterpret_cast<u32x4*>(tile + item_r * kPitch + item_seg * 64);
#pragma unroll
      for (int i = 0; i < 8; ++i) dst[i] = d[i];
    }
    lds_barrier();
    if (step + 2 < n_steps) fetch(raw, step + 2);

    // ---- logits S^T: lane (g, n) gets rows 16*rt + 4g + i of head n
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    {
      const uint16_t* qr = s_q + n * kPitch + 8 * g;
      const uint16_t* k0 = tile + n * kPitch + 8 * g;
      const uint16_t* k1 = tile + (16 + n) * kPitch + 8 * g;
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const f16x8 qb = as_f16x8(*reinterpret_cast<const u32x4*>(qr + 32 * t));
        sacc[0] = mfma16x16x32_f16(as_f16x8(*reinterpret_cast<const u32x4*>(k0 + 32 * t)), qb, sacc[0]);
        sacc[1] = mfma16x16x32_f16(as_f16x8(*reinterpret_cast<const u32x4*>(k1 + 32 * t)), qb, sacc[1]);
      }
    }
    // ---- online softmax (log2 domain)
    float x[8];
    float mloc = -INFINITY;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * g + i;
        const float v = s_rows[step * kStepRows + r] >= 0 ? sacc[rt][i] * scale_log2 : -INFINITY;
        x[4 * rt + i] = v;
        mloc = fmaxf(mloc, v);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(m_run, mloc);
    float psum = 0.0f;
    uint32_t pw[4];
    if (m_new == -INFINITY) {
      pw[0] = pw[1] = pw[2] = pw[3] = 0u;
    } else {
      float pv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pv[i] = exp2f(x[i] - m_new);
        psum += pv[i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) pw[i] = f32_to_f16_bits(pv[2 * i]) | (f32_to_f16_bits(pv[2 * i + 1]) << 16);
    }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    const float alpha = (m_run == -INFINITY) ? 0.0f : exp2f(m_run - m_new);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (alpha != 1.0f) {
#pragma unroll
      for (int i = 0; i < kDimsPerWave / 16; ++i) o[i] *= alpha;
    }
    // ---- O^T += V^T P^T over this wave's dims (K-slots 8g+s <-> rows 4g+s, 16+4g+s-4)
    const f16x8 pb = as_f16x8(u32x4{pw[0], pw[1], pw[2], pw[3]});
#pragma unroll
    for (int i = 0; i < kDimsPerWave / 16; ++i)
      o[i] = mfma16x16x32_f16(v_fragment(tile, g, n, (kDimsPerWave / 16) * wave + i), pb, o[i]);
  };

  if (n_steps > 0) fetch(raw0, 0);
  if (n_steps > 1) fetch(raw1, 1);
  for (int step = 0; step < n_steps; step += 2) {
    run_step(raw0, step);
    if (step + 1 < n_steps) run_step(raw1, step + 1);
  }

  // ---- partial records: the 16 x 512 output block is staged through LDS so that each
  // head's 2 KB record is written by consecutive lanes in whole cache lines; the
  // (max, sum) pairs go to their own array.
  const int64_t rec0 = ((int64_t)b * n_chunks + chunk) * n_heads + 16 * hg;
  lds_barrier();  // every wave is done with the tiles and the query rows
  if (wave == 0 && g == 0) *reinterpret_cast<f32x2*>(part_ml + (rec0 + n) * 2) = f32x2{m_run, l_run};
  {
    float* orow = s_out + n * kOutPitch + kDimsPerWave * wave + 4 * g;
#pragma unroll
    for (int i = 0; i < kDimsPerWave / 16; ++i) *reinterpret_cast<f32x4*>(orow + 16 * i) = o[i];
  }
  lds_barrier();
  constexpr int kVecPerHead = kDim / 4;
#pragma unroll
  for (int k = 0; k < 16 * kVecPerHead / kAttnThreads; ++k) {
    const int i = threadIdx.x + k * kAttnThreads;
    const int h = i / kVecPerHead, c4 = i - h * kVecPerHead;
    *reinterpret_cast<f32x4*>(part_o + (rec0 + h) * kDim + 4 * c4) =
        *reinterpret_cast<const f32x4*>(s_out + h * kOutPitch + 4 * c4);
  }
}

// One workgroup per (query, head): merges the chunks' (max, sum, O) records.  Up to
// kCombineBatch chunks are read in a single round of independent loads (records, maxima
// and sums together); more chunks take further rounds.
constexpr int kCombineThreads = 128;   // 4 dims each
constexpr int kCombineBatch = 32;

__global__ __launch_bounds__(kCombineThreads) void attention_combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml, int n_heads,
    int n_chunks, uint16_t* __restrict__ out) {
  __shared__ float s_m[kMaxChunks];
  __shared__ float s_l[kMaxChunks];
  const int bh = blockIdx.x;  // b * n_heads + h
  const int b = bh / n_heads, h = bh - b * n_heads;
  const int64_t cstride = (int64_t)n_heads * kDim;
  const float* base = part_o + ((int64_t)b * n_chunks * n_heads + h) * kDim;
  const float* mlb = part_ml + ((int64_t)b * n_chunks * n_heads + h) * 2;
  const int d0 = 4 * threadIdx.x;

  f32x4 v[kCombineBatch];
#pragma unroll
  for (int i = 0; i < kCombineBatch; ++i)
    v[i] = i < n_chunks ? *reinterpret_cast<const f32x4*>(base + i * cstride + d0)
                        : f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c = threadIdx.x; c < n_chunks; c += kCombineThreads) {
    const f32x2 ml = *reinterpret_cast<const f32x2*>(mlb + (int64_t)c * n_heads * 2);
    s_m[c] = ml[0];
    s_l[c] = ml[1];
  }
  lds_barrier();
  // Every thread reduces the (few) maxima and sums itself: no further barriers.
  float mmax = -INFINITY;
  for (int c = 0; c < n_chunks; ++c) mmax = fmaxf(mmax, s_m[c]);
  float den = 0.0f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (mmax != -INFINITY) {
    for (int c0 = 0; c0 < n_chunks; c0 += kCombineBatch) {
      if (c0 > 0) {
#pragma unroll
        for (int i = 0; i < kCombineBatch; ++i)
          v[i] = c0 + i < n_chunks ? *reinterpret_cast<const f32x4*>(base + (c0 + i) * cstride + d0)
                                   : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int i = 0; i < kCombineBatch; ++i) {
        if (c0 + i < n_chunks) {
          const float wt = exp2f(s_m[c0 + i] - mmax);  // 0 for empty chunks (max -inf)
          den += s_l[c0 + i] * wt;
          acc += v[i] * wt;
        }
      }
    }
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  const uint32_t lo = f32_to_bf16_rne(acc[0] * inv) | (f32_to_bf16_rne(acc[1] * inv) << 16);
  const uint32_t hi = f32_to_bf16_rne(acc[2] * inv) | (f32_to_bf16_rne(acc[3] * inv) << 16);
  *reinterpret_cast<u32x2*>(out + (int64_t)bh * kDim + d0) = u32x2{lo, hi};
}

int attention_blocks(int batch, int n_heads, const AttnPlan& plan) {
  const int n_pairs = batch * plan.n_chunks;
  return 8 * (n_heads / 16) * ((n_pairs + 7) / 8);
}

template <int KVFMT, bool CSA>
void launch_chunks(hipStream_t stream, const uint8_t* codes, const uint8_t* scales,
                   int64_t seq_stride, int64_t n_rows, const uint16_t* q, int batch, int n_heads,
                   float scale_log2, const int32_t* topk, int top_k, int window,
                   const AttnPlan& plan, float* part_o, float* part_ml) {
  const dim3 grid(attention_blocks(batch, n_heads, plan));
  const int n_pairs = batch * plan.n_chunks;
#define CSAKV_CHUNK(NB)                                                                         \
  hipLaunchKernelGGL((attention_chunk_kernel<KVFMT, CSA, NB>), grid, dim3(kAttnThreads), 0,      \
                     stream, codes, scales, seq_stride, n_rows, q, n_heads, scale_log2, topk,    \
                     top_k, window, plan.n_list, plan.rows_per_chunk, plan.n_chunks, n_pairs,   \
                     part_o, part_ml)
  if (plan.rows_per_chunk <= kStepRows) CSAKV_CHUNK(1);
  else CSAKV_CHUNK(2);
#undef CSAKV_CHUNK
}

}  // namespace

AttnPlan plan_attention(int batch, int64_t n_list, bool csa, int n_heads) {
  AttnPlan p{};
  p.n_list = n_list;
  // Chunks of whole 32-row steps; about 256 workgroups in all, each one
  // (query, chunk, 16-head group), never more than kMaxChunks chunks per query.
  const int64_t groups = n_heads / 16 > 0 ? n_heads / 16 : 1;
  const int64_t want = (256 + batch * groups - 1) / (batch * groups);
  int64_t rpc = (n_list + want - 1) / want;
  const int64_t floor_rows = (n_list + kMaxChunks - 1) / kMaxChunks;
  if (rpc < floor_rows) rpc = floor_rows;
  if (rpc < kStepRows) rpc = kStepRows;
  rpc = ((rpc + kStepRows - 1) / kStepRows) * kStepRows;
  p.rows_per_chunk = (int)(rpc < kMaxChunkRows ? rpc : kMaxChunkRows);
  p.n_chunks = (int)((n_list + p.rows_per_chunk - 1) / p.rows_per_chunk);
  (void)csa;
  return p;
}

bool attention_supported(const AttnPlan& plan) {
  return plan.n_chunks <= kMaxChunks && plan.rows_per_chunk <= kMaxChunkRows;
}

// Workspace: O records [B][chunks][H][512] fp32, then (max, sum) pairs [B][chunks][H][2].
size_t attention_workspace_bytes(int batch, int n_heads, const AttnPlan& plan) {
  return (size_t)batch * plan.n_chunks * n_heads * (kDim + 2) * sizeof(float);
}

hipError_t launch_attention(int kv_fmt, bool csa, const uint8_t* codes, const uint8_t* scales,
                            int64_t seq_stride, int64_t n_rows, const uint16_t* q, int batch,
                            int n_heads, float softmax_scale, const int32_t* topk, int top_k,
                            int window, const AttnPlan& plan, void* workspace, uint16_t* out,
                            hipStream_t stream) {
  float* part_o = static_cast<float*>(workspace);
  float* part_ml = part_o + (size_t)batch * plan.n_chunks * n_heads * kDim;
  const float sl2 = softmax_scale * kLog2e;
  if (plan.n_chunks > 0) {
#define CSAKV_ATTN(F, C)                                                                        \
  launch_chunks<F, C>(stream, codes, scales, seq_stride, n_rows, q, batch, n_heads, sl2, topk, \
                      top_k, window, plan, part_o, part_ml)
    if (csa) {
      if (kv_fmt == 0) CSAKV_ATTN(0, true);
      else if (kv_fmt == 1) CSAKV_ATTN(1, true);
      else CSAKV_ATTN(2, true);
    } else {
      if (kv_fmt == 0) CSAKV_ATTN(0, false);
      else if (kv_fmt == 1) CSAKV_ATTN(1, false);
      else CSAKV_ATTN(2, false);
    }
#undef CSAKV_ATTN
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(attention_combine_kernel, dim3(batch * n_heads), dim3(kCombineThreads), 0,
                     stream, part_o, part_ml, n_heads, plan.n_chunks, out);
  return hipGetLastError();
}

}  // namespace csakv
