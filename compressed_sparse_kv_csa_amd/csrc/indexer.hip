// Lightning-indexer scoring and top-k selection for CSA decode.
//
// What is computed ("DeepSeek-V4 KV Cache 深度分析", section 四 "索引器（Indexer）机制" and
// the section 十一 forward-flow diagram): the query token's indexer query is scored
// against the indexer key of every compressed entry, and the top-k entries are kept.
// Score s_j = sum_h w_h * ReLU(q_h . k_j); ties are broken toward the smaller index.
//
// Two launches per call:
//   1. scan kernel, about one workgroup per CU.  A workgroup owns a run of consecutive
//      4096-row slices of one query.  Its 8 waves stream 16-row key tiles from HBM
//      straight into registers through a 4-deep prefetch ring that runs on across slice
//      boundaries.  Each tile is one [H_I x 128] x [128 x 16] contraction on 16x16x32
//      MFMA with fp32 accumulation; ReLU, the head weights and the head sum are applied
//      to the accumulators and the scores stay in LDS.  When a slice is complete, one
//      2048-bin histogram of its score keys (between the slice's min and max) gives the
//      lower edge t of the bin holding the slice's P-th largest score.  Every key >= t
//      is emitted as a candidate, and t is recorded as the slice's bound: all keys not
//      emitted lie below it.  The slice's scores are also written out, for the merge's
//      rare second look.
//   2. merge kernel, one workgroup per query: the exact k-th largest candidate key, by a
//      histogram of the candidates and a direct ranking of the one bin that holds it.  A
//      slice whose bound lies above that key may hide further winners; its stored scores
//      are re-read and the selection repeated, so the result is exact for any input.
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

#include <algorithm>

#include "topk_select.h"

namespace csakv {

namespace {

constexpr int kIdxDim = 128;
constexpr int kScanWaves = 8;
constexpr int kScanThreads = kScanWaves * kWave;
constexpr int kRing = 4;   // tiles in flight per wave (a group); divides kSliceRows / 16
constexpr int kMergeThreads = 512;  // one thread per slice count at most kMaxMergeSlices
constexpr int kMergeFirstPerThread = kMergeFirstSlots / kMergeThreads;  // first-round slots per thread
static_assert(kMaxMergeSlices <= kMergeThreads, "the merge reads one slice count per thread");

// ------------------------------------------------------------------ key tiles

// Lane (g, n) owns row n of a 16-row tile and 32 of its 128 channels.  Tiles are read
// through buffer resources whose base is the tile's first row and whose size covers the
// tile's rows that exist: a row past the end reads as zeros (no clamping, no fault), and
// every lane's offset inside a tile is a constant.

// bf16 rows: in K-step t the lane supplies channels 32t + 8g .. 32t + 8g + 7.
struct KeyTileBf16 {
  typedef bf16x8 Op;
  u32x4 c[4];
  static constexpr int kRowBytes = kIdxDim * 2;
  static constexpr bool kScales = false;
  static __device__ __forceinline__ int code_offset(int n, int g) { return n * kRowBytes + 16 * g; }
  static __device__ __forceinline__ int scale_offset(int, int) { return 0; }
  __device__ __forceinline__ void set_lane(int) {}
  __device__ __forceinline__ void load(Rsrc rc, Rsrc, int co, int) {
#pragma unroll
    for (int t = 0; t < 4; ++t) c[t] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, co + 64 * t, 0, 0));
  }
  __device__ __forceinline__ void decode(Op* op) const {
#pragma unroll
    for (int t = 0; t < 4; ++t) op[t] = as_bf16x8(c[t]);
  }
  static __device__ __forceinline__ int q_channel(int g, int t) { return 32 * t + 8 * g; }
  static __device__ __forceinline__ f32x4 mma(Op a, Op b, f32x4 c) { return mfma16x16x32(a, b, c); }
};

// FP4 rows: the lane loads channels 32g .. 32g + 31 (16 code bytes) and the dword of
// scale bytes holding their two scales; in K-step t it supplies channels
// 32g + 8t .. 32g + 8t + 7 as exact fp16.
struct KeyTileFp4 {
  typedef f16x8 Op;
  u32x4 c;
  uint32_t s;   // scales of blocks 4(g >> 1) .. 4(g >> 1) + 3, one byte each
  uint32_t sh;  // 16 for odd g: the lane's two scale bytes are the dword's upper half
  __device__ __forceinline__ void set_lane(int g) { sh = 16u * (g & 1); }
  static constexpr int kRowBytes = kIdxDim / 2;
  static constexpr bool kScales = true;
  static __device__ __forceinline__ int code_offset(int n, int g) { return n * kRowBytes + 16 * g; }
  static __device__ __forceinline__ int scale_offset(int n, int g) { return n * (kIdxDim / 16) + 4 * (g >> 1); }
  __device__ __forceinline__ void load(Rsrc rc, Rsrc rs, int co, int so) {
    c = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, co, 0, 0));
    s = __builtin_amdgcn_raw_buffer_load_b32(rs, so, 0, 0);
  }
  __device__ __forceinline__ void decode(Op* op) const {
    // Both E4M3 scales as an fp16 pair (exact); each multiply broadcasts one of them.
    const f16x2 sp = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s >> sh, 1.0f, false);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const f16x2 sc = t < 2 ? f16x2{sp[0], sp[0]} : f16x2{sp[1], sp[1]};
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

// Query b's indexer query fragments (A operand: head n of each 16-head tile, the lane's
// K-channels) and the weights of the accumulator rows lane (g, n) holds (heads
// 16*ht + 4g + i); heads past n_heads get zeros.
// 8 FP4 codes (one dword) times their E4M3 scale, as exact fp16 values.
__device__ __forceinline__ f16x8 fp4x8_to_f16(uint32_t cw, uint32_t scale_code) {
  const uint32_t sp = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(scale_code, 1.0f, false));
  const f16x2 sc = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(sp, sp, 0x01000100u));
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 0) * sc);
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 1) * sc);
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 2) * sc);
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 3) * sc);
  return as_f16x8(r);
}

// The bf16 indexer-query fragments wave w of NW converts: head tiles w, w + NW, ...; lane
// (g, n) holds head 16 * ht + n's channels KT::q_channel(g, t) (zeros past n_heads).  Loaded
// apart from their conversion so that a kernel can issue them ahead of its key loads and
// wait for them alone: the loads go through a buffer resource over query b's rows (a head
// past n_heads reads zeros), so none of them sits behind a per-lane branch, which would
// make the compiler wait for the earlier ones before issuing the rest.
template <class KT, int HT, int NW>
struct QueryRaw {
  static constexpr int kPer = (HT + NW - 1) / NW;  // head tiles per wave
  u32x4 v[kPer][4];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ q_idx, int b, int n_heads, int wave,
                                       int g, int n) {
    const Rsrc rq = make_rsrc(q_idx + (int64_t)b * n_heads * kIdxDim, (uint32_t)(n_heads * kIdxDim * 2));
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int row = 16 * (wave + NW * i) + n;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v[i][t] = u32x4{0u, 0u, 0u, 0u};
        if (wave + NW * i < HT)  // wave-uniform
          v[i][t] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, (row * kIdxDim + KT::q_channel(g, t)) * 2, 0, 0));
      }
    }
  }
};

// Rotated FP4 queries: whether a second wave quantises half of each head tile, and the
// LDS the preparation needs.
template <int HT, int NW>
constexpr bool kFp4hSplit = 2 * HT <= NW;

template <int HT, int NW>
constexpr size_t fp4h_stage_bytes() {
  return sizeof(f16x8) * HT * 4 * kWave + (kFp4hSplit<HT, NW> ? sizeof(float) * HT * 16 * kWave : 0);
}

// Hadamard-rotated FP4 indexer queries (keys stored in the same form).  Wave w of the NW
// waves prepares head tiles w, w + NW, ...; for head tile ht the 4 lanes g of head n's row hold its channels
// 32g .. 32g+31 in fp64 and rotate the row together (stages h = 1..16 in registers, h = 32
// and 64 across lanes g ^ 1 and g ^ 2; every sum is exact), round each value once to fp32
// and scale it once, quantise their two 16-channel blocks with the FP4 codec, and leave the
// decoded values (exact in fp16, in the FP4 key tile's channel order) in LDS, from where
// every wave takes its A operands.  With at most NW / 2 head tiles, wave ht + NW / 2
// quantises the second block of wave ht's lanes (handed over through LDS) while wave ht
// quantises the first.  `stage` holds HT * 4 * 64 fragments, and then HT * 16 * 64 floats
// when the blocks are split; it is free again when this returns.
template <int HT, int NW>
__device__ __forceinline__ void query_frags_fp4h(const QueryRaw<KeyTileFp4, HT, NW>& raw, int wave, int g,
                                                 f16x8 (&qa)[HT][4], f16x8* stage) {
  constexpr bool kSplit = kFp4hSplit<HT, NW>;
  float* const handover = reinterpret_cast<float*>(stage + HT * 4 * kWave);  // kSplit only
  const int lane = threadIdx.x & (kWave - 1);
  float yf[32];
#pragma unroll
  for (int i = 0; i < QueryRaw<KeyTileFp4, HT, NW>::kPer; ++i) {
    const int ht = wave + NW * i;
    if (ht >= HT) continue;  // wave-uniform
    double y[32];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const u32x4 v = raw.v[i][k];  // channels 32g + 8k .. + 7
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        y[8 * k + 2 * j] = (double)bf16_to_f32(v[j] & 0xFFFFu);
        y[8 * k + 2 * j + 1] = (double)bf16_to_f32(v[j] >> 16);
      }
    }
    hadamard_stages<32>(y);
    hadamard_lane_stage<32>(y, 16, (g & 1) != 0);  // h = 32: lanes g, g ^ 1
    hadamard_lane_stage<32>(y, 32, (g & 2) != 0);  // h = 64: lanes g, g ^ 2
#pragma unroll
    for (int j = 0; j < 32; ++j) yf[j] = hadamard_round_scale(y[j]);
    if constexpr (kSplit) {
#pragma unroll
      for (int j = 0; j < 16; ++j) handover[(ht * 16 + j) * kWave + lane] = yf[16 + j];
    } else {
      u32x2 c0, c1;
      uint32_t s0, s1;
      fp4_block_f32(yf, &c0, &s0);
      fp4_block_f32(yf + 16, &c1, &s1);
      f16x8* out = stage + ht * 4 * kWave + lane;
      out[0 * kWave] = fp4x8_to_f16(c0[0], s0);
      out[1 * kWave] = fp4x8_to_f16(c0[1], s0);
      out[2 * kWave] = fp4x8_to_f16(c1[0], s1);
      out[3 * kWave] = fp4x8_to_f16(c1[1], s1);
    }
  }
  if constexpr (kSplit) {  // kPer is 1: wave ht < HT holds its first block in yf
    lds_barrier();
    const int ht = wave < NW / 2 ? wave : wave - NW / 2;
    if (ht < HT) {  // wave-uniform
      const bool second = wave >= NW / 2;
      if (second) {
#pragma unroll
        for (int j = 0; j < 16; ++j) yf[j] = handover[(ht * 16 + j) * kWave + lane];
      }
      u32x2 c;
      uint32_t sc;
      fp4_block_f32(yf, &c, &sc);
      f16x8* out = stage + (ht * 4 + (second ? 2 : 0)) * kWave + lane;
      out[0] = fp4x8_to_f16(c[0], sc);
      out[kWave] = fp4x8_to_f16(c[1], sc);
    }
  }
  lds_barrier();
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int t = 0; t < 4; ++t) qa[ht][t] = stage[(ht * 4 + t) * kWave + lane];
  lds_barrier();
}

// Head weight h = threadIdx.x of query b (zero past n_heads; threads from 16 * HT on are
// not used), loaded at kernel entry ahead of the key loads.  The weights reach every lane
// through LDS: loaded straight into the registers the tile loop reads, their completion
// would be waited for behind the key prefetches in the tile loop.
template <int HT>
__device__ __forceinline__ float query_weight_load(const float* __restrict__ w_idx, int b,
                                                   int n_heads) {
  // A buffer resource over query b's weights: a thread past n_heads reads zero, no branch.
  const Rsrc rw = make_rsrc(w_idx + (int64_t)b * n_heads, (uint32_t)(n_heads * 4));
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rw, (int)threadIdx.x * 4, 0, 0));
}

// The query fragments of query b, bf16 indexer queries, prepared once per workgroup from
// `raw`: wave w of the NW waves takes the largest magnitudes of head tiles w, w + NW, ...;
// all waves then agree on the query's power-of-two scale (fp16 path), each wave converts its
// tiles' fragments into LDS, and every wave takes all of them.  `red` holds HT floats,
// `stage` HT * 256 fragments; both are free again when this returns.
template <class KT, int HT, int NW>
__device__ __forceinline__ void query_frags_staged(const QueryRaw<KT, HT, NW>& qr, int wave,
                                                   typename KT::Op (&qa)[HT][4], u32x4* stage,
                                                   float* red) {
  typedef typename KT::Op Op;
  const int lane = threadIdx.x & (kWave - 1);
  constexpr int kPer = QueryRaw<KT, HT, NW>::kPer;
  const auto& raw = qr.v;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int ht = wave + NW * i;
    if (ht < HT) {  // wave-uniform
      float qmax = 0.0f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const u32x4 v = raw[i][t];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          qmax = fmaxf(qmax, fmaxf(fabsf(bf16_to_f32(v[j] & 0xFFFFu)), fabsf(bf16_to_f32(v[j] >> 16))));
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) qmax = fmaxf(qmax, __shfl_xor(qmax, off));
      if (lane == 0) red[ht] = qmax;
    }
  }
  lds_barrier();
  float qmax = red[0];
#pragma unroll
  for (int ht = 1; ht < HT; ++ht) qmax = fmaxf(qmax, red[ht]);
  // Power of two putting max|q| in [2^14, 2^15) (used by the fp16 path only).
  int p = 0;
  if (qmax > 0.0f) p = 14 - ((int)((__float_as_uint(qmax) >> 23) & 0xFF) - 127);
  p = max(-100, min(p, 100));
  const float qscale = __builtin_ldexpf(1.0f, p);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int ht = wave + NW * i;
    if (ht < HT) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        stage[(ht * 4 + t) * kWave + lane] = __builtin_bit_cast(u32x4, q_operand(raw[i][t], qscale, (Op*)nullptr));
    }
  }
  lds_barrier();
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int t = 0; t < 4; ++t) qa[ht][t] = __builtin_bit_cast(Op, stage[(ht * 4 + t) * kWave + lane]);
  lds_barrier();
}

// The query fragments and head weights of query b, prepared once per workgroup (every
// wave must call this: it holds barriers).  QH: Hadamard-rotated FP4 queries.  `raw`: this
// wave's QueryRaw::load.  `stage`: LDS for HT * 256 fragments; `red`: LDS for HT floats;
// `s_w`: LDS for 16 * HT floats, which the caller keeps until every wave has left this
// function.  `w_pre`: this thread's query_weight_load.  wv gets the weights of the
// accumulator rows lane (g, n) holds (heads 16*ht + 4g + i).
template <class KT, int HT, bool QH, int NW>
__device__ __forceinline__ void query_setup(const QueryRaw<KT, HT, NW>& raw, float w_pre, int wave, int g,
                                            typename KT::Op (&qa)[HT][4], float (&wv)[HT][4],
                                            void* stage, float* red, float* s_w) {
  if (threadIdx.x < 16 * HT) s_w[threadIdx.x] = w_pre;  // ordered by the barriers below
  if constexpr (QH) {
    static_assert(KT::kScales, "rotated FP4 queries meet rotated FP4 keys");
    query_frags_fp4h<HT, NW>(raw, wave, g, qa, static_cast<f16x8*>(stage));
  } else {
    query_frags_staged<KT, HT, NW>(raw, wave, qa, static_cast<u32x4*>(stage), red);
  }
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[ht][i] = s_w[16 * ht + 4 * g + i];
}

// Lane (g, n)'s share of the score of its tile row n: the sum over the heads it holds
// (16 * ht + 4g + i) of w_h * ReLU(acc).  The four lane groups' shares add up to the
// score.  ReLU is a signed-integer max: negative floats (and -0) have the sign bit set.
template <int N, int HT>
__device__ __forceinline__ float weighted_relu_share(const f32x4 (&acc)[N], const float (&wv)[HT][4],
                                                     int hg, float sc = 0.0f) {
#pragma unroll
  for (int ht = 0; ht < N; ++ht)
#pragma unroll
    for (int i = 0; i < 4; ++i) sc += wv[hg + ht][i] * __int_as_float(max(__float_as_int(acc[ht][i]), 0));
  return sc;
}

// Lane (g, n)'s share of the score of key-tile row n for all HT head tiles: the MFMAs of
// up to 4 head tiles at a time (so that at most 4 accumulators are live), each group's
// ReLU-weighted heads added to the share.
template <class KT, int HT>
__device__ __forceinline__ float tile_share(const typename KT::Op (&qa)[HT][4],
                                            const typename KT::Op (&kb)[4], const float (&wv)[HT][4]) {
  constexpr int G = HT < 4 ? HT : 4;
  float sc = 0.0f;
#pragma unroll
  for (int hg = 0; hg < HT; hg += G) {
    f32x4 acc[G];
#pragma unroll
    for (int i = 0; i < G; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < G; ++i) acc[i] = KT::mma(qa[hg + i][t], kb[t], acc[i]);
    sc = weighted_relu_share<G, HT>(acc, wv, hg, sc);
  }
  return sc;
}

// ------------------------------------------------------------------ scan kernel


// Per-call buffers of the indexer, carved from the caller's workspace.

template <class KT, int HT, bool QH, bool PG>
__global__ __launch_bounds__(kScanThreads) void indexer_scan_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t seq_stride,
    const int32_t* __restrict__ page_table, int page_shift, int table_stride, int64_t n_c,
    const int32_t* __restrict__ seq_rows, const uint16_t* __restrict__ q_idx,
    const float* __restrict__ w_idx, int n_heads, int n_slices, int slices_per_wg,
    int wg_per_query, int prefix, int cap, IndexerWs ws) {
  typedef typename KT::Op Op;
  // Per row of the current slice, the four lane groups' shares of its score (float4);
  // first the query setup's staging area.
  __shared__ __attribute__((aligned(16))) float s_part[kSliceRows * 4];
  __shared__ uint32_t s_score[kSliceRows];  // order keys of the slice's scores
  __shared__ SelectSmem sm;
  __shared__ uint32_t s_next;  // the next group of the current slice to hand out

  args_in_sgprs(codes, scales, seq_stride, page_table, page_shift, table_stride, n_c, seq_rows, q_idx,
                w_idx, n_heads, n_slices, slices_per_wg, wg_per_query, prefix, cap, ws.cand, ws.bound,
                ws.count, ws.scores);
  const int b = blockIdx.x / wg_per_query;
  const int slice0 = (blockIdx.x - b * wg_per_query) * slices_per_wg;
  const int n_sl = min(slices_per_wg, n_slices - slice0);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // scalar tile math
  const int lane = threadIdx.x & (kWave - 1);
  const int g = lane >> 4;
  const int n = lane & 15;
  const int64_t row_base = (int64_t)slice0 * kSliceRows;              // compressed row index
  const int64_t n_cb = seq_len(seq_rows, b, n_c);                     // this sequence's rows
  const int64_t rows_total = max(min((int64_t)n_sl * kSliceRows, n_cb - row_base), (int64_t)0);
  const int64_t seq_row0 = (int64_t)b * seq_stride + row_base;
  // Slices of the run past the sequence's end send nothing.
  const int n_done = (int)((rows_total + kSliceRows - 1) / kSliceRows);
  if (threadIdx.x < n_sl - n_done) {
    const int64_t si = (int64_t)b * n_slices + slice0 + n_done + threadIdx.x;
    ws.count[si] = 0u;
    ws.bound[si] = 0ull;
  }
  if (n_done == 0) return;  // the whole workgroup: no barrier is left waiting

  // Work balancing.  A slice's rows are taken in groups of RING 16-row tiles, one ring's
  // worth.  Each wave starts a slice on its own group (group `wave`) and takes further
  // groups from a workgroup counter in LDS, so that waves the SIMD serves unequally (it
  // favours the older of the two waves it holds) still finish a slice together.  The ring
  // holds the current group's tiles and is refilled, tile by tile, with the next group's,
  // which is known one group ahead (its counter value is fetched while the group before it
  // runs).  Once a slice's groups are handed out, a wave's next group is its own group of
  // the following slice, so the ring runs on across slices and starts every slice at slot
  // 0.  Every refill loads (rows past the end read zeros); a row past the end lands in its
  // slice's buffer at or after the slice's last row, where nothing reads it.  Groups are
  // numbered across the workgroup's slices: group G belongs to slice G / kSliceGroups.
  // With more than 64 heads the bf16 ring is halved: 128 heads' query fragments take 128
  // registers.
  constexpr int RING = (HT > 4 && !KT::kScales) ? 2 : kRing;
  constexpr int kGroupRows = 16 * RING;
  constexpr int kSliceGroups = kSliceRows / kGroupRows;
  const uint8_t* kcodes = codes + seq_row0 * KT::kRowBytes;
  const uint8_t* kscales = KT::kScales ? scales + seq_row0 * (kIdxDim / 16) : nullptr;
  const int lane_co = KT::code_offset(n, g), lane_so = KT::scale_offset(n, g);
  const int rows_wg = (int)rows_total;  // at most 512 slices of 4096 rows: 32-bit math
  auto load_tile = [&](KT& kt, int grp, int d) {
    const int r0 = grp * kGroupRows + 16 * d;  // wave-uniform (scalar)
    // The resource covers the rows from r0 to the end of the workgroup's rows; the tile
    // reads at most 16 of them.
    const int live = max(rows_wg - r0, 0);
    const uint8_t* tc = kcodes + (int64_t)r0 * KT::kRowBytes;
    const uint8_t* ts = KT::kScales ? kscales + (int64_t)r0 * (kIdxDim / 16) : nullptr;
    if constexpr (PG) {  // paged: a 16-row tile lies within one page (pages hold 2^k >= 16 rows)
      const int64_t r = row_base + r0;  // row of the sequence
      // (a tile past the end reads nothing; its table index is kept inside the table)
      // (read-only and wave-uniform: a scalar load, waited for apart from the key loads)
      const int64_t e = min(r >> page_shift, (int64_t)table_stride - 1);
      const int64_t pr = ((int64_t)page_table[(int64_t)b * table_stride + e] << page_shift) +
                         (r & ((1 << page_shift) - 1));
      tc = codes + pr * KT::kRowBytes;
      if (KT::kScales) ts = scales + pr * (kIdxDim / 16);
    }
    const Rsrc rc = make_rsrc(tc, (uint32_t)(live * KT::kRowBytes));
    const Rsrc rs = KT::kScales ? make_rsrc(ts, (uint32_t)(live * (kIdxDim / 16))) : rc;
    kt.load(rc, rs, lane_co, lane_so);
  };

  // The query's raw fragments and head weights go out first, so that the set-up waits for
  // them alone; the ring's first loads (the wave's group of the first slice) follow and
  // overlap the set-up.
  QueryRaw<KT, HT, kScanWaves> qraw;
  qraw.load(q_idx, b, n_heads, wave, g, n);
  const float w_pre = query_weight_load<HT>(w_idx, b, n_heads);
  KT ring[RING];
#pragma unroll
  for (int d = 0; d < RING; ++d) {
    ring[d].set_lane(g);
    load_tile(ring[d], wave, d);
  }
  if (threadIdx.x == 0) s_next = kScanWaves;  // the first slice's counter, ordered by the set-up's barriers

  // Indexer query fragments and head weights.
  Op qa[HT][4];
  float wv[HT][4];
  static_assert(sizeof(s_part) >= sizeof(f16x8) * HT * 4 * kWave, "query stage");
  static_assert(!QH || sizeof(s_part) >= fp4h_stage_bytes<HT, kScanWaves>(), "rotated query stage");
  static_assert(sizeof(sm.hist) >= sizeof(float) * 16 * HT, "weight stage");
  static_assert(sizeof(sm.red32) >= sizeof(float) * HT, "query maxima");
  query_setup<KT, HT, QH, kScanWaves>(qraw, w_pre, wave, g, qa, wv, s_part,
                                      reinterpret_cast<float*>(sm.red32), reinterpret_cast<float*>(sm.hist));

  // Lane (g, n)'s share of the score of slice row r goes to s_part[4 * r + g].
  const int lane_part = 4 * n + g;
  int gc = wave;  // the group in the ring
  for (int j = 0;; ++j) {
    const int64_t srow0 = row_base + (int64_t)j * kSliceRows;
    const int rows = (int)min((int64_t)kSliceRows, n_cb - srow0);
    const int n_groups = (rows + kGroupRows - 1) / kGroupRows;
    // The group that follows counter value c of this slice.
    auto group_after = [&](uint32_t c) -> int {
      return (int)c < n_groups ? kSliceGroups * j + (int)c : kSliceGroups * (j + 1) + wave;
    };
    // The group after the wave's first of this slice (the counter was set before the last
    // barrier every wave has passed).
    uint32_t cv = 0u;
    if (lane == 0) cv = atomicAdd(&s_next, 1u);
    int gn = group_after(__builtin_amdgcn_readfirstlane(cv));
    while (gc < kSliceGroups * (j + 1)) {  // the ring holds a group of slice j
      const bool more = gn < kSliceGroups * (j + 1);
      cv = 0u;
      if (more && lane == 0) cv = atomicAdd(&s_next, 1u);  // the group after gn, read after this one
      float* const gpart = s_part + 4 * kGroupRows * (gc - kSliceGroups * j) + lane_part;
#pragma unroll
      for (int d = 0; d < RING; ++d) {
        // Keep each tile's instructions together: hoisting a later tile's decode above
        // this point would wait on that tile's key load, which is still in flight.
        __builtin_amdgcn_sched_barrier(0);
        Op kb[4];
        ring[d].decode(kb);
        load_tile(ring[d], gn, d);  // past the end: reads zeros
        // Each lane stores its share; the shares are added when the slice is complete.
        gpart[4 * 16 * d] = tile_share<KT, HT>(qa, kb, wv);
      }
      __builtin_amdgcn_sched_barrier(0);
      gc = gn;
      gn = more ? group_after(__builtin_amdgcn_readfirstlane(cv)) : -1;
    }

    // ---- slice complete: emit its candidates, its bound and its scores
    const int64_t si = (int64_t)b * n_slices + slice0 + j;
    lds_barrier();  // every wave's shares of the slice are in
    // Thread t adds up the shares of rows t + 512r and keeps their keys in registers, on
    // the way clearing the histogram and taking the keys' minimum and maximum.
    constexpr int kRpt = kSliceRows / kScanThreads;
    uint32_t* sc_out = ws.scores + (int64_t)b * n_c + srow0;
    uint32_t key[kRpt];
    uint32_t mn = ~0u, mx = 0u;
#pragma unroll
    for (int r = 0; r < kRpt; ++r) {
      const int i = threadIdx.x + kScanThreads * r;
      key[r] = 0u;
      if (i < rows) {
        const f32x4 p = *reinterpret_cast<const f32x4*>(s_part + 4 * i);
        key[r] = f32_order_key((p[0] + p[1]) + (p[2] + p[3]));
        s_score[i] = key[r];
        sc_out[i] = key[r];
        mn = key[r] < mn ? key[r] : mn;
        mx = key[r] > mx ? key[r] : mx;
      }
    }
    for (int i = threadIdx.x; i < kHistBins; i += kScanThreads) sm.hist[i] = 0;
    wave_minmax_u32(mn, mx);
    if (lane == 0) {
      sm.red32[wave] = mn;
      sm.red32[16 + wave] = mx;
    }
    lds_barrier();
    mn = sm.red32[0];
    mx = sm.red32[16];
#pragma unroll
    for (int w = 1; w < kScanWaves; ++w) {
      mn = sm.red32[w] < mn ? sm.red32[w] : mn;
      mx = sm.red32[16 + w] > mx ? sm.red32[16 + w] : mx;
    }
    const int pe = min(prefix, rows);
    uint32_t t32 = 0u, cnt = (uint32_t)rows;
    if (pe < rows) slice_threshold<kScanThreads>(key, rows, pe, mn, mx, sm, &t32, &cnt);
    uint64_t* dst = ws.cand + si * cap;
    uint64_t bound;
    uint32_t emitted;
    if (cnt <= (uint32_t)cap) {  // every key whose score is >= t32, wave by wave, row order
      uint32_t wc = 0;
#pragma unroll
      for (int r = 0; r < kRpt; ++r)
        wc += (uint32_t)__builtin_popcountll(
            __ballot((int)threadIdx.x + kScanThreads * r < rows && key[r] >= t32));
      if (lane == 0) sm.wsum[wave] = wc;
      lds_barrier();
      uint32_t pos = 0;
      emitted = 0;
#pragma unroll
      for (int w = 0; w < kScanWaves; ++w) {
        const uint32_t c = sm.wsum[w];
        pos += w < wave ? c : 0u;
        emitted += c;
      }
#pragma unroll
      for (int r = 0; r < kRpt; ++r) {
        const int i = threadIdx.x + kScanThreads * r;
        const bool take = i < rows && key[r] >= t32;
        const uint64_t m = __ballot(take);
        if (take)
          dst[pos + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u))] =
              compose_key(key[r], (uint32_t)(srow0 + i));
        pos += (uint32_t)__builtin_popcountll(m);
      }
      bound = pe < rows ? ((uint64_t)t32 << 32) : 0ull;
    } else {  // too many keys share the boundary bin: the exact top-cap instead
      auto key_at = [&](int i) -> uint64_t { return compose_key(s_score[i], (uint32_t)(srow0 + i)); };
      uint64_t t64, unused;
      block_select2<kScanThreads>(key_at, rows, cap, cap, sm, &t64, &unused);
      uint32_t c = 0;
      for (int i = threadIdx.x; i < rows; i += kScanThreads) c += key_at(i) >= t64;
      uint32_t pos = block_exclusive_scan<kScanThreads>(c, sm.wsum, &emitted);
      for (int i = threadIdx.x; i < rows; i += kScanThreads) {
        const uint64_t key = key_at(i);
        if (key >= t64) dst[pos++] = key;
      }
      bound = t64;
    }
    if (threadIdx.x == 0) {
      ws.count[si] = emitted;
      ws.bound[si] = bound;
      s_next = kScanWaves;  // the next slice's counter
    }
    lds_barrier();  // s_score and sm are free, the counter set, for the next slice
    if (j + 1 >= n_done) break;
  }
}

// ------------------------------------------------------------------ merge kernel

__global__ __launch_bounds__(kMergeThreads) void indexer_merge_kernel(
    IndexerWs ws, int64_t n_c, const int32_t* __restrict__ seq_rows, int top_k, int n_slices,
    int cap, int first, int32_t* __restrict__ topk) {
  __shared__ MergeSmem ms;
  args_in_sgprs(ws.cand, ws.bound, ws.count, ws.scores, n_c, seq_rows, top_k, n_slices, cap, first, topk);
  const int b = blockIdx.x;
  merge_query<kMergeThreads, kMergeFirstPerThread>(ws, n_c, seq_rows, top_k, n_slices, cap, first, b,
                                                   ms, topk + (int64_t)b * top_k, nullptr);
}

// ------------------------------------------------------------------ CSA2 reindex

// Two launches.  The score kernel spreads the pool over many workgroups: each one scores
// kReindexPartRows pool slots of one query, lane (g, n) of wave w reading pool row
// pool[part * kReindexPartRows + 16w + n], exactly as the scan scores a tile, and leaves
// every slot's selection key (0 for an empty slot) in the workspace.  The select kernel
// then keeps the top-k of each query's keys in LDS.  Rows are addressed by 32-bit
// offsets inside a buffer resource over the query's sequence (or the page pool); an
// empty slot is read past that range, which returns zeros without touching memory.
constexpr int kReindexScoreWaves = 4;
constexpr int kReindexScoreThreads = kReindexScoreWaves * kWave;
constexpr int kReindexPartRows = 16 * kReindexScoreWaves;  // one tile per wave
constexpr int kReindexThreads = 512;                        // select kernel
constexpr uint32_t kAbsentKeyOffset = kReindexMaxSeqBytes;

template <class KT, int HT, bool QH>
__global__ __launch_bounds__(kReindexScoreThreads) void reindex_score_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t seq_stride,
    Paging pg, int64_t n_c_max, const int32_t* __restrict__ seq_rows,
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx, int n_heads,
    const int32_t* __restrict__ pool, int n_pool, int n_parts, uint64_t* __restrict__ keys) {
  typedef typename KT::Op Op;
  // Query fragments of the HT head tiles (and, for rotated queries split over two waves,
  // the handed-over values).
  constexpr size_t kStageBytes = QH ? fp4h_stage_bytes<HT, kReindexScoreWaves>() : sizeof(u32x4) * HT * 4 * kWave;
  __shared__ u32x4 s_stage[kStageBytes / sizeof(u32x4)];
  __shared__ float s_red[HT];
  __shared__ float s_w[16 * HT];
  args_in_sgprs(codes, scales, seq_stride, pg.table, pg.page_shift, pg.table_stride, n_c_max, seq_rows,
                q_idx, w_idx, n_heads, pool, n_pool, n_parts, keys);
  const int b = blockIdx.x / n_parts;
  const int part = blockIdx.x - b * n_parts;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  const int g = lane >> 4, n = lane & 15;
  const int64_t n_c = seq_len(seq_rows, b, n_c_max);  // this sequence's rows

  const int pos = part * kReindexPartRows + 16 * wave + n;  // lane n's pool slot
  const int32_t r = pos < n_pool ? pool[(int64_t)b * n_pool + pos] : -1;
  QueryRaw<KT, HT, kReindexScoreWaves> qraw;
  qraw.load(q_idx, b, n_heads, wave, g, n);
  const float w_pre = query_weight_load<HT>(w_idx, b, n_heads);
  Op qa[HT][4];
  float wv[HT][4];
  query_setup<KT, HT, QH, kReindexScoreWaves>(qraw, w_pre, wave, g, qa, wv, s_stage, s_red, s_w);

  const int row = (r >= 0 && r < n_c) ? r : -1;
  const int at = row < 0 || !pg.table
                     ? row
                     : (pg.table[(int64_t)b * pg.table_stride + (row >> pg.page_shift)] << pg.page_shift) +
                           (row & ((1 << pg.page_shift) - 1));
  // Rows are addressed inside the sequence's rows, or inside the page pool when paged.
  const Rsrc rc = pg.table ? make_rsrc(codes, kReindexMaxSeqBytes)
                           : make_rsrc(codes + (int64_t)b * seq_stride * KT::kRowBytes,
                                       (uint32_t)(n_c * KT::kRowBytes));
  const Rsrc rs = !KT::kScales ? rc
                  : pg.table   ? make_rsrc(scales, kReindexMaxSeqBytes)
                               : make_rsrc(scales + (int64_t)b * seq_stride * (kIdxDim / 16),
                                           (uint32_t)(n_c * (kIdxDim / 16)));
  KT kt;
  kt.set_lane(g);
  kt.load(rc, rs,
          at >= 0 ? (uint32_t)at * KT::kRowBytes + KT::code_offset(0, g) : kAbsentKeyOffset,
          at >= 0 ? (uint32_t)at * (kIdxDim / 16) + KT::scale_offset(0, g) : kAbsentKeyOffset);
  Op kb[4];
  kt.decode(kb);
  const float sc = wave_sum_rows(tile_share<KT, HT>(qa, kb, wv));
  if (g == 0 && pos < n_pool)
    keys[(int64_t)b * n_pool + pos] = row >= 0 ? compose_key(f32_order_key(sc), (uint32_t)row) : 0ull;
}

// One workgroup per query: the query's nonzero keys, compacted in pool order, and the
// top_k of them written in that order.
__global__ __launch_bounds__(kReindexThreads) void reindex_select_kernel(
    const uint64_t* __restrict__ keys, int n_pool, int top_k, int32_t* __restrict__ topk) {
  constexpr int NT = kReindexThreads;
  constexpr int kPer = kMaxPool / NT;
  __shared__ uint64_t s_val[kMaxPool];
  __shared__ uint64_t s_list[kMergeListCap];
  __shared__ SelectSmem sm;
  args_in_sgprs(keys, n_pool, top_k, topk);
  const int b = blockIdx.x;
  const uint64_t* kq = keys + (int64_t)b * n_pool;
  const int q0 = threadIdx.x * kPer;  // a contiguous run of slots keeps pool order
  uint64_t kr[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) kr[j] = q0 + j < n_pool ? kq[q0 + j] : 0ull;
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) c += kr[j] != 0ull;
  uint32_t n_valid;
  uint32_t wpos = block_exclusive_scan<NT>(c, sm.wsum, &n_valid);
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (kr[j] != 0ull) s_val[wpos++] = kr[j];
  lds_barrier();

  int32_t* out = topk + (int64_t)b * top_k;
  const int k1 = min(top_k, (int)n_valid);
  for (int i = k1 + threadIdx.x; i < top_k; i += NT) out[i] = -1;
  if (k1 == 0) return;
  const uint64_t kth = (int)n_valid > k1 ? block_kth_exact<NT>(s_val, (int)n_valid, k1, sm, s_list) : 1ull;
  const int chunk = ((int)n_valid + NT - 1) / NT;
  const int p0 = threadIdx.x * chunk, p1 = min(p0 + chunk, (int)n_valid);
  uint32_t cw = 0;
  for (int p = p0; p < p1; ++p) cw += s_val[p] >= kth;
  uint32_t total;
  uint32_t opos = block_exclusive_scan<NT>(cw, sm.wsum, &total);
  for (int p = p0; p < p1; ++p)  // (the bound only matters for a pool that repeats a row)
    if (s_val[p] >= kth && opos < (uint32_t)k1) out[opos++] = key_index(s_val[p]);
}

template <class KT, bool QH>
void launch_reindex_ht(int ht, hipStream_t stream, const uint8_t* codes, const uint8_t* scales,
                       int64_t seq_stride, const Paging& pg, int64_t n_c, const int32_t* seq_rows,
                       const uint16_t* q_idx, const float* w_idx, int batch, int n_heads,
                       const int32_t* pool, int n_pool, uint64_t* keys) {
  const int n_parts = (n_pool + kReindexPartRows - 1) / kReindexPartRows;
  const dim3 grid((unsigned)(batch * n_parts));
#define CSAKV_REINDEX(H)                                                                        \
  hipLaunchKernelGGL((reindex_score_kernel<KT, H, QH>), grid, dim3(kReindexScoreThreads), 0,     \
                     stream, codes, scales, seq_stride, pg, n_c, seq_rows, q_idx, w_idx, n_heads, \
                     pool, n_pool, n_parts, keys)
  switch (ht) {
    case 1: CSAKV_REINDEX(1); break;
    case 2: CSAKV_REINDEX(2); break;
    case 3: CSAKV_REINDEX(3); break;
    case 4: CSAKV_REINDEX(4); break;
    default: CSAKV_REINDEX(8); break;  // 65..128 heads (heads past n_heads are zero)
  }
#undef CSAKV_REINDEX
}

template <class KT, int HT, bool QH>
void launch_scan(hipStream_t stream, const uint8_t* codes, const uint8_t* scales,
                 int64_t seq_stride, const Paging& pg, int64_t n_c, const int32_t* seq_rows,
                 const uint16_t* q_idx, const float* w_idx, int batch, int n_heads,
                 const IndexerPlan& plan, const IndexerWs& ws) {
  // The paged variant is its own kernel: a table lookup behind a branch in the tile
  // loop would make the compiler wait for every key load in flight at each tile.
  if (pg.table)
    hipLaunchKernelGGL((indexer_scan_kernel<KT, HT, QH, true>), dim3(batch * plan.wg_per_query),
                       dim3(kScanThreads), 0, stream, codes, scales, seq_stride, pg.table, pg.page_shift,
                       pg.table_stride, n_c, seq_rows,
                       q_idx, w_idx, n_heads, plan.n_slices, plan.slices_per_wg, plan.wg_per_query,
                       plan.prefix, plan.cap, ws);
  else
    hipLaunchKernelGGL((indexer_scan_kernel<KT, HT, QH, false>), dim3(batch * plan.wg_per_query),
                       dim3(kScanThreads), 0, stream, codes, scales, seq_stride, pg.table, pg.page_shift,
                       pg.table_stride, n_c, seq_rows,
                       q_idx, w_idx, n_heads, plan.n_slices, plan.slices_per_wg, plan.wg_per_query,
                       plan.prefix, plan.cap, ws);
}

template <class KT, bool QH = false>
void launch_scan_ht(int ht, hipStream_t stream, const uint8_t* codes, const uint8_t* scales,
                    int64_t seq_stride, const Paging& pg, int64_t n_c, const int32_t* seq_rows,
                    const uint16_t* q_idx, const float* w_idx, int batch, int n_heads,
                    const IndexerPlan& plan, const IndexerWs& ws) {
#define CSAKV_SCAN(H)                                                                         \
  launch_scan<KT, H, QH>(stream, codes, scales, seq_stride, pg, n_c, seq_rows, q_idx, w_idx,    \
                         batch, n_heads, plan, ws)
  switch (ht) {
    case 1: CSAKV_SCAN(1); break;
    case 2: CSAKV_SCAN(2); break;
    case 3: CSAKV_SCAN(3); break;
    case 4: CSAKV_SCAN(4); break;
    default: CSAKV_SCAN(8); break;  // 65..128 heads (heads past n_heads are zero)
  }
#undef CSAKV_SCAN
}

}  // namespace

IndexerPlan plan_indexer(int batch, int64_t n_c, int top_k) {
  IndexerPlan p{};
  // 4096-row slices, about one scan workgroup per CU (256), each owning a run of slices
  // of one query.  A slice sends its top-P or a few more (at least 4x its expected
  // share k / n_slices of the winners); the merge buffer holds every slice's cap.
  p.n_c = n_c;
  p.slice_rows = kSliceRows;
  p.n_slices = n_c > 0 ? (int)((n_c + kSliceRows - 1) / kSliceRows) : 0;
  if (p.n_slices > 0) {
    int64_t wg = (256 + batch - 1) / batch;
    if (wg > p.n_slices) wg = p.n_slices;
    p.slices_per_wg = (int)((p.n_slices + wg - 1) / wg);
    p.wg_per_query = (p.n_slices + p.slices_per_wg - 1) / p.slices_per_wg;
    p.cap = (int)std::min<int64_t>(kSliceRows, kMergeCap / p.n_slices);
    if (p.n_slices == 1) {
      p.prefix = top_k;
    } else {
      int64_t want = (4 * (int64_t)top_k + p.n_slices - 1) / p.n_slices;
      if (want < 16) want = 16;
      p.prefix = (int)std::min<int64_t>(want, p.cap / 2);
    }
    // The merge reads the first `first` slots of every slice (kMergeFirstSlots in all) in the same
    // round as the counts; a slice that sent more has the rest read afterwards.
    const int64_t room = std::min<int64_t>(p.cap, kMergeFirstSlots / p.n_slices);
    p.first = 1;
    while (2 * (int64_t)p.first <= room) p.first *= 2;
  }
  return p;
}

size_t indexer_workspace_bytes(int batch, const IndexerPlan& plan) {
  const size_t ns = (size_t)batch * plan.n_slices;
  return align256(ns * plan.cap * sizeof(uint64_t)) + align256(ns * sizeof(uint64_t)) +
         align256(ns * sizeof(uint32_t)) + align256((size_t)batch * plan.n_c * sizeof(uint32_t));
}

bool indexer_supported(const IndexerPlan& plan) {
  return plan.n_slices <= kMaxMergeSlices && (plan.n_slices == 0 || plan.prefix >= 1);
}

hipError_t launch_indexer(int key_fmt, const uint8_t* codes, const uint8_t* scales,
                          int64_t seq_stride, const Paging& pg, int64_t n_c,
                          const int32_t* seq_rows, const uint16_t* q_idx, const float* w_idx,
                          int batch, int n_heads, int top_k, const IndexerPlan& plan,
                          void* workspace, int32_t* topk, hipStream_t stream, int stages) {
  const IndexerWs ws = carve_indexer_ws(workspace, batch, plan);
  if (plan.n_slices > 0 && (stages & kStageScan)) {
    const int ht = (n_heads + 15) / 16;
    if (key_fmt == 0)
      launch_scan_ht<KeyTileBf16>(ht, stream, codes, scales, seq_stride, pg, n_c, seq_rows, q_idx, w_idx, batch,
                                  n_heads, plan, ws);
    else if (key_fmt == 1)
      launch_scan_ht<KeyTileFp4>(ht, stream, codes, scales, seq_stride, pg, n_c, seq_rows, q_idx, w_idx, batch,
                                 n_heads, plan, ws);
    else  // Hadamard-rotated FP4 keys: the query is rotated and quantised the same way
      launch_scan_ht<KeyTileFp4, true>(ht, stream, codes, scales, seq_stride, pg, n_c, seq_rows, q_idx, w_idx,
                                       batch, n_heads, plan, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & kStageMerge)
    hipLaunchKernelGGL(indexer_merge_kernel, dim3(batch), dim3(kMergeThreads), 0, stream, ws, n_c, seq_rows,
                       top_k, plan.n_slices, plan.cap, plan.first, topk);
  return hipGetLastError();
}

bool reindex_supported(int key_fmt, int64_t n_c) {
  const int64_t row_bytes = key_fmt == 0 ? KeyTileBf16::kRowBytes : KeyTileFp4::kRowBytes;
  return n_c >= 0 && n_c * row_bytes <= (int64_t)kReindexMaxSeqBytes;
}

size_t reindex_workspace_bytes(int batch, int n_pool) {
  return (size_t)batch * (size_t)n_pool * sizeof(uint64_t);
}

hipError_t launch_reindex(int key_fmt, const uint8_t* codes, const uint8_t* scales,
                          int64_t seq_stride, const Paging& pg, int64_t n_c,
                          const int32_t* seq_rows, const uint16_t* q_idx, const float* w_idx,
                          int batch, int n_heads, const int32_t* pool, int n_pool, int top_k,
                          int32_t* topk, void* workspace, hipStream_t stream) {
  const int ht = (n_heads + 15) / 16;
  uint64_t* keys = static_cast<uint64_t*>(workspace);
  if (key_fmt == 0)
    launch_reindex_ht<KeyTileBf16, false>(ht, stream, codes, scales, seq_stride, pg, n_c, seq_rows,
                                          q_idx, w_idx, batch, n_heads, pool, n_pool, keys);
  else if (key_fmt == 1)
    launch_reindex_ht<KeyTileFp4, false>(ht, stream, codes, scales, seq_stride, pg, n_c, seq_rows,
                                         q_idx, w_idx, batch, n_heads, pool, n_pool, keys);
  else
    launch_reindex_ht<KeyTileFp4, true>(ht, stream, codes, scales, seq_stride, pg, n_c, seq_rows,
                                        q_idx, w_idx, batch, n_heads, pool, n_pool, keys);
  hipLaunchKernelGGL(reindex_select_kernel, dim3(batch), dim3(kReindexThreads), 0, stream, keys,
                     n_pool, top_k, topk);
  return hipGetLastError();
}

}  // namespace csakv
