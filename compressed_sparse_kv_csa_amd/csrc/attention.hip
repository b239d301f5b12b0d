// Multi-query softmax attention over gathered shared-KV rows (CSA sparse, HCA dense).
//
// What is computed ("DeepSeek-V4 KV Cache 深度分析", section 三 for the CSA/HCA row sets,
// section 五 for one entry serving as both key and value, and the section 十一 diagram):
//   o[h] = sum_r softmax_r(scale * q[h] . e_r) * e_r
// over the rows r of one query: CSA = the window rows plus the selected compressed
// rows (one softmax over their union), HCA = every row of the sequence.
//
// Structure: one workgroup per (query, chunk of its row list, block of up to 64 heads);
// the head blocks of one chunk run on one XCD and share its L2 for the gathered rows.  A
// workgroup first resolves the chunk's row indices into LDS, then per 32-row step
// gathers whole rows (coalesced 16-byte loads, several steps ahead of the one
// computing), stores them into a row-major LDS tile (bf16 rows as they are, FP8 and FP4
// rows decoded exactly to fp16) that all of its heads use, and runs, per 16-head group,
//   S^T[32 rows x 16 heads] = K[32 x 512] . Q^T            (16x16x32 MFMA)
//   O^T[512 x 16 heads]    += V^T[512 x 32] . P^T[32 x 16]  (16x16x32 MFMA)
// with an online softmax in fp32 (exp2 domain) whose reference maximum moves only when
// a step's maximum exceeds it by more than 2^8.  The same tile serves both products:
// K fragments are plain 16-byte LDS reads, V^T fragments come from transposing LDS
// reads (ds_read_b64_tr_b16), so no transposed copy is ever written.
//
// Precision: bf16 rows meet the bf16 query on bf16 MFMA, each probability entering P.V
// as two bf16 terms (about 16 significant bits).  FP8 (E4M3) and FP4 (E2M1 x E4M3)
// values are exact in fp16 and meet the query rounded to fp16 (exact from 2^-14 to
// 65504; smaller magnitudes keep an absolute error below 2^-25), probabilities as one
// fp16 term.  Products are exact in fp32 and accumulate in fp32.
// Each chunk writes (max, sum, unnormalised O) per head; a combine kernel merges the
// chunks and rounds to bf16.
#include "csakv_device.h"
#include "csakv_launch.h"

#include <algorithm>

namespace csakv {

namespace {

constexpr int kDim = 512;
constexpr int kNope = 448;
constexpr int kStepRows = 32;
constexpr int kPitch = kDim + 16;     // fp16 elements per LDS row (32-byte pad)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyLog2 = 8.0f;  // rescale the accumulators once the maximum grows by 2^8
// Buffer offset given to an absent row: at or past the end of every sequence the
// launcher accepts (sequence bytes are checked against it on the host).
constexpr uint32_t kAbsentOffset = kAttnMaxSeqBytes;

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

// One step's gathered rows: every thread loads a fixed set of 16-byte pieces and
// later stores them, decoded to fp16, into the row-major tile.  Pieces are assigned so
// that the 64 lanes of one load instruction read consecutive bytes of the cached rows
// (whole cache lines, not one 16-byte piece of 64 different lines), and so that the
// assignment depends only on the thread, not on the step.  Raw data is kept in scalar
// arrays so that it stays in registers.  `rows` points at the step's 32 sequence rows
// (-1: absent); an absent row is read at an offset past the sequence, which returns
// zeros without touching memory.
__device__ __forceinline__ void load16(uint32_t* w, Rsrc rc, uint32_t off) {
  const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, off, 0, 0));
  w[0] = v[0];
  w[1] = v[1];
  w[2] = v[2];
  w[3] = v[3];
}
__device__ __forceinline__ void store16(uint16_t* dst, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  *reinterpret_cast<u32x4*>(dst) = u32x4{a, b, c, d};
}
// A workgroup-uniform 64-bit value, held in scalar registers (buffer resources built from
// it then need no per-lane loop around each load).
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ uint32_t row_offset(int row, uint32_t row_bytes, uint32_t in_row) {
  return row >= 0 ? (uint32_t)row * row_bytes + in_row : kAbsentOffset;
}

constexpr int kWideThreads = 512;                 // 8 waves
constexpr int kWideWaves = kWideThreads / kWave;
constexpr int kHeadGroups = 4;                    // 16-head groups per workgroup
constexpr int kBlockHeads = 16 * kHeadGroups;     // heads per workgroup
constexpr int kHalfDim = kDim / 2;                // dims of one wave's products
constexpr int kAttnTargetBlocks = 256;            // workgroups a launch aims for (one per CU)
constexpr int64_t kWideMinRows = 2048;            // lists at least this long run on wide workgroups

template <int KVFMT>
struct StepRaw;

// bf16 rows (1 KB): load k of wave w reads step row 4w + k whole, lane l its bytes
// 16l .. 16l + 15 (dims 8l .. 8l + 7).  The row is wave-uniform.
template <>
struct StepRaw<0> {
  static constexpr uint32_t kRowBytes = kDim * 2;
  static constexpr uint32_t kScaleRowBytes = 0;
  static constexpr int kAhead = 2;  // steps fetched ahead of the one computing
  static constexpr int kRowsPerWave = kStepRows / kWideWaves;
  uint32_t w[4 * kRowsPerWave];
  __device__ __forceinline__ void load(Rsrc rc, Rsrc, const int* rows, int tid) {
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid & (kWave - 1);
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k) {
      const int row = __builtin_amdgcn_readfirstlane(rows[kRowsPerWave * wave + k]);
      load16(w + 4 * k, rc, row_offset(row, kRowBytes, 16 * lane));
    }
  }
  __device__ __forceinline__ void store(uint16_t* tile, int tid) const {  // as bf16
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid & (kWave - 1);
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k)
      store16(tile + (kRowsPerWave * wave + k) * kPitch + 8 * lane, w[4 * k], w[4 * k + 1],
              w[4 * k + 2], w[4 * k + 3]);
  }
};

// Mixed rows (576 B: 448 E4M3 codes, then 64 bf16).  The step's 32 x 28 E4M3 pieces
// (16 dims each) are numbered row-major, piece p = 512k + tid: every thread takes one in
// the first round, waves 0..5 one more in the second (896 pieces).  The 32 x 8 bf16
// pieces (8 dims each) go to waves 4..7, one per thread.  Every thread issues the same
// three loads (a thread without a piece reads at the absent offset, which returns zeros
// and touches no memory), so the outstanding-load count is the same on every path; only
// the LDS stores are skipped, on wave-uniform branches.
template <>
struct StepRaw<1> {
  static constexpr uint32_t kRowBytes = kNope + 2 * (kDim - kNope);
  static constexpr uint32_t kScaleRowBytes = 0;
  static constexpr int kAhead = 3;
  static constexpr int kFp8Pieces = kStepRows * (kNope / 16);  // 896
  static constexpr int kSecondRoundWaves = (kFp8Pieces - kWideThreads) / kWave;  // 6
  static constexpr int kBf16Pieces = kStepRows * ((kDim - kNope) / 8);           // 256
  static constexpr int kBf16Wave0 = kWideWaves - kBf16Pieces / kWave;            // 4
  uint32_t e[8];  // two E4M3 pieces
  uint32_t r[4];  // one bf16 piece
  __device__ __forceinline__ void load(Rsrc rc, Rsrc, const int* rows, int tid) {
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int p = kWideThreads * k + tid;
      const int rl = p / (kNope / 16), c = p - rl * (kNope / 16);
      const bool has = k == 0 || wave < kSecondRoundWaves;
      load16(e + 4 * k, rc, has ? row_offset(rows[rl], kRowBytes, 16 * c) : kAbsentOffset);
    }
    const int q = (tid - kBf16Wave0 * kWave) & (kBf16Pieces - 1);
    load16(r, rc, wave >= kBf16Wave0 ? row_offset(rows[q >> 3], kRowBytes, kNope + 16 * (q & 7))
                                     : kAbsentOffset);
  }
  __device__ __forceinline__ void store(uint16_t* tile, int tid) const {
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (k == 1 && wave >= kSecondRoundWaves) break;
      const int p = kWideThreads * k + tid;
      const int rl = p / (kNope / 16), c = p - rl * (kNope / 16);
      uint16_t* dst = tile + rl * kPitch + 16 * c;
      uint32_t h[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {  // 4 E4M3 codes -> 4 fp16 (exact)
        h[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(e[4 * k + i], 1.0f, false));
        h[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(e[4 * k + i], 1.0f, true));
      }
      store16(dst, h[0], h[1], h[2], h[3]);
      store16(dst + 8, h[4], h[5], h[6], h[7]);
    }
    if (wave >= kBf16Wave0) {
      const int q = tid - kBf16Wave0 * kWave;
      store16(tile + (q >> 3) * kPitch + kNope + 8 * (q & 7), bf16x2_to_f16x2(r[0]),
              bf16x2_to_f16x2(r[1]), bf16x2_to_f16x2(r[2]), bf16x2_to_f16x2(r[3]));
    }
  }
};

// FP4 rows (256 code bytes, 32 E4M3 scale bytes, one per 16 dims): thread t takes row
// t / 16, code bytes 16c .. 16c + 15 with c = t % 16 (dims 32c .. 32c + 31), and the two
// scale bytes of those dims.
template <>
struct StepRaw<2> {
  static constexpr uint32_t kRowBytes = kDim / 2;
  static constexpr uint32_t kScaleRowBytes = kDim / 16;
  static constexpr int kAhead = 4;
  uint32_t c[4];
  uint32_t s;  // the aligned dword holding the piece's two scale bytes
  __device__ __forceinline__ void load(Rsrc rc, Rsrc rs, const int* rows, int tid) {
    const int row = rows[tid >> 4];
    load16(c, rc, row_offset(row, kRowBytes, 16 * (tid & 15)));
    s = __builtin_amdgcn_raw_buffer_load_b32(rs, row_offset(row, kScaleRowBytes, 4 * ((tid & 15) >> 1)), 0, 0);
  }
  __device__ __forceinline__ void store(uint16_t* tile, int tid) const {
    uint16_t* dst = tile + (tid >> 4) * kPitch + 32 * (tid & 15);
    // Both scales as an fp16 pair (exact), each broadcast to both halves of a pair.
    const uint32_t s2 = s >> (16 * (tid & 1));
    const uint32_t sp = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s2, 1.0f, false));
    const f16x2 s0 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(sp, sp, 0x01000100u));
    const f16x2 s1 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(sp, sp, 0x03020302u));
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // code dword j holds dims 8j .. 8j + 7 (scale j / 2)
      const uint32_t cw = c[j];
      const f16x2 sc = j < 2 ? s0 : s1;
      store16(dst + 8 * j,
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 0) * sc),
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 1) * sc),
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 2) * sc),
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 3) * sc));
    }
  }
};

// ---------------------------------------------------------------- partial records

// A chunk's partial output is stored divided by the chunk's own sum of probabilities: a
// convex combination of the chunk's rows, so no element exceeds the rows' largest.  For
// FP8 and FP4 rows, which reach the products as fp16 and meet fp16 probabilities, the
// records are fp16 (rounded to nearest even; in range by the rows' bound below 65504);
// for bf16 rows they stay fp32.  Four consecutive elements at a time.
template <int KVFMT>
struct PartialRecord {
  static constexpr bool kHalf = KVFMT != 0;
};

template <bool H16>
__device__ __forceinline__ void store_partial4(float* part_o, int64_t elem, f32x4 v) {
  if constexpr (H16) {
    const f16x2 lo = {(_Float16)v[0], (_Float16)v[1]};
    const f16x2 hi = {(_Float16)v[2], (_Float16)v[3]};
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(part_o) + elem) =
        u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
  } else {
    *reinterpret_cast<f32x4*>(part_o + elem) = v;
  }
}

template <bool H16>
__device__ __forceinline__ f32x4 load_partial4(Rsrc r, uint32_t byte_off) {
  if constexpr (H16) {
    // The whole 8-byte load is reinterpreted at once: hipcc folded a bit-cast of the
    // second element of a two-element vector into one of the first.
    typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
    const f16x4 h = __builtin_bit_cast(f16x4, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0));
    return f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
  } else {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
  }
}

// ---------------------------------------------------------------- narrow workgroups
// Short row lists (CSA: window + top-k rows) run on narrow workgroups of 16 heads and 4
// waves, which spread one query's list over more compute units; long lists (HCA) run on
// wide workgroups of 64 heads and 8 waves, which decode each row once for all heads.
constexpr int kNarrowThreads = 256;  // 4 waves
constexpr int kNarrowDims = kDim / 4;  // output dims per wave
constexpr int kOutPitch = kDim + 4;    // floats per LDS row when staging the output

template <int KVFMT>
struct NarrowRaw;

// Narrow workgroups (256 threads).  bf16 rows (1 KB): load k of wave w reads step row 8w + k whole, lane l its bytes
// 16l .. 16l + 15 (dims 8l .. 8l + 7).  The row is wave-uniform.
template <>
struct NarrowRaw<0> {
  static constexpr uint32_t kRowBytes = kDim * 2;
  static constexpr uint32_t kScaleRowBytes = 0;
  uint32_t w[32];
  __device__ __forceinline__ void load(Rsrc rc, Rsrc, const int* rows, int tid) {
    const int wave = tid / kWave, lane = tid & (kWave - 1);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int row = __builtin_amdgcn_readfirstlane(rows[8 * wave + k]);
      load16(w + 4 * k, rc, row_offset(row, kRowBytes, 16 * lane));
    }
  }
  __device__ __forceinline__ void store(uint16_t* tile, int tid) const {  // as bf16
    const int wave = tid / kWave, lane = tid & (kWave - 1);
#pragma unroll
    for (int k = 0; k < 8; ++k)
      store16(tile + (8 * wave + k) * kPitch + 8 * lane, w[4 * k], w[4 * k + 1], w[4 * k + 2],
              w[4 * k + 3]);
  }
};

// Mixed rows (576 B: 448 E4M3 codes, then 64 bf16).  The step's 32 x 28 E4M3 pieces
// are numbered row-major, piece p = 256k + tid (k < 4; the last round covers 128 of
// them), each 16 dims; the 32 x 8 bf16 pieces go one per thread (8 dims each).  The
// threads of the last E4M3 round that have no piece read nothing and write their 32
// bytes into the tile's row padding (dims 512 .. 527, which no product reads).
template <>
struct NarrowRaw<1> {
  static constexpr uint32_t kRowBytes = kNope + 2 * (kDim - kNope);
  static constexpr uint32_t kScaleRowBytes = 0;
  static constexpr int kFp8Pieces = kStepRows * (kNope / 16);  // 896
  uint32_t e[16];  // four E4M3 pieces
  uint32_t r[4];   // one bf16 piece
  __device__ __forceinline__ void load(Rsrc rc, Rsrc, const int* rows, int tid) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int p = 256 * k + tid;
      const int rl = p / (kNope / 16), c = p - rl * (kNope / 16);
      const int row = p < kFp8Pieces ? rows[rl < kStepRows ? rl : kStepRows - 1] : -1;
      load16(e + 4 * k, rc, row_offset(row, kRowBytes, 16 * c));
    }
    load16(r, rc, row_offset(rows[tid >> 3], kRowBytes, kNope + 16 * (tid & 7)));
  }
  __device__ __forceinline__ void store(uint16_t* tile, int tid) const {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int p = 256 * k + tid;
      const int rl = p / (kNope / 16), c = p - rl * (kNope / 16);
      uint16_t* dst = p < kFp8Pieces ? tile + rl * kPitch + 16 * c : tile + (p & 31) * kPitch + kDim;
      uint32_t h[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {  // 4 E4M3 codes -> 4 fp16 (exact)
        h[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(e[4 * k + i], 1.0f, false));
        h[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(e[4 * k + i], 1.0f, true));
      }
      store16(dst, h[0], h[1], h[2], h[3]);
      store16(dst + 8, h[4], h[5], h[6], h[7]);
    }
    store16(tile + (tid >> 3) * kPitch + kNope + 8 * (tid & 7), bf16x2_to_f16x2(r[0]),
            bf16x2_to_f16x2(r[1]), bf16x2_to_f16x2(r[2]), bf16x2_to_f16x2(r[3]));
  }
};

// FP4 rows (256 code bytes, 32 E4M3 scale bytes, one per 16 dims): piece p = 256k + tid
// (k < 2) is row p / 16, code bytes 16c .. 16c + 15 with c = p % 16 (dims 32c .. 32c + 31),
// and the two scale bytes of those dims.
template <>
struct NarrowRaw<2> {
  static constexpr uint32_t kRowBytes = kDim / 2;
  static constexpr uint32_t kScaleRowBytes = kDim / 16;
  uint32_t c[8];
  uint32_t s[2];
  __device__ __forceinline__ void load(Rsrc rc, Rsrc rs, const int* rows, int tid) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int p = 256 * k + tid;
      const int row = rows[p >> 4];
      load16(c + 4 * k, rc, row_offset(row, kRowBytes, 16 * (p & 15)));
      s[k] = __builtin_amdgcn_raw_buffer_load_b16(rs, row_offset(row, kScaleRowBytes, 2 * (p & 15)), 0, 0);
    }
  }
  __device__ __forceinline__ void store(uint16_t* tile, int tid) const {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int p = 256 * k + tid;
      uint16_t* dst = tile + (p >> 4) * kPitch + 32 * (p & 15);
      // Both scales as an fp16 pair (exact), each broadcast to both halves of a pair.
      const uint32_t sp = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s[k], 1.0f, false));
      const f16x2 s0 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(sp, sp, 0x01000100u));
      const f16x2 s1 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(sp, sp, 0x03020302u));
#pragma unroll
      for (int j = 0; j < 4; ++j) {  // code dword j holds dims 8j .. 8j + 7 (scale j / 2)
        const uint32_t cw = c[4 * k + j];
        const f16x2 sc = j < 2 ? s0 : s1;
        store16(dst + 8 * j,
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 0) * sc),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 1) * sc),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 2) * sc),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 3) * sc));
      }
    }
  }
};

// V^T fragment of dims 16*dt .. 16*dt+15 for the K-slots of lane group g (rows 4g..4g+3
// and 16+4g..16+4g+3 of the tile): two transposing reads.  Within each 16-lane group
// the hardware hands lane i, slot j, element i%4 of the 8 bytes addressed by lane
// 4j + i/4; lane k therefore addresses row base + k/4, dims 16*dt + 4*(k%4).
__device__ __forceinline__ u32x4 v_fragment(const uint16_t* tile, int g, int k, int dt) {
  const uint16_t* p = tile + (4 * g + (k >> 2)) * kPitch + 16 * dt + 4 * (k & 3);
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 16 * kPitch));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  return u32x4{l2[0], l2[1], h2[0], h2[1]};
}

// The tile's arithmetic.  bf16 rows stay bf16 in the tile and meet the bf16 queries on
// bf16 MFMA; their probabilities go in as two bf16 terms (high part, then the rounded
// remainder: 16 significant bits).  FP8 and FP4 rows decode exactly to fp16 and meet
// fp16 queries on fp16 MFMA with one fp16 term per probability.
template <int KVFMT>
struct TileMath {
  typedef f16x8 Op;
  static __device__ __forceinline__ Op q_op(u32x4 v) {
    return as_f16x8(u32x4{bf16x2_to_f16x2(v[0]), bf16x2_to_f16x2(v[1]), bf16x2_to_f16x2(v[2]),
                          bf16x2_to_f16x2(v[3])});
  }
  static __device__ __forceinline__ Op op(u32x4 v) { return as_f16x8(v); }
  static __device__ __forceinline__ f32x4 mma(Op a, Op b, f32x4 c) { return mfma16x16x32_f16(a, b, c); }
  static constexpr int kPTerms = 1;
  // The probabilities of K-slots 8g .. 8g + 7 (rows 4g..4g+3, 16+4g..16+4g+3) as term `t`.
  static __device__ __forceinline__ Op p_term(const float (&pv)[8], int) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = f32_to_f16_bits(pv[2 * i]) | (f32_to_f16_bits(pv[2 * i + 1]) << 16);
    return as_f16x8(r);
  }
};
template <>
struct TileMath<0> {
  typedef bf16x8 Op;
  static __device__ __forceinline__ Op q_op(u32x4 v) { return as_bf16x8(v); }
  static __device__ __forceinline__ Op op(u32x4 v) { return as_bf16x8(v); }
  static __device__ __forceinline__ f32x4 mma(Op a, Op b, f32x4 c) { return mfma16x16x32(a, b, c); }
  static constexpr int kPTerms = 2;
  static __device__ __forceinline__ Op p_term(const float (&pv)[8], int t) {
    Op r;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const __bf16 hi = (__bf16)pv[i];  // round to nearest even
      r[i] = t == 0 ? hi : (__bf16)(pv[i] - (float)hi);  // the remainder is exact in fp32
    }
    return r;
  }
};

// Workgroup -> (query b, chunk, head block).  Workgroups are dispatched round-robin over
// the 8 XCDs by index, so the head blocks of one (query, chunk) pair are given indices
// that are equal modulo 8: they run on one XCD and share its L2 for the gathered rows.
__device__ __forceinline__ bool attn_block(int n_pairs, int n_blocks, int n_chunks, int* b,
                                           int* chunk, int* blk) {
  const int x = blockIdx.x & 7, k = blockIdx.x >> 3;
  *blk = k % n_blocks;
  const int pair = x + 8 * (k / n_blocks);
  if (pair >= n_pairs) return false;
  *b = pair / n_chunks;
  *chunk = pair - *b * n_chunks;
  return true;
}

// One workgroup: 16 heads, one chunk of a query's row list.  All 4 waves gather and
// decode; each wave then computes the logits of all 16 heads (the K tile and the query
// rows are shared in LDS) and the output for its own 128 dims.  One decode tile: a step
// takes three barriers (previous tile consumed; tile complete; logit halves written).
constexpr int kNarrowTileBytes = kStepRows * kPitch * 2;
constexpr int kNarrowOutBytes = 16 * kOutPitch * 4;
constexpr int kNarrowMemBytes = kNarrowTileBytes > kNarrowOutBytes ? kNarrowTileBytes : kNarrowOutBytes;

// LDS of a narrow workgroup: the decode tile (later the output staging area), the
// chunk's row indices, and the two halves of each step's logits.
struct NarrowSmem {
  __attribute__((aligned(16))) uint8_t mem[kNarrowMemBytes];
  __attribute__((aligned(16))) int rows[kMaxChunkRows + 2 * kStepRows];
  __attribute__((aligned(16))) float logit[2][kStepRows][16];  // per K half
};

// One chunk of query b's row list for head group hg.  For CSA, sel points at the query's
// selected compressed-row indices (in the workspace, or in LDS when the selection was
// just computed by the same workgroup).
template <int KVFMT, bool CSA, bool PG>
__device__ __forceinline__ void narrow_chunk(
    NarrowSmem& sm, const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    int64_t seq_stride, const Paging& pg, int64_t n_rows_max, const int32_t* __restrict__ seq_rows,
    const uint16_t* __restrict__ q, int n_heads, float scale_log2, const int32_t* sel, int window,
    int64_t n_list, int rows_per_chunk, int n_chunks, float* __restrict__ part_o,
    float* __restrict__ part_ml, int b, int chunk, int hg) {
  constexpr int kTileElems = kStepRows * kPitch;
  uint8_t* const s_mem = sm.mem;
  int* const s_rows = sm.rows;
  auto& s_logit = sm.logit;
  uint16_t* const s_kv0 = reinterpret_cast<uint16_t*>(s_mem);
  float* const s_out = reinterpret_cast<float*>(s_mem);
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int g = lane >> 4;
  const int n = lane & 15;

  const int64_t p_begin = (int64_t)chunk * rows_per_chunk;
  const int64_t p_end = min(p_begin + rows_per_chunk, n_list);
  const int n_steps = (int)((p_end - p_begin + kStepRows - 1) / kStepRows);
  const int64_t n_rows = uniform64(seq_len(seq_rows, b, n_rows_max));  // this sequence's rows
  const int64_t n_c = n_rows - window;

  // Sequence row of every list position of the chunk (-1: absent or out of range), and
  // two steps of -1 past the end for the fetches that run ahead of the last step; for a
  // paged cache, the row's place in the page pool instead.
  for (int i = threadIdx.x; i < (n_steps + 2) * kStepRows; i += kNarrowThreads) {
    const int64_t p = p_begin + i;
    int row = -1;
    if (p < p_end) {
      if (!CSA || p < window) {
        row = p < n_rows ? (int)p : -1;
      } else {
        const int32_t j = sel[p - window];
        row = (j >= 0 && j < n_c) ? window + j : -1;
      }
    }
    if (PG && row >= 0)
      row = (pg.table[(int64_t)b * pg.table_stride + (row >> pg.page_shift)] << pg.page_shift) +
            (row & ((1 << pg.page_shift) - 1));
    s_rows[i] = row;
  }
  // The wave's logit B operands, kept in registers: wave w multiplies row tile w & 1
  // over dims 256 * (w >> 1) .. +255, lane (g, n) supplying head n, dims
  // 256 * (w >> 1) + 32t + 8g .. +7 of K-step t, in the tile's operand type.
  typedef TileMath<KVFMT> TM;
  typename TM::Op qf[8];
  {
    const uint16_t* qr = q + ((int64_t)b * n_heads + 16 * hg + n) * kDim + 256 * (wave >> 1) + 8 * g;
    u32x4 qv[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) qv[t] = *reinterpret_cast<const u32x4*>(qr + 32 * t);
#pragma unroll
    for (int t = 0; t < 8; ++t) qf[t] = TM::q_op(qv[t]);
  }
  lds_barrier();

  f32x4 o[kNarrowDims / 16];
#pragma unroll
  for (int i = 0; i < kNarrowDims / 16; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // m_run starts at a finite floor instead of -inf: the first step with a present row
  // always moves it (grow), so no probability is ever taken against the floor, and no
  // exponential sees -inf - -inf.  A chunk without present rows records -inf.
  float m_run = -__FLT_MAX__, l_run = 0.0f;

  // Two steps are fetched ahead (raw0 / raw1 alternate), so both steps of a 64-row chunk
  // are in flight as soon as the row indices are known.  Rows are read through buffer
  // resources over this query's sequence.  Every fetch is issued unconditionally (the
  // steps past the end have only absent rows, which read nothing); an absent row's logit
  // is masked to -inf, so its probability is exactly 0.  With no branch around the
  // loads, both fetched steps stay in flight across the step being computed.
  typedef NarrowRaw<KVFMT> Raw;
  Raw raw0, raw1;
  // Rows are addressed inside the sequence's rows, or inside the page pool when paged.
  const int64_t seq0 = uniform64((int64_t)b * seq_stride);
  const Rsrc rc = PG ? make_rsrc(codes, kAttnMaxSeqBytes)
                     : make_rsrc(codes + uniform64(seq0 * Raw::kRowBytes),
                                 __builtin_amdgcn_readfirstlane((uint32_t)(n_rows * Raw::kRowBytes)));
  const Rsrc rs = Raw::kScaleRowBytes == 0 ? rc
                  : PG ? make_rsrc(scales, kAttnMaxSeqBytes)
                       : make_rsrc(scales + uniform64(seq0 * Raw::kScaleRowBytes),
                                   __builtin_amdgcn_readfirstlane((uint32_t)(n_rows * Raw::kScaleRowBytes)));
  auto fetch = [&](Raw& raw, int step) { raw.load(rc, rs, s_rows + step * kStepRows, threadIdx.x); };

  auto run_step = [&](Raw& raw, int step) {
    uint16_t* tile = s_kv0;
    if (step > 0) lds_barrier();  // the previous step's tile is consumed
    // ---- decode the fetched rows into the tile (fp16, row-major)
    raw.store(tile, threadIdx.x);
    lds_barrier();
    fetch(raw, step + 2);

    // ---- logits S^T, split over the waves: wave w computes row tile w & 1 over dims
    // 256 * (w >> 1) .. +255 (lane (g, n): rows 16*rt + 4g + i, head n); the two halves
    // meet in LDS and every wave reads the full 32 x 16 block.
    {
      const int rt = wave & 1, kh = wave >> 1;
      const uint16_t* kr = tile + (16 * rt + n) * kPitch + 256 * kh + 8 * g;
      f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 8; ++t)
        part = TM::mma(TM::op(*reinterpret_cast<const u32x4*>(kr + 32 * t)), qf[t], part);
#pragma unroll
      for (int i = 0; i < 4; ++i) s_logit[kh][16 * rt + 4 * g + i][n] = part[i];
    }
    lds_barrier();
    f32x4 sacc[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sacc[rt][i] = s_logit[0][16 * rt + 4 * g + i][n] + s_logit[1][16 * rt + 4 * g + i][n];
    // ---- online softmax (log2 domain).  Row r of the step is present when bit r of
    // `present` is set; only a step with absent rows runs the masking (a uniform
    // branch: the row list is full except at its end).  Exponentials are the hardware's base-2 exponential: a
    // probability below 2^-126 of the reference maximum flushes to 0, far below what
    // its fp16 or bf16 operand resolves next to the maximum's 1.
    const uint32_t present =
        (uint32_t)__ballot(s_rows[step * kStepRows + (lane & (kStepRows - 1))] >= 0);
    float x[8];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[4 * rt + i] = sacc[rt][i] * scale_log2;
    if (__builtin_expect(present != 0xFFFFFFFFu, 0)) {  // a step with absent rows
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!((present >> (16 * rt + 4 * g + i)) & 1u)) x[4 * rt + i] = -INFINITY;
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) mloc = fmaxf(mloc, x[i]);
    mloc = wave_max_rows(mloc);
    // The reference maximum m_run moves only when a step's maximum exceeds it by more
    // than 2^kLazyLog2: the probabilities then stay below 2^kLazyLog2 (within fp16's
    // range, rounded with its full precision), and the accumulators are rescaled only on
    // those rare steps instead of whenever a head's maximum grows.
    const bool grow = mloc > m_run + kLazyLog2;  // m_run at its floor: any present row
    float alpha = 1.0f;
    if (grow) {
      alpha = __builtin_amdgcn_exp2f(m_run - mloc);  // 0 from the floor
      m_run = mloc;
    }
    float psum = 0.0f;
    float pv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pv[i] = __builtin_amdgcn_exp2f(x[i] - m_run);  // absent rows: exp2(-inf) = 0
      psum += pv[i];
    }
    psum = wave_sum_rows(psum);
    l_run = l_run * alpha + psum;
    if (__any(grow)) {
#pragma unroll
      for (int i = 0; i < kNarrowDims / 16; ++i) o[i] *= alpha;
    }
    // ---- O^T += V^T P^T over this wave's dims (K-slots 8g+s <-> rows 4g+s, 16+4g+s-4)
#pragma unroll
    for (int t = 0; t < TM::kPTerms; ++t) {
      const typename TM::Op pb = TM::p_term(pv, t);
#pragma unroll
      for (int i = 0; i < kNarrowDims / 16; ++i)
        o[i] = TM::mma(TM::op(v_fragment(tile, g, n, (kNarrowDims / 16) * wave + i)), pb, o[i]);
    }
  };

  // The first fetches are issued in order (the scheduler may not interleave them), so
  // that each step waits only for its own rows.
  fetch(raw0, 0);
  __builtin_amdgcn_sched_barrier(0);
  fetch(raw1, 1);
  __builtin_amdgcn_sched_barrier(0);
  int step = 0;
  for (; step + 1 < n_steps; step += 2) {
    run_step(raw0, step);
    run_step(raw1, step + 1);
  }
  if (step < n_steps) run_step(raw0, step);

  // ---- partial records: the 16 x 512 output block, divided by each head's sum, is
  // staged through LDS so that each head's record is written by consecutive lanes in
  // whole cache lines; the (max, sum) pairs go to their own array.
  const int64_t rec0 = ((int64_t)b * n_chunks + chunk) * n_heads + 16 * hg;
  lds_barrier();  // every wave is done with the tiles and the query rows
  if (wave == 0 && g == 0)
    *reinterpret_cast<f32x2*>(part_ml + (rec0 + n) * 2) = f32x2{l_run > 0.0f ? m_run : -INFINITY, l_run};
  {
    const float il = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    float* orow = s_out + n * kOutPitch + kNarrowDims * wave + 4 * g;
#pragma unroll
    for (int i = 0; i < kNarrowDims / 16; ++i) *reinterpret_cast<f32x4*>(orow + 16 * i) = o[i] * il;
  }
  lds_barrier();
  constexpr int kVecPerHead = kDim / 4;
#pragma unroll
  for (int k = 0; k < 16 * kVecPerHead / kNarrowThreads; ++k) {
    const int i = threadIdx.x + k * kNarrowThreads;
    const int h = i / kVecPerHead, c4 = i - h * kVecPerHead;
    store_partial4<PartialRecord<KVFMT>::kHalf>(part_o, (rec0 + h) * kDim + 4 * c4,
                                                *reinterpret_cast<const f32x4*>(s_out + h * kOutPitch + 4 * c4));
  }
}

template <int KVFMT, bool CSA, bool PG>
__global__ __launch_bounds__(kNarrowThreads) void attention_narrow_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t seq_stride,
    Paging pg, int64_t n_rows_max, const int32_t* __restrict__ seq_rows,
    const uint16_t* __restrict__ q,
    int n_heads, float scale_log2,
    const int32_t* __restrict__ topk, int top_k, int window, int64_t n_list, int rows_per_chunk,
    int n_chunks, int n_pairs, float* __restrict__ part_o, float* __restrict__ part_ml) {
  __shared__ NarrowSmem sm;
  args_in_sgprs(codes, scales, seq_stride, pg.table, pg.page_shift, pg.table_stride, n_rows_max,
                seq_rows, q, n_heads, scale_log2, topk, top_k, window, n_list, rows_per_chunk,
                n_chunks, n_pairs, part_o, part_ml);
  int b, chunk, hg;
  if (!attn_block(n_pairs, n_heads / 16, n_chunks, &b, &chunk, &hg)) return;
  b = __builtin_amdgcn_readfirstlane(b);
  chunk = __builtin_amdgcn_readfirstlane(chunk);
  hg = __builtin_amdgcn_readfirstlane(hg);
  narrow_chunk<KVFMT, CSA, PG>(sm, codes, scales, seq_stride, pg, n_rows_max, seq_rows, q, n_heads,
                               scale_log2, CSA ? topk + (int64_t)b * top_k : nullptr, window,
                               n_list, rows_per_chunk, n_chunks, part_o, part_ml, b, chunk, hg);
}

// One workgroup: up to 64 heads (four 16-head groups), one chunk of a query's row list.
// All 8 waves gather and decode each 32-row step into one LDS tile that every head
// uses.  Wave w serves head group w / 2 over dims 256 * (w % 2) .. +255: it computes the
// logits' partial sums over those dims, the two halves of each logit meet in LDS, both
// waves of the pair run the same softmax, and each accumulates the output of its own
// dims.  Two tiles alternate, so a step takes two barriers (tile complete; logit halves
// written).  Waves of a head group past the last head only gather and decode.
template <int KVFMT, bool CSA, bool PG>
__global__ __launch_bounds__(kWideThreads) void attention_wide_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t seq_stride,
    Paging pg, int64_t n_rows_max, const int32_t* __restrict__ seq_rows,
    const uint16_t* __restrict__ q,
    int n_heads, float scale_log2,
    const int32_t* __restrict__ topk, int top_k, int window, int64_t n_list, int rows_per_chunk,
    int n_chunks, int n_pairs, int n_blocks, float* __restrict__ part_o, float* __restrict__ part_ml) {
  typedef StepRaw<KVFMT> Raw;
  constexpr int kAhead = Raw::kAhead;
  constexpr int kTileElems = kStepRows * kPitch;
  __shared__ __attribute__((aligned(16))) uint16_t s_tile[2 * kTileElems];
  __shared__ __attribute__((aligned(16))) int s_rows[kMaxChunkRows + kAhead * kStepRows];
  // Partial logits: [dim half][head group][value j of the lane][lane].
  __shared__ __attribute__((aligned(16))) float s_logit[2][kHeadGroups][8][kWave];

  args_in_sgprs(codes, scales, seq_stride, pg.table, pg.page_shift, pg.table_stride, n_rows_max,
                seq_rows, q, n_heads, scale_log2, topk, top_k, window, n_list, rows_per_chunk,
                n_chunks, n_pairs, n_blocks, part_o, part_ml);
  int b, chunk, blk;
  if (!attn_block(n_pairs, n_blocks, n_chunks, &b, &chunk, &blk)) return;
  b = __builtin_amdgcn_readfirstlane(b);
  chunk = __builtin_amdgcn_readfirstlane(chunk);
  blk = __builtin_amdgcn_readfirstlane(blk);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int hg = wave >> 1, kh = wave & 1;
  const int lane = threadIdx.x & (kWave - 1);
  const int g = lane >> 4;
  const int n = lane & 15;
  const int head0 = kBlockHeads * blk + 16 * hg;  // first head of the wave's group
  const bool active = head0 < n_heads;

  const int64_t p_begin = (int64_t)chunk * rows_per_chunk;
  const int64_t p_end = min(p_begin + rows_per_chunk, n_list);
  const int n_steps = (int)((p_end - p_begin + kStepRows - 1) / kStepRows);
  const int64_t n_rows = uniform64(seq_len(seq_rows, b, n_rows_max));  // this sequence's rows
  const int64_t n_c = n_rows - window;

  // Sequence row of every list position of the chunk (-1: absent or out of range), and
  // kAhead steps of -1 past the end for the fetches that run ahead of the last step; for
  // a paged cache, the row's place in the page pool instead.
  for (int i = threadIdx.x; i < (n_steps + kAhead) * kStepRows; i += kWideThreads) {
    const int64_t p = p_begin + i;
    int row = -1;
    if (p < p_end) {
      if (!CSA || p < window) {
        row = p < n_rows ? (int)p : -1;
      } else {
        const int32_t j = topk[(int64_t)b * top_k + (p - window)];
        row = (j >= 0 && j < n_c) ? window + j : -1;
      }
    }
    if (PG && row >= 0)
      row = (pg.table[(int64_t)b * pg.table_stride + (row >> pg.page_shift)] << pg.page_shift) +
            (row & ((1 << pg.page_shift) - 1));
    s_rows[i] = row;
  }
  // The wave's logit B operands, kept in registers: lane (g, n) supplies head n of the
  // group, dims 256 * kh + 32t + 8g .. +7 of K-step t, in the tile's operand type.
  typedef TileMath<KVFMT> TM;
  typename TM::Op qf[kHalfDim / 32];
  if (active) {
    const uint16_t* qr = q + ((int64_t)b * n_heads + head0 + n) * kDim + kHalfDim * kh + 8 * g;
    u32x4 qv[kHalfDim / 32];
#pragma unroll
    for (int t = 0; t < kHalfDim / 32; ++t) qv[t] = *reinterpret_cast<const u32x4*>(qr + 32 * t);
#pragma unroll
    for (int t = 0; t < kHalfDim / 32; ++t) qf[t] = TM::q_op(qv[t]);
  }
  lds_barrier();

  // O^T accumulators of the wave's dims: o[i] holds dims 256 * kh + 16i + 4g .. +3 of
  // head n (lane (g, n)).
  f32x4 o[kHalfDim / 16];
#pragma unroll
  for (int i = 0; i < kHalfDim / 16; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // m_run starts at a finite floor instead of -inf: the first step with a present row
  // always moves it (grow), so no probability is ever taken against the floor, and no
  // exponential sees -inf - -inf.  A chunk without present rows records -inf.
  float m_run = -__FLT_MAX__, l_run = 0.0f;

  // kAhead steps are fetched ahead (a ring of raw buffers), so a short chunk has all its
  // steps in flight as soon as the row indices are known.  Rows are read through buffer
  // resources over this query's sequence.  Every fetch is issued unconditionally (the
  // steps past the end have only absent rows, which read nothing); an absent row's logit
  // is masked to -inf, so its probability is exactly 0.
  Raw raw[kAhead];
  // Rows are addressed inside the sequence's rows, or inside the page pool when paged.
  // Offsets and sizes are made explicitly uniform, so the resources sit in scalar registers.
  const int64_t seq0 = uniform64((int64_t)b * seq_stride);
  const Rsrc rc = PG ? make_rsrc(codes, kAttnMaxSeqBytes)
                     : make_rsrc(codes + uniform64(seq0 * Raw::kRowBytes),
                                 __builtin_amdgcn_readfirstlane((uint32_t)(n_rows * Raw::kRowBytes)));
  const Rsrc rs = Raw::kScaleRowBytes == 0 ? rc
                  : PG ? make_rsrc(scales, kAttnMaxSeqBytes)
                       : make_rsrc(scales + uniform64(seq0 * Raw::kScaleRowBytes),
                                   __builtin_amdgcn_readfirstlane((uint32_t)(n_rows * Raw::kScaleRowBytes)));
  auto fetch = [&](Raw& r, int step) { r.load(rc, rs, s_rows + step * kStepRows, threadIdx.x); };

  auto run_step = [&](Raw& r, int step) {
    uint16_t* tile = s_tile + (step & 1) * kTileElems;
    // ---- decode the fetched rows into the tile (fp16 or bf16, row-major).  The tile
    // was last read two steps ago, before every wave passed the previous step's barriers.
    r.store(tile, threadIdx.x);
    lds_barrier();
    fetch(r, step + kAhead);

    // ---- logits S^T over the wave's dims: lane (g, n) gets rows 16rt + 4g + i of head n.
    // Two accumulator chains per row tile (even and odd K-steps) halve the chain of
    // dependent MFMAs; the halves add in the same order in both waves of the pair.
    f32x4 part[2];
    if (active) {
      const uint16_t* kr = tile + n * kPitch + kHalfDim * kh + 8 * g;
      f32x4 acc[2][2] = {};
#pragma unroll
      for (int t = 0; t < kHalfDim / 32; ++t)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
          acc[rt][t & 1] = TM::mma(TM::op(*reinterpret_cast<const u32x4*>(kr + 16 * rt * kPitch + 32 * t)),
                                   qf[t], acc[rt][t & 1]);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) part[rt] = acc[rt][0] + acc[rt][1];
#pragma unroll
      for (int j = 0; j < 8; ++j) s_logit[kh][hg][j][lane] = part[j >> 2][j & 3];
    }
    lds_barrier();
    if (!active) return;
    // The two halves add in either order to the same fp32 logit, so both waves of the
    // pair see identical logits and keep identical softmax states.
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = (part[j >> 2][j & 3] + s_logit[kh ^ 1][hg][j][lane]) * scale_log2;
    // ---- online softmax (log2 domain).  Row r of the step is present when bit r of
    // `present` is set; only a step with absent rows runs the masking (a uniform branch:
    // the row list is full except at its end).  Exponentials are the hardware's base-2
    // exponential: a probability below 2^-126 of the reference maximum flushes to 0, far
    // below what its fp16 or bf16 operand resolves next to the maximum's 1.
    const uint32_t present =
        (uint32_t)__ballot(s_rows[step * kStepRows + (lane & (kStepRows - 1))] >= 0);
    if (__builtin_expect(present != 0xFFFFFFFFu, 0)) {  // a step with absent rows
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!((present >> (16 * rt + 4 * g + i)) & 1u)) x[4 * rt + i] = -INFINITY;
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) mloc = fmaxf(mloc, x[i]);
    mloc = wave_max_rows(mloc);
    // The reference maximum m_run moves only when a step's maximum exceeds it by more
    // than 2^kLazyLog2: the probabilities then stay below 2^kLazyLog2 (within fp16's
    // range, rounded with its full precision), and the accumulators are rescaled only on
    // those rare steps instead of whenever a head's maximum grows.
    const bool grow = mloc > m_run + kLazyLog2;  // m_run at its floor: any present row
    float alpha = 1.0f;
    if (grow) {
      alpha = __builtin_amdgcn_exp2f(m_run - mloc);  // 0 from the floor
      m_run = mloc;
    }
    float psum = 0.0f;
    float pv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pv[i] = __builtin_amdgcn_exp2f(x[i] - m_run);  // absent rows: exp2(-inf) = 0
      psum += pv[i];
    }
    psum = wave_sum_rows(psum);
    l_run = l_run * alpha + psum;
    if (__any(grow)) {
#pragma unroll
      for (int i = 0; i < kHalfDim / 16; ++i) o[i] *= alpha;
    }
    // ---- O^T += V^T P^T over the wave's dims (K-slots 8g+s <-> rows 4g+s, 16+4g+s-4)
#pragma unroll
    for (int t = 0; t < TM::kPTerms; ++t) {
      const typename TM::Op pb = TM::p_term(pv, t);
#pragma unroll
      for (int i = 0; i < kHalfDim / 16; ++i)
        o[i] = TM::mma(TM::op(v_fragment(tile, g, n, (kHalfDim / 16) * kh + i)), pb, o[i]);
    }
  };

  // The first fetches are issued in ring order (the scheduler may not interleave them),
  // so that, as in the loop, the oldest outstanding loads are the next step's: each step
  // then waits only for its own rows.
#pragma unroll
  for (int k = 0; k < kAhead; ++k) {
    fetch(raw[k], k);
    __builtin_amdgcn_sched_barrier(0);
  }
  // Whole rounds of kAhead steps run without a branch between them, so the loop carries
  // the same outstanding loads around every iteration and each step waits only for its
  // own; the last, partial round follows.
  int step = 0;
  for (; step + kAhead <= n_steps; step += kAhead) {
#pragma unroll
    for (int k = 0; k < kAhead; ++k) run_step(raw[k], step + k);
  }
#pragma unroll
  for (int k = 0; k < kAhead - 1; ++k)
    if (step + k < n_steps) run_step(raw[k], step + k);
  if (!active) return;

  // ---- partial records: (max, sum) per head, and the wave's 256 dims of each head's O
  // divided by the head's sum (four lanes write contiguous pieces of one head's record).
  const int64_t rec = ((int64_t)b * n_chunks + chunk) * n_heads + head0 + n;
  if (kh == 0 && g == 0)
    *reinterpret_cast<f32x2*>(part_ml + rec * 2) = f32x2{l_run > 0.0f ? m_run : -INFINITY, l_run};
  const float il = l_run > 0.0f ? 1.0f / l_run : 0.0f;
  const int64_t e0 = rec * kDim + kHalfDim * kh + 4 * g;
#pragma unroll
  for (int i = 0; i < kHalfDim / 16; ++i)
    store_partial4<PartialRecord<KVFMT>::kHalf>(part_o, e0 + 16 * i, o[i] * il);
}

// One workgroup per (query, head): merges the chunks' (max, sum, O / sum) records (fp16
// records when H16).  NB chunks (the launch picks the smallest of 2, 4, 8, 12, 16 and
// kCombineMaxBatch that covers the chunk count) are read in a single round of
// independent loads; more chunks take further rounds.
constexpr int kCombineThreads = 128;   // 4 dims each
constexpr int kCombineMaxBatch = 32;

template <int NB, bool H16>
__global__ __launch_bounds__(kCombineThreads) void attention_combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml, int n_heads,
    int n_chunks, uint16_t* __restrict__ out) {
  // The launch picks NB < kCombineMaxBatch only for at most NB chunks, so NB slots then
  // hold every chunk's maximum and sum.
  constexpr int kSlots = NB < kCombineMaxBatch ? NB : kMaxChunks;
  __shared__ float s_m[kSlots];
  __shared__ float s_l[kSlots];
  args_in_sgprs(part_o, part_ml, n_heads, n_chunks, out);
  const int bh = blockIdx.x;  // b * n_heads + h
  const int b = bh / n_heads, h = bh - b * n_heads;
  // Chunk c's record of this head starts cstride bytes after chunk c - 1's.  The records
  // are read through buffer resources that end with the last chunk's, so every load of a
  // round is issued unconditionally (a chunk past the last one reads zeros) and the
  // round's loads are in flight together.  The largest resource, 4096 chunks of 128
  // heads of fp32 records, spans 1 GiB; with no chunks (an empty row list) both are empty.
  constexpr uint32_t kElemBytes = H16 ? 2 : 4;
  const uint32_t cstride = (uint32_t)n_heads * kDim * kElemBytes;
  const int64_t rec0 = (int64_t)b * n_chunks * n_heads + h;
  const Rsrc ro = make_rsrc(reinterpret_cast<const uint8_t*>(part_o) + rec0 * kDim * kElemBytes,
                            n_chunks > 0 ? (uint32_t)(n_chunks - 1) * cstride + kDim * kElemBytes : 0u);
  const Rsrc rm = make_rsrc(part_ml + rec0 * 2, n_chunks > 0 ? (uint32_t)(n_chunks - 1) * n_heads * 8 + 8 : 0u);
  const uint32_t d0 = 4 * threadIdx.x;

  f32x4 v[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
    v[i] = load_partial4<H16>(ro, kElemBytes * d0 + i * cstride);
  for (int c = threadIdx.x; c < n_chunks; c += kCombineThreads) {
    const f32x2 ml =
        __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(rm, (uint32_t)c * n_heads * 8, 0, 0));
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
    for (int c0 = 0; c0 < n_chunks; c0 += NB) {
      if (c0 > 0) {
#pragma unroll
        for (int i = 0; i < NB; ++i)
          v[i] = load_partial4<H16>(ro, kElemBytes * d0 + (uint32_t)(c0 + i) * cstride);
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        if (c0 + i < n_chunks) {
          const float wt = s_l[c0 + i] * exp2f(s_m[c0 + i] - mmax);  // 0 for empty chunks
          den += wt;
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

// Heads one workgroup serves: 64 (wide) or 16 (narrow).
int attention_wg_heads(const AttnPlan& plan) { return plan.wide ? kBlockHeads : 16; }

int attention_head_blocks(int n_heads, const AttnPlan& plan) {
  const int h = attention_wg_heads(plan);
  return (n_heads + h - 1) / h;
}

int attention_blocks(int batch, int n_heads, const AttnPlan& plan) {
  const int n_pairs = batch * plan.n_chunks;
  return 8 * attention_head_blocks(n_heads, plan) * ((n_pairs + 7) / 8);
}

template <int KVFMT, bool CSA>
void launch_chunks(hipStream_t stream, const uint8_t* codes, const uint8_t* scales,
                   int64_t seq_stride, const Paging& pg, int64_t n_rows, const int32_t* seq_rows,
                   const uint16_t* q, int batch, int n_heads,
                   float scale_log2, const int32_t* topk, int top_k, int window,
                   const AttnPlan& plan, float* part_o, float* part_ml) {
  const dim3 grid(attention_blocks(batch, n_heads, plan));
  const int n_pairs = batch * plan.n_chunks;
  // A paged cache has its own kernels so that the contiguous ones carry no trace of the
  // page lookup.
#define CSAKV_WIDE(PG)                                                                          \
  hipLaunchKernelGGL((attention_wide_kernel<KVFMT, CSA, PG>), grid, dim3(kWideThreads), 0,        \
                     stream, codes, scales, seq_stride, pg, n_rows, seq_rows, q, n_heads,         \
                     scale_log2, topk, top_k, window, plan.n_list, plan.rows_per_chunk,           \
                     plan.n_chunks, n_pairs, attention_head_blocks(n_heads, plan), part_o, part_ml)
#define CSAKV_NARROW(PG)                                                                        \
  hipLaunchKernelGGL((attention_narrow_kernel<KVFMT, CSA, PG>), grid, dim3(kNarrowThreads), 0,    \
                     stream, codes, scales, seq_stride, pg, n_rows, seq_rows, q, n_heads,         \
                     scale_log2, topk, top_k, window, plan.n_list, plan.rows_per_chunk,           \
                     plan.n_chunks, n_pairs, part_o, part_ml)
  if (plan.wide) {
    if (pg.table) CSAKV_WIDE(true);
    else CSAKV_WIDE(false);
  } else {
    if (pg.table) CSAKV_NARROW(true);
    else CSAKV_NARROW(false);
  }
#undef CSAKV_WIDE
#undef CSAKV_NARROW
}

// Output RoPE with position -i on the 64 RoPE dims of every output row, in place: one
// thread per (query, head, pair k); pair (448 + 2k, 448 + 2k + 1) turns by angle
// -position * base^(-2k/64).  The angle and its sine and cosine are computed in fp64
// (positions reach 2^20 and beyond), the rotation in fp32, the result rounded to bf16.
__global__ __launch_bounds__(256) void rope_output_kernel(uint16_t* __restrict__ out,
                                                          int64_t n_items, int n_heads,
                                                          const int64_t* __restrict__ positions,
                                                          double base) {
#pragma clang fp contract(off)
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < n_items;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int k = (int)(t & 31);
    const int64_t bh = t >> 5;
    const int64_t b = bh / n_heads;
    const double theta = pow(base, -2.0 * k / 64.0);
    double sd, cd;
    sincos(-(double)positions[b] * theta, &sd, &cd);
    uint32_t* p = reinterpret_cast<uint32_t*>(out + bh * kDim + kNope + 2 * k);
    const uint32_t w = *p;
    const float x = bf16_to_f32(w & 0xFFFFu), y = bf16_to_f32(w >> 16);
    const float c = (float)cd, sn = (float)sd;
    const float rx = x * c - y * sn;
    const float ry = x * sn + y * c;
    *p = f32_to_bf16_rne(rx) | (f32_to_bf16_rne(ry) << 16);
  }
}

}  // namespace

hipError_t launch_rope_output(uint16_t* out, int batch, int n_heads, const int64_t* positions,
                              double base, hipStream_t stream) {
  const int64_t items = (int64_t)batch * n_heads * 32;
  if (items == 0) return hipSuccess;
  const int64_t grid = std::min<int64_t>((items + 255) / 256, 4096);
  hipLaunchKernelGGL(rope_output_kernel, dim3((unsigned)grid), dim3(256), 0, stream, out, items,
                     n_heads, positions, base);
  return hipGetLastError();
}

AttnPlan plan_attention(int batch, int64_t n_list, bool csa, int n_heads) {
  AttnPlan p{};
  p.n_list = n_list;
  p.wide = n_list >= kWideMinRows;
  // Chunks of whole 32-row steps; about one workgroup per compute unit in all, each one
  // (query, chunk, head block), never more than kMaxChunks chunks per query.
  const int64_t blocks = std::max(1, attention_head_blocks(n_heads, p));
  const int64_t want = (kAttnTargetBlocks + batch * blocks - 1) / (batch * blocks);
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

bool attention_supported(const AttnPlan& plan, int kv_fmt, int64_t n_rows) {
  const int64_t row_bytes = kv_fmt == 0 ? StepRaw<0>::kRowBytes
                            : kv_fmt == 1 ? StepRaw<1>::kRowBytes
                                          : StepRaw<2>::kRowBytes;
  return plan.n_chunks <= kMaxChunks && plan.rows_per_chunk <= kMaxChunkRows && n_rows >= 0 &&
         n_rows * row_bytes <= (int64_t)kAttnMaxSeqBytes;
}

// Workspace: O records [B][chunks][H][512] fp32 (fp16 records for FP8 and FP4 rows fill
// the first half of the same space), then (max, sum) pairs [B][chunks][H][2].
size_t attention_workspace_bytes(int batch, int n_heads, const AttnPlan& plan) {
  return (size_t)batch * plan.n_chunks * n_heads * (kDim + 2) * sizeof(float);
}

template <bool H16>
void launch_combine(hipStream_t stream, int batch, int n_heads, int n_chunks, const float* part_o,
                    const float* part_ml, uint16_t* out) {
  // A round's loads past the last chunk read nothing but still pass through the address
  // unit, so the round is as short as the chunk count allows.
#define CSAKV_COMBINE(NB)                                                                       \
  hipLaunchKernelGGL((attention_combine_kernel<NB, H16>), dim3(batch * n_heads), dim3(kCombineThreads), \
                     0, stream, part_o, part_ml, n_heads, n_chunks, out)
  if (n_chunks <= 2) CSAKV_COMBINE(2);
  else if (n_chunks <= 4) CSAKV_COMBINE(4);
  else if (n_chunks <= 8) CSAKV_COMBINE(8);
  else if (n_chunks <= 12) CSAKV_COMBINE(12);
  else if (n_chunks <= 16) CSAKV_COMBINE(16);
  else CSAKV_COMBINE(kCombineMaxBatch);
#undef CSAKV_COMBINE
}

hipError_t launch_attention(int kv_fmt, bool csa, const uint8_t* codes, const uint8_t* scales,
                            int64_t seq_stride, const Paging& pg, int64_t n_rows,
                            const int32_t* seq_rows, const uint16_t* q, int batch,
                            int n_heads, float softmax_scale, const int32_t* topk, int top_k,
                            int window, const AttnPlan& plan, void* workspace, uint16_t* out,
                            hipStream_t stream) {
  float* part_o = static_cast<float*>(workspace);
  float* part_ml = part_o + (size_t)batch * plan.n_chunks * n_heads * kDim;
  const float sl2 = softmax_scale * kLog2e;
  if (plan.n_chunks > 0) {
#define CSAKV_ATTN(F, C)                                                                        \
  launch_chunks<F, C>(stream, codes, scales, seq_stride, pg, n_rows, seq_rows, q, batch, n_heads, sl2, topk, \
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
  // The combine reads the records the chunk kernel wrote for this row format (FP8 and
  // FP4 rows share the fp16 records).
  if (kv_fmt == 0) launch_combine<PartialRecord<0>::kHalf>(stream, batch, n_heads, plan.n_chunks, part_o, part_ml, out);
  else launch_combine<PartialRecord<1>::kHalf>(stream, batch, n_heads, plan.n_chunks, part_o, part_ml, out);
  return hipGetLastError();
}

}  // namespace csakv
