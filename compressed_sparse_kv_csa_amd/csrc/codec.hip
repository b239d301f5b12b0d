// Cache-write codecs: FP4 block quantisation, mixed FP8/BF16 rows, and the exact
// decode of every cache format back to bf16.
//
// Formats ("DeepSeek-V4 KV Cache 深度分析", sections 二 and 六, for the 576-byte mixed
// entry; "DeepSeek, KV 캐시를 토큰당 890바이트로 줄인 V4.1-Flash 공개", section 핵심 내용,
// for E2M1 values with one E4M3 scale per 16 channels):
//   FP4 block: scale = E4M3FN(amax / 6), code = E2M1(x / scale) (all zero when the
//   scale decodes to 0); round to nearest even, saturating, sign kept.
//   Mixed row: E4M3FN(x[0:nope]) bytes, then the bf16 bytes of x[nope:dim].
// One thread handles one 16-channel block; consecutive threads take consecutive
// blocks, so every load and store of a wave is contiguous.
#include "csakv_device.h"
#include "csakv_launch.h"

namespace csakv {

namespace {

// One 16-channel block of bf16 values (two 16-byte words) -> 8 bytes of FP4 codes and
// the E4M3 scale byte.
__device__ __forceinline__ void fp4_block(u32x4 w0, u32x4 w1, u32x2* codes, uint32_t* scale) {
  const uint32_t w[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
  float v[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
  fp4_block_f32(v, codes, scale);
}

// 16 bf16 values -> 16 E4M3FN bytes.
__device__ __forceinline__ u32x4 e4m3_block(u32x4 w0, u32x4 w1) {
  uint32_t w[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
  uint32_t o[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t lo = f32_to_e4m3(bf16_to_f32(w[i] & 0xFFFFu));
    const uint32_t hi = f32_to_e4m3(bf16_to_f32(w[i] >> 16));
    o[i >> 1] |= (lo | (hi << 8)) << (16 * (i & 1));
  }
  return u32x4{o[0], o[1], o[2], o[3]};
}

__global__ __launch_bounds__(256) void quantize_fp4_kernel(const uint16_t* __restrict__ x,
                                                           int64_t n_blocks,
                                                           uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales) {
  for (int64_t blk = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; blk < n_blocks;
       blk += (int64_t)gridDim.x * blockDim.x) {
    const u32x4* src = reinterpret_cast<const u32x4*>(x + blk * 16);
    u32x2 c;
    uint32_t sc;
    fp4_block(src[0], src[1], &c, &sc);
    reinterpret_cast<u32x2*>(codes)[blk] = c;
    scales[blk] = (uint8_t)sc;
  }
}

__global__ __launch_bounds__(256) void quantize_fp8_mixed_kernel(const uint16_t* __restrict__ x,
                                                                 int64_t rows, int dim, int nope,
                                                                 uint8_t* __restrict__ out) {
  const int chunks = dim / 16;
  const int64_t row_bytes = nope + 2 * (int64_t)(dim - nope);
  const int64_t total = rows * chunks;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = t / chunks;
    const int c = (int)(t - r * chunks);
    const u32x4* src = reinterpret_cast<const u32x4*>(x + r * dim + 16 * c);
    u32x4 w0 = src[0], w1 = src[1];
    uint8_t* dst_row = out + r * row_bytes;
    if (16 * c < nope) {
      *reinterpret_cast<u32x4*>(dst_row + 16 * c) = e4m3_block(w0, w1);
    } else {
      u32x4* dst = reinterpret_cast<u32x4*>(dst_row + nope + 2 * (16 * c - nope));
      dst[0] = w0;
      dst[1] = w1;
    }
  }
}

// Decode-step cache write: one thread per 16-channel block of the B x n new rows.  Row
// r = b * n + i goes to cache row dst[r] of sequence b (skipped outside [0, n_rows)).
// FMT is the cache format (0 bf16, 1 mixed with 448 E4M3 dims, 2 FP4).
template <int FMT>
__global__ __launch_bounds__(256) void cache_write_kernel(const uint16_t* __restrict__ x,
                                                          const int32_t* __restrict__ dst,
                                                          int64_t n_new, int n, int dim,
                                                          int64_t seq_stride, int64_t n_rows,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  const int chunks = dim / 16;
  const int64_t total = n_new * chunks;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = t / chunks;
    const int c = (int)(t - r * chunks);
    const int32_t d = dst[r];
    if (d < 0 || d >= n_rows) continue;
    const int64_t row = (r / n) * seq_stride + d;
    const u32x4* src = reinterpret_cast<const u32x4*>(x + r * dim + 16 * c);
    const u32x4 w0 = src[0], w1 = src[1];
    if (FMT == 0) {
      u32x4* out = reinterpret_cast<u32x4*>(codes + row * dim * 2 + 32 * c);
      out[0] = w0;
      out[1] = w1;
    } else if (FMT == 1) {
      constexpr int kNope = 448;
      uint8_t* out = codes + row * (kNope + 2 * (512 - kNope));
      if (16 * c < kNope) {
        *reinterpret_cast<u32x4*>(out + 16 * c) = e4m3_block(w0, w1);
      } else {
        u32x4* o = reinterpret_cast<u32x4*>(out + kNope + 2 * (16 * c - kNope));
        o[0] = w0;
        o[1] = w1;
      }
    } else {
      u32x2 cw;
      uint32_t sc;
      fp4_block(w0, w1, &cw, &sc);
      *reinterpret_cast<u32x2*>(codes + row * (dim / 2) + 8 * c) = cw;
      scales[row * (dim / 16) + c] = (uint8_t)sc;
    }
  }
}

// Hadamard-rotated FP4 indexer keys: 16 lanes per 128-wide bf16 row, lane j holding
// channels 8j .. 8j + 7 in fp64.  Butterflies h = 1, 2, 4 run in registers and h = 8 .. 64
// across lanes j ^ 1 .. j ^ 8; every sum is exact, so the fp32 value of each channel is the
// exact H x rounded once, then scaled once.  The 16-channel FP4 blocks span lane pairs
// (2k, 2k + 1): their amax is exchanged, each lane encodes its 8 codes (one dword) and
// the even lane stores the block's scale byte.
__global__ __launch_bounds__(256) void quantize_fp4h_kernel(const uint16_t* __restrict__ x,
                                                            int64_t rows,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales) {
  const int j = threadIdx.x & 15;  // lane of the row's 16
  const int64_t groups = (int64_t)gridDim.x * (blockDim.x / 16);
  for (int64_t r = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) / 16; r < rows; r += groups) {
    // (r is uniform over the 16 lanes of a row, so all of them take part in every shuffle)
    const u32x4 w = reinterpret_cast<const u32x4*>(x + r * 128)[j];
    double y[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      y[2 * i] = (double)bf16_to_f32(w[i] & 0xFFFFu);
      y[2 * i + 1] = (double)bf16_to_f32(w[i] >> 16);
    }
    hadamard_stages<8>(y);
#pragma unroll
    for (int m = 1; m < 16; m *= 2) hadamard_lane_stage<8>(y, m, (j & m) != 0);
    float v[8];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] = hadamard_round_scale(y[i]);
      amax = fmaxf(amax, fabsf(v[i]));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    const uint32_t sc = f32_to_e4m3(amax / 6.0f);
    const float s = e4m3_to_f32(sc);
    uint32_t packed = 0u;
    if (s != 0.0f) {
#pragma unroll
      for (int i = 0; i < 8; ++i) packed |= f32_to_e2m1(v[i] / s) << (4 * i);
    }
    reinterpret_cast<uint32_t*>(codes + r * 64)[j] = packed;
    if ((j & 1) == 0) scales[r * 8 + (j >> 1)] = (uint8_t)sc;
  }
}

__global__ __launch_bounds__(256) void dequantize_kernel(int fmt, const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ scales,
                                                         int64_t rows, int dim, int nope,
                                                         uint16_t* __restrict__ out) {
  const int chunks = dim / 16;
  const int64_t total = rows * chunks;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = t / chunks;
    const int c = (int)(t - r * chunks);
    u32x4* dst = reinterpret_cast<u32x4*>(out + r * dim + 16 * c);
    if (fmt == 0) {  // bf16
      const u32x4* src = reinterpret_cast<const u32x4*>(codes + (r * dim + 16 * c) * 2);
      dst[0] = src[0];
      dst[1] = src[1];
    } else if (fmt == 1) {  // mixed
      const int64_t row_bytes = nope + 2 * (int64_t)(dim - nope);
      const uint8_t* row = codes + r * row_bytes;
      if (16 * c < nope) {
        u32x4 b = *reinterpret_cast<const u32x4*>(row + 16 * c);
        u32x4 o0, o1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(b[i], false);
          f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(b[i], true);
          uint32_t p0 = pack_bf16_exact(lo[0], lo[1]);
          uint32_t p1 = pack_bf16_exact(hi[0], hi[1]);
          if (i < 2) { o0[2 * i] = p0; o0[2 * i + 1] = p1; }
          else { o1[2 * (i - 2)] = p0; o1[2 * (i - 2) + 1] = p1; }
        }
        dst[0] = o0;
        dst[1] = o1;
      } else {
        const u32x4* src = reinterpret_cast<const u32x4*>(row + nope + 2 * (16 * c - nope));
        dst[0] = src[0];
        dst[1] = src[1];
      }
    } else {  // fp4
      u32x2 cw = reinterpret_cast<const u32x2*>(codes)[r * chunks + c];
      float s = e4m3_to_f32(scales[r * chunks + c]);
      dst[0] = fp4x8_to_bf16(cw[0], s);
      dst[1] = fp4x8_to_bf16(cw[1], s);
    }
  }
}

inline int grid_for(int64_t work, int block) {
  int64_t g = (work + block - 1) / block;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

hipError_t launch_quantize_fp4(const uint16_t* x, int64_t rows, int dim, uint8_t* codes,
                               uint8_t* scales, hipStream_t stream) {
  int64_t n_blocks = rows * (dim / 16);
  if (n_blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_fp4_kernel, dim3(grid_for(n_blocks, 256)), dim3(256), 0, stream, x,
                     n_blocks, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8_mixed(const uint16_t* x, int64_t rows, int dim, int nope,
                                     uint8_t* out, hipStream_t stream) {
  int64_t work = rows * (dim / 16);
  if (work == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_fp8_mixed_kernel, dim3(grid_for(work, 256)), dim3(256), 0, stream, x,
                     rows, dim, nope, out);
  return hipGetLastError();
}

hipError_t launch_quantize_fp4h(const uint16_t* x, int64_t rows, uint8_t* codes, uint8_t* scales,
                                hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_fp4h_kernel, dim3(grid_for(rows * 16, 256)), dim3(256), 0, stream, x,
                     rows, codes, scales);
  return hipGetLastError();
}

hipError_t launch_cache_write(int fmt, int dim, void* codes, uint8_t* scales, int64_t seq_stride,
                              int64_t n_rows, int batch, int n, const uint16_t* x,
                              const int32_t* dst, hipStream_t stream) {
  const int64_t n_new = (int64_t)batch * n;
  const int64_t work = n_new * (dim / 16);
  if (work == 0) return hipSuccess;
  uint8_t* c = static_cast<uint8_t*>(codes);
#define CSAKV_WRITE(F)                                                                         \
  hipLaunchKernelGGL((cache_write_kernel<F>), dim3(grid_for(work, 256)), dim3(256), 0, stream, x, \
                     dst, n_new, n, dim, seq_stride, n_rows, c, scales)
  if (fmt == 0) CSAKV_WRITE(0);
  else if (fmt == 1) CSAKV_WRITE(1);
  else CSAKV_WRITE(2);
#undef CSAKV_WRITE
  return hipGetLastError();
}

hipError_t launch_dequantize(int fmt, const void* codes, const uint8_t* scales, int64_t rows,
                             int dim, int nope, uint16_t* out, hipStream_t stream) {
  int64_t work = rows * (dim / 16);
  if (work == 0) return hipSuccess;
  hipLaunchKernelGGL(dequantize_kernel, dim3(grid_for(work, 256)), dim3(256), 0, stream, fmt,
                     static_cast<const uint8_t*>(codes), scales, rows, dim, nope, out);
  return hipGetLastError();
}

}  // namespace csakv
