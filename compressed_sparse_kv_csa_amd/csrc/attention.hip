// Multi-query softmax attention over gathered shared-KV rows (CSA sparse, HCA dense).
//
// What is computed ("DeepSeek-V4 KV Cache 深度分析", section 三 for the CSA/HCA row sets,
// section 五 for one entry serving as both key and value, and the section 十一 diagram):
//   o[h] = sum_r softmax_r(scale * q[h] . e_r) * e_r
// over the rows r of one query: CSA = the window rows plus the selected compressed
// rows (one softmax over their union), HCA = every row of the sequence.
//
// Structure: grid (chunks, B).  A workgroup owns one chunk of a query's row list and
// all heads (one wave per 16 heads).  Per step it gathers 32 rows (whole rows,
// coalesced) and decodes them into LDS twice: row-major bf16 for the logits and
// dim-major fp16 for the value product.  It then runs
//   S^T[32 rows x 16 heads] = K[32 x 512] . Q^T           (16x16x32 bf16 MFMA)
//   O^T[512 x 16 heads]    += V^T[512 x 32] . P^T[32 x 16] (16x16x32 f16 MFMA)
// with an online softmax in fp32 (exp2 domain).  Logit products are exact (bf16 x
// bf16); every decoded cache value is exact in fp16 as well (down to 2^-24), and the
// probabilities, being in [0, 1], keep 11 significant bits in fp16 instead of bf16's 8.  The next step's rows are fetched
// into registers while the current step computes.  Each chunk writes (max, sum,
// unnormalised O) per head; a combine kernel merges the chunks and rounds to bf16.
#include "csakv_device.h"
#include "csakv_launch.h"

namespace csakv {

namespace {

constexpr int kDim = 512;
constexpr int kNope = 448;
constexpr int kStepRows = 32;
constexpr int kKPitch = kDim + 8;         // bf16 elements per row-major LDS row
constexpr int kVPitch = kStepRows + 8;    // fp16 elements per dim-major LDS row
constexpr int kPartStride = kDim + 4;     // floats per (chunk, head) partial record
constexpr float kLog2e = 1.4426950408889634f;

// Raw bytes of one (row, 64-dim segment) work item, before decoding.
template <int KVFMT>
struct SegRaw;

template <>
struct SegRaw<0> {  // bf16: 128 bytes
  u32x4 v[8];
  __device__ __forceinline__ void load(const uint8_t* codes, const uint8_t*, int64_t row, int seg) {
    const u32x4* p = reinterpret_cast<const u32x4*>(codes + row * (kDim * 2) + seg * 128);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = p[i];
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = u32x4{0u, 0u, 0u, 0u};
  }
  // 32 dwords of bf16 pairs for dims seg*64 .. seg*64+63
  __device__ __forceinline__ void decode(int, uint32_t* out) const {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) out[4 * i + j] = v[i][j];
  }
};

template <>
struct SegRaw<1> {  // mixed: 64 E4M3 bytes (segments 0..6) or 128 bf16 bytes (segment 7)
  u32x4 v[8];
  __device__ __forceinline__ void load(const uint8_t* codes, const uint8_t*, int64_t row, int seg) {
    const uint8_t* base = codes + row * (kNope + 2 * (kDim - kNope));
    if (seg < 7) {
      const u32x4* p = reinterpret_cast<const u32x4*>(base + seg * 64);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = p[i];
    } else {
      const u32x4* p = reinterpret_cast<const u32x4*>(base + kNope);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = p[i];
    }
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = u32x4{0u, 0u, 0u, 0u};
  }
  __device__ __forceinline__ void decode(int seg, uint32_t* out) const {
    if (seg < 7) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(v[i][j], false);
          f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(v[i][j], true);
          out[8 * i + 2 * j] = pack_bf16_exact(lo[0], lo[1]);
          out[8 * i + 2 * j + 1] = pack_bf16_exact(hi[0], hi[1]);
        }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) out[4 * i + j] = v[i][j];
    }
  }
};

template <>
struct SegRaw<2> {  // FP4: 32 code bytes + 4 E4M3 scale bytes
  u32x4 c[2];
  uint32_t s;
  __device__ __forceinline__ void load(const uint8_t* codes, const uint8_t* scales, int64_t row,
                                       int seg) {
    const u32x4* p = reinterpret_cast<const u32x4*>(codes + row * (kDim / 2) + seg * 32);
    c[0] = p[0];
    c[1] = p[1];
    s = *reinterpret_cast<const uint32_t*>(scales + row * (kDim / 16) + seg * 4);
  }
  __device__ __forceinline__ void zero() {
    c[0] = c[1] = u32x4{0u, 0u, 0u, 0u};
    s = 0u;
  }
  __device__ __forceinline__ void decode(int, uint32_t* out) const {
#pragma unroll
    for (int w = 0; w < 8; ++w) {  // 8 dwords of codes, 8 elements each; 2 dwords per scale
      const uint32_t cw = c[w >> 2][w & 3];
      const float sc = e4m3_to_f32((s >> (8 * (w >> 1))) & 0xFFu);
      const u32x4 d = fp4x8_to_bf16(cw, sc);
#pragma unroll
      for (int b = 0; b < 4; ++b) out[4 * w + b] = d[b];
    }
  }
};

// Position of row r (0..31) inside a dim-major LDS row: the 8 K-slots of lane group g
// are rows 4g..4g+3 and 16+4g..16+4g+3, stored contiguously.
__device__ __forceinline__ int vpos(int r) {
  const int rt = r >> 4, rr = r & 15;
  return 8 * (rr >> 2) + 4 * rt + (rr & 3);
}

template <int KVFMT, bool CSA, int HG>
__global__ __launch_bounds__(64 * HG) void attention_chunk_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t seq_stride,
    int64_t n_rows, const uint16_t* __restrict__ q, int n_heads, float scale_log2,
    const int32_t* __restrict__ topk, int top_k, int window, int64_t n_list, int rows_per_chunk,
    int n_chunks, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t s_k[kStepRows * kKPitch];
  __shared__ __attribute__((aligned(16))) uint16_t s_v[kDim * kVPitch];
  __shared__ int s_valid[kStepRows];

  const int chunk = blockIdx.x;
  const int b = blockIdx.y;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int g = lane >> 4;
  const int n = lane & 15;
  const int head = 16 * wave + n;

  const int64_t p_begin = (int64_t)chunk * rows_per_chunk;
  const int64_t p_end = min(p_begin + rows_per_chunk, n_list);
  const int n_steps = (int)((p_end - p_begin + kStepRows - 1) / kStepRows);
  const int64_t n_c = n_rows - window;

  // Row of the sequence at list position p, or -1 when absent.
  auto row_of = [&](int64_t p) -> int64_t {
    if (p >= p_end) return -1;
    if (!CSA) return p;
    if (p < window) return p;
    const int32_t j = topk[(int64_t)b * top_k + (p - window)];
    return (j >= 0 && j < n_c) ? window + j : -1;
  };

  // Query fragments (B operand): head `head`, dims 32t + 8g .. +7, t = 0..15.
  bf16x8 qf[16];
  {
    const uint16_t* qh = q + ((int64_t)b * n_heads + head) * kDim + 8 * g;
#pragma unroll
    for (int t = 0; t < 16; ++t) qf[t] = as_bf16x8(*reinterpret_cast<const u32x4*>(qh + 32 * t));
  }

  f32x4 o[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;

  // Work items of this thread inside a step: item = row r * 8 + 64-dim segment seg.
  constexpr int kThreads = 64 * HG;
  constexpr int kItems = (kStepRows * 8 + kThreads - 1) / kThreads;
  SegRaw<KVFMT> raw[kItems];
  int64_t raw_row[kItems];

  auto fetch = [&](int step) {
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
      const int item = threadIdx.x + it * kThreads;
      if (item < kStepRows * 8) {
        const int r = item >> 3, seg = item & 7;
        const int64_t row = row_of(p_begin + (int64_t)step * kStepRows + r);
        raw_row[it] = row;
        if (row >= 0) raw[it].load(codes, scales, (int64_t)b * seq_stride + row, seg);
        else raw[it].zero();
      }
    }
  };

  if (n_steps > 0) fetch(0);
  for (int step = 0; step < n_steps; ++step) {
    // ---- decode the fetched rows into LDS
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
      const int item = threadIdx.x + it * kThreads;
      if (item < kStepRows * 8) {
        const int r = item >> 3, seg = item & 7;
        uint32_t d[32];
        raw[it].decode(seg, d);
        u32x4* kd = reinterpret_cast<u32x4*>(s_k + r * kKPitch + seg * 64);
#pragma unroll
        for (int i = 0; i < 8; ++i) kd[i] = u32x4{d[4 * i], d[4 * i + 1], d[4 * i + 2], d[4 * i + 3]};
        const int vp = vpos(r);
        uint16_t* vd = s_v + (seg * 64) * kVPitch + vp;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          vd[(2 * i) * kVPitch] = (uint16_t)f32_to_f16_bits(bf16_to_f32(d[i] & 0xFFFFu));
          vd[(2 * i + 1) * kVPitch] = (uint16_t)f32_to_f16_bits(bf16_to_f32(d[i] >> 16));
        }
        if (seg == 0) s_valid[r] = raw_row[it] >= 0;
      }
    }
    __syncthreads();
    if (step + 1 < n_steps) fetch(step + 1);

    // ---- logits S^T: lane (g, n) gets rows 16*rt + 4g + i of head `head`
    f32x4 sacc[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      sacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint16_t* kr = s_k + (16 * rt + n) * kKPitch + 8 * g;
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(kr + 32 * t));
        sacc[rt] = mfma16x16x32(a, qf[t], sacc[rt]);
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
        float v = s_valid[r] ? sacc[rt][i] * scale_log2 : -INFINITY;
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
      for (int i = 0; i < 32; ++i) o[i] *= alpha;
    }
    // ---- O^T += V^T P^T
    const f16x8 pb = as_f16x8(u32x4{pw[0], pw[1], pw[2], pw[3]});
    const uint16_t* vr = s_v + n * kVPitch + 8 * g;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      f16x8 a = as_f16x8(*reinterpret_cast<const u32x4*>(vr + (16 * dt) * kVPitch));
      o[dt] = mfma16x16x32_f16(a, pb, o[dt]);
    }
    __syncthreads();
  }

  // ---- partial record: [m, l, -, -, O[0..512)]
  float* rec = part + (((int64_t)b * n_chunks + chunk) * n_heads + head) * kPartStride;
  if (g == 0) {
    rec[0] = m_run;
    rec[1] = l_run;
  }
#pragma unroll
  for (int dt = 0; dt < 32; ++dt)
    *reinterpret_cast<f32x4*>(rec + 4 + 16 * dt + 4 * g) = o[dt];
}

__global__ __launch_bounds__(128) void attention_combine_kernel(const float* __restrict__ part,
                                                                int n_heads, int n_chunks,
                                                                uint16_t* __restrict__ out) {
  const int bh = blockIdx.x;  // b * n_heads + h
  const int b = bh / n_heads, h = bh - b * n_heads;
  float mmax = -INFINITY;
  for (int c = 0; c < n_chunks; ++c)
    mmax = fmaxf(mmax, part[(((int64_t)b * n_chunks + c) * n_heads + h) * kPartStride]);
  float den = 0.0f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int d0 = 4 * threadIdx.x;
  if (mmax != -INFINITY) {
    for (int c = 0; c < n_chunks; ++c) {
      const float* rec = part + (((int64_t)b * n_chunks + c) * n_heads + h) * kPartStride;
      const float m = rec[0];
      if (m == -INFINITY) continue;
      const float wgt = exp2f(m - mmax);
      den += rec[1] * wgt;
      acc += *reinterpret_cast<const f32x4*>(rec + 4 + d0) * wgt;
    }
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  uint32_t lo = f32_to_bf16_rne(acc[0] * inv) | (f32_to_bf16_rne(acc[1] * inv) << 16);
  uint32_t hi = f32_to_bf16_rne(acc[2] * inv) | (f32_to_bf16_rne(acc[3] * inv) << 16);
  *reinterpret_cast<u32x2*>(out + (int64_t)bh * kDim + d0) = u32x2{lo, hi};
}

template <int KVFMT, bool CSA>
void launch_chunks(dim3 grid, hipStream_t stream, const uint8_t* codes, const uint8_t* scales,
                   int64_t seq_stride, int64_t n_rows, const uint16_t* q, int n_heads,
                   float scale_log2, const int32_t* topk, int top_k, int window,
                   const AttnPlan& plan, float* part) {
#define CSAKV_CHUNK(HG)                                                                        \
  hipLaunchKernelGGL((attention_chunk_kernel<KVFMT, CSA, HG>), grid, dim3(64 * HG), 0, stream,  \
                     codes, scales, seq_stride, n_rows, q, n_heads, scale_log2, topk, top_k,    \
                     window, plan.n_list, plan.rows_per_chunk, plan.n_chunks, part)
  switch (n_heads / 16) {
    case 1: CSAKV_CHUNK(1); break;
    case 2: CSAKV_CHUNK(2); break;
    case 3: CSAKV_CHUNK(3); break;
    default: CSAKV_CHUNK(4); break;
  }
#undef CSAKV_CHUNK
}

}  // namespace

AttnPlan plan_attention(int batch, int64_t n_list, bool csa) {
  AttnPlan p{};
  p.n_list = n_list;
  int64_t rpc;
  if (csa) {
    rpc = 64;
  } else {
    // About 512 workgroups in all, chunks of whole 32-row steps.
    int64_t want = (512 + batch - 1) / batch;
    rpc = (n_list + want - 1) / want;
    if (rpc < 64) rpc = 64;
  }
  rpc = ((rpc + kStepRows - 1) / kStepRows) * kStepRows;
  p.rows_per_chunk = (int)rpc;
  p.n_chunks = (int)((n_list + rpc - 1) / rpc);
  return p;
}

size_t attention_workspace_bytes(int batch, int n_heads, const AttnPlan& plan) {
  return (size_t)batch * plan.n_chunks * n_heads * kPartStride * sizeof(float);
}

hipError_t launch_attention(int kv_fmt, bool csa, const uint8_t* codes, const uint8_t* scales,
                            int64_t seq_stride, int64_t n_rows, const uint16_t* q, int batch,
                            int n_heads, float softmax_scale, const int32_t* topk, int top_k,
                            int window, const AttnPlan& plan, void* workspace, uint16_t* out,
                            hipStream_t stream) {
  float* part = static_cast<float*>(workspace);
  const float sl2 = softmax_scale * kLog2e;
  if (plan.n_chunks > 0) {
    dim3 grid(plan.n_chunks, batch);
#define CSAKV_ATTN(F, C)                                                                     \
  launch_chunks<F, C>(grid, stream, codes, scales, seq_stride, n_rows, q, n_heads, sl2, topk, \
                      top_k, window, plan, part)
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
  hipLaunchKernelGGL(attention_combine_kernel, dim3(batch * n_heads), dim3(128), 0, stream, part,
                     n_heads, plan.n_chunks, out);
  return hipGetLastError();
}

}  // namespace csakv
