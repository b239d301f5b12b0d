// Device-side helpers shared by the csakv HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csakv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- buffer resources

// A raw buffer resource over [base, base + bytes): a load at an offset at or past the
// end returns zeros and touches no memory.  base must be wave-uniform.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// ---------------------------------------------------------------- kernel arguments

// Kernel arguments are read from the argument segment by scalar loads that the compiler
// places at each argument's first use, so a prologue with branches pays one round trip
// per group of first uses.  Naming every argument as a scalar-register input of an empty
// asm statement at kernel entry issues all of those loads together, behind one wait.
template <class T>
__device__ __forceinline__ void arg_in_sgprs(T v) {
  asm volatile("" ::"s"(v));
}
template <class... T>
__device__ __forceinline__ void args_in_sgprs(T... v) {
  (arg_in_sgprs(v), ...);
}

// ---------------------------------------------------------------- bf16 bits

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even fp32 -> bf16 bit pattern (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t lsb = (u >> 16) & 1u;
  return (u + 0x7FFFu + lsb) >> 16;
}

// Two fp32 values that are exactly representable in bf16 -> packed bf16x2 bits.
__device__ __forceinline__ uint32_t pack_bf16_exact(float lo, float hi) {
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
}

// ---------------------------------------------------------------- OCP E4M3FN

// Value of an E4M3FN code (NaN codes are never produced by this library's encoders
// and are decoded as the pattern the hardware conversion gives).
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  f32x2 v = __builtin_amdgcn_cvt_pk_f32_fp8(code & 0xFFu, false);
  return v[0];
}

// E4M3FN code of x: round to nearest even on the finite grid, saturating at +-448,
// sign kept.  Exact integer/power-of-two arithmetic only.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  float a = fabsf(x);
  if (!(a < 448.0f)) return sign | 0x7Eu;                 // also catches +inf
  int e = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;  // floor(log2 a) for normal a
  if (e < -6) e = -6;                                      // subnormal quantum 2^-9
  float q = __builtin_ldexpf(a, 3 - e);                    // a / 2^(e-3), exact
  int n = (int)__builtin_rintf(q);                         // round half to even
  int code = (e + 7) * 8 + n - 8;
  if (code > 0x7E) code = 0x7E;
  return sign | (uint32_t)code;
}

// ---------------------------------------------------------------- OCP E2M1

// E2M1 code of r: nearest of {0,.5,1,1.5,2,3,4,6}, ties to the even code, saturating.
__device__ __forceinline__ uint32_t f32_to_e2m1(float r) {
  uint32_t sign = (__float_as_uint(r) >> 28) & 0x8u;
  float a = fabsf(r);
  uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) +
               (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  return sign | c;
}

// One 16-channel block of fp32 values -> FP4 codes (element 2i in the low nibble of
// byte i) and the E4M3 scale byte: scale = E4M3(amax / 6), code = E2M1(x / scale), both
// divisions single fp32 divisions; all codes 0 when the scale decodes to 0.
__device__ __forceinline__ void fp4_block_f32(const float* v, u32x2* codes, uint32_t* scale) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const uint32_t sc = f32_to_e4m3(amax / 6.0f);
  const float s = e4m3_to_f32(sc);
  uint32_t packed[2] = {0u, 0u};
  if (s != 0.0f) {
#pragma unroll
    for (int i = 0; i < 16; ++i) packed[i >> 3] |= f32_to_e2m1(v[i] / s) << (4 * (i & 7));
  }
  *codes = u32x2{packed[0], packed[1]};
  *scale = sc;
}

// ---------------------------------------------------------------- Hadamard rotation

// The indexer's 128-wide Hadamard rotation, H x / sqrt(128) with H the Sylvester matrix:
// the product H x is formed exactly (fast-transform butterflies in fp64: for bf16 rows whose
// nonzero magnitudes span at most 38 binades every sum is exact, so the butterfly order
// does not matter), rounded once to fp32, then multiplied once by fp32(1/sqrt(128)).
constexpr float kHadamardScale = 0x1.6a09e6p-4f;  // fp32(1 / sqrt(128))

// The in-register butterfly stages h = 1 .. N/2 of N consecutive channels.
template <int N, class T>
__device__ __forceinline__ void hadamard_stages(T* y) {
#pragma unroll
  for (int h = 1; h < N; h *= 2)
#pragma unroll
    for (int i = 0; i < N; ++i)
      if ((i & h) == 0) {
        const T a = y[i], b = y[i + h];
        y[i] = a + b;
        y[i + h] = a - b;
      }
}

// One butterfly stage across lanes: the lane holding the upper half of each pair (`upper`)
// takes partner - own, the lower one own + partner; `mask` selects the partner lane.
template <int N>
__device__ __forceinline__ void hadamard_lane_stage(double* y, int mask, bool upper) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const double p = __shfl_xor(y[i], mask);
    y[i] = upper ? p - y[i] : y[i] + p;
  }
}

// An exact H x value, rounded once to fp32 and scaled once (both round to nearest even).
__device__ __forceinline__ float hadamard_round_scale(double v) {
#pragma clang fp contract(off)
  return (float)v * kHadamardScale;
}

// ---------------------------------------------------------------- FP4 block decode

// Eight E2M1 codes (one dword, element 2i in the low nibble of byte i) times the block
// scale s -> eight bf16 values, packed in pairs.  Exact: an E2M1 value times an E4M3
// value has at most 6 significant bits.
__device__ __forceinline__ u32x4 fp4x8_to_bf16(uint32_t codes, float s) {
  f32x2 e0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
  f32x2 e1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
  f32x2 e2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
  f32x2 e3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
  return u32x4{pack_bf16_exact(e0[0] * s, e0[1] * s), pack_bf16_exact(e1[0] * s, e1[1] * s),
               pack_bf16_exact(e2[0] * s, e2[1] * s), pack_bf16_exact(e3[0] * s, e3[1] * s)};
}

// ---------------------------------------------------------------- sequence lengths

// Rows of sequence b: n, or seq_rows[b] clamped to [0, n] when per-sequence lengths
// are given.
__device__ __forceinline__ int64_t seq_len(const int32_t* seq_rows, int b, int64_t n) {
  if (!seq_rows) return n;
  const int64_t r = seq_rows[b];
  return r < 0 ? 0 : (r > n ? n : r);
}

// ---------------------------------------------------------------- order keys

// Monotone map fp32 -> uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- barriers

// Workgroup barrier that orders LDS only: global loads still in flight stay in flight
// (a full __syncthreads() also waits for every outstanding global access).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------- wave scans (DPP)

// Inclusive prefix sum over the 64 lanes of a wave: row shifts within 16-lane rows,
// then row broadcasts across rows (no LDS round trips).
__device__ __forceinline__ uint32_t wave_incl_scan_add(uint32_t x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// One step of a 64-bit min/max scan: combine with the lane CTRL selects (lanes without
// a source keep the identity).
template <int CTRL, int ROWMASK>
__device__ __forceinline__ void minmax_step(uint64_t& mn, uint64_t& mx) {
  const uint32_t a_lo = __builtin_amdgcn_update_dpp(0xFFFFFFFFu, (uint32_t)mn, CTRL, ROWMASK, 0xF, false);
  const uint32_t a_hi = __builtin_amdgcn_update_dpp(0xFFFFFFFFu, (uint32_t)(mn >> 32), CTRL, ROWMASK, 0xF, false);
  const uint32_t b_lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)mx, CTRL, ROWMASK, 0xF, false);
  const uint32_t b_hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(mx >> 32), CTRL, ROWMASK, 0xF, false);
  const uint64_t a = ((uint64_t)a_hi << 32) | a_lo, b = ((uint64_t)b_hi << 32) | b_lo;
  mn = a < mn ? a : mn;
  mx = b > mx ? b : mx;
}

// Wave-wide minimum and maximum of 64-bit values (result uniform across the wave).
__device__ __forceinline__ void wave_minmax_u64(uint64_t& mn, uint64_t& mx) {
  minmax_step<0x111, 0xF>(mn, mx);
  minmax_step<0x112, 0xF>(mn, mx);
  minmax_step<0x114, 0xF>(mn, mx);
  minmax_step<0x118, 0xF>(mn, mx);
  minmax_step<0x142, 0xA>(mn, mx);
  minmax_step<0x143, 0xC>(mn, mx);
  // (readlane returns a signed int: widen through uint32_t, never sign-extend)
  mn = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((uint32_t)(mn >> 32), 63) << 32) |
       (uint32_t)__builtin_amdgcn_readlane((uint32_t)mn, 63);
  mx = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((uint32_t)(mx >> 32), 63) << 32) |
       (uint32_t)__builtin_amdgcn_readlane((uint32_t)mx, 63);
}

// Wave-wide minimum and maximum of 32-bit values (result uniform across the wave).
template <int CTRL, int ROWMASK>
__device__ __forceinline__ void minmax_step32(uint32_t& mn, uint32_t& mx) {
  const uint32_t a = __builtin_amdgcn_update_dpp(0xFFFFFFFFu, mn, CTRL, ROWMASK, 0xF, false);
  const uint32_t b = __builtin_amdgcn_update_dpp(0u, mx, CTRL, ROWMASK, 0xF, false);
  mn = a < mn ? a : mn;
  mx = b > mx ? b : mx;
}
__device__ __forceinline__ void wave_minmax_u32(uint32_t& mn, uint32_t& mx) {
  minmax_step32<0x111, 0xF>(mn, mx);
  minmax_step32<0x112, 0xF>(mn, mx);
  minmax_step32<0x114, 0xF>(mn, mx);
  minmax_step32<0x118, 0xF>(mn, mx);
  minmax_step32<0x142, 0xA>(mn, mx);
  minmax_step32<0x143, 0xC>(mn, mx);
  mn = (uint32_t)__builtin_amdgcn_readlane(mn, 63);
  mx = (uint32_t)__builtin_amdgcn_readlane(mx, 63);
}

// Sum of a value over the four 16-lane rows of a wave, in every lane (lane l gets
// x[l%16] + x[l%16+16] + x[l%16+32] + x[l%16+48]).
__device__ __forceinline__ float wave_sum_rows(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t v = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Maximum of a value over the four 16-lane rows of a wave, in every lane.
__device__ __forceinline__ float wave_max_rows(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t v = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// ---------------------------------------------------------------- MFMA

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16x16x32_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) {
  return __builtin_bit_cast(f16x8, v);
}

// fp32 -> IEEE half bit pattern, round to nearest even.
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

}  // namespace csakv
