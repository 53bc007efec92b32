// Device helpers shared by the libqsa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

enum { DT_F16 = 0, DT_BF16 = 1 };

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// ---------------------------------------------------------------------------
// 16x16x32 MFMA, fp32 accumulate.  A is 16 (M) x 32 (K): lane l holds row
// l%16, K slots 8*(l/16)..+7.  B is 32 (K) x 16 (N): lane l holds column
// l%16, the same K slots.  D is 16 x 16: lane l holds rows 4*(l/16)+r
// (r = 0..3) of column l%16.
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (DT == DT_F16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// Number formats.  16-bit values travel as raw bits.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bits_to_f32(uint32_t h, int dt) {
  if (dt == DT_F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
  return __uint_as_float(h << 16);
}

template <int DT>
__device__ __forceinline__ float bits_to_f32_t(uint32_t h) {
  if constexpr (DT == DT_F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
  else return __uint_as_float(h << 16);
}

// float -> 16-bit, round to nearest even (gfx950 converts in one
// instruction, two values at a time with pack2).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int DT>
__device__ __forceinline__ uint32_t f32_to_bits(float x) {
  if constexpr (DT == DT_F16) return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
  else return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
}

// Two floats -> two 16-bit values packed low | high << 16.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  if constexpr (DT == DT_F16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
  else return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint32_t f32_to_bits_rt(float x, int dt) {
  return dt == DT_F16 ? f32_to_bits<DT_F16>(x) : f32_to_bits<DT_BF16>(x);
}

// double -> float rounded to odd: truncate, then force the last bit on when
// the value was inexact.  Rounding that result to nearest-even in any format
// with at least two fewer significant bits equals one direct rounding of the
// double.
__device__ __forceinline__ float f64_to_f32_odd(double x) {
  float f = __double2float_rz(x);
  if ((double)f != x) f = __uint_as_float(__float_as_uint(f) | 1u);
  return f;
}

// double -> 16-bit with a single round-to-nearest-even.
__device__ __forceinline__ uint32_t f64_to_bits(double x, int dt) {
  return f32_to_bits_rt(f64_to_f32_odd(x), dt);
}

// ---------------------------------------------------------------------------
// Wave utilities.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ int shfl_i(int v, int src) { return __shfl(v, src, 64); }

__device__ __forceinline__ bool wave_any(bool p) { return __ballot(p) != 0ull; }

__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void st16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }

// Pack two 16-bit halves: low from a, high from b (selected by hi flags).
__device__ __forceinline__ uint32_t pack_lo_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ uint32_t u4_at(const u32x4 &v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

}  // namespace qsa
