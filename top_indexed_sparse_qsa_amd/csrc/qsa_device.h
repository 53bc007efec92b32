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

// An fp32 query value as the 16-bit pieces the block scoring multiplies
// (fp16 MFMA operands, for either activation dtype): piece 0 is x rounded to
// fp16, piece 1 the rounded remainder (11 + 11 significant bits).  Stored
// 128 elements apart.
constexpr int kQPieces = 2;

__device__ __forceinline__ void store_q_pieces(uint16_t *dst, float x) {
  float r = x;
#pragma unroll
  for (int p = 0; p < kQPieces; ++p) {
    const uint32_t h = f32_to_bits<DT_F16>(r);
    r -= bits_to_f32_t<DT_F16>(h);
    dst[128 * p] = (uint16_t)h;
  }
}

// Two bf16 values (low, high halves) as two fp16 values: exact for
// magnitudes in fp16's normal range [2^-14, 65504]; smaller ones round to
// fp16's subnormal steps of 2^-24.  Block scoring takes bf16 kbar this way,
// so that both dtypes score with the same fp16 MFMA and two query pieces.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t v) {
  return pack2<DT_F16>(__uint_as_float(v << 16), __uint_as_float(v & 0xffff0000u));
}
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 v) {
  return u32x4{bf16x2_to_f16x2(v[0]), bf16x2_to_f16x2(v[1]), bf16x2_to_f16x2(v[2]), bf16x2_to_f16x2(v[3])};
}

// double -> float rounded to odd: x itself when exact, else whichever of its
// two float neighbours has its last bit set.  Rounding that result to
// nearest-even in any format with at least two fewer significant bits equals
// one direct rounding of the double.  From the nearest float f: f is that
// neighbour when it is exact or odd; an even, inexact f is replaced by its
// odd neighbour on x's side (one step away from or towards zero).
__device__ __forceinline__ float f64_to_f32_odd(double x) {
  const float f = (float)x;
  const double fd = (double)f;
  const uint32_t b = __float_as_uint(f);
  if (fd == x || (b & 1u)) return f;
  return __uint_as_float(fabs(x) > fabs(fd) ? b + 1u : b - 1u);
}

// 1 / sqrt(v) for a normal v > 0: the hardware estimate (about 23 correct
// bits) refined by two Newton steps r += r (1 - v r^2) / 2, within about an
// fp64 ulp of the correctly rounded value (a correctly rounded sqrt and
// divide take ~26 instructions; this takes 9).  Every use rounds the
// normalised value once more, to fp32 or 16 bits, where an fp64 ulp decides
// the rounding only for values within ~2^-29 (fp32) of a tie.
__device__ __forceinline__ double inv_sqrt_f64(double v) {
  double r = __builtin_amdgcn_rsq(v);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const double e = fma(-(v * r), r, 1.0);
    r = fma(0.5 * r, e, r);
  }
  return r;
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

// ---------------------------------------------------------------------------
// fp64 helpers of the query / key preparation (RMSNorm and RoPE in fp64).
// ---------------------------------------------------------------------------
// sin and cos of an angle |x| < 2^24 (positions below 2^24 times
// frequencies <= 1): x - k*pi/2 with pi/2 split into parts of 29, 25 and 53
// significant bits (so k*P1 and k*P2 are exact for |k| < 2^24; the reduced
// argument is within ~1e-16 of the exact one), then the library sincos on
// |r| <= pi/4 and the quadrant k mod 4.  This keeps the library's reduction
// of large arguments (a table walk) off the query prep's critical path.
__device__ __forceinline__ void sincos_angle(double x, double *s, double *c) {
  constexpr double kTwoOverPi = 0.6366197723675814;
  const double P1 = 0x1.921fb54p+0, P2 = 0x1.10b461p-30, P3 = 0x1.a62633145c06ep-58;
  const double k = rint(x * kTwoOverPi);
  const double r = ((x - k * P1) - k * P2) - k * P3;
  double sr, cr;
  sincos(r, &sr, &cr);
  const int q = (int)k & 3;
  *s = q == 0 ? sr : q == 1 ? cr : q == 2 ? -sr : -cr;
  *c = q == 0 ? cr : q == 1 ? -sr : q == 2 ? -cr : sr;
}

// One in-row DPP shift of a double (both 32-bit halves move); a source lane
// outside the row reads 0 (bound_ctrl), so no zero fill precedes the moves.
template <int CTRL>
__device__ __forceinline__ double dpp_row_shr_f64(double v) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)b, CTRL, 0xf, 0xf, true);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), CTRL, 0xf, 0xf, true);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// v + v[lane ^ 16] (X16) or v + v[lane ^ 32]: the gfx950 lane swap hands
// every lane its own value and its partner's, one in each output, so their
// sum is the pair's sum whichever output holds which.
template <bool X16>
__device__ __forceinline__ double add_swapped_f64(double v) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)b, hi = (uint32_t)(b >> 32);
  const auto l = X16 ? __builtin_amdgcn_permlane16_swap(lo, lo, false, false)
                     : __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  const auto h = X16 ? __builtin_amdgcn_permlane16_swap(hi, hi, false, false)
                     : __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  const double d0 = __longlong_as_double((long long)(((unsigned long long)h[0] << 32) | l[0]));
  const double d1 = __longlong_as_double((long long)(((unsigned long long)h[1] << 32) | l[1]));
  return d0 + d1;
}

// Sum of v over the wave, in every lane: an inclusive scan within each row
// of 16 lanes (lane 16r + 15 ends with row r's sum), the rows' sums added
// across lanes l ^ 32 and then l ^ 16, and lane 15's total read back.
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_row_shr_f64<0x111>(v);  // row_shr:1
  v += dpp_row_shr_f64<0x112>(v);  // row_shr:2
  v += dpp_row_shr_f64<0x114>(v);  // row_shr:4
  v += dpp_row_shr_f64<0x118>(v);  // row_shr:8
  v = add_swapped_f64<false>(v);   // rows 0 + 2, 1 + 3
  v = add_swapped_f64<true>(v);    // all four
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, 15);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 15);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

}  // namespace qsa
