// Fused front end: packed QKV -> per-head qk-norm (gains already folded to
// 1 + w) -> partial RoPE -> Q, dense K/V mirrors and the leading head_dim
// columns of the paged K/V pool rows; in decode the same kernel appends the
// new token.
//
// Method: TensorRT-Edge-LLM "Qsa Attention Plugin", fused step 1 (packed-QKV
// split + per-head qk-norm + partial RoPE + paged-KV write + dense K/V
// mirrors; decode's rope-append) and its "KV pool contract (widened rows)":
// a pool row's leading head_size elements hold roped K / raw V, the tail is
// the indexer's and is never written here.
//
// Precision: norm and RoPE in fp64, one rounding to the 16-bit dtype (as the
// indexer's pooling); V is copied bit for bit.
#include <math.h>

#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

constexpr int kFeRows = 4;  // token rows per workgroup (one per wave for the RoPE table)

// One head vector per wave: lane l holds dims E*l .. E*l + E-1 (E = D / 64).
template <int D>
__global__ __launch_bounds__(256) void front_end_kernel(FrontEndArgs a) {
  constexpr int E = D / 64;
  __shared__ double s_cs[kFeRows][64][2];  // cos, sin of the row's angles (i < rot/2)
  const int lane = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long long nrows = (long long)a.B * a.S;
  const long long row0 = (long long)blockIdx.x * kFeRows;
  const int half = a.rot >> 1;
  {
    const long long r = row0 + wv;
    if (r < nrows && lane < half) {
      const int b = (int)(r / a.S), t = (int)(r % a.S);
      const double pos = (double)((a.start ? a.start[b] : 0) + t);
      double sn, cs;
      sincos_angle(pos * a.freq[lane], &sn, &cs);
      s_cs[wv][lane][0] = cs;
      s_cs[wv][lane][1] = sn;
    }
  }
  __syncthreads();
  const int NH = a.Hq + 2 * a.Hkv;
  const int items = kFeRows * NH;
  for (int it = wv; it < items; it += 4) {
    const int rl = it / NH, h = it % NH;
    const long long r = row0 + rl;
    if (r >= nrows) break;  // items run row by row: every later item is past the rows too
    const int b = (int)(r / a.S), t = (int)(r % a.S);
    const int pos = (a.start ? a.start[b] : 0) + t;
    const bool live = pos < a.ctx[b];
    const uint16_t *src = a.qkv + (size_t)r * NH * D + (size_t)h * D + E * lane;
    uint32_t raw = E == 2 ? *reinterpret_cast<const uint32_t *>(src) : (uint32_t)*src;
    // pool row of this token in plane 0 (K) or 1 (V), or -1
    auto pool_off = [&](int plane, int kvh) -> long long {
      if (!a.pool || !live) return -1;
      const int pi = pos >> 7;
      if (pos < 0 || pi >= a.max_pages) return -1;
      const int pg = a.pt[((size_t)b * 2 + plane) * a.max_pages + pi];
      if ((unsigned)pg >= (unsigned)a.num_flat_pages) return -1;
      return (((long long)pg * 128 + (pos & 127)) * a.Hkv + kvh) * a.PHD;
    };
    if (h >= a.Hq + a.Hkv) {  // V: copied unchanged
      const int kvh = h - a.Hq - a.Hkv;
      if (a.v_out) {
        uint16_t *dst = a.v_out + ((size_t)r * a.Hkv + kvh) * D + E * lane;
        if (E == 2) *reinterpret_cast<uint32_t *>(dst) = raw;
        else *dst = (uint16_t)raw;
      }
      const long long o = pool_off(1, kvh);
      if (o >= 0) {
        if (E == 2) *reinterpret_cast<uint32_t *>(a.pool + o + E * lane) = raw;
        else a.pool[o + lane] = (uint16_t)raw;
      }
      continue;
    }
    const bool is_q = h < a.Hq;
    const float *gamma = is_q ? a.q_gamma : a.k_gamma;
    double x[E];
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = (double)bits_to_f32((raw >> (16 * e)) & 0xffffu, a.dt);
    double ss = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e) ss += x[e] * x[e];
    ss = wave_sum_f64(ss);
    const double den = sqrt(ss / (double)D + a.eps);
    double y[E];
#pragma unroll
    for (int e = 0; e < E; ++e) y[e] = x[e] / den * (double)gamma[E * lane + e];
    // RoPE: pair (i, i + half) for i < half; the partner of dim d is held by
    // lane pd / E as element pd % E
    double o[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int d = E * lane + e;
      const int pd = d < a.rot ? (d < half ? d + half : d - half) : d;
      double p0 = __shfl(y[0], pd / E, 64), p1 = E == 2 ? __shfl(y[E - 1], pd / E, 64) : p0;
      const double yp = (pd % E) ? p1 : p0;
      if (d < a.rot) {
        const int i = d < half ? d : d - half;
        const double c = s_cs[rl][i][0], sn = s_cs[rl][i][1];
        o[e] = d < half ? y[e] * c - yp * sn : y[e] * c + yp * sn;
      } else {
        o[e] = y[e];
      }
    }
    uint32_t packed = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) packed |= f64_to_bits(o[e], a.dt) << (16 * e);
    uint16_t *dst;
    long long po = -1;
    if (is_q) {
      dst = a.q_out + ((size_t)r * a.Hq + h) * D + E * lane;
    } else {
      const int kvh = h - a.Hq;
      dst = a.k_out ? a.k_out + ((size_t)r * a.Hkv + kvh) * D + E * lane : nullptr;
      po = pool_off(0, kvh);
    }
    if (dst) {
      if (E == 2) *reinterpret_cast<uint32_t *>(dst) = packed;
      else *dst = (uint16_t)packed;
    }
    if (po >= 0) {
      if (E == 2) *reinterpret_cast<uint32_t *>(a.pool + po + E * lane) = packed;
      else a.pool[po + lane] = (uint16_t)packed;
    }
  }
}

hipError_t launch_front_end(const FrontEndArgs &a_in, int D, hipStream_t s) {
  FrontEndArgs a = a_in;
  for (int i = 0; i < 64; ++i) a.freq[i] = i < (a.rot >> 1) ? pow(a.theta, (-2.0 * (double)i) / (double)a.rot) : 0.0;
  const long long rows = (long long)a.B * a.S;
  const unsigned grid = (unsigned)((rows + kFeRows - 1) / kFeRows);
  if (D == 128) hipLaunchKernelGGL(front_end_kernel<128>, dim3(grid), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(front_end_kernel<64>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace qsa
