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
constexpr int kFeInFlight = 8;  // head vectors whose loads a wave issues together

// One head vector per wave and item: lane l holds dims E*l .. E*l + E-1
// (E = D / 64).  Per row, the RoPE table, and the pool offsets of the row
// in both planes, are set up once in LDS; the gains are loaded once per
// wave; a wave's items then go kFeInFlight at a time, all their loads issued
// before the first is used (the loop is otherwise one load round trip per
// item).
template <int D>
__global__ __launch_bounds__(256) void front_end_kernel(FrontEndArgs a) {
  constexpr int E = D / 64, U = kFeInFlight;
  __shared__ double s_cs[kFeRows][64][2];  // cos, sin of the row's angles (i < rot/2)
  __shared__ long long s_po[kFeRows][2];   // element offset of the row's pool row (KV head 0), plane 0 / 1, or -1
  const int lane = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long long nrows = (long long)a.B * a.S;
  const long long row0 = (long long)blockIdx.x * kFeRows;
  const int half = a.rot >> 1;
  {
    const long long r = row0 + wv;
    if (r < nrows) {
      const int b = (int)(r / a.S), t = (int)(r % a.S);
      const int pos = (a.start ? a.start[b] : 0) + t;
      if (lane < half) {
        double sn, cs;
        sincos_angle((double)pos * a.freq[lane], &sn, &cs);
        s_cs[wv][lane][0] = cs;
        s_cs[wv][lane][1] = sn;
      }
      if (lane < 2) {
        // rows at or past the total length, and rows whose page-table entry
        // is out of range, are not written to the pool
        long long o = -1;
        if (a.pool && pos < a.ctx[b] && pos >= 0 && (pos >> 7) < a.max_pages) {
          const int pg = a.pt[((size_t)b * 2 + lane) * a.max_pages + (pos >> 7)];
          if ((unsigned)pg < (unsigned)a.num_flat_pages) o = ((long long)pg * 128 + (pos & 127)) * a.Hkv * a.PHD;
        }
        s_po[wv][lane] = o;
      }
    }
  }
  float gq[E], gk[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    gq[e] = a.q_gamma[E * lane + e];
    gk[e] = a.k_gamma[E * lane + e];
  }
  // this lane's dims d = E lane + e: RoPE partner lane and element, angle
  // index, whether d is rotated and whether its sine term is subtracted
  int pdl[E], pde[E], ci[E];
  bool in_rot[E], neg[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int d = E * lane + e;
    const int pd = d < a.rot ? (d < half ? d + half : d - half) : d;
    pdl[e] = pd / E;
    pde[e] = pd % E;
    in_rot[e] = d < a.rot;
    neg[e] = d < half;
    ci[e] = d < a.rot ? (d < half ? d : d - half) : 0;
  }
  __syncthreads();
  const int NH = a.Hq + 2 * a.Hkv;
  const int items = (int)min((long long)kFeRows, nrows - row0) * NH;  // row by row
  auto process = [&](int it, uint32_t raw) {
    const int rl = it / NH, h = it % NH;
    const long long r = row0 + rl;
    if (h >= a.Hq + a.Hkv) {  // V: copied unchanged
      const int kvh = h - a.Hq - a.Hkv;
      if (a.v_out) {
        uint16_t *dst = a.v_out + ((size_t)r * a.Hkv + kvh) * D + E * lane;
        if (E == 2) *reinterpret_cast<uint32_t *>(dst) = raw;
        else *dst = (uint16_t)raw;
      }
      const long long o = s_po[rl][1];
      if (o >= 0) {
        uint16_t *dst = a.pool + o + (long long)kvh * a.PHD + E * lane;
        if (E == 2) *reinterpret_cast<uint32_t *>(dst) = raw;
        else *dst = (uint16_t)raw;
      }
      return;
    }
    const bool is_q = h < a.Hq;
    double x[E];
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = (double)bits_to_f32((raw >> (16 * e)) & 0xffffu, a.dt);
    double ss = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e) ss += x[e] * x[e];
    ss = wave_sum_f64(ss);
    // one inverse square root per lane (the same for every lane) instead of
    // a division per element: x * (1 / den) and x / den differ by about an
    // fp64 ulp, far below the 16-bit rounding that follows
    const double inv = inv_sqrt_f64(ss / (double)D + a.eps);
    double y[E];
#pragma unroll
    for (int e = 0; e < E; ++e) y[e] = x[e] * inv * (double)(is_q ? gq[e] : gk[e]);
    // RoPE: pair (i, i + half) for i < half: o_i = y_i c - y_{i+half} s,
    // o_{i+half} = y_{i+half} c + y_i s.  The partner of dim d is held by lane
    // pd / E as element pd % E, which is element e itself when half is a
    // multiple of E (two shuffles instead of four).
    double yp[E];
    if (half % E == 0) {
#pragma unroll
      for (int e = 0; e < E; ++e) yp[e] = __shfl(y[e], pdl[e], 64);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const double p0 = __shfl(y[0], pdl[e], 64), p1 = E == 2 ? __shfl(y[E - 1], pdl[e], 64) : p0;
        yp[e] = pde[e] ? p1 : p0;
      }
    }
    double o[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const double c = s_cs[rl][ci[e]][0], sn = s_cs[rl][ci[e]][1];
      o[e] = in_rot[e] ? y[e] * c + yp[e] * (neg[e] ? -sn : sn) : y[e];
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
      po = s_po[rl][0] >= 0 ? s_po[rl][0] + (long long)kvh * a.PHD : -1;
    }
    if (dst) {
      if (E == 2) *reinterpret_cast<uint32_t *>(dst) = packed;
      else *dst = (uint16_t)packed;
    }
    if (po >= 0) {
      if (E == 2) *reinterpret_cast<uint32_t *>(a.pool + po + E * lane) = packed;
      else a.pool[po + lane] = (uint16_t)packed;
    }
  };
  for (int it0 = wv; it0 < items; it0 += 4 * U) {
    // every load unconditional (a clamped item), issued before any is used
    uint32_t raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int it = min(it0 + 4 * u, items - 1);
      const int rl = it / NH, h = it % NH;
      const uint16_t *src = a.qkv + (size_t)(row0 + rl) * NH * D + (size_t)h * D + E * lane;
      raw[u] = E == 2 ? *reinterpret_cast<const uint32_t *>(src) : (uint32_t)*src;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (it0 + 4 * u < items) process(it0 + 4 * u, raw[u]);
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
