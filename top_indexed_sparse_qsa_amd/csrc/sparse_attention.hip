// Sparse GQA attention over index lists: prefill (dense BSND K/V) and
// single-token split-K decode (paged pool).
//
// Contract: TensorRT-Edge-LLM "Cute Dsl Qsa Sparse Runner", structs
// QsaSparsePrefillParams and QsaSparseDecodeParams -- lists of distinct ids,
// -1 padded on the right, no positional mask, zero rows past the live
// length, only pool columns [0, headDim) read, V page ids pre-offset.
//
// Work split: one wave per (query row, KV head) in prefill and per (sequence,
// KV head, split) in decode.  The GQA head group of one KV head (up to 16
// query heads) is the 16-wide MFMA tile.  Per chunk of 32 list slots a wave
//   * gathers the 32 K rows straight into MFMA A-fragments (each lane reads
//     16 contiguous bytes of one row; four lanes cover 64 bytes of a row),
//   * gathers the 32 V rows with each 16-lane group reading whole rows
//     (fully coalesced 256-byte rows for D = 128),
//   * computes S^T = K Q^T (two 16-key tiles), so every lane ends up owning
//     the scores of one query head m = lane % 16 for eight keys,
//   * runs the fp32 online softmax in the exp2 domain,
//   * feeds those eight probabilities, unchanged in place, as the B operand
//     of O^T += V^T P^T; the V^T A-operand is an in-register 8x8 transpose of
//     16-bit values (v_perm) because a lane already holds eight keys x eight
//     dims of V.  Output dim d = 8*row + e, so lane (q, m) accumulates the 32
//     contiguous dims [32q, 32q+32) of head m.
// No LDS is needed on the prefill path; decode stages its page-table row in
// LDS.  The next chunk's gathers are in flight while the current one
// computes, and ids run two chunks ahead.
#include <math.h>

#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

template <int D>
struct Frag {
  static constexpr int NKS = D / 32;
  u32x4 kf[2][NKS];  // K, A-operand layout, tiles of keys 0..15 and 16..31
  u32x4 vf[8];       // V rows of the lane's eight key slots, dims 8c..8c+7
  uint32_t valid;    // bit i: key slot i of this lane is usable
};

// Key slot i of lane group q: keys 4q+i (i < 4) and 16+4q+(i-4) (i >= 4).
__device__ __forceinline__ int slot_of(int q4, int i) { return i < 4 ? 4 * q4 + i : 12 + 4 * q4 + i; }

struct DenseKV {
  const uint16_t *k, *v;  // row 0 of this sequence, this KV head
  size_t row_stride;      // elements between consecutive tokens
  int limit;              // ids in [0, limit) are usable
  __device__ const uint16_t *krow(int id) const { return k + (size_t)id * row_stride; }
  __device__ const uint16_t *vrow(int id) const { return v + (size_t)id * row_stride; }
};

struct PagedKV {
  const uint16_t *pool;   // pool + kvh * PHD
  const int32_t *pk, *pv; // LDS copies of the sequence's page-table rows
  size_t row_stride;      // Hkv * PHD
  int num_flat_pages;
  int limit;
  __device__ const uint16_t *row(const int32_t *pt, int id) const {
    int pg = pt[id >> 7];
    if ((unsigned)pg >= (unsigned)num_flat_pages) pg = 0;
    return pool + ((size_t)pg * 128 + (id & 127)) * row_stride;
  }
  __device__ const uint16_t *krow(int id) const { return row(pk, id); }
  __device__ const uint16_t *vrow(int id) const { return row(pv, id); }
};

template <int D, int DT, class KV>
__device__ __forceinline__ void issue_chunk(Frag<D> &f, int idv, const KV &kv, int q4, int r16) {
  int kid0 = shfl_i(idv, r16), kid1 = shfl_i(idv, 16 + r16);
  kid0 = ((unsigned)kid0 < (unsigned)kv.limit) ? kid0 : 0;
  kid1 = ((unsigned)kid1 < (unsigned)kv.limit) ? kid1 : 0;
  const uint16_t *k0 = kv.krow(kid0) + 8 * q4;
  const uint16_t *k1 = kv.krow(kid1) + 8 * q4;
#pragma unroll
  for (int ks = 0; ks < Frag<D>::NKS; ++ks) {
    f.kf[0][ks] = ld16(k0 + 32 * ks);
    f.kf[1][ks] = ld16(k1 + 32 * ks);
  }
  uint32_t valid = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int id = shfl_i(idv, slot_of(q4, i));
    bool ok = (unsigned)id < (unsigned)kv.limit;
    valid |= (uint32_t)ok << i;
    if (D == 128 || r16 < D / 8) f.vf[i] = ld16(kv.vrow(ok ? id : 0) + 8 * r16);
    else f.vf[i] = u32x4{0u, 0u, 0u, 0u};
  }
  f.valid = valid;
}

template <int D, int DT>
__device__ __forceinline__ void consume_chunk(const Frag<D> &f, const u32x4 (&qf)[D / 32], float sl2,
                                              float &m_run, float &l_run, f32x4 (&acc)[8]) {
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < Frag<D>::NKS; ++ks) {
    s0 = mfma16x16x32<DT>(f.kf[0][ks], qf[ks], s0);
    s1 = mfma16x16x32<DT>(f.kf[1][ks], qf[ks], s1);
  }
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = ((f.valid >> i) & 1u) ? s0[i] * sl2 : -INFINITY;
    x[4 + i] = ((f.valid >> (4 + i)) & 1u) ? s1[i] * sl2 : -INFINITY;
  }
  float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
  mx = fmaxf(mx, shfl_xor_f(mx, 16));
  mx = fmaxf(mx, shfl_xor_f(mx, 32));
  const float m_new = fmaxf(m_run, mx);
  const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
  const float alpha = exp2f(m_run - m_use);
  uint32_t pb[4];
  float psum = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t h0 = f32_to_bits<DT>(exp2f(x[2 * w] - m_use));
    uint32_t h1 = f32_to_bits<DT>(exp2f(x[2 * w + 1] - m_use));
    psum += bits_to_f32_t<DT>(h0) + bits_to_f32_t<DT>(h1);  // normalise by the rounded weights
    pb[w] = h0 | (h1 << 16);
  }
  l_run = l_run * alpha + psum;
  m_run = m_new;
  const u32x4 bop = {pb[0], pb[1], pb[2], pb[3]};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    acc[e] *= alpha;
    u32x4 a;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t lo = u4_at(f.vf[2 * w], e >> 1), hi = u4_at(f.vf[2 * w + 1], e >> 1);
      a[w] = (e & 1) ? pack_hi_hi(lo, hi) : pack_lo_lo(lo, hi);
    }
    acc[e] = mfma16x16x32<DT>(a, bop, acc[e]);
  }
}

// Runs the online softmax over list slots [0, n_slots).  Processing stops at
// the first 32-slot chunk that holds no usable id.
template <int D, int DT, class KV>
__device__ void run_list(const int32_t *__restrict__ list, int n_slots, const KV &kv,
                         const u32x4 (&qf)[D / 32], float sl2, float &m_run, float &l_run,
                         f32x4 (&acc)[8]) {
  const int lane = lane_id(), q4 = lane >> 4, r16 = lane & 15;
  const int nchunks = (n_slots + 31) >> 5;
  auto load_id = [&](int c) -> int {
    int s = (c << 5) + (lane & 31);
    return (c < nchunks && s < n_slots) ? list[s] : -1;
  };
  auto usable = [&](int idv) { return wave_any((unsigned)idv < (unsigned)kv.limit); };

  Frag<D> fa, fb;
  int id_a = load_id(0);
  int id_b = load_id(1);
  if (!usable(id_a)) return;
  issue_chunk<D, DT>(fa, id_a, kv, q4, r16);
  int id_c = load_id(2);
  for (int c = 0;; c += 2) {
    // fa holds chunk c; id_b / id_c are the ids of chunks c+1 / c+2.
    const bool b_ok = usable(id_b);
    int id_d = -1;
    if (b_ok) {
      issue_chunk<D, DT>(fb, id_b, kv, q4, r16);
      id_d = load_id(c + 3);
    }
    consume_chunk<D, DT>(fa, qf, sl2, m_run, l_run, acc);
    if (!b_ok) break;
    const bool c_ok = usable(id_c);
    int id_e = -1;
    if (c_ok) {
      issue_chunk<D, DT>(fa, id_c, kv, q4, r16);
      id_e = load_id(c + 4);
    }
    consume_chunk<D, DT>(fb, qf, sl2, m_run, l_run, acc);
    if (!c_ok) break;
    id_b = id_d;
    id_c = id_e;
  }
}

template <int D>
__device__ __forceinline__ void load_q(u32x4 (&qf)[D / 32], const uint16_t *qhead0, int G, int q4, int r16) {
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
    qf[ks] = (r16 < G) ? ld16(qhead0 + (size_t)r16 * D + 32 * ks + 8 * q4) : u32x4{0u, 0u, 0u, 0u};
}

// Row t of every sequence before row t-1: long lists are dispatched first.
template <int D, int DT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void sparse_prefill_kernel(PrefillAttnArgs a) {
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= a.B * a.S * a.Hkv) return;
  const int kvh = item % a.Hkv;
  const int rest = item / a.Hkv;
  const int b = rest % a.B;
  const int t = a.S - 1 - rest / a.B;
  const int lane = lane_id(), q4 = lane >> 4, r16 = lane & 15;
  const int live = min(a.ctx[b], a.S);
  const size_t qo_off = (((size_t)b * a.S + t) * a.Hq + (size_t)kvh * a.G) * D;

  f32x4 acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  if (t < live) {
    u32x4 qf[D / 32];
    load_q<D>(qf, a.q + qo_off, a.G, q4, r16);
    DenseKV kv;
    kv.k = a.k + ((size_t)b * a.S * a.Hkv + kvh) * D;
    kv.v = a.v + ((size_t)b * a.S * a.Hkv + kvh) * D;
    kv.row_stride = (size_t)a.Hkv * D;
    kv.limit = live;
    run_list<D, DT>(a.indices + ((size_t)b * a.S + t) * a.top_k, a.top_k, kv, qf, a.sl2, m_run, l_run, acc);
  }
  float l = l_run + shfl_xor_f(l_run, 16);
  l += shfl_xor_f(l, 32);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (r16 < a.G && 32 * q4 < D) {
    uint16_t *dst = a.o + qo_off + (size_t)r16 * D + 32 * q4;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      u32x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = f32_to_bits<DT>(acc[2 * j][rr] * inv) | (f32_to_bits<DT>(acc[2 * j + 1][rr] * inv) << 16);
      st16(dst + 8 * rr, w);
    }
  }
}

// One wave per (sequence, KV head, split).  Each split stores its unnormalised
// accumulator and (max, sum) per head row; the last split to arrive (counter
// after a release fence) merges all splits in split order, so the result does
// not depend on arrival order, then resets the counter to zero.
template <int D, int DT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2))) void sparse_decode_kernel(DecodeAttnArgs a) {
  extern __shared__ int32_t s_pt[];  // [2][max_pages]
  const int item = blockIdx.x;
  const int split = item % a.nsplits;
  const int rest = item / a.nsplits;
  const int kvh = rest % a.Hkv;
  const int b = rest / a.Hkv;
  const int lane = lane_id(), q4 = lane >> 4, r16 = lane & 15;
  const int ctx = min(max(a.ctx[b], 0), a.max_pages * 128);
  const int npages = (ctx + 127) >> 7;
  const int32_t *ptb = a.pt + (size_t)b * 2 * a.max_pages;
  for (int i = lane; i < npages; i += 64) {
    s_pt[i] = ptb[i];
    s_pt[a.max_pages + i] = ptb[a.max_pages + i];
  }
  __syncthreads();

  f32x4 acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const int s0 = split * a.split_slots;
  const int n_slots = min(a.top_k - s0, a.split_slots);
  if (ctx > 0 && n_slots > 0) {
    u32x4 qf[D / 32];
    load_q<D>(qf, a.q + ((size_t)b * a.Hq + (size_t)kvh * a.G) * D, a.G, q4, r16);
    PagedKV kv;
    kv.pool = a.pool + (size_t)kvh * a.PHD;
    kv.pk = s_pt;
    kv.pv = s_pt + a.max_pages;
    kv.row_stride = (size_t)a.Hkv * a.PHD;
    kv.num_flat_pages = a.num_flat_pages;
    kv.limit = ctx;
    run_list<D, DT>(a.indices + (size_t)b * a.top_k + s0, n_slots, kv, qf, a.sl2, m_run, l_run, acc);
  }
  float l = l_run + shfl_xor_f(l_run, 16);
  l += shfl_xor_f(l, 32);

  const int pair = b * a.Hkv + kvh;
  const size_t slot0 = (size_t)pair * 16;  // QSA_MAX_SPLITS slots per pair
  float *po = a.part_o + (slot0 + split) * 16 * D;
  float *ps = a.part_stats + (slot0 + split) * 32;
  if (32 * q4 < D) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      float *dst = po + (size_t)r16 * D + 32 * q4 + 8 * rr;
      *reinterpret_cast<f32x4 *>(dst) = f32x4{acc[0][rr], acc[1][rr], acc[2][rr], acc[3][rr]};
      *reinterpret_cast<f32x4 *>(dst + 4) = f32x4{acc[4][rr], acc[5][rr], acc[6][rr], acc[7][rr]};
    }
  }
  if (q4 == 0) {
    ps[r16] = m_run;
    ps[16 + r16] = l;
  }
  __threadfence();
  int last = 0;
  if (lane == 0) last = (atomicAdd(&a.counters[pair], 1) == a.nsplits - 1);
  last = __shfl(last, 0, 64);
  if (!last) return;
  __threadfence();

  if (r16 < a.G && 32 * q4 < D) {
    const float *pso = a.part_stats + slot0 * 32;
    float M = -INFINITY;
    for (int s = 0; s < a.nsplits; ++s) M = fmaxf(M, pso[s * 32 + r16]);
    float L = 0.f;
    float o[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) o[j] = 0.f;
    for (int s = 0; s < a.nsplits; ++s) {
      const float ms = pso[s * 32 + r16];
      const float w = (ms == -INFINITY) ? 0.f : exp2f(ms - M);
      L += pso[s * 32 + 16 + r16] * w;
      const float *src = a.part_o + ((slot0 + s) * 16 + r16) * D + 32 * q4;
#pragma unroll
      for (int j = 0; j < 32; j += 4) {
        f32x4 v = *reinterpret_cast<const f32x4 *>(src + j);
        o[j] += v[0] * w;
        o[j + 1] += v[1] * w;
        o[j + 2] += v[2] * w;
        o[j + 3] += v[3] * w;
      }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    uint16_t *dst = a.o + ((size_t)b * a.Hq + (size_t)kvh * a.G + r16) * D + 32 * q4;
#pragma unroll
    for (int j = 0; j < 32; j += 8) {
      u32x4 w;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        w[k] = f32_to_bits<DT>(o[j + 2 * k] * inv) | (f32_to_bits<DT>(o[j + 2 * k + 1] * inv) << 16);
      st16(dst + j, w);
    }
  }
  if (lane == 0) __hip_atomic_store(&a.counters[pair], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, int DT>
static hipError_t launch_prefill_t(const PrefillAttnArgs &a, hipStream_t s) {
  const long long items = (long long)a.B * a.S * a.Hkv;
  const unsigned grid = (unsigned)((items + 3) / 4);
  hipLaunchKernelGGL((sparse_prefill_kernel<D, DT>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sparse_prefill(const PrefillAttnArgs &a, int D, int dt, hipStream_t s) {
  if (D == 128) return dt == DT_F16 ? launch_prefill_t<128, DT_F16>(a, s) : launch_prefill_t<128, DT_BF16>(a, s);
  return dt == DT_F16 ? launch_prefill_t<64, DT_F16>(a, s) : launch_prefill_t<64, DT_BF16>(a, s);
}

template <int D, int DT>
static hipError_t launch_decode_t(const DecodeAttnArgs &a, hipStream_t s) {
  const unsigned grid = (unsigned)(a.B * a.Hkv * a.nsplits);
  const size_t lds = (size_t)2 * a.max_pages * sizeof(int32_t);
  hipLaunchKernelGGL((sparse_decode_kernel<D, DT>), dim3(grid), dim3(64), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_sparse_decode(const DecodeAttnArgs &a, int D, int dt, hipStream_t s) {
  if (D == 128) return dt == DT_F16 ? launch_decode_t<128, DT_F16>(a, s) : launch_decode_t<128, DT_BF16>(a, s);
  return dt == DT_F16 ? launch_decode_t<64, DT_F16>(a, s) : launch_decode_t<64, DT_BF16>(a, s);
}

}  // namespace qsa
