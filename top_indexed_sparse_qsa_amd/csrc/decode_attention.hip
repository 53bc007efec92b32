// Sparse GQA attention over index lists, single-token split-K decode over the
// paged pool (also the rows of a prefill chunk), and the decode step's
// select + attention kernel.  The per-chunk machinery shared with prefill is
// in attention_core.h; the workgroup select in select_core.h.
#include <math.h>

#include <algorithm>

#include "attention_core.h"
#include "qsa_device.h"
#include "qsa_launch.h"
#include "select_core.h"

namespace qsa {

// Decode: one wave per (sequence, KV head, split); the waves of a workgroup
// (up to kDecWaves = 8) take consecutive splits of the same (sequence, KV head),
// share its page-table row in LDS, and merge their partial softmax states in
// LDS in split order.  When a (sequence, KV head) needs more splits than one
// workgroup holds, each workgroup stores its merged partial (unnormalised O,
// running max, running sum) and a second small kernel merges the workgroup
// partials, again in a fixed order.  The order never depends on timing, so
// results are deterministic.  No cross-workgroup flags are used: on this
// part each XCD has its own L2, and a kernel boundary is the cheap place to
// make one workgroup's stores visible to another.

// LDS of a decode workgroup of nw waves, sized to nw: per wave a K tile
// (32 rows of 256 B) during the walk; once every wave has finished its list
// (a workgroup barrier separates the two uses) the merge scratch -- per wave
// 16 rows of D + 4 floats of O, then the running max and sum of each row --
// overlays the K tiles.  The page-table rows follow.
template <int D>
struct DecLds {
  static constexpr int RS = D + 4;  // padded row stride (floats)
  static constexpr size_t kTile = 32 * 16 * sizeof(u32x4);
  static constexpr size_t kMerge = (16 * RS + 2 * 16) * sizeof(float);
  static constexpr size_t per_wave = kTile > kMerge ? kTile : kMerge;
  static __host__ __device__ size_t bytes(int nw) { return per_wave * nw; }
  unsigned char *base;
  int nw;
  __device__ u32x4 *ktile(int w) const { return reinterpret_cast<u32x4 *>(base + kTile * w); }
  __device__ float *acc(int w) const { return reinterpret_cast<float *>(base) + (size_t)16 * RS * w; }
  __device__ float *m(int w) const { return reinterpret_cast<float *>(base) + (size_t)16 * RS * nw + 16 * w; }
  __device__ float *l(int w) const { return m(nw) + 16 * w; }
};

template <int D, int DT>
__device__ __forceinline__ void decode_merge_store(const DecodeAttnArgs &a, const DecLds<D> &mg, int pair, int group,
                                                   int br, int kvh, float m_run, float l_run, const f32x4 (&acc)[8]);

// Lane (q, r) of wave w merges row r, dims [d0, d0 + D/16).
template <int D, int DT>
__global__ __launch_bounds__(64 * kDecWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void sparse_decode_kernel(DecodeAttnArgs a) {
  extern __shared__ __align__(16) unsigned char s_raw[];
  const int wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const DecLds<D> mg{s_raw, nw};
  uint64_t *s_pb = reinterpret_cast<uint64_t *>(s_raw + DecLds<D>::bytes(nw));  // [2][max_pages] page byte offsets
  const int group = blockIdx.x % a.ngroups;
  const int pair = blockIdx.x / a.ngroups;  // (query row, KV head)
  const int br = pair / a.Hkv, kvh = pair % a.Hkv;
  const int b = br / a.C, row = br % a.C;
  const int split = group * a.wpg + wv;
  const int lane = lane_id(), q4 = lane >> 4, r16 = lane & 15;
  // Everything the walk needs first is issued at once -- the first two
  // chunks' ids, Q, the context length and both page-table rows (whole
  // rows, so that the copy does not wait for the context length) -- so that
  // one round trip precedes the first gathers.
  const int s0 = split * a.split_slots;
  const int n_slots = split < a.nsplits ? min(a.top_k - s0, a.split_slots) : 0;
  const int32_t *row_ids = a.indices + (size_t)br * a.top_k;
  const int32_t *list = row_ids + s0;
  const int sl = lane & 31;
  // unconditional loads of the first two chunks' ids (clamped to the row)
  const int raw_a = row_ids[min(s0 + sl, a.top_k - 1)];
  const int raw_b = row_ids[min(s0 + sl + 32, a.top_k - 1)];
  const int id_a = sl < n_slots ? raw_a : -1;
  const int id_b = sl + 32 < n_slots ? raw_b : -1;
  u32x4 qf[D / 32];
  load_q<D>(qf, a.q + ((size_t)br * a.Hq + (size_t)kvh * a.G) * D, a.G, q4, r16);
  const int ctx_in = a.ctx[b];
  const int pos = a.start ? a.start[b] + row : ctx_in - 1;  // the row's position
  {
    const int32_t *ptb = a.pt + (size_t)b * 2 * a.max_pages;  // rows 0 and 1 are contiguous
    const int npt = 2 * a.max_pages;
    const uint64_t row_bytes = (uint64_t)a.Hkv * a.PHD * sizeof(uint16_t);
    constexpr int U = 4;
    for (int i0 = threadIdx.x; i0 < npt; i0 += U * (int)blockDim.x) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = ptb[min(i0 + u * (int)blockDim.x, npt - 1)];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u * (int)blockDim.x;
        if (i < npt) s_pb[i] = page_bytes_of(v[u], a.num_flat_pages, row_bytes);
      }
    }
  }
  __syncthreads();
  const int ctx = min(max(ctx_in, 0), a.max_pages * 128);

  f32x4 acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  if (ctx > 0 && n_slots > 0 && pos >= 0 && pos < ctx_in) {
    PagedKV kv;
    kv.pool = reinterpret_cast<const char *>(a.pool + (size_t)kvh * a.PHD);
    kv.pk = s_pb;
    kv.pv = s_pb + a.max_pages;
    kv.row_bytes = (uint64_t)a.Hkv * a.PHD * sizeof(uint16_t);
    kv.limit = ctx;
    run_list_ids<D, DT>(list, n_slots, kv, qf, a.sl2, m_run, l_run, acc, mg.ktile(wv), id_a, id_b);
  }
  decode_merge_store<D, DT>(a, mg, pair, group, br, kvh, m_run, l_run, acc);
}

// The workgroup's splits (one per wave: m_run, l_run, acc) merged in split
// order, then stored as output rows (one workgroup per pair) or as the
// workgroup's partial.
template <int D, int DT>
__device__ __forceinline__ void decode_merge_store(const DecodeAttnArgs &a, const DecLds<D> &mg, int pair, int group,
                                                   int br, int kvh, float m_run, float l_run, const f32x4 (&acc)[8]) {
  const int wv = threadIdx.x >> 6, nw = mg.nw;
  const int lane = lane_id(), q4 = lane >> 4, r16 = lane & 15;
  __syncthreads();  // every K tile is dead before the merge scratch is written
  float l = l_run + shfl_xor_f(l_run, 16);
  l += shfl_xor_f(l, 32);
  if (32 * q4 < D) {
    float *dst = mg.acc(wv) + r16 * DecLds<D>::RS + 32 * q4;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      *reinterpret_cast<f32x4 *>(dst + 8 * rr) = f32x4{acc[0][rr], acc[1][rr], acc[2][rr], acc[3][rr]};
      *reinterpret_cast<f32x4 *>(dst + 8 * rr + 4) = f32x4{acc[4][rr], acc[5][rr], acc[6][rr], acc[7][rr]};
    }
  }
  if (q4 == 0) {
    mg.m(wv)[r16] = m_run;
    mg.l(wv)[r16] = l;
  }
  __syncthreads();

  // Merge the workgroup's splits in split order.  The head dims form 16
  // slices of D/16; lane (q, r) of wave w takes row r and slices w*4+q,
  // w*4+q + 4*nw, ...  The sums are explicit fmas, so that every kernel
  // that inlines this merge (whatever it knows of nw) rounds them alike.
  constexpr int ND = D / 16;
  float M = -INFINITY;
  for (int w = 0; w < nw; ++w) M = fmaxf(M, mg.m(w)[r16]);
  float L = 0.f, sc[kDecWaves];
#pragma unroll
  for (int w = 0; w < kDecWaves; ++w) {
    const float mw = w < nw ? mg.m(w)[r16] : -INFINITY;
    sc[w] = mw == -INFINITY ? 0.f : exp2f(mw - M);
    L = __builtin_fmaf(w < nw ? mg.l(w)[r16] : 0.f, sc[w], L);
  }
  if (r16 >= a.G) return;
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const size_t slot = (size_t)pair * kDecMaxGroups + group;
  for (int sl = wv * 4 + q4; sl < 16; sl += 4 * nw) {
    const int d0 = sl * ND;
    float o[ND];
#pragma unroll
    for (int j = 0; j < ND; ++j) o[j] = 0.f;
    for (int w = 0; w < nw; ++w) {
      const float *src = mg.acc(w) + r16 * DecLds<D>::RS + d0;
#pragma unroll
      for (int j = 0; j < ND; ++j) o[j] = __builtin_fmaf(src[j], sc[w], o[j]);
    }
    if (a.ngroups == 1) {
      uint16_t *out = a.o + ((size_t)br * a.Hq + (size_t)kvh * a.G + r16) * D + d0;
#pragma unroll
      for (int j = 0; j < ND; j += 2)
        *reinterpret_cast<uint32_t *>(out + j) =
            pack2<DT>(o[j] * inv, o[j + 1] * inv);
    } else {
      float *po = a.part_o + (slot * 16 + r16) * D + d0;
#pragma unroll
      for (int j = 0; j < ND; j += 4) *reinterpret_cast<f32x4 *>(po + j) = f32x4{o[j], o[j + 1], o[j + 2], o[j + 3]};
    }
  }
  if (a.ngroups > 1 && wv == 0 && q4 == 0) {
    a.part_stats[slot * 32 + r16] = M;
    a.part_stats[slot * 32 + 16 + r16] = L;
  }
}

// Merges the workgroup partials of one (sequence, KV head) in group order.
template <int D, int DT>
__global__ __launch_bounds__(64) void sparse_decode_merge_kernel(DecodeAttnArgs a) {
  const int pair = blockIdx.x;  // (query row, KV head)
  const int br = pair / a.Hkv, kvh = pair % a.Hkv;
  const int lane = lane_id(), q4 = lane >> 4, r16 = lane & 15;
  if (r16 >= a.G) return;
  constexpr int NDL = D / 4;  // dims per lane
  const int d0 = q4 * NDL;
  const size_t slot0 = (size_t)pair * kDecMaxGroups;
  float M = -INFINITY;
  for (int g = 0; g < a.ngroups; ++g) M = fmaxf(M, a.part_stats[(slot0 + g) * 32 + r16]);
  float L = 0.f, o[NDL];
#pragma unroll
  for (int j = 0; j < NDL; ++j) o[j] = 0.f;
  for (int g = 0; g < a.ngroups; ++g) {
    const float mg = a.part_stats[(slot0 + g) * 32 + r16];
    const float sc = mg == -INFINITY ? 0.f : exp2f(mg - M);
    L += a.part_stats[(slot0 + g) * 32 + 16 + r16] * sc;
    const float *src = a.part_o + ((slot0 + g) * 16 + r16) * D + d0;
#pragma unroll
    for (int j = 0; j < NDL; j += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(src + j);
      o[j] += v[0] * sc;
      o[j + 1] += v[1] * sc;
      o[j + 2] += v[2] * sc;
      o[j + 3] += v[3] * sc;
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t *out = a.o + ((size_t)br * a.Hq + (size_t)kvh * a.G + r16) * D + d0;
#pragma unroll
  for (int j = 0; j < NDL; j += 8) {
    u32x4 w;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = pack2<DT>(o[j + 2 * k] * inv, o[j + 2 * k + 1] * inv);
    st16(out + j, w);
  }
}

// ---------------------------------------------------------------------------
// Decode step: the indexer's select (decode B3) and the sparse decode in one
// kernel.  One workgroup of kDecWaves waves per (sequence, KV head) reads
// the sequence's block scores, runs the workgroup select (select_core.h) --
// the workgroups of all KV heads of a sequence run the same select, so the
// list never has to reach memory before the walk -- and walks that list
// straight from LDS.  The workgroup of KV head 0 also stores the list, as
// the indexer would.  The scores of the whole row width go out with the
// context length, Q and the page-table rows (masked once the length is
// known), so one round trip precedes the select and one more the first
// gathers.  Splits, walk and merge are those of sparse_decode_kernel with
// one workgroup per pair, so the output is the same bit for bit.
// ---------------------------------------------------------------------------

// The list of one decode row, made from its kept blocks lb (ascending):
// slot i < head is token r*lb[i/r] + i%r, then the causal tail i + tail0
// below len, then -1; s0 offsets the slots (a split's first slot).  With
// head = 0 the list is 0..len-1.
struct KeptList {
  const uint16_t *lb;
  int s0, r, head, len, tail0;
  __device__ int operator[](int slot) const {
    const int i = s0 + slot;
    if (i < head) {
      const int j = r == 4 ? i >> 2 : i / r;
      return r * (int)lb[j] + (i - r * j);
    }
    return i < len ? i + tail0 : -1;
  }
};

// LDS of the decode step: the select's histograms share the front with the
// walk's tiles and merge scratch (the select ends before the walk starts),
// then both page-table rows, then the kept blocks.
template <int D>
__host__ __device__ constexpr size_t step_front_bytes() {
  return DecLds<D>::bytes(kDecWaves) > sizeof(WgSelLds<64 * kDecWaves>) ? DecLds<D>::bytes(kDecWaves)
                                                                         : sizeof(WgSelLds<64 * kDecWaves>);
}

template <int D, int DT, int KPT>
__global__ __launch_bounds__(64 * kDecWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_select_attend_kernel(
    DecodeAttnArgs a) {
  constexpr int NT = 64 * kDecWaves;
  extern __shared__ __align__(16) unsigned char s_raw[];
  const int tid = threadIdx.x, wv = tid >> 6;
  const DecLds<D> mg{s_raw, kDecWaves};
  WgSelLds<NT> &sel = *reinterpret_cast<WgSelLds<NT> *>(s_raw);
  uint64_t *s_pb = reinterpret_cast<uint64_t *>(s_raw + step_front_bytes<D>());  // [2][max_pages] page byte offsets
  uint16_t *s_lb = reinterpret_cast<uint16_t *>(s_pb + 2 * a.max_pages);
  const int pair = blockIdx.x;  // (sequence, KV head)
  const int b = pair / a.Hkv, kvh = pair % a.Hkv;
  const int lane = lane_id(), q4 = lane >> 4, r16 = lane & 15;

  const int ctx_in = a.ctx[b];
  const float *srow = a.scores + (size_t)b * a.score_stride;
  // Every load is unconditional (a load on one branch only makes the
  // compiler wait for it where the branches join, one load at a time):
  // slots past the row width read the row's last four scores and are
  // masked once the context length is known.
  // Thread j's keys of round r are blocks 4*NT*r + 4j + c (select_core.h).
  float sv[KPT];
#pragma unroll
  for (int r = 0; r < KPT / 4; ++r) {
    const f32x4 v = *reinterpret_cast<const f32x4 *>(srow + min(4 * NT * r + 4 * tid, a.score_stride - 4));
#pragma unroll
    for (int c = 0; c < 4; ++c) sv[4 * r + c] = v[c];
  }
  u32x4 qf[D / 32];
  load_q<D>(qf, a.q + ((size_t)b * a.Hq + (size_t)kvh * a.G) * D, a.G, q4, r16);
  wg_select_clear<NT>(sel);
  {
    const int32_t *ptb = a.pt + (size_t)b * 2 * a.max_pages;  // rows 0 and 1 are contiguous
    const int npt = 2 * a.max_pages;
    const uint64_t row_bytes = (uint64_t)a.Hkv * a.PHD * sizeof(uint16_t);
    constexpr int U = 4;
    for (int k0 = tid; k0 < npt; k0 += U * NT) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = ptb[min(k0 + u * NT, npt - 1)];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = k0 + u * NT;
        if (k < npt) s_pb[k] = page_bytes_of(v[u], a.num_flat_pages, row_bytes);
      }
    }
  }
  __syncthreads();

  // the row's list, as the indexer's decode select makes it
  const int c = min(ctx_in, a.max_pages * 128);
  const int r = a.ratio;
  const int nc = c > 0 ? c / r : 0;
  KeptList list{s_lb, 0, r, 0, c > 0 ? c : 0, 0};
  if (nc > a.budget) {  // uniform over the workgroup
    uint32_t key[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) key[j] = 4 * NT * (j >> 2) + 4 * tid + (j & 3) < nc ? score_key(sv[j]) : 0xffffffffu;
    wg_select_blocks<NT, KPT>(key, nc, a.budget, sel, s_lb);
    list.head = r * a.budget;
    list.len = list.head + c - r * nc;
    list.tail0 = r * nc - list.head;
  }
  if (kvh == 0) {
    int32_t *out = a.lists_out + (size_t)b * a.top_k;
    for (int i = tid; i < a.top_k; i += NT) out[i] = list[i];
  }

  const int s0 = wv * a.split_slots;
  const int n_slots = wv < a.nsplits ? min(a.top_k - s0, a.split_slots) : 0;
  KeptList mine = list;
  mine.s0 = s0;
  const int sl = lane & 31;
  const int raw_a = mine[sl], raw_b = mine[sl + 32];  // LDS reads, any slot
  const int id_a = sl < n_slots ? raw_a : -1;
  const int id_b = sl + 32 < n_slots ? raw_b : -1;
  const int ctx = min(max(ctx_in, 0), a.max_pages * 128);
  f32x4 acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  if (ctx > 0 && n_slots > 0) {
    PagedKV kv;
    kv.pool = reinterpret_cast<const char *>(a.pool + (size_t)kvh * a.PHD);
    kv.pk = s_pb;
    kv.pv = s_pb + a.max_pages;
    kv.row_bytes = (uint64_t)a.Hkv * a.PHD * sizeof(uint16_t);
    kv.limit = ctx;
    run_list_ids<D, DT>(mine, n_slots, kv, qf, a.sl2, m_run, l_run, acc, mg.ktile(wv), id_a, id_b);
  }
  decode_merge_store<D, DT>(a, mg, pair, 0, b, kvh, m_run, l_run, acc);
}

template <int D, int DT>
static hipError_t launch_decode_t(const DecodeAttnArgs &a, hipStream_t s) {
  const unsigned pairs = (unsigned)((long long)a.B * a.C * a.Hkv);
  const size_t lds = DecLds<D>::bytes(a.wpg) + (size_t)2 * a.max_pages * sizeof(uint64_t);
  if (lds > 65536)
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&sparse_decode_kernel<D, DT>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL((sparse_decode_kernel<D, DT>), dim3(pairs * a.ngroups), dim3(64 * a.wpg), lds, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.ngroups == 1) return e;
  hipLaunchKernelGGL((sparse_decode_merge_kernel<D, DT>), dim3(pairs), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sparse_decode(const DecodeAttnArgs &a, int D, int dt, hipStream_t s) {
  if (D == 128) return dt == DT_F16 ? launch_decode_t<128, DT_F16>(a, s) : launch_decode_t<128, DT_BF16>(a, s);
  return dt == DT_F16 ? launch_decode_t<64, DT_F16>(a, s) : launch_decode_t<64, DT_BF16>(a, s);
}

template <int D, int DT, int KPT>
static hipError_t launch_step_t(const DecodeAttnArgs &a, hipStream_t s) {
  // the kept-block list: the select runs only when budget < nc <= gmax
  const size_t lb_bytes = ((size_t)std::min(a.budget, a.gmax) * sizeof(uint16_t) + 15) & ~(size_t)15;
  const size_t lds = step_front_bytes<D>() + (size_t)2 * a.max_pages * sizeof(uint64_t) + lb_bytes;
  const void *fn = reinterpret_cast<const void *>(&decode_select_attend_kernel<D, DT, KPT>);
  if (lds > 65536) (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL((decode_select_attend_kernel<D, DT, KPT>), dim3((unsigned)((long long)a.B * a.Hkv)),
                     dim3(64 * kDecWaves), lds, s, a);
  return hipGetLastError();
}

template <int D, int DT>
static hipError_t launch_step_d(const DecodeAttnArgs &a, hipStream_t s) {
  // thread j holds the scores of blocks [j*KPT, (j+1)*KPT)
  if (a.gmax <= 64 * kDecWaves * 16) return launch_step_t<D, DT, 16>(a, s);
  return launch_step_t<D, DT, 32>(a, s);
}

hipError_t launch_decode_select_attend(const DecodeAttnArgs &a, int D, int dt, hipStream_t s) {
  if (a.gmax > kStepMaxBlocks || a.ngroups != 1 || a.wpg > kDecWaves) return hipErrorInvalidValue;
  if (D == 128) return dt == DT_F16 ? launch_step_d<128, DT_F16>(a, s) : launch_step_d<128, DT_BF16>(a, s);
  return dt == DT_F16 ? launch_step_d<64, DT_F16>(a, s) : launch_step_d<64, DT_BF16>(a, s);
}

}  // namespace qsa
