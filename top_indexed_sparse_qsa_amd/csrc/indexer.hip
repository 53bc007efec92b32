// QSA indexer kernels: query prep, block-key pooling, weight-free block
// scoring, per-row top-budget block select + expansion into token lists, and
// the decode step that keeps the indexer state in the KV-pool tails.
//
// Method: TensorRT-Edge-LLM "Qsa Attention Plugin" (class description: the
// indexer steps, decode B1/B2/B3; "KV pool contract (widened rows)"), and
// atlasinference "spark_model/layers/ops/qsa.rs" (doc comments of
// qsa_block_pool, qsa_qprep, qsa_score, qsa_score_rows).
//
// Precision: pooling, RMSNorm and RoPE run in fp64 and round once (kbar to
// the activation dtype, queries to fp32).  Scoring is an MFMA contraction of
// the fp32 queries, split exactly into two fp16 or three bf16 pieces, against
// the 16-bit kbar, accumulated in fp32.  Scores are kept unscaled by
// 1/sqrt(hd): a positive factor does not change which blocks win.
#include <math.h>

#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

__device__ __forceinline__ double bits_to_f64(uint32_t h, int dt) { return (double)bits_to_f32(h, dt); }

// Sum over the block (blockDim.x = 128 = two waves).
__device__ __forceinline__ double block_sum128(double v, double *red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  __syncthreads();
  if (lane_id() == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return red[0] + red[1];
}

// y = RoPE_pos(x / sqrt(mean(x^2) + eps) * (1 + w)) for one 128-vector held one
// element per thread.  Pairs (i, i + rot/2), angle pos * theta^(-2i/rot).
__device__ double norm_rope(double x, double w, double pos, int rot, double theta, double eps,
                            double *sx, double *red) {
  const int d = threadIdx.x;
  const double ms = block_sum128(x * x, red) / 128.0;
  const double y = x / sqrt(ms + eps) * (1.0 + w);
  sx[d] = y;
  __syncthreads();
  const int half = rot >> 1;
  double out = y;
  if (d < rot) {
    const int i = d < half ? d : d - half;
    const double ang = pos * pow(theta, (-2.0 * (double)i) / (double)rot);
    double sn, cs;
    sincos(ang, &sn, &cs);
    out = d < half ? y * cs - sx[d + half] * sn : y * cs + sx[d - half] * sn;
  }
  __syncthreads();
  return out;
}

// grid: B*S query rows, then B*Gmax blocks; block: 128 threads (hd = 128).
__global__ __launch_bounds__(128) void idx_prep_kernel(IdxPrepArgs a) {
  __shared__ double sx[128];
  __shared__ double red[2];
  const int d = threadIdx.x;
  const long long nrows = (long long)a.B * a.S;
  const long long bid = blockIdx.x;
  if (bid < nrows) {
    const int b = (int)(bid / a.S), t = (int)(bid % a.S);
    if (t >= min(a.ctx[b], a.S)) return;
    const double w = (double)a.wq[d];
    for (int h = 0; h < a.Hi; ++h) {
      const size_t off = ((size_t)bid * a.Hi + h) * 128 + d;
      const double x = bits_to_f64(a.idx_q[off], a.dt);
      a.qhat[off] = (float)norm_rope(x, w, (double)t, a.rot, a.theta, a.eps, sx, red);
    }
  } else {
    const long long k = bid - nrows;
    const int b = (int)(k / a.Gmax), g = (int)(k % a.Gmax);
    if (g >= min(a.ctx[b], a.S) / a.ratio) return;
    double m = 0.0;
    for (int j = 0; j < a.ratio; ++j)
      m += bits_to_f64(a.idx_k[((size_t)b * a.S + (size_t)a.ratio * g + j) * 128 + d], a.dt);
    m /= (double)a.ratio;
    const double y = norm_rope(m, (double)a.wk[d], (double)a.ratio * g, a.rot, a.theta, a.eps, sx, red);
    a.kbar[((size_t)b * a.Gmax + g) * 128 + d] = (uint16_t)f64_to_bits(y, a.dt);
  }
}

// fp32 -> exact sum of NP 16-bit pieces (two fp16 or three bf16).
template <int DT>
struct QSplit {
  static constexpr int NP = DT == DT_F16 ? 2 : 3;
};

template <int DT>
__device__ __forceinline__ void split8(const float (&x)[8], u32x4 (&out)[QSplit<DT>::NP]) {
  float r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = x[i];
#pragma unroll
  for (int p = 0; p < QSplit<DT>::NP; ++p) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t h0 = f32_to_bits<DT>(r[2 * w]), h1 = f32_to_bits<DT>(r[2 * w + 1]);
      r[2 * w] -= bits_to_f32_t<DT>(h0);
      r[2 * w + 1] -= bits_to_f32_t<DT>(h1);
      out[p][w] = h0 | (h1 << 16);
    }
  }
}

__device__ __forceinline__ void load8f(float (&x)[8], const float *p) {
  f32x4 a = *reinterpret_cast<const f32x4 *>(p), b = *reinterpret_cast<const f32x4 *>(p + 4);
  x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
  x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
}

// Prefill scoring.  One wave per 4 consecutive rows: the MFMA M tile is
// (row, head) with the head fastest, so each lane group ends with the four
// head dots of one row and one block and sums their relus without any
// cross-lane step.  Tiles of 16 blocks run up to the last row's complete
// count; the kbar tile of the next step is fetched while this one computes.
template <int DT>
__global__ __launch_bounds__(256) void idx_score_kernel(IdxScoreArgs a) {
  constexpr int NP = QSplit<DT>::NP;
  const int lane = lane_id(), q4 = lane >> 4, r16 = lane & 15;
  const int T4 = (a.S + 3) >> 2;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= a.B * T4) return;
  const int b = item % a.B;
  const int t0 = 4 * (T4 - 1 - item / a.B);
  const int live = min(a.ctx[b], a.S);
  if (t0 >= live) return;

  u32x4 qa[NP][4];
  {
    const int t = t0 + (r16 >> 2), h = r16 & 3;
    const bool ok = t < live && h < a.Hi;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float x[8];
      if (ok) load8f(x, a.qhat + (((size_t)b * a.S + t) * a.Hi + h) * 128 + 32 * ks + 8 * q4);
      else
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = 0.f;
      u32x4 pieces[NP];
      split8<DT>(x, pieces);
#pragma unroll
      for (int p = 0; p < NP; ++p) qa[p][ks] = pieces[p];
    }
  }
  const int t_out = t0 + q4;
  const int nc_out = t_out < live ? (t_out + 1) / a.ratio : 0;
  const int nc_hi = (min(t0 + 3, live - 1) + 1) / a.ratio;
  const uint16_t *kb0 = a.kbar + (size_t)b * a.Gmax * 128 + 8 * q4;
  float *srow = a.scores + ((size_t)b * a.S + t_out) * a.stride;

  auto load_tile = [&](int g0, u32x4 (&kb)[4]) {
    const int g = min(g0 + r16, max(a.Gmax - 1, 0));
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kb[ks] = ld16(kb0 + (size_t)g * 128 + 32 * ks);
  };
  u32x4 cur[4], nxt[4];
  if (nc_hi > 0) load_tile(0, cur);
  for (int g0 = 0; g0 < nc_hi; g0 += 16) {
    if (g0 + 16 < nc_hi) load_tile(g0 + 16, nxt);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int p = 0; p < NP; ++p) acc = mfma16x16x32<DT>(qa[p][ks], cur[ks], acc);
    const float s = fmaxf(acc[0], 0.f) + fmaxf(acc[1], 0.f) + fmaxf(acc[2], 0.f) + fmaxf(acc[3], 0.f);
    if (g0 + r16 < nc_out) srow[g0 + r16] = s;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) cur[ks] = nxt[ks];
  }
}

// ---------------------------------------------------------------------------
// Select + expand.  One workgroup (256 threads) per row.  Scores are
// non-negative, so their fp32 bit patterns (sign cleared) order like the
// values.  An MSB-first radix select (four 8-bit digits, LDS histograms with
// wave-aggregated increments) finds the budget-th largest key T; the kept
// set is every key > T plus the lowest-index keys == T until the budget is
// met.  An ordered ballot scan then writes the kept blocks in ascending
// order, each as ratio consecutive token ids, followed by the causal tail
// and -1 padding.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t score_key(float s) { return __float_as_uint(s) & 0x7fffffffu; }

// Exclusive prefix count of `flag` over the NT threads in thread order;
// returns this thread's prefix and sets *total.
template <int NT>
__device__ __forceinline__ int block_scan_flag(bool flag, int *s_wave, int *total) {
  constexpr int NW = NT / 64;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const unsigned long long m = __ballot(flag);
  const int in_wave = __popcll(m & ((1ull << lane) - 1ull));
  __syncthreads();
  if (lane == 0) s_wave[wv] = __popcll(m);
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int c = s_wave[w];
    before += w < wv ? c : 0;
    tot += c;
  }
  *total = tot;
  return before + in_wave;
}

template <int NT>
__global__ __launch_bounds__(NT) void idx_select_kernel(IdxSelectArgs a) {
  constexpr int NW = NT / 64;
  extern __shared__ uint32_t s_key[];
  __shared__ uint32_t hist[256];
  __shared__ int s_wave[NW > 4 ? NW : 4];
  __shared__ uint32_t s_digit, s_above;
  const int tid = threadIdx.x, lane = lane_id();

  int b, t, live;
  int32_t *out;
  const float *srow;
  if (a.decode) {
    b = blockIdx.x;
    const int c = min(a.ctx[b], a.max_ctx);
    t = c - 1;
    live = c > 0;
    out = a.out + (size_t)b * a.top_k;
    srow = a.scores + (size_t)b * a.row_stride;
  } else {
    // longest rows first
    const int r = blockIdx.x;
    b = r % a.B;
    t = a.S - 1 - r / a.B;
    live = t < min(a.ctx[b], a.S);
    out = a.out + ((size_t)b * a.S + t) * a.top_k;
    srow = a.scores + ((size_t)b * a.S + t) * a.row_stride;
  }
  if (!live) {
    for (int i = tid; i < a.top_k; i += NT) out[i] = -1;
    return;
  }
  const int r = a.ratio;
  const int nc = (t + 1) / r;
  if (nc <= a.budget) {  // every complete block is kept: the list is 0..t
    for (int i = tid; i < a.top_k; i += NT) out[i] = i <= t ? i : -1;
    return;
  }

  // Stage the row's keys in LDS.  Rows start 64-byte aligned; four float4
  // loads per thread are in flight before the first LDS store.
  {
    const int n4 = nc >> 2;
    const f32x4 *src4 = reinterpret_cast<const f32x4 *>(srow);
    for (int base = 0; base < n4; base += 4 * NT) {
      f32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i4 = base + u * NT + tid;
        if (i4 < n4) v[u] = src4[i4];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i4 = base + u * NT + tid;
        if (i4 < n4) {
          s_key[4 * i4] = score_key(v[u][0]);
          s_key[4 * i4 + 1] = score_key(v[u][1]);
          s_key[4 * i4 + 2] = score_key(v[u][2]);
          s_key[4 * i4 + 3] = score_key(v[u][3]);
        }
      }
    }
    for (int i = 4 * n4 + tid; i < nc; i += NT) s_key[i] = score_key(srow[i]);
  }
  uint32_t prefix = 0, pmask = 0;
  uint32_t remaining = (uint32_t)a.budget;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    const int iters = (nc + NT - 1) / NT;
    for (int it = 0; it < iters; ++it) {
      const int i = it * NT + tid;
      bool act = false;
      uint32_t dig = 0;
      if (i < nc) {
        const uint32_t k = s_key[i];
        act = (k & pmask) == prefix;
        dig = (k >> shift) & 255u;
      }
      // Peel off the most common digit of the wave with one increment.
      unsigned long long pend = __ballot(act);
      for (int rep = 0; rep < 4 && pend; ++rep) {
        const int leader = __ffsll((long long)pend) - 1;
        const uint32_t ld = (uint32_t)__shfl((int)dig, leader, 64);
        const unsigned long long same = __ballot(act && dig == ld);
        if (lane == leader) atomicAdd(&hist[ld], (uint32_t)__popcll(same));
        if (act && dig == ld) act = false;
        pend &= ~same;
      }
      if (act) atomicAdd(&hist[dig], 1u);
    }
    __syncthreads();
    // Suffix counts over digits 255..0: thread j < 256 holds digit 255 - j.
    const uint32_t c = tid < 256 ? hist[255 - tid] : 0u;
    uint32_t incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t v = (uint32_t)__shfl_up((int)incl, o, 64);
      if (lane >= o) incl += v;
    }
    if (tid < 256 && lane == 63) s_wave[tid >> 6] = (int)incl;
    __syncthreads();
    if (tid < 256) {
      uint32_t before = 0;
      for (int w = 0; w < (tid >> 6); ++w) before += (uint32_t)s_wave[w];
      incl += before;
      const uint32_t excl = incl - c;
      if (excl < remaining && incl >= remaining) {  // exactly one thread
        s_digit = 255u - (uint32_t)tid;
        s_above = excl;
      }
    }
    __syncthreads();
    prefix |= s_digit << shift;
    pmask |= 255u << shift;
    remaining -= s_above;
    __syncthreads();
  }
  const uint32_t T = prefix;
  const int need_eq = (int)remaining;          // keys equal to T still to take
  int eq_base = 0, sel_base = 0;
  for (int base = 0; base < nc; base += NT) {
    const int g = base + tid;
    const uint32_t k = g < nc ? s_key[g] : 0u;
    const bool gt = g < nc && k > T;
    const bool eq = g < nc && k == T;
    int eq_tot;
    const int eq_rank = eq_base + block_scan_flag<NT>(eq, s_wave, &eq_tot);
    const bool sel = gt || (eq && eq_rank < need_eq);
    int sel_tot;
    const int pos = sel_base + block_scan_flag<NT>(sel, s_wave, &sel_tot);
    if (sel)
      for (int j = 0; j < r; ++j) out[(size_t)r * pos + j] = r * g + j;
    eq_base += eq_tot;
    sel_base += sel_tot;
  }
  const int head = r * a.budget;
  const int len = head + (t + 1) - r * nc;
  for (int i = head + tid; i < a.top_k; i += NT) out[i] = i < len ? r * nc + (i - head) : -1;
}

// ---------------------------------------------------------------------------
// Decode B1: queries at p = ctx-1 and the tail update.  grid B, block 128.
// ---------------------------------------------------------------------------
__device__ __forceinline__ long long pool_row_off(const int32_t *ptrow, int token, int max_pages,
                                                  int num_flat_pages, int Hkv, int PHD) {
  const int pi = token >> 7;
  if (token < 0 || pi >= max_pages) return -1;
  const int pg = ptrow[pi];
  if ((unsigned)pg >= (unsigned)num_flat_pages) return -1;
  return (((long long)pg * 128 + (token & 127)) * Hkv) * PHD;
}

__global__ __launch_bounds__(128) void idx_dec_prep_kernel(IdxDecPrepArgs a) {
  __shared__ double sx[128];
  __shared__ double red[2];
  const int b = blockIdx.x, d = threadIdx.x;
  const int ctx = min(a.ctx[b], a.max_pages * 128);
  if (ctx <= 0) return;
  const int p = ctx - 1;
  const double wq = (double)a.wq[d];
  for (int h = 0; h < a.Hi; ++h) {
    const size_t off = ((size_t)b * a.Hi + h) * 128 + d;
    a.qhat[off] = (float)norm_rope(bits_to_f64(a.idx_q[off], a.dt), wq, (double)p, a.rot, a.theta, a.eps, sx, red);
  }
  const int32_t *ptk = a.pt + (size_t)b * 2 * a.max_pages;
  const int32_t *ptv = ptk + a.max_pages;
  const uint16_t knew = a.idx_k[(size_t)b * 128 + d];
  if (ctx % a.ratio != 0) {
    const long long o = pool_row_off(ptk, p, a.max_pages, a.num_flat_pages, a.Hkv, a.PHD);
    if (o >= 0) a.pool[o + a.D + d] = knew;
    return;
  }
  const int g = ctx / a.ratio - 1;
  const int base = a.ratio * g;
  double m = 0.0;
  bool ok = true;
  for (int j = 0; j < a.ratio - 1; ++j) {
    const long long o = pool_row_off(ptk, base + j, a.max_pages, a.num_flat_pages, a.Hkv, a.PHD);
    ok = ok && o >= 0;
    if (o >= 0) m += bits_to_f64(a.pool[o + a.D + d], a.dt);
  }
  m += bits_to_f64(knew, a.dt);
  m /= (double)a.ratio;
  const double y = norm_rope(m, (double)a.wk[d], (double)base, a.rot, a.theta, a.eps, sx, red);
  const long long ov = pool_row_off(ptv, base, a.max_pages, a.num_flat_pages, a.Hkv, a.PHD);
  if (ok && ov >= 0) a.pool[ov + a.D + d] = (uint16_t)f64_to_bits(y, a.dt);
}

// ---------------------------------------------------------------------------
// Decode B2: scores of blocks g < ctx/ratio from the V-row tails.  Each wave
// takes kScoreTilesPerWave tiles of 16 blocks and issues all their tail
// loads before the first MFMA.  A = kbar (rows = blocks), B = query pieces
// (columns = heads); the relus of the heads are summed across lanes.
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(256) void idx_dec_score_kernel(IdxDecScoreArgs a) {
  constexpr int NP = QSplit<DT>::NP;
  constexpr int TPW = kScoreTilesPerWave;
  const int lane = lane_id(), q4 = lane >> 4, r16 = lane & 15;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= a.B * a.waves_per_seq) return;
  const int b = item / a.waves_per_seq, chunk = item % a.waves_per_seq;
  const int ctx = min(a.ctx[b], a.max_pages * 128);
  const int nc = ctx > 0 ? ctx / a.ratio : 0;
  const int g_begin = chunk * TPW * 16;
  if (g_begin >= nc) return;

  u32x4 qb[NP][4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    float x[8];
    if (r16 < a.Hi) load8f(x, a.qhat + ((size_t)b * a.Hi + r16) * 128 + 32 * ks + 8 * q4);
    else
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = 0.f;
    u32x4 pieces[NP];
    split8<DT>(x, pieces);
#pragma unroll
    for (int p = 0; p < NP; ++p) qb[p][ks] = pieces[p];
  }
  const int32_t *ptv = a.pt + (size_t)b * 2 * a.max_pages + a.max_pages;
  u32x4 kb[TPW][4];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int g = g_begin + tt * 16 + r16;
    long long o = g < nc ? pool_row_off(ptv, a.ratio * g, a.max_pages, a.num_flat_pages, a.Hkv, a.PHD) : -1;
    if (o < 0) o = 0;
    const uint16_t *src = a.pool + o + a.D + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kb[tt][ks] = ld16(src + 32 * ks);
  }
  float *srow = a.scores + (size_t)b * a.stride;
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int p = 0; p < NP; ++p) acc = mfma16x16x32<DT>(kb[tt][ks], qb[p][ks], acc);
    float v[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      float s = fmaxf(acc[rr], 0.f);
      s += shfl_xor_f(s, 1);
      s += shfl_xor_f(s, 2);
      v[rr] = s;
    }
    const int g4 = g_begin + tt * 16 + 4 * q4;
    if (r16 == 0 && g4 < nc) {
      if (g4 + 3 < nc) *reinterpret_cast<f32x4 *>(srow + g4) = f32x4{v[0], v[1], v[2], v[3]};
      else
        for (int rr = 0; rr < 4 && g4 + rr < nc; ++rr) srow[g4 + rr] = v[rr];
    }
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_idx_prep(const IdxPrepArgs &a, hipStream_t s) {
  const long long nblk = (long long)a.B * a.S + (long long)a.B * a.Gmax;
  hipLaunchKernelGGL(idx_prep_kernel, dim3((unsigned)nblk), dim3(128), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_idx_score(const IdxScoreArgs &a, int dt, hipStream_t s) {
  const long long waves = (long long)a.B * ((a.S + 3) / 4);
  const unsigned grid = (unsigned)((waves + 3) / 4);
  if (dt == DT_F16) hipLaunchKernelGGL(idx_score_kernel<DT_F16>, dim3(grid), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(idx_score_kernel<DT_BF16>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_idx_select(const IdxSelectArgs &a, int nc_max, hipStream_t s) {
  const unsigned rows = (unsigned)(a.decode ? a.B : (long long)a.B * a.S);
  const size_t lds = (size_t)(nc_max > 0 ? nc_max : 1) * sizeof(uint32_t);
  // Decode has one long row per sequence: a wide workgroup per row.
  if (a.decode) hipLaunchKernelGGL(idx_select_kernel<1024>, dim3(rows), dim3(1024), lds, s, a);
  else hipLaunchKernelGGL(idx_select_kernel<256>, dim3(rows), dim3(256), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_idx_dec_prep(const IdxDecPrepArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(idx_dec_prep_kernel, dim3((unsigned)a.B), dim3(128), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_idx_dec_score(const IdxDecScoreArgs &a, int dt, hipStream_t s) {
  const long long waves = (long long)a.B * a.waves_per_seq;
  const unsigned grid = (unsigned)((waves + 3) / 4);
  if (dt == DT_F16) hipLaunchKernelGGL(idx_dec_score_kernel<DT_F16>, dim3(grid), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(idx_dec_score_kernel<DT_BF16>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace qsa
