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
// the fp32 queries, split into two fp16 pieces (hi + lo: about 22 of their
// 24 significant bits), against the kbar taken as fp16 (bf16 kbar
// converted), accumulated in fp32.  Scores are kept unscaled by 1/sqrt(hd):
// a positive factor does not change which blocks win.
#include <math.h>

#include <algorithm>

#include "qsa_device.h"
#include "qsa_launch.h"
#include "select_core.h"

namespace qsa {

__device__ __forceinline__ double bits_to_f64(uint32_t h, int dt) { return (double)bits_to_f32(h, dt); }

// One 128-vector per wave: lane l holds dims l and l + 64.  RoPE pairs dims
// (i, i + rot/2) and turns them by pos * theta^(-2i/rot); dims >= rot pass
// through.  The frequencies are computed once on the host (fp64 pow) and
// passed with the kernel arguments, and the cos/sin of one position serve
// every head at that position.
struct Rope2 {
  double c0, s0, c1, s1;  // rotation of dims lane and lane + 64
};

static void fill_freq(double *freq, int rot, double theta) {
  for (int i = 0; i < 64; ++i) freq[i] = i < (rot >> 1) ? pow(theta, (-2.0 * (double)i) / (double)rot) : 0.0;
}

// The lane's two frequencies, read once per kernel before any other load:
// the table sits in the kernel arguments but is indexed per lane, so it is
// a vector load, and one issued after a batch of loads waits for all of
// them.
struct RopeLane {
  double f0, f1;
  bool same;  // dims lane and lane + 64 share a frequency (rot = 128)
};

__device__ __forceinline__ RopeLane rope_lane(const double *freq, int rot) {
  const int lane = lane_id(), half = rot >> 1;
  const int d0 = lane, d1 = lane + 64;
  const int i0 = d0 < half ? d0 : d0 - half, i1 = d1 < half ? d1 : d1 - half;
  // indexes past the table (dims >= rot, which do not rotate) are clamped
  return RopeLane{freq[min(max(i0, 0), 63)], freq[min(max(i1, 0), 63)], i1 == i0};
}

__device__ __forceinline__ Rope2 rope_at(double pos, const RopeLane &f, int rot) {
  const int lane = lane_id();
  Rope2 r{1.0, 0.0, 1.0, 0.0};
  const int d0 = lane, d1 = lane + 64;
  if (d0 < rot) sincos_angle(pos * f.f0, &r.s0, &r.c0);
  if (d1 < rot) {
    if (d0 < rot && f.same) {
      r.c1 = r.c0;
      r.s1 = r.s0;
    } else {
      sincos_angle(pos * f.f1, &r.s1, &r.c1);
    }
  }
  return r;
}

// (o0, o1) = RoPE(x / sqrt(mean(x^2) + eps) * (1 + w)) for the lane's two dims.
__device__ __forceinline__ void norm_rope2(double x0, double x1, double w0, double w1, double eps, int rot,
                                           const Rope2 &r, double &o0, double &o1) {
  const double ss = wave_sum_f64(x0 * x0 + x1 * x1);
  // one inverse square root per lane: x * (1 / den) and x / den differ by
  // about an fp64 ulp, far below the one rounding at the end
  const double inv = inv_sqrt_f64(ss / 128.0 + eps);
  const double y0 = x0 * inv * (1.0 + w0), y1 = x1 * inv * (1.0 + w1);
  const int lane = lane_id(), half = rot >> 1;
  const int d0 = lane, d1 = lane + 64;
  const int q0 = d0 < rot ? (d0 < half ? d0 + half : d0 - half) : d0;
  const int q1 = d1 < rot ? (d1 < half ? d1 + half : d1 - half) : d1;
  const double a0 = __shfl(y0, q0 & 63, 64), b0 = __shfl(y1, q0 & 63, 64);
  const double a1 = __shfl(y0, q1 & 63, 64), b1 = __shfl(y1, q1 & 63, 64);
  const double p0 = (q0 >> 6) ? b0 : a0, p1 = (q1 >> 6) ? b1 : a1;
  o0 = d0 < rot ? (d0 < half ? y0 * r.c0 - p0 * r.s0 : y0 * r.c0 + p0 * r.s0) : y0;
  o1 = d1 < rot ? (d1 < half ? y1 * r.c1 - p1 * r.s1 : y1 * r.c1 + p1 * r.s1) : y1;
}

// Element offset of KV head 0 of `token`'s row in the paged pool (128 tokens
// per page; ptrow is the sequence's K or V page-table row, V pages already
// offset by numPages), or -1 when its page-table entry is out of range.
__device__ __forceinline__ long long pool_row_off(const int32_t *ptrow, int token, int max_pages,
                                                  int num_flat_pages, int Hkv, int PHD) {
  const int pi = token >> 7;
  if (token < 0 || pi >= max_pages) return -1;
  const int pg = ptrow[pi];
  if ((unsigned)pg >= (unsigned)num_flat_pages) return -1;
  return (((long long)pg * 128 + (token & 127)) * Hkv) * PHD;
}

// Workgroups go round-robin over the eight XCDs.  For work whose cost
// follows the item's sequence (item mod B, live lengths differ), the n-th set
// of eight workgroups takes items 8n + ((x + n) mod 8) on XCD x: each XCD
// cycles through every residue instead of keeping the ones that B ties to
// its index.  Launches round the grid up to a multiple of eight and
// bound-check the item.
__device__ __forceinline__ int xcd_spread(int blk) {
  const int n = blk >> 3;
  return (n << 3) | (((blk & 7) + n) & 7);
}

// Items: B*S query rows, then B*Gmax blocks, a.per_wave consecutive items
// per wave (up to kPrepItemsPerWave, fewer when that would leave the chip
// short of waves), four waves per workgroup; a wave holds rows only or
// blocks only.  A wave issues every load of its next item before it works
// on the current one.  (The item's stores could alias its loads as far as
// the compiler knows, so loads written inside the per-head loop would each
// wait for the previous head's stores: one memory round trip per head.)
constexpr int kPrepItemsPerWave = 4;

// One item's inputs, lane l's dims l and l + 64: a row's heads (slot h =
// head h) or a block's raw keys (slot j = token j).  Slots past Hi (ratio)
// repeat the last real one, so the loads are issued unconditionally.
template <int N>
struct PrepIn {
  uint32_t x[N][2];
  int ctx;
};

__device__ __forceinline__ void prep_row_loads(const IdxPrepArgs &a, long long item, int lane, PrepIn<4> &in) {
  in.ctx = a.ctx[item / a.S];
  const uint16_t *src = a.idx_q + (size_t)item * a.Hi * 128 + lane;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int hh = min(h, a.Hi - 1);
    in.x[h][0] = src[hh * 128];
    in.x[h][1] = src[hh * 128 + 64];
  }
}

__device__ __forceinline__ void prep_block_loads(const IdxPrepArgs &a, long long kk, int lane, PrepIn<8> &in) {
  const int b = (int)(kk / a.Gmax), g = (int)(kk % a.Gmax);
  in.ctx = a.ctx[b];
  const uint16_t *src = a.idx_k + ((size_t)b * a.S + (size_t)a.ratio * g) * 128 + lane;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int jj = min(j, a.ratio - 1);
    in.x[j][0] = src[jj * 128];
    in.x[j][1] = src[jj * 128 + 64];
  }
}

__global__ __launch_bounds__(256) void idx_prep_kernel(IdxPrepArgs a) {
  const RopeLane rl = rope_lane(a.freq, a.rot);
  const int lane = lane_id();
  const long long wave = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const long long nrows = (long long)a.B * a.S, nblocks = (long long)a.B * a.Gmax;
  const long long row_waves = (nrows + a.per_wave - 1) / a.per_wave;
  double o0, o1;
  if (wave < row_waves) {
    const long long first = wave * a.per_wave, end = min(first + a.per_wave, nrows);
    const double w0 = a.wq[lane], w1 = a.wq[lane + 64];
    PrepIn<4> cur;
    prep_row_loads(a, first, lane, cur);
    for (long long item = first; item < end; ++item) {
      PrepIn<4> nxt;
      prep_row_loads(a, min(item + 1, end - 1), lane, nxt);
      const int t = (int)(item % a.S);
      if (t < min(cur.ctx, a.S)) {
        const Rope2 r = rope_at((double)t, rl, a.rot);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          if (h >= a.Hi) break;
          norm_rope2(bits_to_f64(cur.x[h][0], a.dt), bits_to_f64(cur.x[h][1], a.dt), w0, w1, a.eps, a.rot, r, o0,
                     o1);
          // q-hat rounded once to fp32, stored as the scoring's 16-bit pieces
          uint16_t *qp = a.qhat + ((size_t)item * a.Hi + h) * 128 * kQPieces;
          store_q_pieces(qp + lane, (float)o0);
          store_q_pieces(qp + 64 + lane, (float)o1);
        }
      }
      cur = nxt;
    }
    return;
  }
  const long long first = (wave - row_waves) * a.per_wave, end = min(first + a.per_wave, nblocks);
  if (first >= end) return;
  const double w0 = a.wk[lane], w1 = a.wk[lane + 64];
  // one item's loads at a time here (blocks are a quarter of the items or
  // fewer; a second buffer of eight slots would cost the row waves'
  // occupancy as well)
  for (long long kk = first; kk < end; ++kk) {
    PrepIn<8> cur;
    prep_block_loads(a, kk, lane, cur);
    const int b = (int)(kk / a.Gmax), g = (int)(kk % a.Gmax);
    if (g < min(cur.ctx, a.S) / a.ratio) {
      // mean over the block's tokens, summed in token order from +0
      double m0 = 0.0, m1 = 0.0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j >= a.ratio) break;
        m0 += bits_to_f64(cur.x[j][0], a.dt);
        m1 += bits_to_f64(cur.x[j][1], a.dt);
      }
      m0 /= (double)a.ratio;
      m1 /= (double)a.ratio;
      const Rope2 r = rope_at((double)a.ratio * g, rl, a.rot);
      norm_rope2(m0, m1, w0, w1, a.eps, a.rot, r, o0, o1);
      const size_t ob = ((size_t)b * a.Gmax + g) * 128;
      a.kbar[ob + lane] = (uint16_t)f64_to_bits(o0, a.dt);
      a.kbar[ob + 64 + lane] = (uint16_t)f64_to_bits(o1, a.dt);
    }
  }
}

// Prefill -> decode handoff: the indexer state a decode step continues from,
// in the pool tails (columns [D, D + 128) of KV head 0 rows).  Wave item
// (b, g), g < Gmax: block g's kbar, as pooled above, into the V-row tail of
// token ratio*g when the block is complete; item (b, Gmax): the raw keys of
// the trailing incomplete block into the K-row tails of its tokens.  Rows
// whose page-table entry is out of range are skipped.
__global__ __launch_bounds__(256) void idx_handoff_kernel(IdxPrepArgs a) {
  const int lane = lane_id();
  const long long item = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= (long long)a.B * (a.Gmax + 1)) return;
  const int b = (int)(item / (a.Gmax + 1)), g = (int)(item % (a.Gmax + 1));
  const int live = min(a.ctx[b], a.S), nc = live / a.ratio;
  const int32_t *ptk = a.pt + (size_t)b * 2 * a.max_pages, *ptv = ptk + a.max_pages;
  if (g < a.Gmax) {
    if (g >= nc) return;
    const long long o = pool_row_off(ptv, a.ratio * g, a.max_pages, a.num_flat_pages, a.Hkv, a.PHD);
    if (o < 0) return;
    const uint16_t *kb = a.kbar + ((size_t)b * a.Gmax + g) * 128;
    a.pool[o + a.D + lane] = kb[lane];
    a.pool[o + a.D + 64 + lane] = kb[lane + 64];
    return;
  }
  for (int t = nc * a.ratio; t < live; ++t) {
    const long long o = pool_row_off(ptk, t, a.max_pages, a.num_flat_pages, a.Hkv, a.PHD);
    if (o < 0) continue;
    const uint16_t *k = a.idx_k + ((size_t)b * a.S + t) * 128;
    a.pool[o + a.D + lane] = k[lane];
    a.pool[o + a.D + 64 + lane] = k[lane + 64];
  }
}

// Chunked prefill, step 1: the indexer state the chunk's rows score against.
// Chunk row t of sequence b sits at position start[b] + t.  Wave items:
//   * (b, t), t < C: the queries of a live row at its position -> qhat;
//   * (b, g), g < Gmax: every complete block g < ctx/ratio into the dense
//     kbar workspace -- copied from its V-row tail when it was complete
//     before the chunk, else pooled from the raw keys of its tokens (the
//     stored K-row tails of tokens before the chunk, the chunk's idx_k for
//     the rest) and also stored in its V-row tail;
//   * (b, Gmax): the chunk's tokens of the trailing incomplete block -> their
//     raw keys into their K-row tails.
// The tails these items read (V rows of blocks complete before the chunk, K
// rows of tokens before it) and those they write are disjoint.
__global__ __launch_bounds__(256) void idx_chunk_prep_kernel(IdxChunkPrepArgs a) {
  const RopeLane rl = rope_lane(a.freq, a.rot);
  const int lane = lane_id();
  const long long item = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const long long per_seq = (long long)a.C + a.Gmax + 1;
  if (item >= (long long)a.B * per_seq) return;
  const int b = (int)(item / per_seq), k = (int)(item % per_seq);
  const int P = a.start[b];
  if (P < 0) return;
  // positions past the chunk have no keys here (a total length past
  // start + C breaks the contract): they are treated as absent
  const int ctx = (int)min((long long)min(a.ctx[b], a.max_pages * 128), (long long)P + a.C);
  if (ctx <= P) return;
  const int32_t *ptk = a.pt + (size_t)b * 2 * a.max_pages, *ptv = ptk + a.max_pages;
  const int r = a.ratio;
  double o0, o1;
  if (k < a.C) {  // queries of row k
    const int pos = P + k;
    if (pos >= ctx) return;
    // every head's inputs loaded before the first store (as in the prefill
    // prep: a store may alias a later head's input as far as the compiler
    // knows, so per-head loads would each wait for the previous stores)
    const size_t row_off = ((size_t)b * a.C + k) * a.Hi * 128;
    uint32_t x[4][2];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const size_t off = row_off + (size_t)min(h, a.Hi - 1) * 128;
      x[h][0] = a.idx_q[off + lane];
      x[h][1] = a.idx_q[off + 64 + lane];
    }
    const double w0 = a.wq[lane], w1 = a.wq[lane + 64];
    const Rope2 rp = rope_at((double)pos, rl, a.rot);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      if (h >= a.Hi) break;
      norm_rope2(bits_to_f64(x[h][0], a.dt), bits_to_f64(x[h][1], a.dt), w0, w1, a.eps, a.rot, rp, o0, o1);
      uint16_t *qp = a.qhat + (row_off + (size_t)h * 128) * kQPieces;
      store_q_pieces(qp + lane, (float)o0);
      store_q_pieces(qp + 64 + lane, (float)o1);
    }
    return;
  }
  const int nc = ctx / r;
  if (k < a.C + a.Gmax) {  // block g
    const int g = k - a.C;
    if (g >= nc) return;
    uint16_t *kb = a.kbar + ((size_t)b * a.Gmax + g) * 128;
    const long long ov = pool_row_off(ptv, r * g, a.max_pages, a.num_flat_pages, a.Hkv, a.PHD);
    if (r * g + r <= P) {  // complete before the chunk: its tail holds kbar
      kb[lane] = ov >= 0 ? a.pool[ov + a.D + lane] : 0;
      kb[lane + 64] = ov >= 0 ? a.pool[ov + a.D + 64 + lane] : 0;
      return;
    }
    double m0 = 0.0, m1 = 0.0;
    bool ok = true;
    for (int j = 0; j < r; ++j) {
      const int tok = r * g + j;
      if (tok < P) {
        const long long o = pool_row_off(ptk, tok, a.max_pages, a.num_flat_pages, a.Hkv, a.PHD);
        ok = ok && o >= 0;
        if (o >= 0) {
          m0 += bits_to_f64(a.pool[o + a.D + lane], a.dt);
          m1 += bits_to_f64(a.pool[o + a.D + 64 + lane], a.dt);
        }
      } else {
        const size_t off = ((size_t)b * a.C + (tok - P)) * 128;
        m0 += bits_to_f64(a.idx_k[off + lane], a.dt);
        m1 += bits_to_f64(a.idx_k[off + 64 + lane], a.dt);
      }
    }
    m0 /= (double)r;
    m1 /= (double)r;
    const Rope2 rp = rope_at((double)(r * g), rl, a.rot);
    norm_rope2(m0, m1, (double)a.wk[lane], (double)a.wk[lane + 64], a.eps, a.rot, rp, o0, o1);
    const uint16_t k0 = (uint16_t)f64_to_bits(o0, a.dt), k1 = (uint16_t)f64_to_bits(o1, a.dt);
    kb[lane] = k0;
    kb[lane + 64] = k1;
    if (ok && ov >= 0) {
      a.pool[ov + a.D + lane] = k0;
      a.pool[ov + a.D + 64 + lane] = k1;
    }
    return;
  }
  // the chunk's tokens of the trailing incomplete block
  for (int tok = max(P, r * nc); tok < ctx; ++tok) {
    const long long o = pool_row_off(ptk, tok, a.max_pages, a.num_flat_pages, a.Hkv, a.PHD);
    if (o < 0) continue;
    const uint16_t *src = a.idx_k + ((size_t)b * a.C + (tok - P)) * 128;
    a.pool[o + a.D + lane] = src[lane];
    a.pool[o + a.D + 64 + lane] = src[lane + 64];
  }
}

// A kbar piece (eight 16-bit values) as the fp16 MFMA operand.
template <int DT>
__device__ __forceinline__ u32x4 kbar_operand(u32x4 v) {
  if constexpr (DT == DT_F16) return v;
  else return bf16x8_to_f16x8(v);
}

// Prefill scoring.  A workgroup takes 32 consecutive rows and a run of
// chunks of kScoreChunk complete blocks (whole rows or kScoreRun chunks, as
// the launcher decides; the rows' query pieces, prepared by the prep kernel,
// are loaded once per run; short prefills take shorter runs so the grid
// still fills the chip); runs of the last rows are dispatched first, all
// runs of a row group on one XCD.
// Per chunk the kbar rows are staged in LDS, 16-byte pieces XOR-swizzled by
// row so that MFMA fragment reads are conflict-free; each wave
// computes 8 rows against the chunk.  The MFMA M tile is (row, head) with the
// head fastest, so each 16-lane group ends with the four head dots of one row
// and one block and sums their relus in-lane; a wave's two M tiles share every
// kbar fragment.  The chunk's 32 x kScoreChunk scores are assembled in LDS and
// stored as whole 512-byte row segments.
template <int DT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void idx_score_kernel(
    IdxScoreArgs a) {
  constexpr int NP = kQPieces;
  constexpr int CB = kScoreChunk;
  __shared__ __align__(16) uint32_t s_kb[CB * 64];     // CB rows x 256 B
  __shared__ __align__(16) float s_sc[32][CB + 4];    // scores of the chunk
  const int lane = lane_id(), q4 = lane >> 4, r16 = lane & 15, wv = threadIdx.x >> 6;
  const int tid = threadIdx.x;
  const int T32 = (a.S + 31) >> 5;
  // Workgroups go round-robin over the eight XCDs.  All runs of a row group
  // run on one XCD, so they share the group's queries through its L2.  The
  // n-th group of XCD x is group level (n mod L8) * 8 + x (level 0 = the last
  // 32 rows) of sequence n / L8, L8 = ceil(levels / 8): an XCD takes one
  // sequence at a time (its kbar stays in the XCD's L2), longest rows first,
  // and every XCD takes the same levels of every sequence, so ragged batches
  // load the XCDs evenly.
  const int xcd = blockIdx.x & 7;
  const long long n = blockIdx.x >> 3;
  const int run = (int)(n % a.nchunk);
  const long long k = n / a.nchunk;
  const long long L8 = (T32 + 7) / 8;
  const int b = (int)(k / L8);
  const long long level = (k % L8) * 8 + xcd;
  if (level >= T32) return;
  const int tg = 32 * (T32 - 1 - (int)level);
  // row t sits at position off + t; rows [0, live) are live
  const int off = a.start ? a.start[b] : 0;
  // positions stay below Gmax * ratio, the blocks the kbar rows hold
  const int lim = a.start ? min(a.ctx[b], a.Gmax * a.ratio) : a.ctx[b];
  const int live = max(0, min(lim - off, a.S));
  if (tg >= live) return;
  const int nc_hi = (off + min(tg + 31, live - 1) + 1) / a.ratio;
  const int run_lo = run * a.run_chunks * CB;
  const int run_hi = min(run_lo + a.run_chunks * CB, nc_hi);
  if (run_lo >= run_hi) return;

  // kbar rows of a chunk: global -> registers (issued a chunk ahead) -> LDS
  constexpr int NV = CB * 16 / 256;  // 16-byte pieces per thread
  u32x4 v[NV];
  auto load_chunk = [&](int g_lo) {
    const int npiece = (min(g_lo + CB, run_hi) - g_lo) * 16;
    const uint16_t *src = a.kbar + ((size_t)b * a.Gmax + g_lo) * 128;
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int i = tid + 256 * u;
      if (i < npiece) v[u] = ld16(src + 8 * i);
    }
  };
  auto stage_chunk = [&](int g_lo) {
    const int npiece = (min(g_lo + CB, run_hi) - g_lo) * 16;
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int i = tid + 256 * u;
      const int row = i >> 4, pc = i & 15;
      if (i < npiece) *reinterpret_cast<u32x4 *>(&s_kb[row * 64 + 4 * (pc ^ (row & 15))]) = kbar_operand<DT>(v[u]);
    }
  };
  load_chunk(run_lo);  // in flight while the queries are loaded and split

  const int t0 = tg + 8 * wv;
  // the rows' query pieces (written by the prep), zero for dead rows and
  // heads; the loads are unconditional (a clamped row and head)
  u32x4 qa[2][NP][4];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int t = t0 + 4 * m + (r16 >> 2), h = r16 & 3;
    const bool ok = t < live && h < a.Hi;
    const uint16_t *qp = a.qhat + (((size_t)b * a.S + min(t, a.S - 1)) * a.Hi + min(h, a.Hi - 1)) * NP * 128 + 8 * q4;
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4 v = ld16(qp + 128 * p + 32 * ks);
        qa[m][p][ks] = ok ? v : u32x4{0u, 0u, 0u, 0u};
      }
  }
  const int nc_wave = t0 < live ? (off + min(t0 + 7, live - 1) + 1) / a.ratio : 0;
  // score stores: thread tid owns columns 4 (tid % 32) .. +3 of rows tid / 32 + 8 j
  static_assert(CB == 128, "store mapping assumes 32 float4 columns per chunk");
  const int st_row0 = tid >> 5, st_c4 = 4 * (tid & 31);
  int st_nc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = tg + st_row0 + 8 * j;
    st_nc[j] = t < live ? (off + t + 1) / a.ratio : 0;
  }
  float *const st_base = a.scores + ((size_t)b * a.S + tg + st_row0) * a.stride;

  stage_chunk(run_lo);
  __syncthreads();
  for (int g_lo = run_lo; g_lo < run_hi; g_lo += CB) {
    const int g_hi = min(g_lo + CB, run_hi);
    const bool more = g_lo + CB < run_hi;
    if (more) load_chunk(g_lo + CB);  // in flight during this chunk's MFMAs
    const int g_end = min(g_hi, nc_wave);
    for (int g0 = g_lo; g0 < g_end; g0 += 16) {
      const int lb = g0 - g_lo + r16;  // local kbar row; lb & 15 == r16
      u32x4 kb[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kb[ks] = *reinterpret_cast<const u32x4 *>(&s_kb[lb * 64 + 4 * ((4 * ks + q4) ^ r16)]);
      // two independent accumulator chains (the M tiles), interleaved
      f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
          for (int m = 0; m < 2; ++m) acc[m] = mfma16x16x32<DT_F16>(qa[m][p][ks], kb[ks], acc[m]);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const f32x4 d = acc[m];
        s_sc[8 * wv + 4 * m + q4][lb] = fmaxf(d[0], 0.f) + fmaxf(d[1], 0.f) + fmaxf(d[2], 0.f) + fmaxf(d[3], 0.f);
      }
    }
    __syncthreads();  // this chunk's kbar is consumed and its scores are in LDS
    // Stage the next chunk before storing this one's scores: the stage waits
    // on vmcnt, which counts stores too, so with this chunk's stores still in
    // flight it would wait for them as well.
    if (more) stage_chunk(g_lo + CB);
    // store the chunk's scores: 32 rows x (g_hi - g_lo) floats, 16 B per lane;
    // thread tid writes columns c4 of rows tid / 32 + 8 j
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = st_row0 + 8 * j;
      const int ncr = st_nc[j] - g_lo;  // this row's blocks in the chunk (<= 0: none, or dead row)
      if (st_c4 >= ncr) continue;
      float *dst = st_base + (size_t)(8 * j) * a.stride + g_lo + st_c4;
      const f32x4 v4 = *reinterpret_cast<const f32x4 *>(&s_sc[r][st_c4]);
      if (st_c4 + 4 <= ncr) *reinterpret_cast<f32x4 *>(dst) = v4;
      else
        for (int q = 0; q < ncr - st_c4; ++q) dst[q] = v4[q];
    }
    __syncthreads();  // the next chunk's kbar is staged; the score tile is free
  }
}


// ---------------------------------------------------------------------------
// Select + expand for prefill rows of up to 128*KPL blocks: NW = 1 wave per
// row (four rows per workgroup, no barriers) or NW = 2 waves per row (one
// row per 128-thread workgroup: half the keys and registers per wave, so
// long rows run at higher occupancy and half the latency).  Wave h holds
// the keys of blocks h*64*KPL + 256g + 4l + c (lane l, g < KPL/4, c < 4),
// loaded as float4s; slots past the row hold 0xffffffff (real keys have
// bit 31 clear).  The cut is narrowed over key ranges as in the workgroup
// select (select_core.h): the first range runs from the smallest non-zero
// key to the largest in up to 2048 bins (1024 in the one-wave kernels),
// later ones split the cut bin into
// up to 256; the row's histogram lives in LDS (plain atomic increments under
// a wave-uniform branch, keys outside the range into spare words), and
// every wave of the row finds the cut bin itself with DPP scans of per-lane
// bin sums, then inside the one lane range that holds it.  The select stops
// as soon as the cut bin holds exactly the keys still needed (the usual
// case); otherwise it refines to single keys and keeps the lowest-index
// keys equal to the cut.  Emission keeps index order: per 256-block group,
// ballots of the kept slots and mbcnt give each lane its positions.  Each
// wave stages its kept blocks in its own LDS list (when the lists fit), and
// the row is stored with the causal tail and -1 padding in one coalesced
// pass.
// ---------------------------------------------------------------------------
template <int NW>
__device__ __forceinline__ void row_sync() {
  if constexpr (NW == 1) __builtin_amdgcn_wave_barrier();
  else __syncthreads();
}

// First-pass bits of the per-row select: 11 (2048 bins) for two-wave rows,
// 10 for the one-wave kernels (rows of up to 4096 blocks).  One wave's
// histogram clear and first cut search halve; at up to 32 keys per lane
// (62-64 registers, eight waves per SIMD) four 2048-bin histograms per
// workgroup would also have held the kernel at four waves per SIMD by LDS.
// Two-wave rows (8192 keys) measured no faster with 1024 bins.  Ten
// first-pass bits and three passes of eight still reach single keys.
__host__ __device__ constexpr int sel_rows_first_bits(int KPL, int NW) { return NW == 1 && KPL <= 64 ? 10 : 11; }
__host__ __device__ constexpr int sel_rows_hist_words(int KPL, int NW) {
  return (1 << sel_rows_first_bits(KPL, NW)) + ((1 << sel_rows_first_bits(KPL, NW)) >> 3);
}

template <int KPL, int NW, bool STAGE>
__global__ __launch_bounds__(256) void idx_select_rows_kernel(IdxSelectArgs a) {
  constexpr int NG = KPL / 4;
  constexpr int SPAN = 64 * KPL;  // blocks held by one wave
  extern __shared__ __align__(16) uint32_t s_dyn[];
  __shared__ int s_x[3][4];       // two-wave rows: per wave kmax, kmin, kept, equal count; [2]: cut
  const int wv = threadIdx.x >> 6, lane = lane_id();
  const int h = NW == 1 ? 0 : wv;
  const int tid = NW == 1 ? lane : (int)threadIdx.x, nthr = 64 * NW;
  const int wg = xcd_spread((int)blockIdx.x);
  const int row = a.row0 + (NW == 1 ? wg * 4 + wv : wg);
  if (row >= a.row0 + a.nrows) return;  // a two-wave workgroup holds one row
  const int b = row % a.B;
  const int tl = a.S - 1 - row / a.B;  // longest rows first; the row's position is off + tl
  const int t = (a.start ? a.start[b] : 0) + tl;
  const bool live = t >= 0 && t < min(a.ctx[b], a.max_ctx);
  int32_t *out = a.out + ((size_t)b * a.S + tl) * a.top_k;
  if (!live) {
    for (int i = tid; i < a.top_k; i += nthr) out[i] = -1;
    return;
  }
  const int r = a.ratio;
  const int nc = (t + 1) / r;
  // chunk rows reach every launch (their lengths are device data): a row
  // longer than this kernel holds is the workgroup select's
  if (a.start && nc > NW * SPAN) return;
  if (nc <= a.budget) {
    for (int i = tid; i < a.top_k; i += nthr) out[i] = i <= t ? i : -1;
    return;
  }
  uint32_t *region = s_dyn + (NW == 1 ? wv : 0) * a.wave_words;
  uint32_t *hist = region;
  // Staged lists hold the kept block indices (16 bits: blocks < QSA_MAX_BLOCKS),
  // a.list_words words per wave.  One wave: the list overlays the histogram;
  // two waves: [hist | list0 | list1].  Unstaged: expanded ids go straight out.
  uint16_t *lb0 =
      reinterpret_cast<uint16_t *>(region + (NW == 1 ? 0 : kSelHistWords + kSelTrash + kSelSmallWords + kSelTrash));
  uint16_t *lb = lb0 + 2 * h * a.list_words;
  const float *srow = a.scores + ((size_t)b * a.S + tl) * a.row_stride;
  const int base_i = h * SPAN;
  uint32_t key[KPL];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    // unconditional loads (a load on one branch only is waited for alone
    // where the branches join): slots past the row read its last scores
    const int i0 = base_i + 256 * g + 4 * lane;
    const f32x4 v = *reinterpret_cast<const f32x4 *>(srow + min((long long)i0, a.row_stride - 4));
#pragma unroll
    for (int c = 0; c < 4; ++c) key[4 * g + c] = i0 + c < nc ? score_key(v[c]) : 0xffffffffu;
  }
  // Largest key, smallest non-zero key and the non-zero count (groups of
  // 256 blocks that start past the row hold no real key: skipped).  As
  // signed values the empty-slot marker is -1, below every key; k - 1 wraps
  // a zero key past every real one; the count is taken by ballots.
  int kmax_s = 0;
  uint32_t kmin1 = 0xffffffffu, nnz = 0u;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    if (base_i + 256 * g < nc) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t k = key[4 * g + c], km1 = k - 1u;
        kmax_s = max(kmax_s, (int)k);
        kmin1 = min(kmin1, km1);
        nnz += (uint32_t)__popcll(__ballot(km1 < 0x7fffffffu));
      }
    }
  }
  uint32_t kmax = __builtin_amdgcn_readlane(
      wave_incl_op((uint32_t)kmax_s, 0u, [](uint32_t x, uint32_t y) { return max(x, y); }), 63);
  uint32_t kmin = __builtin_amdgcn_readlane(
      wave_incl_op(kmin1, 0xffffffffu, [](uint32_t x, uint32_t y) { return min(x, y); }), 63);
  if constexpr (NW == 2) {
    if (lane == 0) {
      s_x[wv][0] = (int)kmax;
      s_x[wv][1] = (int)kmin;
      s_x[wv][2] = (int)nnz;
    }
    __syncthreads();
    kmax = max((uint32_t)s_x[0][0], (uint32_t)s_x[1][0]);
    kmin = min((uint32_t)s_x[0][1], (uint32_t)s_x[1][1]);
    nnz = (uint32_t)(s_x[0][2] + s_x[1][2]);
  }
  kmin += 1u;  // used only when some key is non-zero (then below 2^31)
  // The cut is narrowed over key ranges [lo, hi) as in the workgroup select
  // (select_core.h): zeros are left out of the first range unless fewer than
  // `budget` keys are non-zero; the first pass takes up to 2048 bins (1024,
  // sel_rows_first_bits), later ones 256.  Keys outside the range count into spare words (no lane is
  // masked off); two-wave rows alternate two histograms, so a wave may clear
  // the next pass's while the other still reads this one's.
  uint32_t lo, hi;
  int remaining = a.budget;
  bool whole_bin = false;
  if ((int)nnz < a.budget) {  // every non-zero key, then the first zeros
    lo = 0u;
    hi = 1u;
    remaining = a.budget - (int)nnz;
  } else {
    lo = kmin;
    hi = kmax + 1u;
    for (int pass = 0; pass < 4; ++pass) {
      const uint32_t range = hi - lo;
      const int bl = range > 1u ? 32 - __clz((int)(range - 1u)) : 0;
      const int s = max(0, bl - (pass == 0 ? sel_rows_first_bits(KPL, NW) : 8));
      const int nb = (((int)((range - 1u) >> s) >> 8) + 1) << 8;  // bins in use, rounded up to 256
      uint32_t *H = NW == 2 && (pass & 1) ? region + kSelHistWords + kSelTrash : hist;
      uint32_t *spare = H + (H == hist ? sel_rows_hist_words(KPL, NW) : kSelSmallWords) + (lane & (kSelTrash - 1));
      const int nvec = (hpad(nb - 1) + 4) >> 2;
      for (int j = tid; j < nvec; j += nthr) reinterpret_cast<u32x4 *>(H)[j] = u32x4{0u, 0u, 0u, 0u};
      row_sync<NW>();
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if (base_i + 256 * g < nc) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            // k in [lo, hi) as one unsigned compare of k - lo
            const uint32_t d = key[4 * g + c] - lo;
            const bool in = d < range;
            if (__ballot(in) != 0ull) {
              const uint32_t bin = d >> s;
              atomicAdd(in ? H + bin + ((bin >> 5) << 2) : spare, 1u);  // H[hpad(bin)]
            }
          }
        }
      }
      row_sync<NW>();
      int dsel, above, cnt;
      sel_find_cut(H, nb, remaining, dsel, above, cnt);  // every wave of the row
      remaining -= above;
      lo += (uint32_t)dsel << s;
      hi = min(hi, lo + (1u << s));
      if (cnt == remaining) {  // the whole bin is kept
        whole_bin = true;
        break;
      }
      if (s == 0) break;  // single keys: the lowest-index ones of the cut key are kept
    }
  }

  // Keys >= hi are kept; of those in [lo, hi), the first `remaining` in
  // index order (all of them when whole_bin).  A byte per lane and group
  // (bit c: block 256 g + 4 lane + c at or above hi; bit 4 + c: in [lo,
  // hi)), then lane l turns the bytes of blocks [32 j, 32 j + 32) of the
  // wave's span, j = l + 64 u, into two 32-bit masks, and a wave scan of
  // their counts places each mask's kept blocks in the wave's list.  A
  // two-wave row's cut-bin keys in its first wave come before those in its
  // second.  The flags overlay the histograms (past the staged list).
  row_sync<NW>();  // every wave has read the histograms
  uint8_t *fl = reinterpret_cast<uint8_t *>(NW == 1 ? region + (STAGE ? a.list_words : 0) : region + h * 16 * NG);
  {
    const uint32_t above = 0x80000000u - hi, range = hi - lo;  // real keys are below 2^31
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (base_i + 256 * g < nc) {
        uint32_t byte = 0u;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t k = key[4 * g + c];
          byte |= k - hi < above ? 1u << c : 0u;
          byte |= k - lo < range ? 16u << c : 0u;
        }
        fl[64 * g + lane] = (uint8_t)byte;
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();  // a wave reads only its own flags (LDS is in order per wave)
  constexpr int NU = (8 * NG + 63) / 64;        // masks per lane
  const int jmax = min(8 * NG, max(0, (nc - base_i + 31) >> 5));  // masks holding blocks of the row
  uint32_t gtm[NU], eqm[NU];
  int ex[NU], tot[NU];
  int eq_total = 0;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int j = lane + 64 * u;
    unsigned long long v = 0ull;
    if (j < jmax) v = *reinterpret_cast<const unsigned long long *>(fl + 8 * j);
    gtm[u] = low_nibbles(v);
    eqm[u] = low_nibbles(v >> 4);
    const int cnt = __builtin_popcount(eqm[u]) | (__builtin_popcount(gtm[u]) << 16);
    const int inc = wave_incl_scan(cnt);
    ex[u] = inc - cnt;
    tot[u] = __builtin_amdgcn_readlane(inc, 63);
    eq_total += tot[u] & 0xffff;
  }
  int eq_seen = 0;
  if (NW == 2 && !whole_bin) {  // the second wave's cut-bin keys follow the first's
    if (lane == 0) s_x[wv][3] = eq_total;
    __syncthreads();
    eq_seen = h == 1 ? s_x[0][3] : 0;
  }
  const int take_max = max(0, remaining - eq_seen);  // cut-bin keys this wave keeps at most
  int gt_run = 0, eq_run = 0;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int gt_b = gt_run + (ex[u] >> 16), eq_b = eq_run + (ex[u] & 0xffff);
    const int take = min(__builtin_popcount(eqm[u]), max(0, take_max - eq_b));
    int pos = gt_b + min(eq_b, take_max);
    uint32_t keep = gtm[u], e = eqm[u];
    for (int q = 0; q < take; ++q) {
      keep |= e & (0u - e);
      e &= e - 1u;
    }
    const int blk0 = base_i + 32 * (lane + 64 * u);
    while (keep != 0u) {
      const int g_blk = blk0 + __builtin_ctz(keep);
      keep &= keep - 1u;
      if constexpr (STAGE) {
        lb[pos] = (uint16_t)g_blk;
      } else {
        for (int q = 0; q < r; ++q) out[r * pos + q] = r * g_blk + q;
      }
      ++pos;
    }
    gt_run += tot[u] >> 16;
    eq_run += tot[u] & 0xffff;
  }
  const int kept = gt_run + min(eq_run, take_max);
  if constexpr (NW == 2) {
    if (lane == 0) s_x[wv][2] = kept;
  }
  row_sync<NW>();
  const int head = r * a.budget;
  const int len = head + (t + 1) - r * nc;
  const int kb0 = NW == 2 ? s_x[0][2] : a.budget;  // blocks in the first wave's list
  const uint16_t *lb1 = lb0 + 2 * a.list_words;
  for (int i = (STAGE ? 0 : head) + tid; i < a.top_k; i += nthr) {
    int v;
    if (i < head) {  // staged: kept block j = i / r, expanded
      const int j = r == 4 ? i >> 2 : i / r;
      const int blk = j < kb0 ? lb0[j] : lb1[j - kb0];
      v = r * blk + (i - r * j);
    } else {
      v = i < len ? r * nc + (i - head) : -1;
    }
    out[i] = v;
  }
}

// ---------------------------------------------------------------------------
// Select + expand, one 1024-thread workgroup per row: decode rows (one per
// sequence, up to 32768 blocks), prefill rows over 8192 blocks and chunk
// rows.  Thread j holds four keys per round (blocks 4*1024*r + 4j + c) in
// registers; the workgroup select (select_core.h) stages the kept block
// indices in LDS, and the row is stored expanded, with the causal tail and
// -1 padding, in one coalesced pass.
// ---------------------------------------------------------------------------
constexpr int kSelWgThreads = 1024;

template <int KPT>
__global__ __launch_bounds__(kSelWgThreads) void idx_select_wg_kernel(IdxSelectArgs a) {
  constexpr int NT = kSelWgThreads;
  extern __shared__ uint16_t s_lb[];  // kept block indices [budget]
  __shared__ WgSelLds<NT> s_sel;
  const int tid = threadIdx.x;

  int t, live;
  int32_t *out;
  const float *srow;
  if (a.decode) {
    const int b = blockIdx.x;
    const int c = min(a.ctx[b], a.max_ctx);
    t = c - 1;
    live = c > 0;
    out = a.out + (size_t)b * a.top_k;
    srow = a.scores + (size_t)b * a.row_stride;
  } else {
    const int rw = a.row0 + xcd_spread((int)blockIdx.x);  // longest rows first
    if (rw >= a.row0 + a.nrows) return;  // the grid is rounded up to eight
    const int b = rw % a.B;
    const int tl = a.S - 1 - rw / a.B;   // the row; its position is off + tl
    const int off = a.start ? a.start[b] : 0;
    t = off + tl;
    live = t >= 0 && t < min(a.ctx[b], a.max_ctx);
    // chunk rows of up to wg_min_nc blocks, dead ones included, are the
    // per-row kernel's (launched over the same rows)
    if (a.wg_min_nc > 0 && (!live || (t + 1) / a.ratio <= a.wg_min_nc)) return;
    out = a.out + ((size_t)b * a.S + tl) * a.top_k;
    srow = a.scores + ((size_t)b * a.S + tl) * a.row_stride;
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
  wg_select_clear<NT>(s_sel);
  // thread j's keys of round r: blocks 4*NT*r + 4j + c (unconditional loads,
  // as in the per-row kernel)
  uint32_t key[KPT];
#pragma unroll
  for (int r = 0; r < KPT / 4; ++r) {
    const int i = 4 * NT * r + 4 * tid;
    const f32x4 v = *reinterpret_cast<const f32x4 *>(srow + min((long long)i, a.row_stride - 4));
#pragma unroll
    for (int c = 0; c < 4; ++c) key[4 * r + c] = i + c < nc ? score_key(v[c]) : 0xffffffffu;
  }
  wg_select_blocks<NT, KPT>(key, nc, a.budget, s_sel, s_lb);
  const int head = r * a.budget;
  const int len = head + (t + 1) - r * nc;
  for (int i = tid; i < a.top_k; i += NT) {
    int v;
    if (i < head) {
      const int j = r == 4 ? i >> 2 : i / r;
      v = r * (int)s_lb[j] + (i - r * j);
    } else {
      v = i < len ? r * nc + (i - head) : -1;
    }
    out[i] = v;
  }
}

// ---------------------------------------------------------------------------
// Decode B1 + B2 in one kernel.  A workgroup of four waves takes 128 blocks
// (kDecScoreTiles tiles of 16 per wave) of one sequence, position
// p = ctx - 1:
//   * every wave issues the kbar tail loads of its blocks (V-row tails of
//     tokens ratio*g) first, so that they are in flight during the rest;
//   * wave h < Hi prepares query head h at p (fp64, one rounding to fp32)
//     into LDS -- each workgroup does this for itself, which costs less
//     than a launch of its own;
//   * B1's pool update: when the context length closes a block (ctx mod
//     ratio == 0), the workgroup holding that block pools it from the raw
//     K-row tails of its first ratio-1 tokens plus the new key, stores kbar
//     in the V-row tail of its first token and scores with that value (the
//     tail it loaded is the stale one); otherwise the first workgroup of the
//     sequence stores the new raw key in token p's K-row tail;
//   * the MFMA scoring: A = kbar rows (rows = blocks), B = query pieces
//     (columns = heads), the relus of the heads summed across lanes.
// Nothing else reads or writes the tails this step touches.
// ---------------------------------------------------------------------------
#ifndef QSA_DEC_SCORE_WAVES
#define QSA_DEC_SCORE_WAVES 4
#endif
constexpr int kDecScoreWaves = QSA_DEC_SCORE_WAVES;

template <int DT>
__global__ __launch_bounds__(64 * kDecScoreWaves) __attribute__((amdgpu_waves_per_eu(5))) void idx_dec_score_kernel(
    IdxDecScoreArgs a) {
  constexpr int NP = kQPieces;
  constexpr int TPW = kScoreTilesPerWave;
  __shared__ __align__(16) uint16_t s_qp[4][kQPieces][128];  // query heads as fp16 scoring pieces
  __shared__ __align__(16) uint16_t s_kb[128];
  const RopeLane rl = rope_lane(a.freq, a.rot);
  const int lane = lane_id(), q4 = lane >> 4, r16 = lane & 15;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.x / a.wg_per_seq, wg = blockIdx.x % a.wg_per_seq;
  const int wg_begin = wg * kDecScoreWaves * TPW * 16;
  const int g_begin = wg_begin + wv * TPW * 16;
  const int32_t *ptk = a.pt + (size_t)b * 2 * a.max_pages;
  const int32_t *ptv = ptk + a.max_pages;
  // Loads in the order they are needed (they return in order): the context
  // length; the page-table entries of this wave's blocks (one round trip
  // before the tail loads instead of two); the inputs of query head wv, which
  // the fp64 prep below works on while the tails are in flight (issued after
  // the tails, the prep would wait for all of them).
  const int ctx_raw = a.ctx[b];
  int pte[TPW];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) pte[tt] = ptv[min((a.ratio * (g_begin + tt * 16 + r16)) >> 7, a.max_pages - 1)];
  const size_t qoff = ((size_t)b * a.Hi + min(wv, a.Hi - 1)) * 128;
  const uint32_t qx0 = a.idx_q[qoff + lane], qx1 = a.idx_q[qoff + 64 + lane];
  const float wq0 = a.wq[lane], wq1 = a.wq[lane + 64];
  const int ctx = min(ctx_raw, a.max_pages * 128);
  if (ctx <= 0) return;
  const int p = ctx - 1;
  const int nc = ctx / a.ratio;
  const bool closes = ctx % a.ratio == 0;
  if (wg == 0 && !closes && wv == kDecScoreWaves - 1) {
    // the new token's block stays open: its raw key goes to its K-row tail
    const long long o = pool_row_off(ptk, p, a.max_pages, a.num_flat_pages, a.Hkv, a.PHD);
    if (o >= 0) {
      a.pool[o + a.D + lane] = a.idx_k[(size_t)b * 128 + lane];
      a.pool[o + a.D + 64 + lane] = a.idx_k[(size_t)b * 128 + 64 + lane];
    }
  }
  if (wg_begin >= nc) return;  // uniform over the workgroup

  // kbar tail loads of this wave's blocks, issued before anything else
  u32x4 kb[TPW][4];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int g = g_begin + tt * 16 + r16;
    const int tok = a.ratio * g;
    long long o = 0;
    if (g < nc && (tok >> 7) < a.max_pages && (unsigned)pte[tt] < (unsigned)a.num_flat_pages)
      o = (((long long)pte[tt] * 128 + (tok & 127)) * a.Hkv) * a.PHD;
    const uint16_t *src = a.pool + o + a.D + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kb[tt][ks] = ld16(src + 32 * ks);
  }

  // query head wv at position p
  if (wv < a.Hi) {
    const Rope2 r = rope_at((double)p, rl, a.rot);
    double o0, o1;
    norm_rope2(bits_to_f64(qx0, a.dt), bits_to_f64(qx1, a.dt), (double)wq0, (double)wq1, a.eps, a.rot, r, o0, o1);
    // rounded once to fp32 and split into the pieces here, once per head
    // (every wave reads every head's pieces below)
    store_q_pieces(&s_qp[wv][0][lane], (float)o0);
    store_q_pieces(&s_qp[wv][0][lane + 64], (float)o1);
  }
  // the block this step completes, when this workgroup holds it
  const int g_new = nc - 1;
  const bool pool_new = closes && g_new >= wg_begin && g_new < wg_begin + kDecScoreWaves * TPW * 16;
  if (pool_new && wv == (g_new - wg_begin) / (TPW * 16)) {
    const int base = a.ratio * g_new;
    double m0 = 0.0, m1 = 0.0;
    bool ok = true;
    for (int j = 0; j < a.ratio - 1; ++j) {
      const long long o = pool_row_off(ptk, base + j, a.max_pages, a.num_flat_pages, a.Hkv, a.PHD);
      ok = ok && o >= 0;
      if (o >= 0) {
        m0 += bits_to_f64(a.pool[o + a.D + lane], a.dt);
        m1 += bits_to_f64(a.pool[o + a.D + 64 + lane], a.dt);
      }
    }
    m0 += bits_to_f64(a.idx_k[(size_t)b * 128 + lane], a.dt);
    m1 += bits_to_f64(a.idx_k[(size_t)b * 128 + 64 + lane], a.dt);
    m0 /= (double)a.ratio;
    m1 /= (double)a.ratio;
    const Rope2 r = rope_at((double)base, rl, a.rot);
    double o0, o1;
    norm_rope2(m0, m1, (double)a.wk[lane], (double)a.wk[lane + 64], a.eps, a.rot, r, o0, o1);
    const uint16_t k0 = (uint16_t)f64_to_bits(o0, a.dt), k1 = (uint16_t)f64_to_bits(o1, a.dt);
    s_kb[lane] = k0;
    s_kb[lane + 64] = k1;
    const long long ov = pool_row_off(ptv, base, a.max_pages, a.num_flat_pages, a.Hkv, a.PHD);
    if (ok && ov >= 0) {
      a.pool[ov + a.D + lane] = k0;
      a.pool[ov + a.D + 64 + lane] = k1;
    }
  }
  __syncthreads();  // queries (and the new kbar) are in LDS
  if (g_begin >= nc) return;
  if (pool_new) {
    // the lanes that hold block g_new score it with the value just pooled
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
      if (g_begin + tt * 16 + r16 == g_new)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kb[tt][ks] = *reinterpret_cast<const u32x4 *>(&s_kb[32 * ks + 8 * q4]);
  }

  u32x4 qb[NP][4];
  const bool head_ok = r16 < a.Hi;
  const int hq = min(r16, a.Hi - 1);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const u32x4 v = *reinterpret_cast<const u32x4 *>(&s_qp[hq][pp][32 * ks + 8 * q4]);
      qb[pp][ks] = head_ok ? v : u32x4{0u, 0u, 0u, 0u};
    }
  float *srow = a.scores + (size_t)b * a.stride;
  f32x4 accs[TPW][2];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) accs[tt][0] = accs[tt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int pp = 0; pp < NP; ++pp)
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt)
        accs[tt][ks & 1] = mfma16x16x32<DT_F16>(kbar_operand<DT>(kb[tt][ks]), qb[pp][ks], accs[tt][ks & 1]);
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const f32x4 acc = accs[tt][0] + accs[tt][1];
    float v[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      float sc = fmaxf(acc[rr], 0.f);
      sc += shfl_xor_f(sc, 1);
      sc += shfl_xor_f(sc, 2);
      v[rr] = sc;
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
hipError_t launch_idx_prep(const IdxPrepArgs &a_in, hipStream_t s) {
  IdxPrepArgs a = a_in;
  fill_freq(a.freq, a.rot, a.theta);
  const long long nrows = (long long)a.B * a.S, nblocks = (long long)a.B * a.Gmax;
  a.per_wave = (int)std::min<long long>(kPrepItemsPerWave, std::max<long long>(1, (nrows + nblocks) / 8192));
  const long long waves = (nrows + a.per_wave - 1) / a.per_wave + (nblocks + a.per_wave - 1) / a.per_wave;
  hipLaunchKernelGGL(idx_prep_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_idx_handoff(const IdxPrepArgs &a, hipStream_t s) {
  if (!a.pool) return hipSuccess;
  const long long waves = (long long)a.B * (a.Gmax + 1);
  hipLaunchKernelGGL(idx_handoff_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_idx_score(const IdxScoreArgs &a_in, int dt, hipStream_t s) {
  IdxScoreArgs a = a_in;
  const int chunks = max(1, (a.Gmax + kScoreChunk - 1) / kScoreChunk);
  const long long groups = (long long)a.B * ((a.S + 31) / 32);
  int run = groups >= kScoreWholeRowGroups && chunks <= kScoreWholeRowChunks ? chunks : kScoreRun;
  // halved until ~2048 workgroups (8 waves per CU)
  while (run > 1 && groups * ((chunks + run - 1) / run) < 2048) run >>= 1;
  a.run_chunks = run;
  a.nchunk = (chunks + run - 1) / run;
  // per XCD: B sequences x ceil(levels / 8) groups, nchunk runs each
  const long long per_xcd = (long long)a.B * ((((a.S + 31) / 32) + 7) / 8);
  const unsigned grid = (unsigned)(8 * per_xcd * a.nchunk);
  if (dt == DT_F16) hipLaunchKernelGGL(idx_score_kernel<DT_F16>, dim3(grid), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(idx_score_kernel<DT_BF16>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int KPL, int NW>
static void launch_select_rows(IdxSelectArgs a, int row0, int nrows, hipStream_t s) {
  if (nrows <= 0) return;
  a.row0 = row0;
  a.nrows = nrows;
  // a staged list: the kept block indices, 16 bits each, in whole 4-byte words
  const int list_words = ((a.budget + 1) / 2 + 3) & ~3;
  bool stage;
  unsigned grid, block;
  if (NW == 1) {  // lists staged over the histogram when they fit with the flags, else written straight out
    stage = list_words + 16 * (KPL / 4) <= sel_rows_hist_words(KPL, 1);
    a.list_words = list_words;
    a.wave_words = sel_rows_hist_words(KPL, 1) + kSelTrash;
    grid = (unsigned)(((nrows + 3) / 4 + 7) & ~7);  // whole sets of eight (xcd_spread)
    block = 256;
  } else {        // [histogram | second histogram | list0 | list1]; two waves only when both lists fit
    stage = true;
    a.list_words = list_words;
    a.wave_words = kSelHistWords + kSelTrash + kSelSmallWords + kSelTrash + 2 * list_words;
    grid = (unsigned)((nrows + 7) & ~7);
    block = 128;
  }
  const size_t lds = (size_t)(NW == 1 ? 4 : 1) * a.wave_words * sizeof(uint32_t);
  const void *fn = stage ? reinterpret_cast<const void *>(&idx_select_rows_kernel<KPL, NW, true>)
                         : reinterpret_cast<const void *>(&idx_select_rows_kernel<KPL, NW, false>);
  if (lds > 65536) (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (stage) hipLaunchKernelGGL((idx_select_rows_kernel<KPL, NW, true>), dim3(grid), dim3(block), lds, s, a);
  else hipLaunchKernelGGL((idx_select_rows_kernel<KPL, NW, false>), dim3(grid), dim3(block), lds, s, a);
}

template <int KPT>
static void launch_select_wg(IdxSelectArgs a, int row0, unsigned rows, hipStream_t s) {
  if (rows == 0) return;
  a.row0 = row0;
  a.nrows = (int)rows;
  // the kept block list: fewer than QSA_MAX_BLOCKS entries of 16 bits
  const size_t lds = (size_t)std::min(a.budget, QSA_MAX_BLOCKS) * sizeof(uint16_t);
  const void *fn = reinterpret_cast<const void *>(&idx_select_wg_kernel<KPT>);
  if (lds + sizeof(WgSelLds<kSelWgThreads>) > 65536)
    (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  // decode: one workgroup per sequence; prefill and chunk rows: whole sets
  // of eight workgroups (xcd_spread)
  const unsigned grid = a.decode ? rows : ((rows + 7u) & ~7u);
  hipLaunchKernelGGL((idx_select_wg_kernel<KPT>), dim3(grid), dim3(kSelWgThreads), lds, s, a);
}

static void launch_select_wg_for(const IdxSelectArgs &a, int nc_max, int row0, unsigned rows, hipStream_t s) {
  // one workgroup per row; at most QSA_MAX_BLOCKS = 32 * 1024 blocks
  const int kpt = (nc_max + kSelWgThreads - 1) / kSelWgThreads;
  if (kpt <= 4) launch_select_wg<4>(a, row0, rows, s);
  else if (kpt <= 8) launch_select_wg<8>(a, row0, rows, s);
  else if (kpt <= 16) launch_select_wg<16>(a, row0, rows, s);
  else launch_select_wg<32>(a, row0, rows, s);
}

hipError_t launch_idx_select(const IdxSelectArgs &a, int nc_max, hipStream_t s) {
  if (a.decode) {
    launch_select_wg_for(a, nc_max, 0, (unsigned)a.B, s);
    return hipGetLastError();
  }
  if (a.start) {
    // Chunk rows: their positions are device data, so the host cannot sort
    // them into length classes.  The two-wave per-row kernel runs over every
    // row and takes those of up to 8192 blocks; when the pool can hold
    // longer rows, the workgroup kernel runs over every row as well and
    // takes only those.
    const int total = (int)((long long)a.B * a.S);
    const int list_words = (a.budget * a.ratio + 3) & ~3;
    constexpr int kTwoWaveBlocks = 2 * 64 * 64;
    if (list_words <= 4096) {
      launch_select_rows<64, 2>(a, 0, total, s);
      if (nc_max > kTwoWaveBlocks) {
        IdxSelectArgs w = a;
        w.wg_min_nc = kTwoWaveBlocks;
        launch_select_wg_for(w, nc_max, 0, (unsigned)total, s);
      }
    } else {
      launch_select_wg_for(a, nc_max, 0, (unsigned)total, s);
    }
    return hipGetLastError();
  }
  // Prefill rows go longest first (row = (S - 1 - t) * B + b), so rows whose
  // complete-block count nc = (t + 1) / ratio exceeds K are the first
  // rows_from(K) rows.  Each length class gets the kernel that fits it.
  const long long total = (long long)a.B * a.S;
  auto rows_from = [&](long long k) -> int {  // rows with nc > k, i.e. t >= (k + 1) * ratio - 1
    const long long t0 = (k + 1) * a.ratio - 1;
    return (int)(t0 >= a.S ? 0 : (t0 <= 0 ? total : (long long)a.B * (a.S - t0)));
  };
  const int n_wg = rows_from(64 * 128);           // > 8192 blocks: a 1024-thread workgroup per row
  // 4097..8192 blocks: two waves of 64 keys per lane when both lists fit in
  // LDS (measured ~12 % faster than one wave of 128 on such rows; on shorter
  // rows the two-wave barriers cost more than the occupancy gains), else one
  // wave of 128; 2049..4096: one wave of 64; 1025..2048: one wave of 32; the
  // rest: one wave of 16 (fewer registers, so a short prefill's rows all run
  // at once).
  const int list_words = (a.budget * a.ratio + 3) & ~3;  // expanded ids of one list
  const int n_long = rows_from(64 * 64) - n_wg;
  const int n64 = rows_from(64 * 32) - n_wg - n_long;
  const int n32 = rows_from(64 * 16) - n_wg - n_long - n64;
  const int n16 = (int)total - n_wg - n_long - n64 - n32;
  launch_select_wg_for(a, nc_max, 0, (unsigned)n_wg, s);
  if (list_words <= 4096) launch_select_rows<64, 2>(a, n_wg, n_long, s);
  else launch_select_rows<128, 1>(a, n_wg, n_long, s);
  launch_select_rows<64, 1>(a, n_wg + n_long, n64, s);
  launch_select_rows<32, 1>(a, n_wg + n_long + n64, n32, s);
  launch_select_rows<16, 1>(a, n_wg + n_long + n64 + n32, n16, s);
  return hipGetLastError();
}

hipError_t launch_idx_chunk_prep(const IdxChunkPrepArgs &a_in, hipStream_t s) {
  IdxChunkPrepArgs a = a_in;
  fill_freq(a.freq, a.rot, a.theta);
  const long long waves = (long long)a.B * ((long long)a.C + a.Gmax + 1);
  hipLaunchKernelGGL(idx_chunk_prep_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_idx_dec_score(const IdxDecScoreArgs &a_in, int dt, hipStream_t s) {
  IdxDecScoreArgs a = a_in;
  fill_freq(a.freq, a.rot, a.theta);
  const int per_wg = kDecScoreWaves * kScoreTilesPerWave * 16;
  a.wg_per_seq = (a.gmax + per_wg - 1) / per_wg;
  if (a.wg_per_seq < 1) a.wg_per_seq = 1;  // the first workgroup also writes the open block's raw tail
  const unsigned grid = (unsigned)((long long)a.B * a.wg_per_seq);
  if (dt == DT_F16) hipLaunchKernelGGL(idx_dec_score_kernel<DT_F16>, dim3(grid), dim3(64 * kDecScoreWaves), 0, s, a);
  else hipLaunchKernelGGL(idx_dec_score_kernel<DT_BF16>, dim3(grid), dim3(64 * kDecScoreWaves), 0, s, a);
  return hipGetLastError();
}

}  // namespace qsa
