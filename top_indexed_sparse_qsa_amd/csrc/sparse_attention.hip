// Sparse GQA attention over index lists, prefill (dense BSND K/V): the list
// walk and the list tiles.  The per-chunk machinery shared with decode is in
// attention_core.h.
//
// Prefill rows whose lists cover most of their causal prefix (all of them
// before the budget fills) run as list tiles instead of the list walk: a
// workgroup of four waves takes several consecutive rows of one KV head,
// turns their lists into a per-row key mask in LDS, and walks the keys of the
// prefix densely, each 32-key chunk of K and V staged once in LDS for all its
// (row, head) columns (see "Tiles" below).
#include <math.h>

#include <atomic>

#include "attention_core.h"
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

// Tiles.  Where a row's list covers a large part of its causal prefix —
// before the budget fills (t < top_k) it is the whole prefix, and at short
// lengths it is half or more of it — walking all of the prefix densely with
// a key mask is cheaper than gathering the listed rows: the gathers are
// bound by on-chip gather throughput, the dense walk by MFMA and LDS.  A
// tile workgroup takes 4 * NT * 16 / Gp consecutive rows of one (sequence,
// KV head) (Gp = G rounded up to a power of two, G >= 4; NT 16-column MFMA
// tiles per wave: 16 rows at G = 4, 8 at G = 8 and at G = 16) and packs the
// (row, head) pairs as MFMA columns (column r16 of a tile = head r16 % Gp
// of row r16 / Gp).
//
// First the rows' lists become a key bitmask in LDS (one bit per key of
// [0, t_act) per row, set by LDS atomic-or), read like the walk reads them:
// up to the first 32-slot chunk with no usable id.  The mask reproduces
// exactly the keys the list walk would use, or the tile gives up: an id
// repeated in a list or a key at or past t_act (outside the causal range)
// sends the tile's rows to a cooperative list walk, one row at a time (all
// four waves stage each chunk; lists that break the contract only).
//
// Then the workgroup walks the keys once: every 32-key chunk of K and V is
// gathered once into a double-buffered LDS tile (two chunks in flight in
// registers, one barrier per chunk) and read by all four waves; the K and V
// fragments serve every column tile of a wave; a wave whose columns have no
// key in a chunk skips it, and the mask is applied only where some column
// misses a key.
__host__ __device__ constexpr int tile_heads(int G) { return G <= 4 ? 4 : G <= 8 ? 8 : 16; }
// 16-column MFMA tiles per wave: one (128 VGPRs, four waves per SIMD),
// except at Gp = 16 where a column tile is a single row and two per wave
// (186 VGPRs, two waves per SIMD) keep eight rows per tile.  At Gp = 8 the
// launcher also takes two when the launch has tiles for several rounds
// (two per wave read each K and V fragment once for both: half the LDS
// traffic per column).
__host__ __device__ constexpr int tile_nt(int G) { return tile_heads(G) == 16 ? 2 : 1; }
// rows per tile: 4 * NT 16-column tiles of 16 / Gp rows each (G >= 4 only)
__host__ __device__ constexpr int tile_rows_nt(int G, int nt) { return 4 * nt * (16 / tile_heads(G)); }
// key-mask words of a tile workgroup (rows x 32-key chunks of the tile
// range), at most 16 KB of LDS, which bounds the tiled rows to
// t < 32 * kTileMaskWords / rows per tile.  The launch sizes it to its tile
// range: 4 KB at 4096 rows and eight rows per tile, so that with the 34 KB of
// K/V staging four workgroups fit a CU's 160 KB.
constexpr int kTileMaskWords = 4096;

struct TileStage {
  u32x4 k[2], v[2];  // K and V rows srow and 16 + srow of the chunk, one piece each
};

// LDS of a tile workgroup: K chunks with 16-byte pieces XOR-swizzled by row
// (conflict-free row writes and fragment reads), V chunks row-major with
// rows padded to 288 bytes, so that the transposing reads that build V^T
// (lds_tr16) hit distinct banks and step through d by immediate offsets.
constexpr int kTileVRowPieces = 18;
struct TileLds {
  u32x4 k[2][32 * 16];
  u32x4 v[2][32 * kTileVRowPieces];
};

typedef short s16x4_t __attribute__((ext_vector_type(4)));
// gfx950 transposing LDS read of 16-bit elements: within each 16-lane group,
// lane 4a + b gets element b of the 8-byte chunks addressed by lanes a,
// a + 4, a + 8 and a + 12 of the group.
__device__ __forceinline__ s16x4_t lds_tr16(const char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t *)(p));
}

// Output of the lane's column from accumulators in the tile layout (acc[e][i]
// holds output dim 16 e + 4 q4 + i): O = acc / l, or +0.0 for rows past the
// live length.  dst points at the column's (row, head) output row.
template <int D, int DT>
__device__ __forceinline__ void store_column_tr(uint16_t *dst, const f32x4 (&acc)[8], float l_run, bool write,
                                                bool zero) {
  const int q4 = lane_id() >> 4;
  float l = l_run + shfl_xor_f(l_run, 16);
  l += shfl_xor_f(l, 32);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (write) {
#pragma unroll
    for (int e = 0; e < D / 16; ++e) {
      uint2 w;
      w.x = zero ? 0u : pack2<DT>(acc[e][0] * inv, acc[e][1] * inv);
      w.y = zero ? 0u : pack2<DT>(acc[e][2] * inv, acc[e][3] * inv);
      *reinterpret_cast<uint2 *>(dst + 16 * e + 4 * q4) = w;
    }
  }
}

// Output of the lane's column: O = acc / l, or +0.0 for rows past the live
// length (their accumulators may hold values, times 0 they could give -0.0).
// dst points at the column's (row, head) output row.
template <int D, int DT>
__device__ __forceinline__ void store_column(uint16_t *dst, const f32x4 (&acc)[8], float l_run, bool write,
                                             bool zero) {
  const int q4 = lane_id() >> 4;
  float l = l_run + shfl_xor_f(l_run, 16);
  l += shfl_xor_f(l, 32);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (write && 32 * q4 < D) {
    dst += 32 * q4;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      u32x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = zero ? 0u : pack2<DT>(acc[2 * j][rr] * inv, acc[2 * j + 1][rr] * inv);
      st16(dst + 8 * rr, w);
    }
  }
}

// The key mask of the tile's live rows [t0, t_act): row r's words are
// s_mask[r * W .. r * W + W).  Returns (on every lane of a wave that found
// it) true when the lists need the walk.  Wave w builds rows w, w + 4, ...,
// two rows at a time: lane l reads slot quads l + 64 k of each row (16-byte
// loads; list rows are only 4-byte aligned, which global loads accept),
// kBuildLoads loads per row in flight, and sets its usable ids' bits with
// non-returning LDS or (one per quad when its ids share a 32-bit word, as
// the indexer's 4-key blocks do).  A row is read in order up to its first
// 32-slot chunk with no usable id (lanes 8m .. 8m + 7 of a load hold chunk
// m of its 8), where the walk stops too: the ids before it are the row's
// keys and nothing after it is read.  No key may lie at or past t_act, and
// after a barrier the row's mask must hold as many bits as the row has keys
// (a repeated id sets one bit twice).
constexpr int kBuildLoads = 5;  // 2051 slots: two rounds

__device__ __forceinline__ bool build_key_mask(const PrefillAttnArgs &a, int b, int t0, int t_act, int live, int W,
                                               uint32_t *s_mask, int *s_cnt) {
  typedef int i32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
  const int lane = lane_id(), tid = threadIdx.x, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nr = t_act - t0;
  const int nload = (a.top_k + 255) >> 8;  // 64 quads = 8 chunks per load
  const int nchunk = (a.top_k + 31) >> 5;
  for (int i = tid; i < nr * W; i += 256) s_mask[i] = 0u;
  __syncthreads();
  bool bad = false;
  for (int r = wv; r < nr; r += 8) {
    const int rr[2] = {r, min(r + 4, nr - 1)};
    const int32_t *row[2];
    int cnt[2] = {0, 0};            // this lane's keys per row
    bool open[2] = {true, r + 4 < nr};  // still reading (wave-uniform)
#pragma unroll
    for (int j = 0; j < 2; ++j) row[j] = a.indices + ((size_t)b * a.S + t0 + rr[j]) * a.top_k;
    for (int k0 = 0; k0 < nload && (open[0] || open[1]); k0 += kBuildLoads) {
      // both rows' loads are issued before either is used (clamped: what
      // lies past the list or a closed row is dropped)
      i32x4_a4 v[2][kBuildLoads];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int k = 0; k < kBuildLoads; ++k)
          v[j][k] = *reinterpret_cast<const i32x4_a4 *>(row[j] + min(4 * (64 * (k0 + k) + lane), a.top_k - 4));
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (!open[j]) continue;
#pragma unroll
        for (int k = 0; k < kBuildLoads; ++k) {
          const int kk = k0 + k;
          if (kk >= nload) break;
          const int q = 64 * kk + lane;
          const int s0 = min(4 * q, a.top_k - 4);  // slot of v[j][k].x
          bool u[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // a slot counts once: only in the quad it belongs to (4q .. 4q+3)
            const int sl = s0 + e;
            u[e] = (sl >= 4 * q) & (sl < a.top_k) & ((unsigned)v[j][k][e] < (unsigned)live);
          }
          // bit 8m of f: chunk 8 kk + m holds a usable id
          uint64_t f = __ballot(u[0] | u[1] | u[2] | u[3]);
          f |= f >> 4;
          f |= f >> 2;
          f |= f >> 1;
          const int nex = min(8, nchunk - 8 * kk);  // chunks of the list in this load
          const uint64_t gap = ~f & 0x0101010101010101ull & (nex == 8 ? ~0ull : (1ull << (8 * nex)) - 1);
          if (gap != 0ull) {
            // the list ends before chunk 8 kk + m
            const bool keep = lane < (__builtin_ctzll(gap) & ~7);
#pragma unroll
            for (int e = 0; e < 4; ++e) u[e] &= keep;
            open[j] = false;
          }
          uint32_t bits = 0u;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int id = v[j][k][e];
            cnt[j] += u[e] ? 1 : 0;
            bad |= u[e] & (id >= t_act);
            bits |= (u[e] & (id < t_act)) ? 1u << (id & 31) : 0u;
          }
          const int id0 = v[j][k][0];
          const bool one_word = ((!u[1]) | ((v[j][k][1] >> 5) == (id0 >> 5))) &
                                ((!u[2]) | ((v[j][k][2] >> 5) == (id0 >> 5))) &
                                ((!u[3]) | ((v[j][k][3] >> 5) == (id0 >> 5)));
          uint32_t *mrow = s_mask + rr[j] * W;
          if (u[0] & one_word) {
            if (bits != 0u) __hip_atomic_fetch_or(&mrow[id0 >> 5], bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int id = v[j][k][e];
              if (u[e] & (id < t_act))
                __hip_atomic_fetch_or(&mrow[id >> 5], 1u << (id & 31), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
          }
          if (!open[j]) break;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) cnt[j] += __shfl_xor(cnt[j], o, 64);
    }
    if (lane == 0) {
      s_cnt[r] = cnt[0];
      if (r + 4 < nr) s_cnt[r + 4] = cnt[1];
    }
  }
  __syncthreads();
  for (int r = wv; r < nr; r += 4) {
    int bits = 0;
    for (int w = lane; w < W; w += 64) bits += __builtin_popcount(s_mask[r * W + w]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) bits += __shfl_xor(bits, o, 64);
    bad |= bits != s_cnt[r];
  }
  return bad;
}

// Returns false when the tile's lists need the list walk; nothing is written then.
template <int D, int DT, int NT>
__device__ bool list_tile(const PrefillAttnArgs &a, int b, int kvh, int t0, TileLds &L, uint32_t *s_mask, int *s_cnt,
                          int *s_flag) {
  const int lane = lane_id(), q4 = lane >> 4, r16 = lane & 15;
  const int tid = threadIdx.x, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Gp = tile_heads(a.G), RP = 16 / Gp, R = 4 * NT * RP;
  const int live = min(a.ctx[b], a.S);
  const int t_end = min(t0 + R, a.tile_below);  // the tile's rows are [t0, t_end)
  const int t_act = min(t_end, live);           // of which [t0, t_act) are live
  DenseKV kv;
  kv.k = reinterpret_cast<const char *>(a.k + ((size_t)b * a.S * a.Hkv + kvh) * D);
  kv.v = reinterpret_cast<const char *>(a.v + ((size_t)b * a.S * a.Hkv + kvh) * D);
  kv.row_bytes = (uint32_t)(a.Hkv * D * 2);
  kv.limit = live;

  // columns: tile u of this wave holds local row (2 wv + u) RP + r16 / Gp
  const int h = r16 & (Gp - 1);
  int r_col[NT];
  bool col_live[NT];
  u32x4 qp[NT][D / 32];
  f32x4 acc[NT][8];
  float m_run[NT], l_run[NT];
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    r_col[u] = (NT * wv + u) * RP + r16 / Gp;
    col_live[u] = h < a.G && t0 + r_col[u] < t_act;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[u][e] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[u] = -INFINITY;
    l_run[u] = 0.f;
  }

  bool fail = false;
  if (t_act > t0) {
    const int W = (t_act + 31) >> 5;  // 32-key chunks of [0, t_act), mask words per row
    const bool wave_bad = wave_any(build_key_mask(a, b, t0, t_act, live, W, s_mask, s_cnt));
    if (lane == 0) s_flag[wv] = wave_bad ? 1 : 0;
    __syncthreads();
    // uniform by construction; readfirstlane lets the compiler branch on it
    // instead of running both sides under a lane mask
    fail = __builtin_amdgcn_readfirstlane(s_flag[0] | s_flag[1] | s_flag[2] | s_flag[3]) != 0;
  }
  if (!fail && t_act > t0) {
    const int W = (t_act + 31) >> 5, nch = W;
    // Q after the mask build, so that it does not stay live through it
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      // unconditional loads: a dead column (past the sequence, or a head
      // past G) reads a clamped row and head of this KV head's group
      const uint16_t *qh =
          a.q + (((size_t)b * a.S + min(t0 + r_col[u], a.S - 1)) * a.Hq + (size_t)kvh * a.G + min(h, a.G - 1)) * D;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        const u32x4 v = ld16(qh + 32 * ks + 8 * q4);
        qp[u][ks] = col_live[u] ? v : u32x4{0u, 0u, 0u, 0u};
      }
    }
    const int srow = tid >> 4, piece = tid & 15;
    // dead columns (zero Q) get no key: with no key seen, a column's
    // probabilities are 0 (chunk_probs<.., true>)
    const uint32_t *mrow[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) mrow[u] = s_mask + min(r_col[u], t_act - t0 - 1) * W;
    // Every load is unconditional (clamped addresses; what lies past the
    // keys is dropped): the waits then count exactly.
    auto issue = [&](TileStage &st, int c) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int id = min(32 * c + 16 * hh + srow, t_act - 1);
        if (D == 128 || piece < D / 8) kv.load(id, piece, st.k[hh], st.v[hh]);
      }
    };
    auto store = [&](const TileStage &st, int buf) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int row = 16 * hh + srow;
        if (D == 128 || piece < D / 8) {
          L.k[buf][row * 16 + (piece ^ (row & 15))] = st.k[hh];
          L.v[buf][row * kTileVRowPieces + piece] = st.v[hh];
        }
      }
    };
    // V^T operand of accumulator e, two transposing reads: lane i = a + 4R of
    // group q4 points at V[key slot 4 q4 + R][16 e + 4 a] (key slot
    // 16 + 4 q4 + R for the second read), so lane j of the group gets
    // V[key slots 4 q4 .. 4 q4 + 3][16 e + j]: MFMA A element (m = j,
    // k = 8 q4 + i) is V[key slot slot_of(q4, i)][16 e + j], the key order of
    // the P operand.  Accumulator e then holds output dims 16 e + 4 q4 + i.
    const int v_lane = (4 * q4 + (r16 >> 2)) * (16 * kTileVRowPieces) + (r16 & 3) * 8;
    auto compute = [&](int c, int buf) {
      uint32_t word[NT];
#pragma unroll
      for (int u = 0; u < NT; ++u) word[u] = col_live[u] ? mrow[u][c] : 0u;
      uint32_t any_w = 0u, all_w = 0xffffffffu;
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        any_w |= word[u];
        all_w &= word[u];
      }
      if (!wave_any(any_w != 0u)) return;  // no column of this wave has a key here
      const u32x4 *kt = L.k[buf];
      f32x4 s0[NT], s1[NT];
#pragma unroll
      for (int u = 0; u < NT; ++u) s0[u] = s1[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        const u32x4 k0 = kt[r16 * 16 + ((4 * ks + q4) ^ r16)];
        const u32x4 k1 = kt[(16 + r16) * 16 + ((4 * ks + q4) ^ r16)];
#pragma unroll
        for (int u = 0; u < NT; ++u) {
          s0[u] = mfma16x16x32<DT>(k0, qp[u][ks], s0[u]);
          s1[u] = mfma16x16x32<DT>(k1, qp[u][ks], s1[u]);
        }
      }
      const bool full = !wave_any(all_w != 0xffffffffu);  // every column sees every key
      u32x4 bop[NT];
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[i] = s0[u][i];
          x[4 + i] = s1[u][i];
        }
        if (!full) {
          // key slot slot_of(q4, i) = 4 q4 + i (i < 4), 12 + 4 q4 + i: shift
          // once by 4 q4, then by constants
          // and a signed one-bit extract is the select mask (0 or ~0):
          // x or -inf is one bitwise select per score
          const int wq = (int)(word[u] >> (4 * q4));
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t m = (uint32_t)__builtin_amdgcn_sbfe(wq, i < 4 ? i : 12 + i, 1);
            x[i] = __uint_as_float((__float_as_uint(x[i]) & m) | (0xff800000u & ~m));
          }
        }
        bop[u] = chunk_probs<DT, true>(x, a.sl2, m_run[u], l_run[u], acc[u]);
      }
      const char *vb = reinterpret_cast<const char *>(L.v[buf]) + v_lane;
#pragma unroll
      for (int e = 0; e < D / 16; ++e) {
        const s16x4_t lo = lds_tr16(vb + 32 * e), hi = lds_tr16(vb + 16 * 16 * kTileVRowPieces + 32 * e);
        const u32x4 av = {__builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 0, 1)),
                          __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 2, 3)),
                          __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 0, 1)),
                          __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 2, 3))};
#pragma unroll
        for (int u = 0; u < NT; ++u) acc[u][e] = mfma16x16x32<DT>(av, bop[u], acc[u][e]);
      }
    };

    // Buffer 0 holds even chunks, buffer 1 odd ones; a buffer is refilled
    // only after the barrier that follows every wave's last read of it.
    TileStage sa, sb;
    issue(sa, 0);
    issue(sb, 1);
    store(sa, 0);
    issue(sa, 2);
    __syncthreads();
    for (int c = 0;; c += 2) {
      // buffer 0: chunk c; in flight: sb = chunk c + 1, sa = chunk c + 2
      compute(c, 0);
      if (c + 1 >= nch) break;
      store(sb, 1);
      issue(sb, c + 3);
      __syncthreads();
      compute(c + 1, 1);
      if (c + 2 >= nch) break;
      store(sa, 0);
      issue(sa, c + 4);
      __syncthreads();
    }
  }
  if (fail) return false;
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int t = t0 + r_col[u];
    uint16_t *dst = a.o + (((size_t)b * a.S + t) * a.Hq + (size_t)kvh * a.G + h) * D;
    store_column_tr<D, DT>(dst, acc[u], l_run[u], h < a.G && t < t_end, !col_live[u]);
  }
  return true;
}

// Work order.  Sequences one after another, and within a sequence rows
// longest-first (row t before row t-1).  Workgroups are dispatched
// round-robin over the eight XCDs, each with its own 4 MB L2.  When Hkv
// divides 8, workgroup w runs on XCD w % 8 and that XCD only ever processes
// KV head (w % 8) % Hkv: its gathers then touch one KV head of one sequence
// at a time, which keeps most gathers in L2 even when K/V outgrow it (every
// list walks its ids in ascending order, so concurrent waves touch nearby
// rows).  A workgroup's four waves take four consecutive rows of that head.
// Otherwise a workgroup takes the Hkv heads of consecutive rows.  Tile
// workgroups (list_tile) go out longest tiles first, with the same
// XCD-to-head mapping, except that the workgroups which start together
// take them in snake order: at launch an XCD hands its n-th workgroup to CU
// n mod (its CU count) until every CU holds as many as fit, so in plain
// order the CU with the longest tile also gets the longest of every later
// round and finishes last; reversing every other round evens the CUs'
// sums (the rest go out in order to whichever CU frees first).
__device__ __forceinline__ bool tile_item(const PrefillAttnArgs &a, int blk, int &b, int &kvh, int &t0) {
  const int ntiles = a.tile_nb * a.tile_per_seq;
  int k;
  if ((8 % a.Hkv) == 0) {
    const int xcd = blk & 7;
    int n = blk >> 3;
    if (n < a.tile_snake) {
      const int round = n / a.tile_cus, c = n - round * a.tile_cus;
      n = round * a.tile_cus + ((round & 1) ? a.tile_cus - 1 - c : c);
    }
    kvh = xcd % a.Hkv;
    k = n * (8 / a.Hkv) + xcd / a.Hkv;
  } else {
    kvh = blk % a.Hkv;
    k = blk / a.Hkv;
  }
  if (k >= ntiles) return false;
  b = a.tile_b0 + k % a.tile_nb;
  t0 = (a.tile_per_seq - 1 - k / a.tile_nb) * a.tile_rows;
  return true;
}

static unsigned tile_grid(const PrefillAttnArgs &a) {
  const long long ntiles = (long long)a.tile_nb * a.tile_per_seq;
  if ((8 % a.Hkv) == 0) {
    const long long per_head = 8 / a.Hkv;
    return (unsigned)(8 * ((ntiles + per_head - 1) / per_head));
  }
  return (unsigned)(ntiles * a.Hkv);
}

__device__ __forceinline__ bool prefill_item(const PrefillAttnArgs &a, int blk, int wave, int &b, int &t, int &kvh) {
  int rest;
  if ((8 % a.Hkv) == 0) {
    const int xcd = blk & 7, n = blk >> 3;
    const int per_head = 8 / a.Hkv;  // XCDs sharing one KV head
    kvh = xcd % a.Hkv;
    rest = ((n * per_head + xcd / a.Hkv) << 2) + wave;
    if (rest >= a.nrows) return false;
  } else {
    const int item = blk * 4 + wave;
    if (item >= a.nrows * a.Hkv) return false;
    kvh = item % a.Hkv;
    rest = item / a.Hkv;
  }
  rest += a.row0;
  b = rest / a.S;
  t = a.S - 1 - rest % a.S;
  return true;
}

static unsigned prefill_grid(const PrefillAttnArgs &a) {
  if ((8 % a.Hkv) == 0) {
    const long long quads = ((long long)a.nrows + 3) / 4;
    const long long per_head = 8 / a.Hkv;
    return (unsigned)(8 * ((quads + per_head - 1) / per_head));
  }
  return (unsigned)(((long long)a.nrows * a.Hkv + 3) / 4);
}

// Every list is walked in ascending id order, so waves that start together
// touch nearby K/V rows at the same time and share them through L2.  When a
// KV head's K/V is well past one XCD's L2, that sharing depends on the waves
// staying in step, and they drift apart over successive generations of
// workgroups; splitting the rows into launches of about kSyncWaves waves
// starts every launch in step again.
constexpr size_t kL2BytesPerXcd = 4u << 20;
#ifndef QSA_PREFILL_SYNC_WAVES
#define QSA_PREFILL_SYNC_WAVES 8192
#endif
constexpr int kSyncWaves = QSA_PREFILL_SYNC_WAVES;

static int prefill_rows_per_launch(const PrefillAttnArgs &a, int D) {
  const int total = a.B * a.S;
  const size_t head_kv_bytes = (size_t)a.S * 2 * D * sizeof(uint16_t);
  if (head_kv_bytes <= 2 * kL2BytesPerXcd) return total;
  return max(64, kSyncWaves / a.Hkv);
}

// One row (sequence b, position t, KV head kvh) on the list walk: Q of the
// head group, the walk, the output (zeros past the live length).
template <int D, int DT>
__device__ __forceinline__ void walk_row(const PrefillAttnArgs &a, int b, int t, int kvh, u32x4 *ktile) {
  const int lane = lane_id(), q4 = lane >> 4, r16 = lane & 15;
  const int live = min(a.ctx[b], a.S);
  DenseKV kv;
  kv.k = reinterpret_cast<const char *>(a.k + ((size_t)b * a.S * a.Hkv + kvh) * D);
  kv.v = reinterpret_cast<const char *>(a.v + ((size_t)b * a.S * a.Hkv + kvh) * D);
  kv.row_bytes = (uint32_t)(a.Hkv * D * 2);
  kv.limit = live;
  f32x4 acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const size_t qo_off = (((size_t)b * a.S + t) * a.Hq + (size_t)kvh * a.G) * D;
  if (t < live) {
    u32x4 qf[D / 32];
    load_q<D>(qf, a.q + qo_off, a.G, q4, r16);
    run_list<D, DT>(a.indices + ((size_t)b * a.S + t) * a.top_k, a.top_k, kv, qf, a.sl2, m_run, l_run, acc, ktile);
  }
  store_column<D, DT>(a.o + qo_off + (size_t)r16 * D, acc, l_run, r16 < a.G, false);
}

// The list walk for rows [t0, t_end) of a tile whose lists the key mask
// cannot represent (a repeated id, or a key at or past the tile's causal
// range): one row at a time, all four waves stage each
// 32-slot chunk's K/V rows in LDS and wave 0 runs the online softmax over
// the usable slots, stopping at the first chunk without one — the list
// walk's result, at the tile's small register budget.  Rare (lists that
// break the contract), so simple rather than fast.
template <int D, int DT>
__device__ void tile_walk_rows(const PrefillAttnArgs &a, int b, int kvh, int t0, int t_end, TileLds &L, int *s_slot) {
  const int lane = lane_id(), q4 = lane >> 4, r16 = lane & 15;
  const int tid = threadIdx.x, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int srow = tid >> 4, piece = tid & 15;
  const int live = min(a.ctx[b], a.S);
  DenseKV kv;
  kv.k = reinterpret_cast<const char *>(a.k + ((size_t)b * a.S * a.Hkv + kvh) * D);
  kv.v = reinterpret_cast<const char *>(a.v + ((size_t)b * a.S * a.Hkv + kvh) * D);
  kv.row_bytes = (uint32_t)(a.Hkv * D * 2);
  kv.limit = live;
  u32x4 *kt = L.k[0], *vt = L.v[0];  // 16-byte pieces XOR-swizzled by row, 16 per row
  for (int t = t0; t < t_end; ++t) {
    const int32_t *list = a.indices + ((size_t)b * a.S + t) * a.top_k;
    const size_t qo_off = (((size_t)b * a.S + t) * a.Hq + (size_t)kvh * a.G) * D;
    f32x4 acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    u32x4 qf[D / 32];
    load_q<D>(qf, a.q + qo_off, a.G, q4, r16);
    for (int c = 0; t < live && 32 * c < a.top_k; ++c) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int slot = 16 * hh + srow, sl = 32 * c + slot;
        const int id = sl < a.top_k ? list[sl] : -1;
        const bool ok = (unsigned)id < (unsigned)live;
        u32x4 kd, vd;
        kv.load(ok ? id : 0, piece, kd, vd);
        if (D == 128 || piece < D / 8) {
          kt[slot * 16 + (piece ^ (slot & 15))] = kd;
          vt[slot * 16 + (piece ^ (slot & 15))] = vd;
        }
        if (piece == 0) s_slot[slot] = ok ? 1 : 0;
      }
      __syncthreads();
      const uint32_t word = (uint32_t)__ballot(s_slot[lane & 31] != 0);  // bit s: slot s usable
      if (word == 0u) break;  // the walk stops at a chunk without usable ids (uniform)
      if (wv == 0) {
        float x[8];
        chunk_scores<D, DT>(kt, qf, x);
        const uint32_t wq = word >> (4 * q4);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (wq >> (i < 4 ? i : 12 + i)) & 1u ? x[i] : -INFINITY;
        const u32x4 bop = chunk_probs<DT, true>(x, a.sl2, m_run, l_run, acc);
        u32x4 vf[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int row = slot_of(q4, i);
          vf[i] = (D == 128 || r16 < D / 8) ? vt[row * 16 + (r16 ^ (row & 15))] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = mfma16x16x32<DT>(v_operand(vf, e), bop, acc[e]);
      }
      __syncthreads();  // the chunk's LDS is consumed
    }
    if (wv == 0) store_column<D, DT>(a.o + qo_off + (size_t)r16 * D, acc, l_run, r16 < a.G, false);
    __syncthreads();
  }
}

// Tile workgroups: one tile each (tile_item), with the register budget of
// the tile alone: four waves per SIMD at NT = 1, when the launch-sized key
// mask leaves LDS for four workgroups per CU (three otherwise).
template <int D, int DT, int NT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NT == 1 ? 4 : 2, NT == 1 ? 4 : 2))) void
sparse_prefill_tile_kernel(PrefillAttnArgs a) {
  __shared__ TileLds s_tile;
  extern __shared__ uint32_t s_mask[];  // tile_rows x ceil(tile_below / 32) words (launch-sized)
  __shared__ int s_cnt[32], s_flag[4];
  int b = 0, kvh = 0, t0 = 0;
  if (!tile_item(a, blockIdx.x, b, kvh, t0)) return;
  if (list_tile<D, DT, NT>(a, b, kvh, t0, s_tile, s_mask, s_cnt, s_flag)) return;
  tile_walk_rows<D, DT>(a, b, kvh, t0, min(t0 + a.tile_rows, a.tile_below), s_tile, s_cnt);
}

// Row workgroups: every wave walks its own list; rows below skip_below
// belong to tiles.
template <int D, int DT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void sparse_prefill_kernel(PrefillAttnArgs a) {
  __shared__ u32x4 s_ktile[4][32 * 16];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int b = 0, t = 0, kvh = 0;
  if (!prefill_item(a, blockIdx.x, wv, b, t, kvh) || t < a.skip_below) return;
  walk_row<D, DT>(a, b, t, kvh, s_ktile[wv]);
}

// Tiles take rows t with t + 1 <= kTileRangeX2 / 2 * top_k * R / 16 (R rows
// per tile, kTileRangeX2 / 2 = 3.5).  At R = 16 a dense walk of a 32-key chunk costs a row ~1/2.6 of
// what gathering 32 listed keys costs the list walk (workload 2: all 4096
// rows as tiles 147 us, the 2045 rows t >= top_k on the walk 188 us for half
// the row-keys); a tile's chunk costs the same for any R, so a row's share
// scales with 1/R, while the walk's cost per row does not depend on G.  The
// break-even measured on whole calls sits higher than that ratio (rows near
// it keep the walk's gathers off L2 for the other rows): 3.5 beat 1.5, 2.5
// and 5 on workloads 3 and 5.
#ifndef QSA_TILE_RANGE_X2
#define QSA_TILE_RANGE_X2 7
#endif
constexpr int kTileRangeX2 = QSA_TILE_RANGE_X2;
// The same for two column tiles per wave at Gp = 8, with a key mask of up to
// 32 KB (two workgroups per CU either way).
#ifndef QSA_TILE_RANGE_X2_WIDE
#define QSA_TILE_RANGE_X2_WIDE 8
#endif
constexpr int kTileRangeX2Wide = QSA_TILE_RANGE_X2_WIDE;
constexpr int kTileMaskWordsWide = 8192;

// CUs per XCD of the current device (its CU count / 8), or 0 when that is
// not a whole number.  A read-only device property, looked up once per
// device; concurrent first calls may both look it up and store the same value.
static int xcd_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int c = cache[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
    c = (n > 0 && n % 8 == 0) ? n / 8 : -1;
    cache[dev].store(c, std::memory_order_relaxed);
  }
  return c > 0 ? c : 0;
}

template <int D, int DT>
static hipError_t launch_prefill_t(const PrefillAttnArgs &a0, hipStream_t s) {
  // Rows t < tk of every sequence go to tiles (when G >= 4), the rest to the
  // list walk: rows whose causal range is short enough next to the list
  // (see kTileRangeX2) and whose key mask fits the tile's LDS.  Tiles and
  // rows have kernels of their own (their register budgets differ: three
  // waves per SIMD for tiles, two for the walk).
  PrefillAttnArgs a = a0;
  // the tiled rows t < tile_range(...): the range multiplier, capped so the
  // key mask (rows per tile x 32-key words) fits its LDS
  auto tile_range = [&](int x2, int rows_per_tile, int mask_words) {
    long long r = (long long)x2 * a.top_k * (16 / tile_heads(a.G)) / 4;
    r = std::min(r, (long long)a.S);
    return (int)std::min(r, 32LL * mask_words / rows_per_tile);
  };
  // Two column tiles per wave at Gp = 8 (16 rows per tile, two waves per
  // SIMD, so a larger key mask costs no occupancy and the tiles reach further)
  // when the launch holds tiles for at least two rounds of two per CU: the
  // long prefill (S = 32768, Hkv = 4) gains, while the 512 tiles of S = 4096,
  // Hkv = 2 finish sooner as 1024 smaller ones (0.123 ms against 0.151 ms).
  int nt = tile_nt(a.G), x2 = kTileRangeX2, mask_words = kTileMaskWords;
  if (nt == 1 && tile_heads(a.G) == 8 && xcd_cus() > 0) {
    const int r2 = tile_rows_nt(a.G, 2);
    const long long tiles2 =
        (long long)a.B * a.Hkv * ((tile_range(kTileRangeX2Wide, r2, kTileMaskWordsWide) + r2 - 1) / r2);
    if (tiles2 >= 4LL * 8 * xcd_cus()) {
      nt = 2;
      x2 = kTileRangeX2Wide;
      mask_words = kTileMaskWordsWide;
    }
  }
  a.tile_rows = tile_rows_nt(a.G, nt);
  const int tk = tile_range(x2, a.tile_rows, mask_words);
  const bool tiles_on = a.G >= 4 && a.top_k >= 4;
  a.tile_below = tk;
  a.tile_per_seq = (tk + a.tile_rows - 1) / a.tile_rows;
  a.tile_b0 = a.tile_nb = 0;
  a.skip_below = 0;
  auto rows = [&](PrefillAttnArgs p) -> hipError_t {
    if (p.nrows <= 0) return hipSuccess;
    hipLaunchKernelGGL((sparse_prefill_kernel<D, DT>), dim3(prefill_grid(p)), dim3(256), 0, s, p);
    return hipGetLastError();
  };
  auto tiles = [&](int b0, int nb) -> hipError_t {
    PrefillAttnArgs p = a;
    p.tile_b0 = b0;
    p.tile_nb = nb;
    if (p.tile_per_seq <= 0) return hipSuccess;
    // snake order over the workgroups that start together on an XCD: its
    // CUs times the tile workgroups a CU holds (at NT = 1 up to four, as
    // many as the LDS allows; two at NT = 2, bound by registers), in whole
    // rows of CUs within the XCD's share of the grid
    const size_t mask_bytes = (size_t)p.tile_rows * ((p.tile_below + 31) / 32) * sizeof(uint32_t);
    const size_t lds = sizeof(TileLds) + 36 * sizeof(int) + mask_bytes;
    const int per_cu = nt == 1 ? (int)std::min<size_t>(4, (160 * 1024) / lds) : 2;
    p.tile_cus = xcd_cus();
    p.tile_snake = 0;
    if (p.tile_cus > 0 && (8 % a.Hkv) == 0) {
      const long long per_xcd = tile_grid(p) / 8;
      const long long start = (long long)p.tile_cus * per_cu;
      p.tile_snake = (int)min(start, per_xcd / p.tile_cus * p.tile_cus);
    }
    if (nt == 1) {
      hipLaunchKernelGGL((sparse_prefill_tile_kernel<D, DT, 1>), dim3(tile_grid(p)), dim3(256), mask_bytes, s, p);
    } else {
      if (lds > 65536)  // the wide key mask
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&sparse_prefill_tile_kernel<D, DT, 2>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      hipLaunchKernelGGL((sparse_prefill_tile_kernel<D, DT, 2>), dim3(tile_grid(p)), dim3(256), mask_bytes, s, p);
    }
    return hipGetLastError();
  };
  const int total = a.B * a.S, per = prefill_rows_per_launch(a, D);
  if (!tiles_on) {
    for (int o = 0; o < total; o += per) {
      PrefillAttnArgs p = a;
      p.row0 = o;
      p.nrows = min(per, total - o);
      if (hipError_t e = rows(p)) return e;
    }
    return hipSuccess;
  }
  if (per >= total) {
    if (hipError_t e = tiles(0, a.B)) return e;
    PrefillAttnArgs p = a;
    p.row0 = 0;
    if (a.B == 1) {
      p.nrows = a.S - tk;  // rows t >= tk come first in the work order
    } else {
      p.nrows = total;
      p.skip_below = tk;
    }
    return rows(p);
  }
  // Several row launches (each relies on its workgroups starting together,
  // see prefill_rows_per_launch), then the tiles of every sequence.
  const int n = a.S - tk;  // row-walk rows of a sequence: work order [b S, b S + n)
  for (int b = 0; b < a.B; ++b) {
    for (int o = 0; o < n; o += per) {
      PrefillAttnArgs p = a;
      p.row0 = b * a.S + o;
      p.nrows = min(per, n - o);
      if (hipError_t e = rows(p)) return e;
    }
  }
  return tiles(0, a.B);
}

hipError_t launch_sparse_prefill(const PrefillAttnArgs &a, int D, int dt, hipStream_t s) {
  if (D == 128) return dt == DT_F16 ? launch_prefill_t<128, DT_F16>(a, s) : launch_prefill_t<128, DT_BF16>(a, s);
  return dt == DT_F16 ? launch_prefill_t<64, DT_F16>(a, s) : launch_prefill_t<64, DT_BF16>(a, s);
}

}  // namespace qsa
