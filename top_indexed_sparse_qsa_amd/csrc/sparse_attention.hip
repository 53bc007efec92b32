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
//   * gathers the 32 K rows and the 32 V rows with each 16-lane group
//     reading whole 256-byte rows (a row per 16 lanes is ~3x the L1
//     throughput of spreading one load instruction over 16 rows), so lane
//     (q, c) holds dims 8c..8c+7 of eight keys ("key slots") of K and of V,
//   * writes its K rows to a per-wave LDS tile (16-byte pieces XOR-swizzled
//     by row) and reads them back as MFMA A fragments, both conflict-free,
//   * computes S^T = K Q^T (two 16-key tiles), so every lane ends up owning
//     the scores of one query head m = lane % 16 for its eight key slots,
//   * runs the fp32 online softmax in the exp2 domain,
//   * feeds those eight probabilities, unchanged in place, as the B operand
//     of O^T += V^T P^T; the V^T A-operand is an in-register 8x8 transpose of
//     16-bit values (v_perm) because a lane already holds eight keys x eight
//     dims of V.  Output dim d = 8*row + e, so lane (q, m) accumulates the 32
//     contiguous dims [32q, 32q+32) of head m.
// The next chunk's gathers are in flight while the current one computes, and
// ids run two chunks ahead.
//
// Prefill rows whose lists cover most of their causal prefix (all of them
// before the budget fills) run as list tiles instead: a workgroup of four
// waves takes several consecutive rows of one KV head, turns their lists
// into a per-row key mask in LDS, and walks the keys of the prefix densely,
// each 32-key chunk of K and V staged once in LDS for all its (row, head)
// columns (see "Tiles" below).
#include <math.h>

#include <algorithm>
#include <atomic>

#include "qsa_device.h"
#include "qsa_launch.h"
#include "select_core.h"

namespace qsa {

template <int D>
struct Frag {
  static constexpr int NKS = D / 32;
  u32x4 kf[8];       // K rows of the lane's eight key slots, dims 8c..8c+7
  u32x4 vf[8];       // V rows of the lane's eight key slots, dims 8c..8c+7
  uint32_t valid;    // bit i: key slot i of this lane is usable
  bool full;         // every key slot of the wave is usable (wave-uniform)
};

// Key slot i of lane group q: keys 4q+i (i < 4) and 16+4q+(i-4) (i >= 4).
__device__ __forceinline__ int slot_of(int q4, int i) { return i < 4 ? 4 * q4 + i : 12 + 4 * q4 + i; }

// Dense K/V of one sequence and KV head.  The bases are wave-uniform (scalar
// registers) and a token's 16-byte piece is a 32-bit byte offset shared by
// the K and V loads (the host keeps one sequence's K/V under 4 GiB).
struct DenseKV {
  const char *k, *v;      // row 0 of this sequence, this KV head
  uint32_t row_bytes;     // bytes between consecutive tokens
  int limit;              // ids in [0, limit) are usable
  __device__ void load(int id, int r16, u32x4 &kd, u32x4 &vd) const {
    // ids < 2^24 and row_bytes < 2^24: one full-rate 24-bit multiply
    const uint32_t off = __umul24((uint32_t)id, row_bytes) + 16u * (uint32_t)r16;
    kd = ld16(k + off);
    vd = ld16(v + off);
  }
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
  __device__ void load(int id, int r16, u32x4 &kd, u32x4 &vd) const {
    kd = ld16(row(pk, id) + 8 * r16);
    vd = ld16(row(pv, id) + 8 * r16);
  }
};

// Lanes l and l + 32 hold the id of list slot l % 32; invalid ids become 0
// (a harmless row to load) and are masked by the validity bits.
template <int D, int DT, class KV>
__device__ __forceinline__ void issue_chunk(Frag<D> &f, int idv, const KV &kv, int q4, int r16) {
  const bool ok = (unsigned)idv < (unsigned)kv.limit;
  const int sidv = ok ? idv : 0;
  const uint32_t bal = (uint32_t)__ballot(ok);  // bit s: list slot s is usable
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int id = shfl_i(sidv, slot_of(q4, i));
    if (D == 128 || r16 < D / 8) {
      kv.load(id, r16, f.kf[i], f.vf[i]);
    } else {
      f.kf[i] = u32x4{0u, 0u, 0u, 0u};
      f.vf[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  // key slots 0-3 are list slots 4q.., 4-7 are 16+4q..
  f.valid = ((bal >> (4 * q4)) & 0xfu) | (((bal >> (16 + 4 * q4)) & 0xfu) << 4);
  f.full = bal == 0xffffffffu;
}

// Online-softmax bookkeeping.  m_run is the reference the probabilities are
// taken against; it is raised only when a chunk's max exceeds it by more
// than 2^kLazyLog2 (in the exp2 domain), so most chunks skip the rescale of
// the accumulators, and a probability is at most 2^kLazyLog2.  The row sum
// adds the same 16-bit rounded probabilities the PV product uses, two at a
// time with packed dot products against (1, 1).
constexpr float kLazyLog2 = 8.f;

// Max with lane l ^ 16 / l ^ 32 by the gfx950 lane swaps (no LDS round
// trip): one of the two swapped copies holds the partner, the other the
// lane itself.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(v, fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(v, fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}

template <int DT>
__device__ __forceinline__ float add_pair(uint32_t p2, float acc) {
  if constexpr (DT == DT_F16)
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, p2), __builtin_bit_cast(f16x2_t, 0x3C003C00u), acc,
                                  false);
  else
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, p2),
                                           __builtin_bit_cast(bf16x2_t, 0x3F803F80u), acc, false);
}

// Per-wave LDS tile for one chunk of K: 32 rows of 256 B, 16-byte pieces
// XOR-swizzled by row so that both the row writes and the fragment reads are
// free of bank conflicts.  sl2 (scale * log2 e) is positive, so the max of
// the unscaled scores, times sl2, is the max of the scaled ones.
// Probabilities of one chunk for the lane's column: the column max over the
// 32 scores (8 per lane, lanes l, l ^ 16, l ^ 32, l ^ 48), the lazy rescale,
// exp2 and the 16-bit packing that is the B operand of the PV product.
// MAYBE_EMPTY: a column may have had no key yet (m_run = -inf, masked
// scores -inf); its probabilities must then be exp2(-inf) = 0 rather than
// exp2(-inf + inf).
template <int DT, bool MAYBE_EMPTY = false>
__device__ __forceinline__ u32x4 chunk_probs(const float (&x)[8], float sl2, float &m_run, float &l_run,
                                             f32x4 (&acc)[8]) {
  float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
  mx = max_xor16(mx);
  mx = max_xor32(mx);
  mx *= sl2;
  if (wave_any(mx > m_run + kLazyLog2)) {
    // m_new is finite on every lane of the list walk (every column sees >= 1
    // usable key by its first chunk); a masked column with no key yet keeps
    // -inf and alpha = 0 on its zero accumulators
    const float m_new = fmaxf(m_run, mx);
    const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
    m_run = m_new;
  }
  const float m_ref = MAYBE_EMPTY && m_run == -INFINITY ? 0.f : m_run;
  u32x4 bop;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    bop[w] = pack2<DT>(__builtin_amdgcn_exp2f(fmaf(x[2 * w], sl2, -m_ref)),
                       __builtin_amdgcn_exp2f(fmaf(x[2 * w + 1], sl2, -m_ref)));
    l_run = add_pair<DT>(bop[w], l_run);
  }
  return bop;
}

// A operand of the PV product for accumulator e: V^T built in registers
// from the lane's eight key-slot pieces.
__device__ __forceinline__ u32x4 v_operand(const u32x4 (&vf)[8], int e) {
  u32x4 a;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t lo = u4_at(vf[2 * w], e >> 1), hi = u4_at(vf[2 * w + 1], e >> 1);
    a[w] = (e & 1) ? pack_hi_hi(lo, hi) : pack_lo_lo(lo, hi);
  }
  return a;
}

// Scores of one chunk for one 16-column tile: S^T = K Q^T as two 16-key
// tiles; x[i] is key slot slot_of(q4, i) of column r16.
template <int D, int DT>
__device__ __forceinline__ void chunk_scores(const u32x4 *ktile, const u32x4 (&qf)[D / 32], float (&x)[8]) {
  const int lane = lane_id(), q4 = lane >> 4, r16 = lane & 15;
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < Frag<D>::NKS; ++ks) {
    const u32x4 k0 = ktile[r16 * 16 + ((4 * ks + q4) ^ r16)];
    const u32x4 k1 = ktile[(16 + r16) * 16 + ((4 * ks + q4) ^ r16)];
    s0 = mfma16x16x32<DT>(k0, qf[ks], s0);
    s1 = mfma16x16x32<DT>(k1, qf[ks], s1);
  }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = s0[i];
    x[4 + i] = s1[i];
  }
}

// chunk_math: scores, online softmax and PV for one chunk whose K rows sit
// in an LDS tile and whose V rows (the lane's eight key slots) are in vf.
template <int D, int DT>
__device__ __forceinline__ void chunk_math(const u32x4 *ktile, const u32x4 (&vf)[8], uint32_t valid, bool full,
                                           const u32x4 (&qf)[D / 32], float sl2, float &m_run, float &l_run,
                                           f32x4 (&acc)[8]) {
  float x[8];
  chunk_scores<D, DT>(ktile, qf, x);
  if (!full) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = ((valid >> i) & 1u) ? x[i] : -INFINITY;
  }
  const u32x4 bop = chunk_probs<DT>(x, sl2, m_run, l_run, acc);
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = mfma16x16x32<DT>(v_operand(vf, e), bop, acc[e]);
}

template <int D, int DT>
__device__ __forceinline__ void consume_chunk(const Frag<D> &f, const u32x4 (&qf)[D / 32], float sl2,
                                              float &m_run, float &l_run, f32x4 (&acc)[8], u32x4 *ktile) {
  const int lane = lane_id(), q4 = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = slot_of(q4, i);
    if (D == 128 || r16 < D / 8) ktile[row * 16 + (r16 ^ (row & 15))] = f.kf[i];
  }
  __builtin_amdgcn_wave_barrier();
  chunk_math<D, DT>(ktile, f.vf, f.valid, f.full, qf, sl2, m_run, l_run, acc);
}

// Runs the online softmax over list slots [32 * c0, n_slots), with chunk c0
// already issued into fa and id_b holding the ids of chunk c0 + 1.
// Processing stops at the first 32-slot chunk that holds no usable id.  The
// list is a pointer to the ids in memory or a KeptList (ids made from kept
// blocks in LDS); both are read as list[slot].
template <int D, int DT, class KV, class L>
__device__ void run_chunks(L list, int n_slots, const KV &kv,
                           const u32x4 (&qf)[D / 32], float sl2, float &m_run, float &l_run,
                           f32x4 (&acc)[8], u32x4 *ktile, int c0, Frag<D> &fa, int id_b) {
  const int lane = lane_id(), q4 = lane >> 4, r16 = lane & 15;
  // Every load here is unconditional: a load issued on one path only would
  // make the compiler count the wait for the chunk being consumed as if
  // nothing were in flight after it, so that each consume would also wait
  // for the chunk just issued.  Past the end, ids read slot n_slots - 1 and
  // chunks read key 0, and both are dropped.  A chunk's ids are loaded ahead
  // of the gathers issued before its turn and kept raw (range-masked only
  // when used): loads retire in order, so waiting on an id loaded after a
  // chunk's gathers would wait for those gathers too.
  auto load_id = [&](int c) -> int { return list[min((c << 5) + (lane & 31), n_slots - 1)]; };
  auto in_list = [&](int c, int idv) -> int { return (c << 5) + (lane & 31) < n_slots ? idv : -1; };
  auto usable = [&](int idv) { return wave_any((unsigned)idv < (unsigned)kv.limit); };

  Frag<D> fb;
  int id_c = load_id(c0 + 2);
  for (int c = c0;; c += 2) {
    // fa holds chunk c; id_b / id_c are the raw ids of chunks c+1 / c+2.
    const int ib = in_list(c + 1, id_b);
    const bool b_ok = usable(ib);
    const int id_d = load_id(c + 3);
    issue_chunk<D, DT>(fb, ib, kv, q4, r16);
    consume_chunk<D, DT>(fa, qf, sl2, m_run, l_run, acc, ktile);
    if (!b_ok) break;
    const int ic = in_list(c + 2, id_c);
    const bool c_ok = usable(ic);
    const int id_e = load_id(c + 4);
    issue_chunk<D, DT>(fa, ic, kv, q4, r16);
    consume_chunk<D, DT>(fb, qf, sl2, m_run, l_run, acc, ktile);
    if (!c_ok) break;
    id_b = id_d;
    id_c = id_e;
  }
}

// run_chunks from chunk c0, issuing that chunk first.
template <int D, int DT, class KV>
__device__ void run_list(const int32_t *__restrict__ list, int n_slots, const KV &kv,
                         const u32x4 (&qf)[D / 32], float sl2, float &m_run, float &l_run,
                         f32x4 (&acc)[8], u32x4 *ktile, int c0 = 0) {
  const int lane = lane_id(), q4 = lane >> 4, r16 = lane & 15;
  const int s = (c0 << 5) + (lane & 31);
  // unconditional loads (clamped to the list): a load on one branch only
  // would be waited for on its own
  const int raw_a = list[min(s, n_slots - 1)];
  const int raw_b = list[min(s + 32, n_slots - 1)];
  const int id_a = s < n_slots ? raw_a : -1;
  const int id_b = s + 32 < n_slots ? raw_b : -1;
  if (!wave_any((unsigned)id_a < (unsigned)kv.limit)) return;
  Frag<D> fa;
  issue_chunk<D, DT>(fa, id_a, kv, q4, r16);
  run_chunks<D, DT>(list, n_slots, kv, qf, sl2, m_run, l_run, acc, ktile, c0, fa, id_b);
}

// run_chunks over a list from slot 0, with the raw ids of its first two
// chunks already loaded (slots past n_slots read as -1).
template <int D, int DT, class KV, class L>
__device__ void run_list_ids(L list, int n_slots, const KV &kv,
                             const u32x4 (&qf)[D / 32], float sl2, float &m_run, float &l_run,
                             f32x4 (&acc)[8], u32x4 *ktile, int id_a, int id_b) {
  const int lane = lane_id(), q4 = lane >> 4, r16 = lane & 15;
  if (!wave_any((unsigned)id_a < (unsigned)kv.limit)) return;
  Frag<D> fa;
  issue_chunk<D, DT>(fa, id_a, kv, q4, r16);
  run_chunks<D, DT>(list, n_slots, kv, qf, sl2, m_run, l_run, acc, ktile, 0, fa, id_b);
}

// Q rows of the GQA group as MFMA B fragments (columns past G are zero).
// The loads are unconditional (a clamped row), so that none waits alone.
template <int D>
__device__ __forceinline__ void load_q(u32x4 (&qf)[D / 32], const uint16_t *qhead0, int G, int q4, int r16) {
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    const u32x4 v = ld16(qhead0 + (size_t)min(r16, G - 1) * D + 32 * ks + 8 * q4);
    qf[ks] = r16 < G ? v : u32x4{0u, 0u, 0u, 0u};
  }
}

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
// (186 VGPRs, two waves per SIMD) keep eight rows per tile.
__host__ __device__ constexpr int tile_nt(int G) { return tile_heads(G) == 16 ? 2 : 1; }
// rows per tile: 4 * NT 16-column tiles of 16 / Gp rows each (G >= 4 only)
__host__ __device__ constexpr int tile_rows_for(int G) { return 4 * tile_nt(G) * (16 / tile_heads(G)); }
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
    const int W = (t_act + 31) >> 5, nch = W;  // 32-key chunks of [0, t_act), mask words per row
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

// Decode: one wave per (sequence, KV head, split); the waves of a workgroup
// (up to four) take consecutive splits of the same (sequence, KV head),
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
  int32_t *s_pt = reinterpret_cast<int32_t *>(s_raw + DecLds<D>::bytes(nw));  // [2][max_pages]
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
    constexpr int U = 4;
    for (int i0 = threadIdx.x; i0 < npt; i0 += U * (int)blockDim.x) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = ptb[min(i0 + u * (int)blockDim.x, npt - 1)];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u * (int)blockDim.x;
        if (i < npt) s_pt[i] = v[u];
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
    kv.pool = a.pool + (size_t)kvh * a.PHD;
    kv.pk = s_pt;
    kv.pv = s_pt + a.max_pages;
    kv.row_stride = (size_t)a.Hkv * a.PHD;
    kv.num_flat_pages = a.num_flat_pages;
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
  int32_t *s_pt = reinterpret_cast<int32_t *>(s_raw + step_front_bytes<D>());  // [2][max_pages]
  uint16_t *s_lb = reinterpret_cast<uint16_t *>(s_pt + 2 * a.max_pages);
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
    constexpr int U = 4;
    for (int k0 = tid; k0 < npt; k0 += U * NT) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = ptb[min(k0 + u * NT, npt - 1)];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = k0 + u * NT;
        if (k < npt) s_pt[k] = v[u];
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
    kv.pool = a.pool + (size_t)kvh * a.PHD;
    kv.pk = s_pt;
    kv.pv = s_pt + a.max_pages;
    kv.row_stride = (size_t)a.Hkv * a.PHD;
    kv.num_flat_pages = a.num_flat_pages;
    kv.limit = ctx;
    run_list_ids<D, DT>(mine, n_slots, kv, qf, a.sl2, m_run, l_run, acc, mg.ktile(wv), id_a, id_b);
  }
  decode_merge_store<D, DT>(a, mg, pair, 0, b, kvh, m_run, l_run, acc);
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
  a.tile_rows = tile_rows_for(a.G);
  long long tkl = (long long)kTileRangeX2 * a.top_k * (16 / tile_heads(a.G)) / 4;
  if (tkl > a.S) tkl = a.S;
  if (tkl > 32LL * kTileMaskWords / a.tile_rows) tkl = 32LL * kTileMaskWords / a.tile_rows;
  const int tk = (int)tkl;
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
    const int per_cu = tile_nt(a.G) == 1 ? (int)std::min<size_t>(4, (160 * 1024) / lds) : 2;
    p.tile_cus = xcd_cus();
    p.tile_snake = 0;
    if (p.tile_cus > 0 && (8 % a.Hkv) == 0) {
      const long long per_xcd = tile_grid(p) / 8;
      const long long start = (long long)p.tile_cus * per_cu;
      p.tile_snake = (int)min(start, per_xcd / p.tile_cus * p.tile_cus);
    }
    if (tile_nt(a.G) == 1)
      hipLaunchKernelGGL((sparse_prefill_tile_kernel<D, DT, 1>), dim3(tile_grid(p)), dim3(256), mask_bytes, s, p);
    else
      hipLaunchKernelGGL((sparse_prefill_tile_kernel<D, DT, 2>), dim3(tile_grid(p)), dim3(256), mask_bytes, s, p);
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

template <int D, int DT>
static hipError_t launch_decode_t(const DecodeAttnArgs &a, hipStream_t s) {
  const unsigned pairs = (unsigned)((long long)a.B * a.C * a.Hkv);
  const size_t lds = DecLds<D>::bytes(a.wpg) + (size_t)2 * a.max_pages * sizeof(int32_t);
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
  const size_t lds = step_front_bytes<D>() + (size_t)2 * a.max_pages * sizeof(int32_t) + lb_bytes;
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
