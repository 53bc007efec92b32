// Device pieces of the sparse GQA attention shared by the prefill kernels
// (sparse_attention.hip) and the decode kernels (decode_attention.hip).
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
#pragma once

#include <math.h>

#include "qsa_device.h"
#include "qsa_launch.h"

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

// Paged K/V of one sequence and KV head.  The sequence's page-table rows
// are staged in LDS as byte offsets of the pages (page_bytes_of), so a
// token's K and V pieces are one shared in-page offset plus one LDS read
// each.
struct PagedKV {
  const char *pool;           // the KV head's columns of pool row 0
  const uint64_t *pk, *pv;    // LDS: byte offset of each page of the K / V plane rows
  uint64_t row_bytes;         // Hkv * PHD * 2
  int limit;
  __device__ void load(int id, int r16, u32x4 &kd, u32x4 &vd) const {
    const char *tok = pool + (uint64_t)(uint32_t)(id & 127) * row_bytes + 16u * (uint32_t)r16;
    kd = ld16(tok + pk[id >> 7]);
    vd = ld16(tok + pv[id >> 7]);
  }
};

// Byte offset of page-table entry pg (an entry out of [0, num_flat_pages)
// reads page 0, harmlessly: only a list id past the context could use it).
__device__ __forceinline__ uint64_t page_bytes_of(int pg, int num_flat_pages, uint64_t row_bytes) {
  return (uint64_t)((unsigned)pg < (unsigned)num_flat_pages ? pg : 0) * (128u * row_bytes);
}

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

}  // namespace qsa
