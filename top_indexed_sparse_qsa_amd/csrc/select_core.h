// Top-k block selection pieces shared by the indexer's select kernels and
// the fused decode step (gfx950, wave64).
//
// The selection is the indexer's fused step 2 (TensorRT-Edge-LLM, Qsa
// Attention Plugin, class description; decode B3): keep the `budget`
// highest-scoring complete blocks of a row, ties going to the lower block
// index.  Scores are non-negative, so their fp32 bit patterns (sign cleared)
// order like the values; an MSB-first radix select over those keys narrows
// the cut down to one bin.  Every key above the bin is kept, and of the
// bin's keys the lowest-index ones up to the budget.
#pragma once

#include "qsa_device.h"

namespace qsa {

__device__ __forceinline__ uint32_t score_key(float s) { return __float_as_uint(s) & 0x7fffffffu; }

// Inclusive prefix sum over the 64 lanes of a wave: DPP row shifts inside
// each 16-lane row, then the row broadcasts of lanes 15 and 31.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Radix histograms: the first window has 2048 bins, later ones 256; four pad
// words per 32 bins keep reads of consecutive bins by consecutive lanes free
// of bank conflicts.
constexpr int kSelBins = 2048;
__host__ __device__ constexpr int hpad(int d) { return d + ((d >> 5) << 2); }
constexpr int kSelHistWords = kSelBins + (kSelBins >> 3);

// Inclusive scan of v over the 64 lanes of a wave under a commutative,
// associative op with identity id (DPP as wave_incl_scan); lane 63 ends
// with the op over the whole wave.
template <class Op>
__device__ __forceinline__ uint32_t wave_incl_op(uint32_t v, uint32_t id, Op op) {
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x111, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x112, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x114, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x118, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x142, 0xa, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x143, 0xc, 0xf, false));
  return v;
}

// ---------------------------------------------------------------------------
// Workgroup select over the keys of one row: NT threads, thread j holding in
// round r the four keys of blocks 4*NT*r + 4j + c (c < 4; KPT/4 rounds; one
// float4 load each, coalesced across the workgroup).  Slots past the row
// hold 0xffffffff (real keys have bit 31 clear); a wave skips the rounds
// that start past the row.
//
// The cut is narrowed over key ranges [lo, hi) rather than bit prefixes.
// Zero scores (every head's relu zero) are left out of the first range:
// they are kept only when fewer than `budget` keys are non-zero, and then
// the non-zero keys are all kept and the zeros tie.  The first range is
// [smallest non-zero key, largest key], split into at most 2048 bins of
// 2^s keys each; later passes split the cut bin into at most 256.  Scores
// sit in a few binades, so a range that starts at the smallest non-zero key
// spreads them over far more bins than a window aligned to the bits all
// keys share would, and four passes always reach single keys.  A pass is
// one barrier: the keys count into an LDS histogram (plain atomic
// increments, under a wave-uniform branch; lanes whose key is outside the
// range add to one of 32 spare words instead, so no lane is masked off), and
// then every wave reads the whole histogram and finds the cut bin for itself
// (DPP scans over lane sums of bins, then within the one lane's range that
// holds it), so nothing is broadcast.  Each pass has a histogram of its own,
// all cleared at the start.
//
// Emission: every lane stores one byte per round, its four blocks' "above
// the cut" bits in the low nibble and "in the cut bin" bits in the high one;
// after a barrier thread j turns bytes [8j, 8j+8) into the two 32-bit masks
// of blocks [32j, 32j+32), and one workgroup scan of their counts places the
// kept blocks in ascending order (those above the cut, then the lowest-index
// ones of the cut bin up to the budget).
// ---------------------------------------------------------------------------
constexpr int kSelSmallWords = ((hpad(255) + 4 + 3) / 4) * 4;  // a padded 256-bin histogram
constexpr int kSelTrash = 32;                                    // spare words after each histogram

template <int NT>
struct alignas(16) WgSelLds {
  static constexpr int NW = NT / 64;
  uint32_t hist[kSelHistWords + kSelTrash];         // pass 0 (up to 2048 bins)
  uint32_t small[3][kSelSmallWords + kSelTrash];    // passes 1..3 (up to 256 bins)
  uint32_t red[3 * NW];   // per wave: largest key, smallest non-zero key, non-zero count
  int wt[NW];             // the emission scan
  uint8_t flags[8 * NT];  // per 4 blocks: above-cut bits | in-cut-bin bits << 4
};

// Exclusive prefix sum of v over the workgroup in thread order, with one
// barrier.  s_wt holds one int per wave and is read after that barrier, so
// the caller puts another barrier between two calls.
template <int NT>
__device__ __forceinline__ int wg_exscan(int v, int *s_wt, int *total) {
  constexpr int NW = NT / 64;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) s_wt[wv] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int x = s_wt[w];
    before += w < wv ? x : 0;
    all += x;
  }
  *total = all;
  return before + incl - v;
}

// Clears every histogram; call before the keys are needed, so that the
// stores overlap their loads.  wg_select_blocks reads them after its first
// barrier.
template <int NT>
__device__ __forceinline__ void wg_select_clear(WgSelLds<NT> &S) {
  constexpr int kVecs = (sizeof(S.hist) + sizeof(S.small)) / 16;
  static_assert(sizeof(S.hist) % 16 == 0 && sizeof(S.small) % 16 == 0, "histograms are whole 16-byte words");
  u32x4 *h = reinterpret_cast<u32x4 *>(S.hist);
  for (int j = threadIdx.x; j < kVecs; j += NT) h[j] = u32x4{0u, 0u, 0u, 0u};
}

// Eight bytes (little-endian in v) -> the 32-bit word of their low nibbles
// in order (byte j's nibble at bits 4j..4j+3).
__device__ __forceinline__ uint32_t low_nibbles(unsigned long long v) {
  v &= 0x0F0F0F0F0F0F0F0Full;
  v = (v | (v >> 4)) & 0x00FF00FF00FF00FFull;
  v = (v | (v >> 8)) & 0x0000FFFF0000FFFFull;
  v = (v | (v >> 16)) & 0x00000000FFFFFFFFull;
  return (uint32_t)v;
}

// The cut bin of one pass, found by one wave from the histogram H of nb
// bins (a multiple of 256; bins past the pass's range are empty): dsel, the
// bin holding the remaining-th largest key; above, the keys in bins above
// it; cnt, the keys in it.
__device__ __forceinline__ void sel_find_cut(const uint32_t *H, int nb, int remaining, int &dsel, int &above,
                                             int &cnt) {
  const int lane = lane_id();
  // lane l sums bins [nb - per*(l+1), nb - per*l): lane 0 holds the top bins
  const int per = nb >> 6;  // a multiple of 4
  const int lo = nb - per * (lane + 1);
  int lsum = 0;
  for (int j = 0; j < per; j += 4) {
    const u32x4 hv = *reinterpret_cast<const u32x4 *>(H + hpad(lo + j));
    lsum += (int)(hv[0] + hv[1] + hv[2] + hv[3]);
  }
  const int incl = wave_incl_scan(lsum);
  const int src = __ffsll((long long)__ballot(incl >= remaining)) - 1;
  const int above0 = __builtin_amdgcn_readlane(incl - lsum, src);
  // inside lane src's range, top bin first
  const int hb = lane < per ? (int)H[hpad(nb - 1 - (src * per + lane))] : 0;
  const int incl2 = above0 + wave_incl_scan(hb);
  const int js = __ffsll((long long)__ballot(incl2 >= remaining)) - 1;
  dsel = nb - 1 - (src * per + js);
  above = __builtin_amdgcn_readlane(incl2 - hb, js);
  cnt = __builtin_amdgcn_readlane(hb, js);
}

// Keeps `budget` (< the number of real keys, nc the row length) of the
// workgroup's keys and writes the kept block indices to lb[0, budget) in
// ascending order.  The histograms must have been cleared by
// wg_select_clear.  Ends with a barrier: lb is complete on return.
template <int NT, int KPT>
__device__ void wg_select_blocks(const uint32_t (&key)[KPT], int nc, int budget, WgSelLds<NT> &S, uint16_t *lb) {
  constexpr int NW = NT / 64, R = KPT / 4;
  static_assert(KPT % 4 == 0 && NT * KPT <= 8 * NT * 4, "four keys per round, at most 32 per thread");
  const int tid = threadIdx.x, lane = lane_id(), wv = tid >> 6;
  // rounds this wave holds real keys in (wave-uniform)
  const int nrw = __builtin_amdgcn_readfirstlane(
      nc > 256 * wv ? min(R, (nc - 256 * wv + 4 * NT - 1) / (4 * NT)) : 0);
  // As signed values the empty-slot marker is -1, below every key; k - 1
  // wraps a zero key past every real one (kmin below is the smallest k - 1,
  // plus one); the non-zero count is taken by ballots.
  int kmax_s = 0;
  uint32_t kmin = 0xffffffffu, nnz = 0u;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r < nrw) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t k = key[4 * r + c], km1 = k - 1u;
        kmax_s = max(kmax_s, (int)k);
        kmin = min(kmin, km1);
        nnz += (uint32_t)__popcll(__ballot(km1 < 0x7fffffffu));
      }
    }
  }
  uint32_t kmax = wave_incl_op((uint32_t)kmax_s, 0u, [](uint32_t x, uint32_t y) { return max(x, y); });
  kmin = wave_incl_op(kmin, 0xffffffffu, [](uint32_t x, uint32_t y) { return min(x, y); });
  if (lane == 63) {
    S.red[wv] = kmax;
    S.red[NW + wv] = kmin;
    S.red[2 * NW + wv] = nnz;
  }
  __syncthreads();
  kmax = 0u;
  kmin = 0xffffffffu;
  nnz = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    kmax = max(kmax, S.red[w]);
    kmin = min(kmin, S.red[NW + w]);
    nnz += S.red[2 * NW + w];
  }
  kmin += 1u;  // used only when some key is non-zero (then below 2^31)
  // keys in [lo, hi) are still open; those >= hi are kept
  uint32_t lo, hi;
  int remaining = budget;
  if ((int)nnz < budget) {  // every non-zero key, then the first zeros
    lo = 0u;
    hi = 1u;
    remaining = budget - (int)nnz;
  } else {
    lo = kmin;
    hi = kmax + 1u;
    for (int pass = 0; pass < 4; ++pass) {
      const uint32_t range = hi - lo;
      const int bl = range > 1u ? 32 - __clz((int)(range - 1u)) : 0;
      const int s = max(0, bl - (pass == 0 ? 11 : 8));
      const int nb = (((int)((range - 1u) >> s) >> 8) + 1) << 8;  // bins in use, rounded up to 256
      uint32_t *H = pass == 0 ? S.hist : S.small[pass - 1];
      uint32_t *spare = H + (pass == 0 ? kSelHistWords : kSelSmallWords) + (lane & (kSelTrash - 1));
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (r < nrw) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            // k in [lo, hi) as one unsigned compare of k - lo
            const uint32_t d = key[4 * r + c] - lo;
            const bool in = d < range;
            if (__ballot(in) != 0ull) {
              const uint32_t bin = d >> s;
              atomicAdd(in ? H + bin + ((bin >> 5) << 2) : spare, 1u);  // H[hpad(bin)]
            }
          }
        }
      }
      __syncthreads();
      int dsel, above, cnt;
      sel_find_cut(H, nb, remaining, dsel, above, cnt);
      remaining -= above;
      lo += (uint32_t)dsel << s;
      hi = min(hi, lo + (1u << s));
      if (cnt == remaining || s == 0) break;
    }
  }

  // Per round a byte per lane: bit c = block 4*NT*r + 4*tid + c above the
  // cut (>= hi), bit 4 + c = inside the cut bin ([lo, hi)).  Every round is
  // stored (past the row both nibbles are 0), so the bytes of [0, NT*KPT)
  // are all written.
  const uint32_t above = 0x80000000u - hi, range = hi - lo;  // real keys are below 2^31
#pragma unroll
  for (int r = 0; r < R; ++r) {
    uint32_t byte = 0u;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t k = key[4 * r + c];
      byte |= k - hi < above ? 1u << c : 0u;
      byte |= k - lo < range ? 16u << c : 0u;
    }
    S.flags[NT * r + tid] = (uint8_t)byte;
  }
  __syncthreads();
  // thread j: blocks [32j, 32j+32), bytes [8j, 8j+8)
  uint32_t gt_bits = 0u, eq_bits = 0u;
  if (32 * tid < NT * KPT) {
    const unsigned long long v = *reinterpret_cast<const unsigned long long *>(&S.flags[8 * tid]);
    gt_bits = low_nibbles(v);
    eq_bits = low_nibbles(v >> 4);
  }
  const int n_gt = __builtin_popcount(gt_bits), n_eq = __builtin_popcount(eq_bits);
  // One scan of both counts (n_gt in the high half: fewer than budget < nc
  // <= 32768 keys are above the cut, so neither half overflows).  The keys
  // in the cut bin before this thread's take min(eq_before, remaining)
  // slots, which is also right when the whole bin is kept.
  int tot;
  const int both = wg_exscan<NT>(n_eq | (n_gt << 16), S.wt, &tot);
  const int eq_before = both & 0xffff;
  const int take_eq = min(n_eq, max(0, remaining - eq_before));
  int pos = (both >> 16) + min(eq_before, remaining);
  // kept: above the cut, and the lowest take_eq of the cut bin
  uint32_t keep = gt_bits;
  for (int e = 0; e < take_eq; ++e) {
    keep |= eq_bits & (0u - eq_bits);
    eq_bits &= eq_bits - 1u;
  }
  while (keep != 0u) {
    const int j = __builtin_ctz(keep);
    keep &= keep - 1u;
    lb[pos++] = (uint16_t)(32 * tid + j);
  }
  __syncthreads();
}

}  // namespace qsa
