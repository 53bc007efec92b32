// Kernel argument blocks and host-side launchers (internal to libqsa).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "libqsa.h"

namespace qsa {

// Host-visible argument checks of qsa_indexer_decode (api.cpp).
__attribute__((visibility("hidden"))) qsa_status check_indexer_decode(const qsa_indexer_decode_params *p);

struct PrefillAttnArgs {
  const uint16_t *q, *k, *v;
  uint16_t *o;
  const int32_t *indices, *ctx;
  int B, S, Hq, Hkv, G, top_k;
  float sl2;  // attention scale * log2(e)
  int row0, nrows;  // this launch covers rows [row0, row0 + nrows) of the work order
  // tiles of rows t < tile_below: a tile launch takes the tiles of
  // sequences [tile_b0, tile_b0 + tile_nb), tile_per_seq tiles of tile_rows
  // rows each per sequence
  int tile_rows, tile_per_seq, tile_b0, tile_nb, tile_below;
  // the first tile_snake workgroups of each XCD (whole rows of tile_cus,
  // its CU count) are taken in snake order (set by the launcher; 0: none)
  int tile_cus, tile_snake;
  int skip_below;  // the row walk skips rows t < skip_below (held by tiles)
};

struct DecodeAttnArgs {
  const uint16_t *q;
  uint16_t *o;
  const uint16_t *pool;
  const int32_t *pt, *indices, *ctx;
  float *part_o, *part_stats;  // [pairs * kDecMaxGroups][16][D], [..][2][16]
  int B, Hq, Hkv, G, PHD, num_flat_pages, max_pages, top_k;
  // rows per sequence: 1 in decode (live when ctx > 0); C for a chunk, whose
  // row r of sequence b is live when start[b] + r < ctx[b]
  int C;
  const int32_t *start;
  int nsplits, split_slots;  // split s covers list slots [s*split_slots, (s+1)*split_slots)
  int wpg, ngroups;          // splits (waves) per workgroup, workgroups per (sequence, KV head)
  float sl2;
  // decode step only (select and attention in one kernel): the rows' block
  // scores [B][score_stride] (gmax live width), the select's budget and
  // ratio, and where the rows' lists are stored
  const float *scores;
  int score_stride, gmax, budget, ratio;
  int32_t *lists_out;
};

// Decode: waves (splits) per workgroup, merged in LDS; splits beyond that
// go to further workgroups whose partials a second kernel merges.
#ifndef QSA_DEC_WAVES
#define QSA_DEC_WAVES 8
#endif
constexpr int kDecWaves = QSA_DEC_WAVES;
constexpr int kDecMaxGroups = (16 + kDecWaves - 1) / kDecWaves;  // QSA_MAX_SPLITS / waves per workgroup

// Indexer: query prep + block pooling for prefill.
struct IdxPrepArgs {
  const uint16_t *idx_q, *idx_k;
  const float *wq, *wk;
  const int32_t *ctx;
  uint16_t *qhat;   // [B,S,Hi][pieces][hd]: the fp32 queries as 16-bit MFMA pieces
  uint16_t *kbar;   // [B,Gmax,hd]
  int B, S, Hi, hd, rot, ratio, Gmax;
  double theta, eps;
  int dt;
  int per_wave;     // items per wave (set by the launcher)
  double freq[64];  // RoPE frequencies theta^(-2i/rot), i < rot/2 (set by the launcher)
  // prefill -> decode handoff into the pool tails (pool == nullptr: none)
  uint16_t *pool;
  const int32_t *pt;
  int Hkv, D, PHD, num_flat_pages, max_pages;
};

struct IdxScoreArgs {
  const uint16_t *qhat;  // [B,S,Hi][pieces][hd]
  const uint16_t *kbar;
  float *scores;    // [B,S,stride]
  const int32_t *ctx;
  const int32_t *start;  // row t of sequence b sits at position start[b] + t (null: t)
  int B, S, Hi, Gmax, stride, ratio;
  int nchunk;       // chunk runs per 32-row group (set by the launcher)
  int run_chunks;   // chunks per run (set by the launcher)
};

constexpr int kScoreChunk = 128;           // kbar rows staged at a time in prefill scoring
// Chunks per prefill scoring workgroup (a run).  Whole rows when there are
// at least kScoreWholeRowGroups row groups and a row holds at most
// kScoreWholeRowChunks chunks: the longest run then stays below the average
// work per workgroup slot, so longest-first dispatch finishes evenly, and each
// group loads its queries once.  Otherwise runs of kScoreRun chunks, which
// keep the last runs short.  (Measured over nine shapes from 1 x 8192 to
// 4 x 32768 rows; runs of 8 to 16 chunks were never the fastest.)
constexpr int kScoreRun = 4;
constexpr int kScoreWholeRowGroups = 2048;
constexpr int kScoreWholeRowChunks = 32;

struct IdxSelectArgs {
  const float *scores;
  long long row_stride;
  int32_t *out;
  const int32_t *ctx;
  const int32_t *start;  // prefill rows: row t of sequence b sits at position start[b] + t (null: t)
  int B, S;            // prefill: rows B*S; decode: rows B (S unused)
  int top_k, budget, ratio;
  int decode;          // 1: row of sequence b is position ctx[b]-1
  int max_ctx;         // decode: clamp of ctx (max_pages * 128)
  int wave_words;      // per-row kernels: LDS words per row region (set by the launcher)
  int list_words;      // two-wave kernel: LDS words of each wave's list (set by the launcher)
  int row0, nrows;     // prefill: this launch covers rows [row0, row0 + nrows) (set by the launcher)
  int wg_min_nc;       // chunk rows, workgroup kernel: skip rows of at most this many blocks (0: none)
};

// Indexer decode B1 + B2 (one kernel): query prep, the pool-tail update and
// the block scores of one step.
struct IdxDecScoreArgs {
  const uint16_t *idx_q, *idx_k;
  const float *wq, *wk;
  uint16_t *pool;
  const int32_t *pt, *ctx;
  float *scores;       // [B,stride]
  int B, Hi, hd, rot, ratio, Hkv, D, PHD, num_flat_pages, max_pages, stride;
  int gmax;            // blocks one sequence may hold (max_pages * 128 / ratio)
  int wg_per_seq;      // set by the launcher
  double theta, eps;
  int dt;
  double freq[64];     // RoPE frequencies theta^(-2i/rot), i < rot/2 (set by the launcher)
};

// Chunked prefill, indexer step 1 (queries, kbar of every complete block,
// the chunk's tail writes).
struct IdxChunkPrepArgs {
  const uint16_t *idx_q, *idx_k;   // [B,C,Hi,hd], [B,C,hd]
  const float *wq, *wk;
  uint16_t *pool;
  const int32_t *pt, *ctx, *start;
  uint16_t *qhat;                  // [B,C,Hi][pieces][hd]
  uint16_t *kbar;                  // [B,Gmax,hd]
  int B, C, Hi, hd, rot, ratio, Hkv, D, PHD, num_flat_pages, max_pages, Gmax;
  double theta, eps;
  int dt;
  double freq[64];                 // set by the launcher
};

hipError_t launch_idx_chunk_prep(const IdxChunkPrepArgs &a, hipStream_t s);

// Fused front end (packed QKV -> Q, K/V mirrors, pool rows).
struct FrontEndArgs {
  const uint16_t *qkv;        // [B,S,(Hq+2Hkv)*D]
  const float *q_gamma, *k_gamma;
  const int32_t *ctx, *start;  // start may be null (all 0)
  uint16_t *q_out, *k_out, *v_out;  // k_out / v_out may be null
  uint16_t *pool;             // may be null
  const int32_t *pt;
  int B, S, Hq, Hkv, rot, PHD, num_flat_pages, max_pages;
  double theta, eps;
  int dt;
  double freq[64];            // set by the launcher
};

hipError_t launch_front_end(const FrontEndArgs &a, int D, hipStream_t s);

constexpr int kScoreTilesPerWave = 2;  // decode scoring: tiles of 16 blocks per wave
constexpr float kLog2e = 1.4426950408889634f;

hipError_t launch_sparse_prefill(const PrefillAttnArgs &a, int D, int dt, hipStream_t s);
hipError_t launch_sparse_decode(const DecodeAttnArgs &a, int D, int dt, hipStream_t s);
// Decode step select + attention (one workgroup of kDecWaves splits per
// (sequence, KV head)); gmax <= kStepMaxBlocks.
constexpr int kStepMaxBlocks = 64 * kDecWaves * 32;
hipError_t launch_decode_select_attend(const DecodeAttnArgs &a, int D, int dt, hipStream_t s);
hipError_t launch_idx_prep(const IdxPrepArgs &a, hipStream_t s);
// prefill -> decode handoff into the pool tails (no-op when a.pool is null)
hipError_t launch_idx_handoff(const IdxPrepArgs &a, hipStream_t s);
hipError_t launch_idx_score(const IdxScoreArgs &a, int dt, hipStream_t s);
hipError_t launch_idx_select(const IdxSelectArgs &a, int nc_max, hipStream_t s);
hipError_t launch_idx_dec_score(const IdxDecScoreArgs &a, int dt, hipStream_t s);

}  // namespace qsa
