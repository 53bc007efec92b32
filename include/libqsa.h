/*
 * libqsa -- QSA (Qwen Sparse Attention) hot path for AMD MI355X (gfx950).
 *
 * Entry points, in the order a layer calls them:
 *
 *   front end: qsa_qkv_front_end   -> packed QKV split, qk-norm, partial RoPE,
 *                                     paged K/V write + dense K/V mirrors
 *   prefill:   qsa_indexer_prefill -> int32 index lists [B, S, top_k]
 *              qsa_sparse_prefill  -> sparse GQA attention over the lists
 *   decode:    qsa_indexer_decode  -> indexer state update in the pool tails
 *                                     + lists [B, 1, top_k]
 *              qsa_sparse_decode   -> split-K sparse attention over the pool
 *              qsa_decode_step     -> both, the select fused into the
 *                                     attention kernel
 *   chunked prefill over the pool: qsa_indexer_chunk, qsa_sparse_chunk
 *   allocation-free decode indexer: qsa_indexer_decode_noalloc
 *
 * Sources (pages cited by title and section):
 *   [Runner] TensorRT-Edge-LLM "Cute Dsl Qsa Sparse Runner": structs
 *            QsaSparsePrefillParams and QsaSparseDecodeParams, and the
 *            runners' run() contract.
 *   [Plugin] TensorRT-Edge-LLM "Qsa Attention Plugin": the class
 *            description (indexer steps, decode B1/B2/B3), its Contract
 *            paragraph and the "KV pool contract (widened rows)" paragraph.
 *   [Atlas]  atlasinference "spark_model/layers/ops/qsa.rs": doc comments of
 *            qsa_block_pool, qsa_qprep, qsa_score, qsa_score_rows.
 *
 * Conventions for every call
 *   - All pointers are DEVICE pointers, except the params struct itself and
 *     the config struct, which are read on the host during the call and may
 *     be freed when it returns.  The caller owns every buffer.
 *   - The library never allocates, frees or synchronises, keeps no state
 *     between calls, and enqueues all work on `stream` (a hipStream_t; NULL
 *     is the default stream).  Buffers must stay alive until that work ends.
 *     Calls are reentrant and contain no host-device synchronisation, so they
 *     may be captured in a HIP graph.  The only things the library holds are
 *     read-only device properties it looks up once per device (the CU
 *     count) and, on each GPU that runs it, the scratch of
 *     qsa_indexer_decode_noalloc.
 *   - Floating-point inputs must be finite (the kernels are built without
 *     NaN/Inf semantics): a NaN or Inf in Q, K, V, the pool or the indexer
 *     inputs gives unspecified output values, never a fault.
 *   - Only host-visible arguments are validated.  On any validation failure
 *     the call returns a non-QSA_OK status and enqueues nothing.  Device
 *     contents (list validity, context lengths, page ids) are the caller's
 *     contract; kernels still bound every device-supplied index they use for
 *     an address, so a broken contract gives wrong values, never a fault.
 *   - QSA_ERR_LAUNCH reports a HIP launch error seen right after enqueueing.
 *   - 16-bit tensors are fp16 or bf16 as `dtype` says, contiguous, innermost
 *     dimension last.  Q/K/V/O, pool, indexer input and partial_o base
 *     pointers must be 16-byte aligned (QSA_ERR_BAD_SHAPE otherwise);
 *     workspaces 256-byte aligned.
 */
#ifndef LIBQSA_H
#define LIBQSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QSA_PAGE_TOKENS 128   /* tokens per KV page [Runner: QsaSparseDecodeParams] */
#define QSA_PARTIAL_ROWS 16   /* rows per partial (the MFMA M tile) */
#define QSA_MAX_SPLITS 16     /* largest decode split count this library plans */
#define QSA_MAX_BLOCKS 32768  /* largest complete-block count one row may see */
#define QSA_NOALLOC_SCRATCH_BYTES (16u << 20) /* scratch of qsa_indexer_decode_noalloc, per GPU */

/* The *_RANGE_MIN / *_RANGE_MAX members are not values to use: they give the
 * enums the range of int32_t, so that any int a caller passes (an unknown
 * dtype or status) is a valid value to test and reject. */
typedef enum {
  QSA_FP16 = 0,
  QSA_BF16 = 1,
  QSA_DTYPE_RANGE_MIN = -2147483647 - 1,
  QSA_DTYPE_RANGE_MAX = 2147483647
} qsa_dtype;

typedef enum {
  QSA_OK = 0,
  QSA_ERR_NULL_POINTER = 1,
  QSA_ERR_BAD_SHAPE = 2,
  QSA_ERR_UNSUPPORTED = 3,
  QSA_ERR_WORKSPACE_TOO_SMALL = 4,
  QSA_ERR_LAUNCH = 5,
  QSA_STATUS_RANGE_MIN = -2147483647 - 1,
  QSA_STATUS_RANGE_MAX = 2147483647
} qsa_status;

/* Indexer attributes [Plugin: constructor attributes indexerNumHeads,
 * indexerHeadDim, indexerBudget, indexerCompressRatio, rmsNormEps; Atlas:
 * the rot and theta arguments of qsa_block_pool / qsa_qprep].
 * Supported: num_heads 1..4, head_dim 128, rot_dim even and <= head_dim,
 * compress_ratio 1..8, budget >= 1, rms_eps >= 0, rope_theta > 0. */
typedef struct {
  int32_t num_heads;      /* indexer query heads Hi (one shared key head) */
  int32_t head_dim;       /* indexer head dim hd */
  int32_t rot_dim;        /* leading dims that RoPE rotates, pairs (i, i+rot/2) */
  int32_t compress_ratio; /* tokens per block */
  int32_t budget;         /* blocks kept per row */
  float rope_theta;       /* RoPE base */
  float rms_eps;          /* RMSNorm epsilon, inside the square root */
} qsa_indexer_config;

/* Sparse prefill [Runner: QsaSparsePrefillParams].
 * q, o: [batch, seq_len, num_q_heads, head_dim]; k, v: [batch, seq_len,
 * num_kv_heads, head_dim].  indices: int32 [batch, seq_len, top_k], per row
 * distinct token ids < t+1, any order, -1 padded on the right; one list
 * serves every head of the row.  The kernel applies no positional mask.
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).
 * context_lengths: int32 [batch]; rows t >= context_lengths[b] are written
 * as +0.0 and ids >= context_lengths[b] are never read.  A live row whose
 * list holds no usable id (0 <= id < context_lengths[b]) is +0.0.  A chunk
 * of 32 slots (slots 32c .. 32c+31) that holds no usable id ends the row's
 * list: later slots are not read.
 * Supported: head_dim 64 or 128; num_q_heads a multiple of num_kv_heads with
 * ratio 1..16; top_k >= 1; seq_len < 2^24 and num_kv_heads * head_dim * 2 <
 * 2^24 bytes (token offsets use a 24-bit multiply), and one sequence's K (or
 * V) under 4 GiB; QSA_ERR_UNSUPPORTED otherwise. */
typedef struct {
  const void *q;
  const void *k;
  const void *v;
  void *o;
  const int32_t *indices;
  const int32_t *context_lengths;
  int32_t batch;
  int32_t seq_len;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t top_k;
  float attention_scale; /* multiplies q.k; finite and > 0, not assumed to be 1/sqrt(D) */
  qsa_dtype dtype;
  void *stream;
} qsa_sparse_prefill_params;

/* Split-K sparse decode [Runner: QsaSparseDecodeParams].
 * q, o: [batch, 1, num_q_heads, head_dim].
 * kv_pool: [num_flat_pages, 128, num_kv_heads, pool_head_dim]; only columns
 * [0, head_dim) of each row are read (the tail holds indexer state).
 * page_table: int32 [batch, 2, max_pages_per_seq]; row 0 holds K page ids,
 * row 1 V page ids already offset by num_flat_pages / 2.
 * indices: int32 [batch, 1, top_k] as for prefill.
 * context_lengths: int32 [batch], the TOTAL length including the new token.
 * The list is cut into num_splits contiguous runs of 32-slot chunks (0 lets
 * the library choose; otherwise 1..QSA_MAX_SPLITS), each run one online
 * softmax.  Up to eight splits of one (sequence, KV head) share a workgroup
 * and are merged there in split order, so the library's own plan
 * (num_splits = 0, never more than eight splits -- the pages' kMaxSplits)
 * is a single launch that needs no workspace: partial_o and partial_stats
 * may then be NULL.  An explicit num_splits above eight spreads a (sequence,
 * KV head) over two workgroups whose partials (fp32, partial_o:
 * qsa_sparse_decode_partial_o_elems(), partial_stats:
 * qsa_sparse_decode_partial_stats_elems()) a second small kernel merges, in
 * a fixed order.  Either way the result never depends on timing.  The
 * partials need no initial contents; calls that overlap on the GPU must not
 * share them.
 * Supported: as prefill, plus pool_head_dim >= head_dim, a multiple of 8,
 * and max_pages_per_seq <= 4096. */
typedef struct {
  const void *q;
  void *o;
  const void *kv_pool;
  const int32_t *page_table;
  const int32_t *indices;
  const int32_t *context_lengths;
  float *partial_o;
  float *partial_stats;
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t pool_head_dim;
  int32_t num_flat_pages;   /* 2 * numPages (both planes) */
  int32_t max_pages_per_seq;
  int32_t top_k;
  int32_t num_splits;
  float attention_scale;    /* finite and > 0 */
  qsa_dtype dtype;
  void *stream;
} qsa_sparse_decode_params;

/* Indexer, prefill [Plugin: fused step 2; Atlas: qsa_block_pool,
 * qsa_qprep_rows, qsa_score_rows].
 * idx_q: [batch, seq_len, num_heads, hd] raw indexer queries; idx_k:
 * [batch, seq_len, hd] raw indexer keys (one key head); q_norm_w, k_norm_w:
 * fp32 [hd] raw gains, applied as (1 + w).  context_lengths: int32 [batch].
 * Output indices: int32 [batch, seq_len, top_k].  Row t keeps the `budget`
 * highest-scoring of its floor((t+1)/ratio) complete blocks (all of them if
 * there are no more than `budget`; equal scores favour the lower block),
 * written in ascending block order as ratio consecutive ids each, then its
 * causal tail ratio*floor((t+1)/ratio) .. t, then -1.  Rows t >=
 * context_lengths[b] are all -1.  Scores are computed in fp32 from a
 * two-piece fp16 split of the fp32 queries (22 significant bits) against
 * kbar taken as fp16 (bf16 kbar converted: exact in fp16's normal range;
 * RMSNorm bounds |kbar| by sqrt(128) * max|1 + w_k|, inside fp16's range
 * while max|1 + w_k| < 5000);
 * the pages call such scoring selection-equivalent, so a swap of blocks
 * whose scores sit within that rounding of the cut can differ from a
 * float64 reference.
 * workspace: device scratch of at least
 * qsa_indexer_prefill_workspace_bytes() bytes, 256-byte aligned.
 * Optional prefill -> decode handoff [Plugin: KV pool contract (widened
 * rows)]: with kv_pool not NULL the call also leaves, for every sequence, the
 * indexer state a decode step continues from, in the layout
 * qsa_indexer_decode reads (pool and page table as for qsa_sparse_decode,
 * num_kv_heads, head_dim, pool_head_dim, num_flat_pages and
 * max_pages_per_seq describing them): with c = min(context_lengths[b],
 * seq_len), the kbar of each complete block g < c/ratio (rounded to dtype,
 * the value prefill scores with) in the V-row tail of token ratio*g, and the
 * raw idx_k of each token of the trailing incomplete block ratio*(c/ratio)
 * .. c-1 in its K-row tail.  Only those tails are written (tokens whose
 * page-table entry is out of range are skipped); the rest of the pool is
 * left bit-unchanged.  A qsa_indexer_decode step at context length c+1 then
 * selects for row c as a prefill over c+1 tokens would.  With kv_pool NULL
 * the handoff fields are ignored.
 * Supported: top_k >= budget*ratio + ratio - 1; floor(seq_len/ratio) <=
 * QSA_MAX_BLOCKS; batch*seq_len <= INT32_MAX/2; with the handoff,
 * pool_head_dim >= head_dim + cfg.head_dim, both multiples of 8. */
typedef struct {
  const void *idx_q;
  const void *idx_k;
  const float *q_norm_w;
  const float *k_norm_w;
  const int32_t *context_lengths;
  int32_t *indices;
  void *workspace;
  size_t workspace_bytes;
  int32_t batch;
  int32_t seq_len;
  int32_t top_k;
  qsa_indexer_config cfg;
  qsa_dtype dtype;
  void *stream;
  /* optional handoff (kv_pool NULL: none) */
  void *kv_pool;
  const int32_t *page_table;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t pool_head_dim;
  int32_t num_flat_pages;
  int32_t max_pages_per_seq;
} qsa_indexer_prefill_params;

/* Indexer, one decode step [Plugin: decode B1/B2/B3 and the KV pool
 * contract].  The indexer state lives in columns [head_dim, head_dim + hd)
 * of KV head 0 rows of kv_pool: block g's kbar in the V-row tail of token
 * ratio*g; for the trailing incomplete block only, each token's raw index
 * key in its K-row tail.  With p = context_lengths[b] - 1:
 *   B1  prep the queries at position p; if the block of p stays incomplete
 *       (context length not a multiple of ratio) store idx_k in the K-row
 *       tail of token p, else pool the block from the raw tails of its first
 *       ratio-1 tokens plus idx_k and store kbar in the V-row tail of its
 *       first token;
 *   B2  score the floor(ctx/ratio) blocks from the V-row tails;
 *   B3  select and expand as in prefill, for row p.
 * kv_pool is updated in place (only those tails); everything else in the
 * pool is left bit-unchanged.  idx_q: [batch, 1, num_heads, hd]; idx_k:
 * [batch, 1, hd]; indices out: int32 [batch, 1, top_k].  Page table and
 * pool as for qsa_sparse_decode.  workspace: at least
 * qsa_indexer_decode_workspace_bytes() bytes (the fp32 score row of each
 * sequence); it needs no initial contents, and calls that overlap on the
 * GPU must not share it.  B1 and B2 run as one kernel, B3 as a second.
 * Supported: pool_head_dim >= head_dim + cfg.head_dim;
 * max_pages_per_seq*128/ratio <= QSA_MAX_BLOCKS, and batch times that
 * <= INT32_MAX/2. */
typedef struct {
  const void *idx_q;
  const void *idx_k;
  const float *q_norm_w;
  const float *k_norm_w;
  void *kv_pool;
  const int32_t *page_table;
  const int32_t *context_lengths;
  int32_t *indices;
  void *workspace;
  size_t workspace_bytes;
  int32_t batch;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t pool_head_dim;
  int32_t num_flat_pages;
  int32_t max_pages_per_seq;
  int32_t top_k;
  qsa_indexer_config cfg;
  qsa_dtype dtype;
  void *stream;
} qsa_indexer_decode_params;

/* Fused front end [Plugin: fused step 1 -- packed-QKV split + per-head
 * qk-norm (gammas pre-folded to 1+w) + partial RoPE + paged-KV write + dense
 * K/V mirrors, and in decode the rope-append of the new token; "KV pool
 * contract (widened rows)"].
 * qkv: [batch, seq_len, (num_q_heads + 2*num_kv_heads) * head_dim], each row
 * the query heads, then the key heads, then the value heads.  q_gamma,
 * k_gamma: fp32 [head_dim], the gains already folded (1 + w), one vector for
 * all query heads and one for all key heads.  Row t of sequence b sits at
 * position start_positions[b] + t (start_positions NULL: t; decode passes
 * the past lengths with seq_len 1) and is live while that position is below
 * context_lengths[b] (the TOTAL length).
 * Outputs, for every row: q_out [batch, seq_len, num_q_heads, head_dim] =
 * RoPE(RMSNorm(q) * q_gamma) (eps inside the square root, mean over
 * head_dim; the first rot_dim dims turn as pairs (i, i + rot_dim/2) by
 * position * rope_theta^(-2i/rot_dim)), evaluated in fp64 and rounded once;
 * k_out the same for the key heads with k_gamma; v_out the value heads
 * unchanged.  k_out / v_out are the dense mirrors the prefill attention
 * reads; both may be NULL (decode).  With kv_pool not NULL (pool and page
 * table as for qsa_sparse_decode) each live row's K and V go to columns
 * [0, head_dim) of its token's K-plane and V-plane rows; the tails
 * [head_dim, pool_head_dim) and every other row stay bit-unchanged, and rows
 * whose page-table entry is out of range are skipped.
 * Supported: head_dim 64 or 128, rot_dim even and <= head_dim, num_q_heads
 * and num_kv_heads >= 1, rope_theta > 0, rms_eps >= 0; with the pool,
 * pool_head_dim >= head_dim, a multiple of 8. */
typedef struct {
  const void *qkv;
  const float *q_gamma;
  const float *k_gamma;
  const int32_t *context_lengths;
  const int32_t *start_positions;
  void *q_out;
  void *k_out;
  void *v_out;
  void *kv_pool;
  const int32_t *page_table;
  int32_t batch;
  int32_t seq_len;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t rot_dim;
  int32_t pool_head_dim;
  int32_t num_flat_pages;
  int32_t max_pages_per_seq;
  float rope_theta;
  float rms_eps;
  qsa_dtype dtype;
  void *stream;
} qsa_front_end_params;

qsa_status qsa_qkv_front_end(const qsa_front_end_params *p);
qsa_status qsa_indexer_prefill(const qsa_indexer_prefill_params *p);
qsa_status qsa_sparse_prefill(const qsa_sparse_prefill_params *p);
qsa_status qsa_indexer_decode(const qsa_indexer_decode_params *p);
qsa_status qsa_sparse_decode(const qsa_sparse_decode_params *p);

/* One whole decode step: qsa_indexer_decode(indexer) and then
 * qsa_sparse_decode(attention) over the lists it makes, as the plugin's
 * decode runs B1, B2, B3 and the sparse decode in one enqueue [Plugin: class
 * description, decode B1/B2/B3].  The results are those of the two calls in
 * that order, bit for bit: the pool tails, the lists in indexer->indices and
 * attention->o.  The two structs must describe the same step:
 * attention->indices == indexer->indices, and the same context_lengths,
 * kv_pool, page_table, batch, num_kv_heads, head_dim, pool_head_dim,
 * num_flat_pages, max_pages_per_seq, top_k, dtype and stream, else
 * QSA_ERR_BAD_SHAPE; each struct is validated as its own call would be.
 * Work: B1 + B2 in one kernel, then B3 and the attention in a second (one
 * workgroup per (sequence, KV head) selects from the score rows and walks
 * the list from LDS; the KV head 0 workgroup also stores the list), when
 * max_pages_per_seq*128/ratio <= 16384 and the split plan puts all splits of
 * a (sequence, KV head) in one workgroup (num_splits <= 8); otherwise the
 * two calls' own kernels.  The indexer workspace is used as by
 * qsa_indexer_decode. */
qsa_status qsa_decode_step(const qsa_indexer_decode_params *indexer, const qsa_sparse_decode_params *attention);

/* Chunked prefill over the paged pool: a chunk of chunk_len new tokens per
 * sequence continues a sequence whose earlier tokens are already in the pool
 * (attention K/V in the leading columns, indexer state in the tails, as left
 * by qsa_indexer_prefill's handoff, an earlier chunk or decode steps).  The
 * pages' plugin rejects chunked prefill [Plugin: Contract]; this is our
 * extension, with the list contract: chunk row t of sequence b sits at
 * position start_positions[b] + t (start_positions = the past lengths) and
 * is live while that position is below context_lengths[b] (the TOTAL length
 * after the chunk); its list is exactly the prefill list of that position
 * (top budget blocks of all complete blocks before it, expanded, plus its
 * causal tail; global token ids, -1 padded), and rows that are not live are
 * all -1 / +0.0.  Decode is the chunk of one row.
 *
 * qsa_indexer_chunk: idx_q [batch, chunk_len, num_heads, hd], idx_k [batch,
 * chunk_len, hd] raw; indices out [batch, chunk_len, top_k].  It pools every
 * block the chunk completes (the stored raw keys of its tokens before the
 * chunk plus the chunk's keys) into that block's V-row tail, stores the raw
 * keys of the chunk's tokens of the trailing incomplete block in their K-row
 * tails, and leaves the rest of the pool bit-unchanged -- so the tails then
 * hold what a prefill of context_lengths[b] tokens leaves.  workspace: at
 * least qsa_indexer_chunk_workspace_bytes() bytes, 256-byte aligned (the
 * fp32 queries as 16-bit scoring pieces, kbar of every block, fp32 score
 * rows).  Pool, page table and
 * sizes as for qsa_indexer_decode.
 * qsa_sparse_chunk: q, o [batch, chunk_len, num_q_heads, head_dim]; the
 * attention of every live row over its list, K/V read through the page
 * table (the chunk's own tokens included: write them first, e.g. with
 * qsa_qkv_front_end and start_positions); the split plan is the library's
 * (one workgroup per row and KV head, no workspace).  Supported: as
 * qsa_sparse_decode. */
typedef struct {
  const void *idx_q;
  const void *idx_k;
  const float *q_norm_w;
  const float *k_norm_w;
  void *kv_pool;
  const int32_t *page_table;
  const int32_t *start_positions;
  const int32_t *context_lengths;
  int32_t *indices;
  void *workspace;
  size_t workspace_bytes;
  int32_t batch;
  int32_t chunk_len;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t pool_head_dim;
  int32_t num_flat_pages;
  int32_t max_pages_per_seq;
  int32_t top_k;
  qsa_indexer_config cfg;
  qsa_dtype dtype;
  void *stream;
} qsa_indexer_chunk_params;

typedef struct {
  const void *q;
  void *o;
  const void *kv_pool;
  const int32_t *page_table;
  const int32_t *indices;
  const int32_t *start_positions;
  const int32_t *context_lengths;
  int32_t batch;
  int32_t chunk_len;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t pool_head_dim;
  int32_t num_flat_pages;
  int32_t max_pages_per_seq;
  int32_t top_k;
  float attention_scale;
  qsa_dtype dtype;
  void *stream;
} qsa_sparse_chunk_params;

qsa_status qsa_indexer_chunk(const qsa_indexer_chunk_params *p);
qsa_status qsa_sparse_chunk(const qsa_sparse_chunk_params *p);
size_t qsa_indexer_chunk_workspace_bytes(const qsa_indexer_config *cfg, int32_t batch, int32_t chunk_len,
                                         int32_t max_pages_per_seq);

/* Allocation-free qsa_indexer_decode, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The same step as qsa_indexer_decode,
 * except that its workspace comes from a scratch array libqsa keeps on each
 * GPU it runs on (QSA_NOALLOC_SCRATCH_BYTES, held until the process ends);
 * p->workspace and p->workspace_bytes are ignored.  The GPU is the current
 * HIP device at the call, which must be the device of p->stream.  Returns
 * QSA_ERR_WORKSPACE_TOO_SMALL when qsa_indexer_decode_workspace_bytes() for
 * these arguments exceeds QSA_NOALLOC_SCRATCH_BYTES (e.g. batch 256 at
 * max_pages_per_seq 512 and ratio 4 fits), and the statuses of
 * qsa_indexer_decode otherwise; QSA_ERR_LAUNCH also when the scratch address
 * cannot be looked up.  It calls no allocator.  Every call on one GPU uses
 * that GPU's one array: calls that may overlap on one GPU (other streams,
 * other threads) race and must be serialised by the caller.  Together with
 * qsa_sparse_decode on its default plan (NULL partials) a whole decode step
 * allocates nothing. */
qsa_status qsa_indexer_decode_noalloc(const qsa_indexer_decode_params *p);

/* Workspace sizes (bytes or elements); 0 when the arguments are invalid. */
size_t qsa_indexer_prefill_workspace_bytes(const qsa_indexer_config *cfg, int32_t batch,
                                           int32_t seq_len);
size_t qsa_indexer_decode_workspace_bytes(const qsa_indexer_config *cfg, int32_t batch,
                                          int32_t max_pages_per_seq);
size_t qsa_sparse_decode_partial_o_elems(int32_t batch, int32_t num_kv_heads, int32_t head_dim);
size_t qsa_sparse_decode_partial_stats_elems(int32_t batch, int32_t num_kv_heads);

/* Split count qsa_sparse_decode uses for these arguments (num_splits = 0). */
int32_t qsa_sparse_decode_default_splits(int32_t batch, int32_t num_kv_heads, int32_t top_k);

/* Static, never-NULL description of a status. */
const char *qsa_status_string(qsa_status s);

#ifdef __cplusplus
}
#endif

#endif /* LIBQSA_H */
