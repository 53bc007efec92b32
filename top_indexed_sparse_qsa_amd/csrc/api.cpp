// libqsa C ABI: argument validation, workspace layout, split planning and
// kernel launches on the caller's stream.  Validation happens before any
// HIP call, so a rejected call touches no device state.
#include <hip/hip_runtime.h>
#include <math.h>

#include "libqsa.h"
#include "qsa_launch.h"

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
size_t round16(size_t x) { return (x + 15) / 16 * 16; }

bool dtype_ok(qsa_dtype d) { return d == QSA_FP16 || d == QSA_BF16; }

// Kernels read 16-byte vectors; every device base pointer must allow that.
bool aligned16(const void *p) { return ((uintptr_t)p % 16) == 0; }
template <class... P>
bool all_aligned16(const P *...p) { return (aligned16(p) && ...); }

qsa_status check_heads(int32_t hq, int32_t hkv, int32_t d) {
  if (hq < 1 || hkv < 1) return QSA_ERR_BAD_SHAPE;
  if (hq % hkv != 0) return QSA_ERR_BAD_SHAPE;
  if (hq / hkv > 16) return QSA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return QSA_ERR_UNSUPPORTED;
  return QSA_OK;
}

qsa_status check_cfg(const qsa_indexer_config &c) {
  if (c.num_heads < 1 || c.num_heads > 4) return QSA_ERR_UNSUPPORTED;
  if (c.head_dim != 128) return QSA_ERR_UNSUPPORTED;
  if (c.rot_dim < 0 || c.rot_dim > c.head_dim || (c.rot_dim & 1)) return QSA_ERR_UNSUPPORTED;
  if (c.compress_ratio < 1 || c.compress_ratio > 8) return QSA_ERR_UNSUPPORTED;
  if (c.budget < 1) return QSA_ERR_BAD_SHAPE;
  if (!(c.rope_theta > 0.f) || !(c.rms_eps >= 0.f) || !isfinite(c.rope_theta) || !isfinite(c.rms_eps))
    return QSA_ERR_BAD_SHAPE;
  return QSA_OK;
}

int64_t min_top_k(const qsa_indexer_config &c) {
  return (int64_t)c.budget * c.compress_ratio + c.compress_ratio - 1;
}

// Prefill indexer workspace: queries (fp32 values as two fp16 scoring
// pieces each) | 16-bit kbar | fp32 score rows.
struct PrefillWs {
  size_t qhat, kbar, scores, total;
  int gmax, stride;
};
PrefillWs prefill_ws(const qsa_indexer_config &c, int32_t B, int32_t S) {
  PrefillWs w{};
  w.gmax = S / c.compress_ratio;
  w.stride = (int)round16((size_t)(w.gmax > 0 ? w.gmax : 1));
  w.qhat = 0;
  w.kbar = align_up((size_t)B * S * c.num_heads * c.head_dim * 4);
  w.scores = w.kbar + align_up((size_t)B * (w.gmax > 0 ? w.gmax : 1) * c.head_dim * 2);
  w.total = w.scores + align_up((size_t)B * S * w.stride * 4);
  return w;
}

// Decode indexer workspace: fp32 score rows, one per sequence.
struct DecodeWs {
  size_t scores, total;
  int stride;
};
DecodeWs decode_ws(const qsa_indexer_config &c, int32_t B, int32_t max_pages) {
  DecodeWs w{};
  const size_t gmax = (size_t)max_pages * QSA_PAGE_TOKENS / c.compress_ratio;
  w.stride = (int)round16(gmax > 0 ? gmax : 1);
  w.scores = 0;
  w.total = align_up((size_t)B * w.stride * 4);
  return w;
}

// Chunk indexer workspace: queries (as scoring pieces) | 16-bit kbar of every block a
// sequence may hold | fp32 score rows.
struct ChunkWs {
  size_t qhat, kbar, scores, total;
  int gmax, stride;
};
ChunkWs chunk_ws(const qsa_indexer_config &c, int32_t B, int32_t C, int32_t max_pages) {
  ChunkWs w{};
  w.gmax = max_pages * QSA_PAGE_TOKENS / c.compress_ratio;
  w.stride = (int)round16((size_t)(w.gmax > 0 ? w.gmax : 1));
  w.qhat = 0;
  w.kbar = align_up((size_t)B * C * c.num_heads * c.head_dim * 4);
  w.scores = w.kbar + align_up((size_t)B * w.gmax * c.head_dim * 2);
  w.total = w.scores + align_up((size_t)B * C * w.stride * 4);
  return w;
}

int default_splits_rows(int64_t rows, int32_t hkv, int32_t top_k) {
  const int chunks = (top_k + 31) / 32;
  const int64_t pairs = rows * hkv;
  int64_t want = (1024 + pairs - 1) / pairs;
  if (want > qsa::kDecWaves) want = qsa::kDecWaves;
  if (want > chunks) want = chunks;
  if (want < 1) want = 1;
  return (int)want;
}

int default_splits(int32_t B, int32_t hkv, int32_t top_k) {
  const int chunks = (top_k + 31) / 32;
  const int pairs = B * hkv;
  // aim for ~1024 waves, at most one workgroup of kDecWaves splits per
  // (sequence, KV head) so that the call is a single launch: at 32 sequences
  // x 4 KV heads, 8 splits in one 8-wave workgroup measured 27.6 us per call
  // against 29.1 us as two 4-wave workgroups plus a merge launch
  int want = (1024 + pairs - 1) / pairs;
  if (want > qsa::kDecWaves) want = qsa::kDecWaves;
  if (want > chunks) want = chunks;
  if (want < 1) want = 1;
  return want;
}

qsa_status launched(hipError_t e) { return e == hipSuccess ? QSA_OK : QSA_ERR_LAUNCH; }

// Validates a sparse decode call and fills the kernel arguments.
qsa_status decode_attn_args(const qsa_sparse_decode_params *p, qsa::DecodeAttnArgs &a) {
  if (!p || !p->q || !p->o || !p->kv_pool || !p->page_table || !p->indices || !p->context_lengths)
    return QSA_ERR_NULL_POINTER;
  if (!dtype_ok(p->dtype)) return QSA_ERR_UNSUPPORTED;
  if (p->batch < 1 || p->top_k < 1 || p->num_flat_pages < 1 || p->max_pages_per_seq < 1) return QSA_ERR_BAD_SHAPE;
  if (qsa_status st = check_heads(p->num_q_heads, p->num_kv_heads, p->head_dim)) return st;
  if (p->pool_head_dim < p->head_dim || (p->pool_head_dim % 8) != 0) return QSA_ERR_BAD_SHAPE;
  if (!all_aligned16(p->q, p->o, p->kv_pool)) return QSA_ERR_BAD_SHAPE;
  if (p->max_pages_per_seq > 4096) return QSA_ERR_UNSUPPORTED;
  if (p->num_splits < 0 || p->num_splits > QSA_MAX_SPLITS) return QSA_ERR_BAD_SHAPE;
  if ((int64_t)p->batch * p->num_kv_heads * QSA_MAX_SPLITS > (int64_t)INT32_MAX) return QSA_ERR_UNSUPPORTED;
  if (!isfinite(p->attention_scale) || !(p->attention_scale > 0.f)) return QSA_ERR_BAD_SHAPE;
  int splits = p->num_splits ? p->num_splits : default_splits(p->batch, p->num_kv_heads, p->top_k);
  const int chunks = (p->top_k + 31) / 32;
  const int per = (chunks + splits - 1) / splits;
  splits = (chunks + per - 1) / per;  // drop splits that would get no slots
  const int wpg = splits < qsa::kDecWaves ? splits : qsa::kDecWaves;
  const int ngroups = (splits + wpg - 1) / wpg;
  // more than one workgroup per (sequence, KV head): their partials meet in
  // the caller's buffers
  if (ngroups > 1 && (!p->partial_o || !p->partial_stats)) return QSA_ERR_NULL_POINTER;
  if (ngroups > 1 && !aligned16(p->partial_o)) return QSA_ERR_BAD_SHAPE;
  a = qsa::DecodeAttnArgs{};
  a.q = static_cast<const uint16_t *>(p->q);
  a.o = static_cast<uint16_t *>(p->o);
  a.pool = static_cast<const uint16_t *>(p->kv_pool);
  a.pt = p->page_table;
  a.indices = p->indices;
  a.ctx = p->context_lengths;
  a.part_o = p->partial_o;
  a.part_stats = p->partial_stats;
  a.B = p->batch;
  a.C = 1;
  a.start = nullptr;
  a.Hq = p->num_q_heads;
  a.Hkv = p->num_kv_heads;
  a.G = p->num_q_heads / p->num_kv_heads;
  a.PHD = p->pool_head_dim;
  a.num_flat_pages = p->num_flat_pages;
  a.max_pages = p->max_pages_per_seq;
  a.top_k = p->top_k;
  a.nsplits = splits;
  a.split_slots = per * 32;
  a.wpg = wpg;
  a.ngroups = ngroups;
  a.sl2 = p->attention_scale * qsa::kLog2e;
  return QSA_OK;
}

}  // namespace

extern "C" {

const char *qsa_status_string(qsa_status s) {
  switch (s) {
    case QSA_OK: return "ok";
    case QSA_ERR_NULL_POINTER: return "null pointer argument";
    case QSA_ERR_BAD_SHAPE: return "invalid shape or size argument";
    case QSA_ERR_UNSUPPORTED: return "configuration not supported by the library";
    case QSA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case QSA_ERR_LAUNCH: return "HIP kernel launch failed";
    default: break;
  }
  return "unknown status";
}

size_t qsa_indexer_prefill_workspace_bytes(const qsa_indexer_config *cfg, int32_t batch, int32_t seq_len) {
  if (!cfg || check_cfg(*cfg) != QSA_OK || batch < 1 || seq_len < 1) return 0;
  return prefill_ws(*cfg, batch, seq_len).total;
}

size_t qsa_indexer_decode_workspace_bytes(const qsa_indexer_config *cfg, int32_t batch, int32_t max_pages) {
  if (!cfg || check_cfg(*cfg) != QSA_OK || batch < 1 || max_pages < 1) return 0;
  return decode_ws(*cfg, batch, max_pages).total;
}

size_t qsa_sparse_decode_partial_o_elems(int32_t batch, int32_t hkv, int32_t d) {
  if (batch < 1 || hkv < 1 || d < 1) return 0;
  return (size_t)batch * hkv * qsa::kDecMaxGroups * QSA_PARTIAL_ROWS * d;
}

size_t qsa_sparse_decode_partial_stats_elems(int32_t batch, int32_t hkv) {
  if (batch < 1 || hkv < 1) return 0;
  return (size_t)batch * hkv * qsa::kDecMaxGroups * 2 * QSA_PARTIAL_ROWS;
}

int32_t qsa_sparse_decode_default_splits(int32_t batch, int32_t hkv, int32_t top_k) {
  if (batch < 1 || hkv < 1 || top_k < 1) return 0;
  return default_splits(batch, hkv, top_k);
}

qsa_status qsa_qkv_front_end(const qsa_front_end_params *p) {
  if (!p || !p->qkv || !p->q_gamma || !p->k_gamma || !p->context_lengths || !p->q_out) return QSA_ERR_NULL_POINTER;
  if (!p->k_out != !p->v_out) return QSA_ERR_NULL_POINTER;  // both mirrors or neither
  if (!dtype_ok(p->dtype)) return QSA_ERR_UNSUPPORTED;
  if (p->batch < 1 || p->seq_len < 1 || p->num_q_heads < 1 || p->num_kv_heads < 1) return QSA_ERR_BAD_SHAPE;
  if (p->head_dim != 64 && p->head_dim != 128) return QSA_ERR_UNSUPPORTED;
  if (p->rot_dim < 0 || p->rot_dim > p->head_dim || (p->rot_dim & 1)) return QSA_ERR_UNSUPPORTED;
  if (!(p->rope_theta > 0.f) || !isfinite(p->rope_theta) || !(p->rms_eps >= 0.f) || !isfinite(p->rms_eps))
    return QSA_ERR_BAD_SHAPE;
  if (!all_aligned16(p->qkv, p->q_out, p->k_out, p->v_out)) return QSA_ERR_BAD_SHAPE;
  if ((int64_t)p->batch * p->seq_len * (p->num_q_heads + 2 * p->num_kv_heads) * p->head_dim > ((int64_t)1 << 40))
    return QSA_ERR_UNSUPPORTED;
  if (p->kv_pool) {
    if (!p->page_table) return QSA_ERR_NULL_POINTER;
    if (p->num_flat_pages < 1 || p->max_pages_per_seq < 1) return QSA_ERR_BAD_SHAPE;
    if (p->pool_head_dim < p->head_dim || (p->pool_head_dim % 8) != 0) return QSA_ERR_BAD_SHAPE;
    if (!all_aligned16(p->kv_pool)) return QSA_ERR_BAD_SHAPE;
  }
  qsa::FrontEndArgs a{};
  a.qkv = static_cast<const uint16_t *>(p->qkv);
  a.q_gamma = p->q_gamma;
  a.k_gamma = p->k_gamma;
  a.ctx = p->context_lengths;
  a.start = p->start_positions;
  a.q_out = static_cast<uint16_t *>(p->q_out);
  a.k_out = static_cast<uint16_t *>(p->k_out);
  a.v_out = static_cast<uint16_t *>(p->v_out);
  a.pool = static_cast<uint16_t *>(p->kv_pool);
  a.pt = p->kv_pool ? p->page_table : nullptr;
  a.B = p->batch;
  a.S = p->seq_len;
  a.Hq = p->num_q_heads;
  a.Hkv = p->num_kv_heads;
  a.rot = p->rot_dim;
  a.PHD = p->kv_pool ? p->pool_head_dim : 0;
  a.num_flat_pages = p->kv_pool ? p->num_flat_pages : 0;
  a.max_pages = p->kv_pool ? p->max_pages_per_seq : 0;
  a.theta = (double)p->rope_theta;
  a.eps = (double)p->rms_eps;
  a.dt = (int)p->dtype;
  return launched(qsa::launch_front_end(a, p->head_dim, (hipStream_t)p->stream));
}

qsa_status qsa_sparse_prefill(const qsa_sparse_prefill_params *p) {
  if (!p || !p->q || !p->k || !p->v || !p->o || !p->indices || !p->context_lengths) return QSA_ERR_NULL_POINTER;
  if (!dtype_ok(p->dtype)) return QSA_ERR_UNSUPPORTED;
  if (p->batch < 1 || p->seq_len < 1 || p->top_k < 1) return QSA_ERR_BAD_SHAPE;
  if (qsa_status st = check_heads(p->num_q_heads, p->num_kv_heads, p->head_dim)) return st;
  if (!all_aligned16(p->q, p->k, p->v, p->o)) return QSA_ERR_BAD_SHAPE;
  if ((int64_t)p->batch * p->seq_len * p->num_kv_heads > (int64_t)INT32_MAX - 4) return QSA_ERR_UNSUPPORTED;
  // one sequence's K (or V) is addressed with 32-bit byte offsets, a token's
  // row as a 24-bit multiply of its id by the row bytes
  if ((int64_t)p->seq_len * p->num_kv_heads * p->head_dim * 2 >= ((int64_t)1 << 32)) return QSA_ERR_UNSUPPORTED;
  if (p->seq_len >= (1 << 24) || (int64_t)p->num_kv_heads * p->head_dim * 2 >= (1 << 24)) return QSA_ERR_UNSUPPORTED;
  if (!isfinite(p->attention_scale) || !(p->attention_scale > 0.f)) return QSA_ERR_BAD_SHAPE;
  qsa::PrefillAttnArgs a{};
  a.q = static_cast<const uint16_t *>(p->q);
  a.k = static_cast<const uint16_t *>(p->k);
  a.v = static_cast<const uint16_t *>(p->v);
  a.o = static_cast<uint16_t *>(p->o);
  a.indices = p->indices;
  a.ctx = p->context_lengths;
  a.B = p->batch;
  a.S = p->seq_len;
  a.Hq = p->num_q_heads;
  a.Hkv = p->num_kv_heads;
  a.G = p->num_q_heads / p->num_kv_heads;
  a.top_k = p->top_k;
  a.sl2 = p->attention_scale * qsa::kLog2e;
  return launched(qsa::launch_sparse_prefill(a, p->head_dim, (int)p->dtype, (hipStream_t)p->stream));
}

qsa_status qsa_sparse_decode(const qsa_sparse_decode_params *p) {
  qsa::DecodeAttnArgs a;
  if (qsa_status st = decode_attn_args(p, a)) return st;
  return launched(qsa::launch_sparse_decode(a, p->head_dim, (int)p->dtype, (hipStream_t)p->stream));
}

size_t qsa_indexer_chunk_workspace_bytes(const qsa_indexer_config *cfg, int32_t batch, int32_t chunk_len,
                                          int32_t max_pages) {
  if (!cfg || check_cfg(*cfg) != QSA_OK || batch < 1 || chunk_len < 1 || max_pages < 1) return 0;
  return chunk_ws(*cfg, batch, chunk_len, max_pages).total;
}

qsa_status qsa_sparse_chunk(const qsa_sparse_chunk_params *p) {
  if (!p || !p->q || !p->o || !p->kv_pool || !p->page_table || !p->indices || !p->context_lengths ||
      !p->start_positions)
    return QSA_ERR_NULL_POINTER;
  if (!dtype_ok(p->dtype)) return QSA_ERR_UNSUPPORTED;
  if (p->batch < 1 || p->chunk_len < 1 || p->top_k < 1 || p->num_flat_pages < 1 || p->max_pages_per_seq < 1)
    return QSA_ERR_BAD_SHAPE;
  if (qsa_status st = check_heads(p->num_q_heads, p->num_kv_heads, p->head_dim)) return st;
  if (p->pool_head_dim < p->head_dim || (p->pool_head_dim % 8) != 0) return QSA_ERR_BAD_SHAPE;
  if (!all_aligned16(p->q, p->o, p->kv_pool)) return QSA_ERR_BAD_SHAPE;
  if (p->max_pages_per_seq > 4096) return QSA_ERR_UNSUPPORTED;
  if ((int64_t)p->batch * p->chunk_len * p->num_kv_heads > (int64_t)INT32_MAX / 2) return QSA_ERR_UNSUPPORTED;
  if (!isfinite(p->attention_scale) || !(p->attention_scale > 0.f)) return QSA_ERR_BAD_SHAPE;
  int splits = default_splits_rows((int64_t)p->batch * p->chunk_len, p->num_kv_heads, p->top_k);
  const int chunks = (p->top_k + 31) / 32;
  const int per = (chunks + splits - 1) / splits;
  splits = (chunks + per - 1) / per;
  qsa::DecodeAttnArgs a{};
  a.q = static_cast<const uint16_t *>(p->q);
  a.o = static_cast<uint16_t *>(p->o);
  a.pool = static_cast<const uint16_t *>(p->kv_pool);
  a.pt = p->page_table;
  a.indices = p->indices;
  a.ctx = p->context_lengths;
  a.part_o = nullptr;
  a.part_stats = nullptr;
  a.B = p->batch;
  a.C = p->chunk_len;
  a.start = p->start_positions;
  a.Hq = p->num_q_heads;
  a.Hkv = p->num_kv_heads;
  a.G = p->num_q_heads / p->num_kv_heads;
  a.PHD = p->pool_head_dim;
  a.num_flat_pages = p->num_flat_pages;
  a.max_pages = p->max_pages_per_seq;
  a.top_k = p->top_k;
  a.nsplits = splits;
  a.split_slots = per * 32;
  a.wpg = splits;  // at most kDecWaves: one workgroup per (row, KV head)
  a.ngroups = 1;
  a.sl2 = p->attention_scale * qsa::kLog2e;
  return launched(qsa::launch_sparse_decode(a, p->head_dim, (int)p->dtype, (hipStream_t)p->stream));
}

qsa_status qsa_indexer_chunk(const qsa_indexer_chunk_params *p) {
  if (!p || !p->idx_q || !p->idx_k || !p->q_norm_w || !p->k_norm_w || !p->kv_pool || !p->page_table ||
      !p->context_lengths || !p->start_positions || !p->indices || !p->workspace)
    return QSA_ERR_NULL_POINTER;
  if (!dtype_ok(p->dtype)) return QSA_ERR_UNSUPPORTED;
  if (qsa_status st = check_cfg(p->cfg)) return st;
  if (p->batch < 1 || p->chunk_len < 1 || p->num_kv_heads < 1 || p->num_flat_pages < 1 || p->max_pages_per_seq < 1)
    return QSA_ERR_BAD_SHAPE;
  if (p->head_dim < 1 || p->pool_head_dim < p->head_dim + p->cfg.head_dim || (p->head_dim % 8) != 0 ||
      (p->pool_head_dim % 8) != 0)
    return QSA_ERR_BAD_SHAPE;
  if (p->top_k < min_top_k(p->cfg)) return QSA_ERR_BAD_SHAPE;
  if ((int64_t)p->max_pages_per_seq * QSA_PAGE_TOKENS / p->cfg.compress_ratio > QSA_MAX_BLOCKS)
    return QSA_ERR_UNSUPPORTED;
  const int gmax = p->max_pages_per_seq * QSA_PAGE_TOKENS / p->cfg.compress_ratio;
  if ((int64_t)p->batch * ((int64_t)p->chunk_len + gmax + 1) > (int64_t)INT32_MAX / 2) return QSA_ERR_UNSUPPORTED;
  if ((int64_t)p->batch * p->chunk_len > (int64_t)INT32_MAX / 2) return QSA_ERR_UNSUPPORTED;
  if (!all_aligned16(p->idx_q, p->idx_k, p->kv_pool)) return QSA_ERR_BAD_SHAPE;
  if (((uintptr_t)p->workspace % kAlign) != 0) return QSA_ERR_BAD_SHAPE;
  const ChunkWs w = chunk_ws(p->cfg, p->batch, p->chunk_len, p->max_pages_per_seq);
  if (p->workspace_bytes < w.total) return QSA_ERR_WORKSPACE_TOO_SMALL;
  char *ws = static_cast<char *>(p->workspace);
  const hipStream_t s = (hipStream_t)p->stream;
  const int dt = (int)p->dtype;

  qsa::IdxChunkPrepArgs pa{};
  pa.idx_q = static_cast<const uint16_t *>(p->idx_q);
  pa.idx_k = static_cast<const uint16_t *>(p->idx_k);
  pa.wq = p->q_norm_w;
  pa.wk = p->k_norm_w;
  pa.pool = static_cast<uint16_t *>(p->kv_pool);
  pa.pt = p->page_table;
  pa.ctx = p->context_lengths;
  pa.start = p->start_positions;
  pa.qhat = reinterpret_cast<uint16_t *>(ws + w.qhat);
  pa.kbar = reinterpret_cast<uint16_t *>(ws + w.kbar);
  pa.B = p->batch;
  pa.C = p->chunk_len;
  pa.Hi = p->cfg.num_heads;
  pa.hd = p->cfg.head_dim;
  pa.rot = p->cfg.rot_dim;
  pa.ratio = p->cfg.compress_ratio;
  pa.Hkv = p->num_kv_heads;
  pa.D = p->head_dim;
  pa.PHD = p->pool_head_dim;
  pa.num_flat_pages = p->num_flat_pages;
  pa.max_pages = p->max_pages_per_seq;
  pa.Gmax = w.gmax;
  pa.theta = (double)p->cfg.rope_theta;
  pa.eps = (double)p->cfg.rms_eps;
  pa.dt = dt;
  if (qsa::launch_idx_chunk_prep(pa, s) != hipSuccess) return QSA_ERR_LAUNCH;

  qsa::IdxScoreArgs sa{};
  sa.qhat = pa.qhat;
  sa.kbar = pa.kbar;
  sa.scores = reinterpret_cast<float *>(ws + w.scores);
  sa.ctx = p->context_lengths;
  sa.start = p->start_positions;
  sa.B = p->batch;
  sa.S = p->chunk_len;
  sa.Hi = p->cfg.num_heads;
  sa.Gmax = w.gmax;
  sa.stride = w.stride;
  sa.ratio = p->cfg.compress_ratio;
  if (qsa::launch_idx_score(sa, dt, s) != hipSuccess) return QSA_ERR_LAUNCH;

  qsa::IdxSelectArgs xa{};
  xa.scores = sa.scores;
  xa.row_stride = w.stride;
  xa.out = p->indices;
  xa.ctx = p->context_lengths;
  xa.start = p->start_positions;
  xa.B = p->batch;
  xa.S = p->chunk_len;
  xa.top_k = p->top_k;
  xa.budget = p->cfg.budget;
  xa.ratio = p->cfg.compress_ratio;
  xa.decode = 0;
  xa.max_ctx = p->max_pages_per_seq * QSA_PAGE_TOKENS;
  return launched(qsa::launch_idx_select(xa, gmax, s));
}

qsa_status qsa_indexer_prefill(const qsa_indexer_prefill_params *p) {
  if (!p || !p->idx_q || !p->idx_k || !p->q_norm_w || !p->k_norm_w || !p->context_lengths || !p->indices ||
      !p->workspace)
    return QSA_ERR_NULL_POINTER;
  if (!dtype_ok(p->dtype)) return QSA_ERR_UNSUPPORTED;
  if (qsa_status st = check_cfg(p->cfg)) return st;
  if (p->batch < 1 || p->seq_len < 1) return QSA_ERR_BAD_SHAPE;
  if (p->top_k < min_top_k(p->cfg)) return QSA_ERR_BAD_SHAPE;
  if (p->seq_len / p->cfg.compress_ratio > QSA_MAX_BLOCKS) return QSA_ERR_UNSUPPORTED;
  if (!all_aligned16(p->idx_q, p->idx_k)) return QSA_ERR_BAD_SHAPE;
  if ((int64_t)p->batch * p->seq_len > (int64_t)INT32_MAX / 2) return QSA_ERR_UNSUPPORTED;
  if (((uintptr_t)p->workspace % kAlign) != 0) return QSA_ERR_BAD_SHAPE;
  if (p->kv_pool) {
    if (!p->page_table) return QSA_ERR_NULL_POINTER;
    if (p->num_kv_heads < 1 || p->num_flat_pages < 1 || p->max_pages_per_seq < 1) return QSA_ERR_BAD_SHAPE;
    if (p->head_dim < 1 || p->pool_head_dim < p->head_dim + p->cfg.head_dim || (p->head_dim % 8) != 0 ||
        (p->pool_head_dim % 8) != 0)
      return QSA_ERR_BAD_SHAPE;
    if (!all_aligned16(p->kv_pool)) return QSA_ERR_BAD_SHAPE;
  }
  const PrefillWs w = prefill_ws(p->cfg, p->batch, p->seq_len);
  if (p->workspace_bytes < w.total) return QSA_ERR_WORKSPACE_TOO_SMALL;
  char *ws = static_cast<char *>(p->workspace);
  const hipStream_t s = (hipStream_t)p->stream;
  const int dt = (int)p->dtype;

  qsa::IdxPrepArgs pa{};
  pa.idx_q = static_cast<const uint16_t *>(p->idx_q);
  pa.idx_k = static_cast<const uint16_t *>(p->idx_k);
  pa.wq = p->q_norm_w;
  pa.wk = p->k_norm_w;
  pa.ctx = p->context_lengths;
  pa.qhat = reinterpret_cast<uint16_t *>(ws + w.qhat);
  pa.kbar = reinterpret_cast<uint16_t *>(ws + w.kbar);
  pa.B = p->batch;
  pa.S = p->seq_len;
  pa.Hi = p->cfg.num_heads;
  pa.hd = p->cfg.head_dim;
  pa.rot = p->cfg.rot_dim;
  pa.ratio = p->cfg.compress_ratio;
  pa.Gmax = w.gmax;
  pa.theta = (double)p->cfg.rope_theta;
  pa.eps = (double)p->cfg.rms_eps;
  pa.dt = dt;
  pa.pool = static_cast<uint16_t *>(p->kv_pool);
  pa.pt = p->kv_pool ? p->page_table : nullptr;
  pa.Hkv = p->kv_pool ? p->num_kv_heads : 0;
  pa.D = p->kv_pool ? p->head_dim : 0;
  pa.PHD = p->kv_pool ? p->pool_head_dim : 0;
  pa.num_flat_pages = p->kv_pool ? p->num_flat_pages : 0;
  pa.max_pages = p->kv_pool ? p->max_pages_per_seq : 0;
  if (qsa::launch_idx_prep(pa, s) != hipSuccess) return QSA_ERR_LAUNCH;
  if (qsa::launch_idx_handoff(pa, s) != hipSuccess) return QSA_ERR_LAUNCH;

  qsa::IdxScoreArgs sa{};
  sa.qhat = pa.qhat;
  sa.kbar = pa.kbar;
  sa.scores = reinterpret_cast<float *>(ws + w.scores);
  sa.ctx = p->context_lengths;
  sa.B = p->batch;
  sa.S = p->seq_len;
  sa.Hi = p->cfg.num_heads;
  sa.Gmax = w.gmax;
  sa.stride = w.stride;
  sa.ratio = p->cfg.compress_ratio;
  if (qsa::launch_idx_score(sa, dt, s) != hipSuccess) return QSA_ERR_LAUNCH;

  qsa::IdxSelectArgs xa{};
  xa.scores = sa.scores;
  xa.row_stride = w.stride;
  xa.out = p->indices;
  xa.ctx = p->context_lengths;
  xa.B = p->batch;
  xa.S = p->seq_len;
  xa.top_k = p->top_k;
  xa.budget = p->cfg.budget;
  xa.ratio = p->cfg.compress_ratio;
  xa.decode = 0;
  xa.max_ctx = p->seq_len;
  return launched(qsa::launch_idx_select(xa, w.gmax, s));
}

}  // extern "C"

// Host-visible argument checks of qsa_indexer_decode (shared with its
// allocation-free variant, which checks with its scratch size).
qsa_status qsa::check_indexer_decode(const qsa_indexer_decode_params *p) {
  if (!p || !p->idx_q || !p->idx_k || !p->q_norm_w || !p->k_norm_w || !p->kv_pool || !p->page_table ||
      !p->context_lengths || !p->indices || !p->workspace)
    return QSA_ERR_NULL_POINTER;
  if (!dtype_ok(p->dtype)) return QSA_ERR_UNSUPPORTED;
  if (qsa_status st = check_cfg(p->cfg)) return st;
  if (p->batch < 1 || p->num_kv_heads < 1 || p->num_flat_pages < 1 || p->max_pages_per_seq < 1)
    return QSA_ERR_BAD_SHAPE;
  if (p->head_dim < 1 || p->pool_head_dim < p->head_dim + p->cfg.head_dim || (p->head_dim % 8) != 0 ||
      (p->pool_head_dim % 8) != 0)
    return QSA_ERR_BAD_SHAPE;
  if (p->top_k < min_top_k(p->cfg)) return QSA_ERR_BAD_SHAPE;
  if ((int64_t)p->max_pages_per_seq * QSA_PAGE_TOKENS / p->cfg.compress_ratio > QSA_MAX_BLOCKS)
    return QSA_ERR_UNSUPPORTED;
  // block indices across the batch (score rows, scoring waves) stay in int
  if ((int64_t)p->batch * (p->max_pages_per_seq * QSA_PAGE_TOKENS / p->cfg.compress_ratio) > (int64_t)INT32_MAX / 2)
    return QSA_ERR_UNSUPPORTED;
  if (!all_aligned16(p->idx_q, p->idx_k, p->kv_pool)) return QSA_ERR_BAD_SHAPE;
  if (((uintptr_t)p->workspace % kAlign) != 0) return QSA_ERR_BAD_SHAPE;
  if (p->workspace_bytes < decode_ws(p->cfg, p->batch, p->max_pages_per_seq).total) return QSA_ERR_WORKSPACE_TOO_SMALL;
  return QSA_OK;
}

namespace {

// Decode B1 + B2 (one kernel) of a validated indexer decode call; the score
// rows go to the workspace.
hipError_t launch_dec_score(const qsa_indexer_decode_params *p) {
  const DecodeWs w = decode_ws(p->cfg, p->batch, p->max_pages_per_seq);
  qsa::IdxDecScoreArgs sa{};
  sa.idx_q = static_cast<const uint16_t *>(p->idx_q);
  sa.idx_k = static_cast<const uint16_t *>(p->idx_k);
  sa.wq = p->q_norm_w;
  sa.wk = p->k_norm_w;
  sa.pool = static_cast<uint16_t *>(p->kv_pool);
  sa.pt = p->page_table;
  sa.ctx = p->context_lengths;
  sa.scores = reinterpret_cast<float *>(static_cast<char *>(p->workspace) + w.scores);
  sa.B = p->batch;
  sa.Hi = p->cfg.num_heads;
  sa.hd = p->cfg.head_dim;
  sa.rot = p->cfg.rot_dim;
  sa.ratio = p->cfg.compress_ratio;
  sa.Hkv = p->num_kv_heads;
  sa.D = p->head_dim;
  sa.PHD = p->pool_head_dim;
  sa.num_flat_pages = p->num_flat_pages;
  sa.max_pages = p->max_pages_per_seq;
  sa.stride = w.stride;
  sa.gmax = p->max_pages_per_seq * QSA_PAGE_TOKENS / p->cfg.compress_ratio;
  sa.theta = (double)p->cfg.rope_theta;
  sa.eps = (double)p->cfg.rms_eps;
  sa.dt = (int)p->dtype;
  return qsa::launch_idx_dec_score(sa, (int)p->dtype, (hipStream_t)p->stream);
}

}  // namespace

extern "C" {

qsa_status qsa_indexer_decode(const qsa_indexer_decode_params *p) {
  if (qsa_status st = qsa::check_indexer_decode(p)) return st;
  if (launch_dec_score(p) != hipSuccess) return QSA_ERR_LAUNCH;
  const DecodeWs w = decode_ws(p->cfg, p->batch, p->max_pages_per_seq);
  const int gmax = p->max_pages_per_seq * QSA_PAGE_TOKENS / p->cfg.compress_ratio;
  qsa::IdxSelectArgs xa{};
  xa.scores = reinterpret_cast<const float *>(static_cast<const char *>(p->workspace) + w.scores);
  xa.row_stride = w.stride;
  xa.out = p->indices;
  xa.ctx = p->context_lengths;
  xa.B = p->batch;
  xa.S = 1;
  xa.top_k = p->top_k;
  xa.budget = p->cfg.budget;
  xa.ratio = p->cfg.compress_ratio;
  xa.decode = 1;
  xa.max_ctx = p->max_pages_per_seq * QSA_PAGE_TOKENS;
  return launched(qsa::launch_idx_select(xa, gmax, (hipStream_t)p->stream));
}

qsa_status qsa_decode_step(const qsa_indexer_decode_params *ip, const qsa_sparse_decode_params *ap) {
  if (!ip || !ap) return QSA_ERR_NULL_POINTER;
  if (qsa_status st = qsa::check_indexer_decode(ip)) return st;
  qsa::DecodeAttnArgs a;
  if (qsa_status st = decode_attn_args(ap, a)) return st;
  // both halves describe the same step
  if (ap->indices != ip->indices || ap->context_lengths != ip->context_lengths || ap->kv_pool != ip->kv_pool ||
      ap->page_table != ip->page_table || ap->batch != ip->batch || ap->num_kv_heads != ip->num_kv_heads ||
      ap->head_dim != ip->head_dim || ap->pool_head_dim != ip->pool_head_dim ||
      ap->num_flat_pages != ip->num_flat_pages || ap->max_pages_per_seq != ip->max_pages_per_seq ||
      ap->top_k != ip->top_k || ap->dtype != ip->dtype || ap->stream != ip->stream)
    return QSA_ERR_BAD_SHAPE;
  const int gmax = ip->max_pages_per_seq * QSA_PAGE_TOKENS / ip->cfg.compress_ratio;
  if (gmax > qsa::kStepMaxBlocks || a.ngroups != 1) {  // the two calls, one after the other
    if (qsa_status st = qsa_indexer_decode(ip)) return st;
    return launched(qsa::launch_sparse_decode(a, ap->head_dim, (int)ap->dtype, (hipStream_t)ap->stream));
  }
  if (launch_dec_score(ip) != hipSuccess) return QSA_ERR_LAUNCH;
  const DecodeWs w = decode_ws(ip->cfg, ip->batch, ip->max_pages_per_seq);
  a.scores = reinterpret_cast<const float *>(static_cast<const char *>(ip->workspace) + w.scores);
  a.score_stride = w.stride;
  a.gmax = gmax;
  a.budget = ip->cfg.budget;
  a.ratio = ip->cfg.compress_ratio;
  a.lists_out = ip->indices;
  return launched(qsa::launch_decode_select_attend(a, ap->head_dim, (int)ap->dtype, (hipStream_t)ap->stream));
}

}  // extern "C"
