"""ctypes binding of libqsa (include/libqsa.h).

Argument marshalling only: every step of the hot path runs in libqsa's HIP
kernels.  Functions carry the C names, take torch tensors for device buffers
and enqueue on the current HIP stream unless one is given.  A missing or
unloadable libqsa.so raises immediately; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# LIBQSA_PATH names another build of the same library (the host-sanitized
# one the boundary tests run against); it is never a fallback: a missing
# file still raises.
LIB_PATH = os.environ.get("LIBQSA_PATH") or os.path.join(HERE, "libqsa.so")

QSA_FP16, QSA_BF16 = 0, 1
QSA_PAGE_TOKENS = 128
QSA_PARTIAL_ROWS = 16
QSA_MAX_SPLITS = 16
QSA_MAX_BLOCKS = 32768
QSA_NOALLOC_SCRATCH_BYTES = 16 << 20

STATUS = {0: "QSA_OK", 1: "QSA_ERR_NULL_POINTER", 2: "QSA_ERR_BAD_SHAPE", 3: "QSA_ERR_UNSUPPORTED",
          4: "QSA_ERR_WORKSPACE_TOO_SMALL", 5: "QSA_ERR_LAUNCH"}

EXPORTS = [
    "qsa_indexer_prefill", "qsa_sparse_prefill", "qsa_indexer_decode", "qsa_sparse_decode",
    "qsa_decode_step", "qsa_indexer_decode_noalloc", "qsa_qkv_front_end", "qsa_indexer_chunk", "qsa_sparse_chunk",
    "qsa_indexer_chunk_workspace_bytes",
    "qsa_indexer_prefill_workspace_bytes", "qsa_indexer_decode_workspace_bytes",
    "qsa_sparse_decode_partial_o_elems", "qsa_sparse_decode_partial_stats_elems",
    "qsa_sparse_decode_default_splits", "qsa_status_string",
]

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_f32 = ctypes.c_float
_sz = ctypes.c_size_t


class QsaIndexerConfig(ctypes.Structure):
    _fields_ = [("num_heads", _i32), ("head_dim", _i32), ("rot_dim", _i32), ("compress_ratio", _i32),
                ("budget", _i32), ("rope_theta", _f32), ("rms_eps", _f32)]


class SparsePrefillParams(ctypes.Structure):
    _fields_ = [("q", _vp), ("k", _vp), ("v", _vp), ("o", _vp), ("indices", _vp), ("context_lengths", _vp),
                ("batch", _i32), ("seq_len", _i32), ("num_q_heads", _i32), ("num_kv_heads", _i32),
                ("head_dim", _i32), ("top_k", _i32), ("attention_scale", _f32), ("dtype", ctypes.c_int),
                ("stream", _vp)]


class SparseDecodeParams(ctypes.Structure):
    _fields_ = [("q", _vp), ("o", _vp), ("kv_pool", _vp), ("page_table", _vp), ("indices", _vp),
                ("context_lengths", _vp), ("partial_o", _vp), ("partial_stats", _vp),
                ("batch", _i32), ("num_q_heads", _i32), ("num_kv_heads", _i32), ("head_dim", _i32),
                ("pool_head_dim", _i32), ("num_flat_pages", _i32), ("max_pages_per_seq", _i32),
                ("top_k", _i32), ("num_splits", _i32), ("attention_scale", _f32), ("dtype", ctypes.c_int),
                ("stream", _vp)]


class FrontEndParams(ctypes.Structure):
    _fields_ = [("qkv", _vp), ("q_gamma", _vp), ("k_gamma", _vp), ("context_lengths", _vp),
                ("start_positions", _vp), ("q_out", _vp), ("k_out", _vp), ("v_out", _vp), ("kv_pool", _vp),
                ("page_table", _vp), ("batch", _i32), ("seq_len", _i32), ("num_q_heads", _i32),
                ("num_kv_heads", _i32), ("head_dim", _i32), ("rot_dim", _i32), ("pool_head_dim", _i32),
                ("num_flat_pages", _i32), ("max_pages_per_seq", _i32), ("rope_theta", _f32), ("rms_eps", _f32),
                ("dtype", ctypes.c_int), ("stream", _vp)]


class IndexerPrefillParams(ctypes.Structure):
    _fields_ = [("idx_q", _vp), ("idx_k", _vp), ("q_norm_w", _vp), ("k_norm_w", _vp),
                ("context_lengths", _vp), ("indices", _vp), ("workspace", _vp), ("workspace_bytes", _sz),
                ("batch", _i32), ("seq_len", _i32), ("top_k", _i32), ("cfg", QsaIndexerConfig),
                ("dtype", ctypes.c_int), ("stream", _vp),
                ("kv_pool", _vp), ("page_table", _vp), ("num_kv_heads", _i32), ("head_dim", _i32),
                ("pool_head_dim", _i32), ("num_flat_pages", _i32), ("max_pages_per_seq", _i32)]


class IndexerDecodeParams(ctypes.Structure):
    _fields_ = [("idx_q", _vp), ("idx_k", _vp), ("q_norm_w", _vp), ("k_norm_w", _vp), ("kv_pool", _vp),
                ("page_table", _vp), ("context_lengths", _vp), ("indices", _vp), ("workspace", _vp),
                ("workspace_bytes", _sz), ("batch", _i32), ("num_kv_heads", _i32), ("head_dim", _i32),
                ("pool_head_dim", _i32), ("num_flat_pages", _i32), ("max_pages_per_seq", _i32),
                ("top_k", _i32), ("cfg", QsaIndexerConfig), ("dtype", ctypes.c_int), ("stream", _vp)]


class IndexerChunkParams(ctypes.Structure):
    _fields_ = [("idx_q", _vp), ("idx_k", _vp), ("q_norm_w", _vp), ("k_norm_w", _vp), ("kv_pool", _vp),
                ("page_table", _vp), ("start_positions", _vp), ("context_lengths", _vp), ("indices", _vp),
                ("workspace", _vp), ("workspace_bytes", _sz), ("batch", _i32), ("chunk_len", _i32),
                ("num_kv_heads", _i32), ("head_dim", _i32), ("pool_head_dim", _i32), ("num_flat_pages", _i32),
                ("max_pages_per_seq", _i32), ("top_k", _i32), ("cfg", QsaIndexerConfig), ("dtype", ctypes.c_int),
                ("stream", _vp)]


class SparseChunkParams(ctypes.Structure):
    _fields_ = [("q", _vp), ("o", _vp), ("kv_pool", _vp), ("page_table", _vp), ("indices", _vp),
                ("start_positions", _vp), ("context_lengths", _vp), ("batch", _i32), ("chunk_len", _i32),
                ("num_q_heads", _i32), ("num_kv_heads", _i32), ("head_dim", _i32), ("pool_head_dim", _i32),
                ("num_flat_pages", _i32), ("max_pages_per_seq", _i32), ("top_k", _i32), ("attention_scale", _f32),
                ("dtype", ctypes.c_int), ("stream", _vp)]


class QsaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {STATUS.get(status, status)}")
        self.status = status


_LIB = None


def load() -> ctypes.CDLL:
    """Load libqsa.so from the package directory (build it with
    ``python -m top_indexed_sparse_qsa_amd.build``)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build libqsa first "
                           "(python -m top_indexed_sparse_qsa_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, st in (("qsa_indexer_prefill", IndexerPrefillParams), ("qsa_sparse_prefill", SparsePrefillParams),
                     ("qsa_indexer_decode", IndexerDecodeParams), ("qsa_sparse_decode", SparseDecodeParams),
                     ("qsa_indexer_decode_noalloc", IndexerDecodeParams), ("qsa_qkv_front_end", FrontEndParams),
                     ("qsa_indexer_chunk", IndexerChunkParams), ("qsa_sparse_chunk", SparseChunkParams)):
        fn = getattr(lib, name)
        fn.argtypes = [ctypes.POINTER(st)]
        fn.restype = ctypes.c_int
    lib.qsa_decode_step.argtypes = [ctypes.POINTER(IndexerDecodeParams), ctypes.POINTER(SparseDecodeParams)]
    lib.qsa_decode_step.restype = ctypes.c_int
    lib.qsa_indexer_prefill_workspace_bytes.argtypes = [ctypes.POINTER(QsaIndexerConfig), _i32, _i32]
    lib.qsa_indexer_prefill_workspace_bytes.restype = _sz
    lib.qsa_indexer_decode_workspace_bytes.argtypes = [ctypes.POINTER(QsaIndexerConfig), _i32, _i32]
    lib.qsa_indexer_decode_workspace_bytes.restype = _sz
    lib.qsa_indexer_chunk_workspace_bytes.argtypes = [ctypes.POINTER(QsaIndexerConfig), _i32, _i32, _i32]
    lib.qsa_indexer_chunk_workspace_bytes.restype = _sz
    lib.qsa_sparse_decode_partial_o_elems.argtypes = [_i32, _i32, _i32]
    lib.qsa_sparse_decode_partial_o_elems.restype = _sz
    lib.qsa_sparse_decode_partial_stats_elems.argtypes = [_i32, _i32]
    lib.qsa_sparse_decode_partial_stats_elems.restype = _sz
    lib.qsa_sparse_decode_default_splits.argtypes = [_i32, _i32, _i32]
    lib.qsa_sparse_decode_default_splits.restype = _i32
    lib.qsa_status_string.argtypes = [ctypes.c_int]
    lib.qsa_status_string.restype = ctypes.c_char_p
    _LIB = lib
    return lib


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
def _ptr(t) -> int | None:
    return None if t is None else int(t.data_ptr())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float16:
        return QSA_FP16
    if t.dtype == torch.bfloat16:
        return QSA_BF16
    raise TypeError(f"libqsa takes float16 or bfloat16 tensors, got {t.dtype}")


def _stream(stream) -> int | None:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _check(fn: str, st: int) -> None:
    if st != 0:
        raise QsaError(fn, st)


def indexer_config(num_heads=4, head_dim=128, rot_dim=64, compress_ratio=4, budget=512,
                   rope_theta=1.0e6, rms_eps=1.0e-6) -> QsaIndexerConfig:
    return QsaIndexerConfig(num_heads, head_dim, rot_dim, compress_ratio, budget, rope_theta, rms_eps)


def qsa_status_string(status: int) -> str:
    return load().qsa_status_string(status).decode()


def qsa_indexer_prefill_workspace_bytes(cfg: QsaIndexerConfig, batch: int, seq_len: int) -> int:
    return int(load().qsa_indexer_prefill_workspace_bytes(ctypes.byref(cfg), batch, seq_len))


def qsa_indexer_decode_workspace_bytes(cfg: QsaIndexerConfig, batch: int, max_pages_per_seq: int) -> int:
    return int(load().qsa_indexer_decode_workspace_bytes(ctypes.byref(cfg), batch, max_pages_per_seq))


def qsa_sparse_decode_partial_o_elems(batch: int, num_kv_heads: int, head_dim: int) -> int:
    return int(load().qsa_sparse_decode_partial_o_elems(batch, num_kv_heads, head_dim))


def qsa_sparse_decode_partial_stats_elems(batch: int, num_kv_heads: int) -> int:
    return int(load().qsa_sparse_decode_partial_stats_elems(batch, num_kv_heads))


def qsa_sparse_decode_default_splits(batch: int, num_kv_heads: int, top_k: int) -> int:
    return int(load().qsa_sparse_decode_default_splits(batch, num_kv_heads, top_k))


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------
def qsa_sparse_prefill(q, k, v, o, indices, context_lengths, attention_scale: float, stream=None) -> None:
    """q, o [B,S,Hq,D]; k, v [B,S,Hkv,D]; indices int32 [B,S,top_k]; context_lengths int32 [B]."""
    B, S, Hq, D = q.shape
    p = SparsePrefillParams(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(indices), _ptr(context_lengths),
                            B, S, Hq, k.shape[2], D, indices.shape[-1], float(attention_scale),
                            _dtype_code(q), _stream(stream))
    _check("qsa_sparse_prefill", load().qsa_sparse_prefill(ctypes.byref(p)))


def qsa_sparse_decode(q, o, kv_pool, page_table, indices, context_lengths, partial_o, partial_stats,
                      attention_scale: float, head_dim: int | None = None, num_splits: int = 0,
                      stream=None) -> None:
    """q, o [B,1,Hq,D]; kv_pool [2*numPages,128,Hkv,poolHeadDim]; page_table int32 [B,2,maxPages]."""
    B, _, Hq, D = q.shape
    D = head_dim or D
    p = SparseDecodeParams(_ptr(q), _ptr(o), _ptr(kv_pool), _ptr(page_table), _ptr(indices),
                           _ptr(context_lengths), _ptr(partial_o), _ptr(partial_stats),
                           B, Hq, kv_pool.shape[2], D, kv_pool.shape[3], kv_pool.shape[0],
                           page_table.shape[-1], indices.shape[-1], num_splits, float(attention_scale),
                           _dtype_code(q), _stream(stream))
    _check("qsa_sparse_decode", load().qsa_sparse_decode(ctypes.byref(p)))


def qsa_indexer_prefill(idx_q, idx_k, q_norm_w, k_norm_w, context_lengths, indices, workspace,
                        cfg: QsaIndexerConfig, stream=None, kv_pool=None, page_table=None,
                        head_dim: int | None = None) -> None:
    """idx_q [B,S,Hi,hd]; idx_k [B,S,hd]; q_norm_w/k_norm_w fp32 [hd]; indices int32 [B,S,top_k].
    Optional handoff: kv_pool [2*numPages,128,Hkv,poolHeadDim], page_table int32 [B,2,maxPages],
    head_dim = the attention head dim (the tails start there)."""
    B, S = idx_k.shape[0], idx_k.shape[1]
    p = IndexerPrefillParams(_ptr(idx_q), _ptr(idx_k), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(context_lengths),
                             _ptr(indices), _ptr(workspace), workspace.numel() * workspace.element_size(),
                             B, S, indices.shape[-1], cfg, _dtype_code(idx_q), _stream(stream))
    if kv_pool is not None:
        p.kv_pool, p.page_table = _ptr(kv_pool), _ptr(page_table)
        p.num_kv_heads, p.pool_head_dim, p.num_flat_pages = kv_pool.shape[2], kv_pool.shape[3], kv_pool.shape[0]
        p.head_dim = int(head_dim) if head_dim is not None else 0
        p.max_pages_per_seq = page_table.shape[-1] if page_table is not None else 0
    _check("qsa_indexer_prefill", load().qsa_indexer_prefill(ctypes.byref(p)))


def qsa_indexer_decode(idx_q, idx_k, q_norm_w, k_norm_w, kv_pool, page_table, context_lengths, indices,
                       workspace, cfg: QsaIndexerConfig, head_dim: int, stream=None) -> None:
    """idx_q [B,1,Hi,hd]; idx_k [B,1,hd]; kv_pool updated in place (head-0 tails only)."""
    B = idx_k.shape[0]
    p = IndexerDecodeParams(_ptr(idx_q), _ptr(idx_k), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(kv_pool),
                            _ptr(page_table), _ptr(context_lengths), _ptr(indices), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), B, kv_pool.shape[2], head_dim,
                            kv_pool.shape[3], kv_pool.shape[0], page_table.shape[-1], indices.shape[-1], cfg,
                            _dtype_code(idx_q), _stream(stream))
    _check("qsa_indexer_decode", load().qsa_indexer_decode(ctypes.byref(p)))


def qsa_decode_step(idx_q, idx_k, q_norm_w, k_norm_w, q, o, kv_pool, page_table, context_lengths, indices,
                    workspace, cfg: QsaIndexerConfig, attention_scale: float, partial_o=None, partial_stats=None,
                    head_dim: int | None = None, num_splits: int = 0, stream=None) -> None:
    """One decode step: qsa_indexer_decode then qsa_sparse_decode over its lists, in one call.
    idx_q [B,1,Hi,hd]; idx_k [B,1,hd]; q, o [B,1,Hq,D]; kv_pool [2*numPages,128,Hkv,poolHeadDim]
    (tails updated in place); page_table int32 [B,2,maxPages]; indices int32 [B,1,top_k] (written)."""
    B, _, Hq, D = q.shape
    D = head_dim or D
    st = _stream(stream)
    ip = IndexerDecodeParams(_ptr(idx_q), _ptr(idx_k), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(kv_pool),
                             _ptr(page_table), _ptr(context_lengths), _ptr(indices), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), B, kv_pool.shape[2], D,
                             kv_pool.shape[3], kv_pool.shape[0], page_table.shape[-1], indices.shape[-1], cfg,
                             _dtype_code(idx_q), st)
    ap = SparseDecodeParams(_ptr(q), _ptr(o), _ptr(kv_pool), _ptr(page_table), _ptr(indices),
                            _ptr(context_lengths), _ptr(partial_o), _ptr(partial_stats),
                            B, Hq, kv_pool.shape[2], D, kv_pool.shape[3], kv_pool.shape[0],
                            page_table.shape[-1], indices.shape[-1], num_splits, float(attention_scale),
                            _dtype_code(q), st)
    _check("qsa_decode_step", load().qsa_decode_step(ctypes.byref(ip), ctypes.byref(ap)))


def qsa_indexer_decode_noalloc(idx_q, idx_k, q_norm_w, k_norm_w, kv_pool, page_table, context_lengths, indices,
                               cfg: QsaIndexerConfig, head_dim: int, stream=None) -> None:
    """qsa_indexer_decode with the library's own per-GPU scratch instead of a
    caller workspace (allocation-free; calls that overlap on one GPU race)."""
    B = idx_k.shape[0]
    p = IndexerDecodeParams(_ptr(idx_q), _ptr(idx_k), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(kv_pool),
                            _ptr(page_table), _ptr(context_lengths), _ptr(indices), None, 0, B, kv_pool.shape[2],
                            head_dim, kv_pool.shape[3], kv_pool.shape[0], page_table.shape[-1], indices.shape[-1],
                            cfg, _dtype_code(idx_q), _stream(stream))
    _check("qsa_indexer_decode_noalloc", load().qsa_indexer_decode_noalloc(ctypes.byref(p)))


def qsa_qkv_front_end(qkv, q_gamma, k_gamma, context_lengths, q_out, num_q_heads: int, num_kv_heads: int,
                      rot_dim: int, rope_theta: float = 1.0e6, rms_eps: float = 1.0e-6, k_out=None, v_out=None,
                      start_positions=None, kv_pool=None, page_table=None, stream=None) -> None:
    """qkv [B,S,(Hq+2Hkv)*D]; q_gamma/k_gamma fp32 [D] (folded 1+w); q_out [B,S,Hq,D]; optional mirrors
    k_out/v_out [B,S,Hkv,D], start_positions int32 [B], pool [2*numPages,128,Hkv,poolHeadDim] + page table."""
    B, S = qkv.shape[0], qkv.shape[1]
    D = q_out.shape[-1]
    p = FrontEndParams(_ptr(qkv), _ptr(q_gamma), _ptr(k_gamma), _ptr(context_lengths), _ptr(start_positions),
                       _ptr(q_out), _ptr(k_out), _ptr(v_out), _ptr(kv_pool), _ptr(page_table), B, S, num_q_heads,
                       num_kv_heads, D, rot_dim, kv_pool.shape[3] if kv_pool is not None else 0,
                       kv_pool.shape[0] if kv_pool is not None else 0,
                       page_table.shape[-1] if page_table is not None else 0, float(rope_theta), float(rms_eps),
                       _dtype_code(qkv), _stream(stream))
    _check("qsa_qkv_front_end", load().qsa_qkv_front_end(ctypes.byref(p)))


def qsa_indexer_chunk_workspace_bytes(cfg: QsaIndexerConfig, batch: int, chunk_len: int, max_pages_per_seq: int) -> int:
    return int(load().qsa_indexer_chunk_workspace_bytes(ctypes.byref(cfg), batch, chunk_len, max_pages_per_seq))


def qsa_indexer_chunk(idx_q, idx_k, q_norm_w, k_norm_w, kv_pool, page_table, start_positions, context_lengths,
                      indices, workspace, cfg: QsaIndexerConfig, head_dim: int, stream=None) -> None:
    """idx_q [B,C,Hi,hd]; idx_k [B,C,hd]; start_positions / context_lengths int32 [B] (past / total lengths);
    indices int32 [B,C,top_k]; kv_pool updated in place (head-0 tails only)."""
    B, C = idx_k.shape[0], idx_k.shape[1]
    p = IndexerChunkParams(_ptr(idx_q), _ptr(idx_k), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(kv_pool), _ptr(page_table),
                           _ptr(start_positions), _ptr(context_lengths), _ptr(indices), _ptr(workspace),
                           workspace.numel() * workspace.element_size(), B, C, kv_pool.shape[2], head_dim,
                           kv_pool.shape[3], kv_pool.shape[0], page_table.shape[-1], indices.shape[-1], cfg,
                           _dtype_code(idx_q), _stream(stream))
    _check("qsa_indexer_chunk", load().qsa_indexer_chunk(ctypes.byref(p)))


def qsa_sparse_chunk(q, o, kv_pool, page_table, indices, start_positions, context_lengths, attention_scale: float,
                     head_dim: int | None = None, stream=None) -> None:
    """q, o [B,C,Hq,D]; indices int32 [B,C,top_k]; K/V of every position read through the page table."""
    B, C, Hq, D = q.shape
    D = head_dim or D
    p = SparseChunkParams(_ptr(q), _ptr(o), _ptr(kv_pool), _ptr(page_table), _ptr(indices), _ptr(start_positions),
                          _ptr(context_lengths), B, C, Hq, kv_pool.shape[2], D, kv_pool.shape[3], kv_pool.shape[0],
                          page_table.shape[-1], indices.shape[-1], float(attention_scale), _dtype_code(q),
                          _stream(stream))
    _check("qsa_sparse_chunk", load().qsa_sparse_chunk(ctypes.byref(p)))
