"""libqsa: the QSA (Qwen Sparse Attention) hot path on AMD MI355X (gfx950).

The compute lives in libqsa.so (hand-written HIP kernels behind a C ABI,
declared in include/libqsa.h).  This package is its thin ctypes binding:
the functions below marshal torch tensors into the C parameter structs and
call the library.  Import does not load the library; the first call does,
and raises if it is missing.
"""
from ._lib import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    QSA_BF16,
    QSA_FP16,
    QSA_MAX_BLOCKS,
    QSA_MAX_SPLITS,
    QSA_NOALLOC_SCRATCH_BYTES,
    QSA_PAGE_TOKENS,
    QSA_PARTIAL_ROWS,
    QsaError,
    QsaIndexerConfig,
    indexer_config,
    load,
    qsa_decode_step,
    qsa_indexer_chunk,
    qsa_indexer_chunk_workspace_bytes,
    qsa_indexer_decode,
    qsa_indexer_decode_noalloc,
    qsa_indexer_decode_workspace_bytes,
    qsa_indexer_prefill,
    qsa_indexer_prefill_workspace_bytes,
    qsa_qkv_front_end,
    qsa_sparse_chunk,
    qsa_sparse_decode,
    qsa_sparse_decode_default_splits,
    qsa_sparse_decode_partial_o_elems,
    qsa_sparse_decode_partial_stats_elems,
    qsa_sparse_prefill,
    qsa_status_string,
)
