"""Plain, slow CPU oracle for the QSA (Qwen Sparse Attention) hot path.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The library
(``libqsa``) never calls it and shares no code with it.

Every function computes in float64 from the exact widening of its 16-bit
inputs and rounds once, where the method keeps a narrower type.  Sources (the
pages are cited by title and section):

* [Plugin]  TensorRT-Edge-LLM, "Qsa Attention Plugin": class description,
  fused step 2 (the indexer: weight-free block-compressed scoring, per-row
  top-512 blocks, expand + causal tail into int32 lists [B, S, 2051]); the
  decode description (B1 q-prep + predicated tail write / compress, B2 block
  scores from the kbar tails, B3 deterministic top-512 + expand); the
  "KV pool contract (widened rows)" paragraph (tail layout).
* [Runner]  TensorRT-Edge-LLM, "Cute Dsl Qsa Sparse Runner": struct
  QsaSparsePrefillParams (BSND layout, list contract, zero rows past the live
  length) and struct QsaSparseDecodeParams (paged pool, page table with V
  pages pre-offset by numPages, only columns [0, headDim) read).
* [Plugin]  also its fused step 1 (packed-QKV split + per-head qk-norm with
  gammas pre-folded to 1+w + partial RoPE + paged-KV write + dense K/V
  mirrors; in decode the rope-append of the new token) and its KV pool
  contract: the leading head_size elements of a pool row hold roped K / raw
  V, the tail is the indexer's.
* [Atlas]   atlasinference, "spark_model/layers/ops/qsa.rs": doc comments of
  qsa_block_pool (mean over ratio raw keys, then RMSNorm*(1+w), then rope at
  the block-start position), qsa_qprep (per head RMSNorm*(1+w) + partial rope
  at the query position, kept in FP32), qsa_score (sum over heads of
  relu(q_h . k_b) / sqrt(hd)) and qsa_score_rows (-inf beyond each row's
  complete block count).

Readings where the pages leave a step open:
* RoPE rotates the first ``rot`` dims as pairs (i, i + rot/2) by angle
  pos * theta^(-2i/rot); dims at or past ``rot`` pass through.
* RMSNorm is x / sqrt(mean(x^2) + eps) * (1 + w), mean over the head dim.
* One indexer key head, shared by every indexer query head.
* Row t sees nc(t) = floor((t+1)/ratio) complete blocks; its causal tail is
  the (t+1) mod ratio tokens of its own incomplete block.
* With at most ``budget`` complete blocks every block is kept.  Otherwise the
  ``budget`` highest scores win and equal scores go to the lower block index.
* Lists hold the kept blocks in ascending order, each expanded to its
  ``ratio`` token ids, then the tail, then -1.  Rows at or past the live
  length are all -1.
* kbar is rounded to the activation dtype (it lives in the 16-bit pool tail
  in decode), the prepped queries to float32.
* The 32-bit float parameters the boundary receives (eps, theta, attention
  scale) are used at their float32 values.
* Chunked prefill: chunk row t of sequence b sits at position start[b] + t
  and is live while that position is below the total length ctx[b]; its
  list is the prefill list of that position (global token ids).  The
  indexer state of the positions before the chunk is the one the pool tails
  hold; a block the chunk completes is pooled from the stored raw keys of
  its earlier tokens plus the chunk's keys; after the chunk the tails hold
  what a prefill of length ctx[b] leaves.  Attention reads every key and
  value, the chunk's own included, through the page table.
* Front end: a packed QKV row holds the Hq query heads, then the Hkv key
  heads, then the Hkv value heads, D each.  q-norm and k-norm are RMSNorm
  over D with one gamma vector each (shared by the heads), received already
  folded (gamma = 1 + w); RoPE as for the indexer.  Row t of sequence b sits
  at position start[b] + t (start = 0 without past) and is live while that
  position is below the sequence's total length; only live rows reach the
  pool.  V passes through unchanged.

Storage conventions: fp16 arrays are ``np.float16``; bf16 arrays are uint16
bit patterns.
"""
from __future__ import annotations

import math

import numpy as np

# (significant bits, minimum normal exponent, largest finite value)
_FORMATS = {
    "fp16": (11, -14, 65504.0),
    "bf16": (8, -126, float(np.finfo(np.float32).max)),
    "fp32": (24, -126, float(np.finfo(np.float32).max)),
}


# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------
def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of 16-bit storage (fp16 array or bf16 bit array)."""
    a = np.asarray(a)
    if dtype == "fp16":
        return a.astype(np.float64)
    if dtype == "bf16":
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "fp32":
        return a.astype(np.float64)
    raise ValueError(dtype)


def round_to(x, fmt: str) -> np.ndarray:
    """Round float64 values to the nearest value of ``fmt`` (ties to even),
    in one step.  Returns float64 holding exactly representable values."""
    p, emin, fmax = _FORMATS[fmt]
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                       # |x| in [2^(e-1), 2^e)
    expo = np.maximum(e - 1, emin)           # exponent of the binade (subnormals clamp)
    quantum = np.ldexp(1.0, expo - (p - 1))
    y = np.rint(x / quantum) * quantum
    return np.where(np.abs(y) > fmax, np.copysign(np.inf, x), y)


def narrow(x64: np.ndarray, dtype: str) -> np.ndarray:
    """Storage form of values already representable in ``dtype``."""
    if dtype == "fp16":
        return np.asarray(x64).astype(np.float16)
    if dtype == "bf16":
        return (np.asarray(x64).astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    if dtype == "fp32":
        return np.asarray(x64).astype(np.float32)
    raise ValueError(dtype)


def f32(v: float) -> float:
    """The float32 value a 32-bit float parameter carries."""
    return float(np.float32(v))


# ---------------------------------------------------------------------------
# Indexer building blocks  [Atlas: qsa_block_pool, qsa_qprep]
# ---------------------------------------------------------------------------
def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean_d x_d^2 + eps) * (1 + w) over the last axis."""
    ms = np.mean(np.square(x), axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * (1.0 + np.asarray(w, dtype=np.float64))


def rope(x: np.ndarray, pos, rot: int, theta: float) -> np.ndarray:
    """Partial rotary embedding of the first ``rot`` dims at position ``pos``
    (broadcast against x's leading axes).  Pair (i, i + rot/2) turns by
    pos * theta^(-2i/rot)."""
    y = np.array(x, dtype=np.float64, copy=True)
    half = rot // 2
    if half == 0:
        return y
    i = np.arange(half, dtype=np.float64)
    inv_freq = theta ** ((-2.0 * i) / rot)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    a = x[..., :half]
    b = x[..., half:rot]
    y[..., :half] = a * c - b * s
    y[..., half:rot] = b * c + a * s
    return y


def pool_blocks(k_raw: np.ndarray, first_block: int, w_k, icfg, dtype: str) -> np.ndarray:
    """kbar for consecutive blocks: mean over ``ratio`` raw keys, RMSNorm*(1+w),
    rope at the block's first token position, rounded once to ``dtype``.

    k_raw: float64 [n_blocks * ratio, hd] raw keys of the blocks, in order.
    first_block: index g of the first block (sets the rope positions)."""
    r = icfg.compress_ratio
    n = k_raw.shape[0] // r
    m = k_raw[: n * r].reshape(n, r, k_raw.shape[1]).sum(axis=1) / r
    y = rms_norm(m, widen(w_k, "fp32"), f32(icfg.rms_eps))
    pos = r * (first_block + np.arange(n))
    y = rope(y, pos, icfg.rot_dim, f32(icfg.rope_theta))
    return round_to(y, dtype)


def prep_queries(q_raw: np.ndarray, pos, w_q, icfg) -> np.ndarray:
    """Indexer queries: per head RMSNorm*(1+w) then rope at the row position,
    rounded once to float32.  q_raw: float64 [..., Hi, hd]; pos broadcasts
    against the leading axes (not the head axis)."""
    y = rms_norm(q_raw, widen(w_q, "fp32"), f32(icfg.rms_eps))
    y = rope(y, np.asarray(pos)[..., None], icfg.rot_dim, f32(icfg.rope_theta))
    return round_to(y, "fp32")


def block_scores(qhat: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """s_g = sum_h relu(qhat_h . kbar_g) / sqrt(hd).  qhat [Hi, hd], kbar [n, hd]."""
    dots = kbar @ qhat.T                      # [n, Hi]
    return np.maximum(dots, 0.0).sum(axis=1) / math.sqrt(qhat.shape[-1])


def select_blocks(scores: np.ndarray, budget: int) -> np.ndarray:
    """Indices of the kept blocks, ascending.  All of them when there are at
    most ``budget``; else the ``budget`` largest scores, ties to lower index."""
    n = scores.shape[0]
    if n <= budget:
        return np.arange(n, dtype=np.int64)
    order = np.lexsort((np.arange(n), -scores))   # primary: -score, then index
    return np.sort(order[:budget])


def expand_list(t: int, kept: np.ndarray, icfg, top_k: int) -> np.ndarray:
    """Token ids of row t: each kept block g as ratio*g .. ratio*g + ratio-1,
    then the causal tail ratio*nc(t) .. t, then -1 up to ``top_k``."""
    r = icfg.compress_ratio
    nc = (t + 1) // r
    ids = (r * kept[:, None] + np.arange(r)[None, :]).reshape(-1)
    ids = np.concatenate([ids, np.arange(r * nc, t + 1)])
    assert ids.size <= top_k
    out = np.full(top_k, -1, dtype=np.int32)
    out[: ids.size] = ids
    return out


def list_length(t: int, icfg) -> int:
    """|list(t)| = ratio * min(nc(t), budget) + (t+1) mod ratio."""
    r = icfg.compress_ratio
    return r * min((t + 1) // r, icfg.budget) + (t + 1) % r


# ---------------------------------------------------------------------------
# Indexer, prefill  [Plugin: fused step 2]
# ---------------------------------------------------------------------------
def indexer_prefill(idx_q, idx_k, w_q, w_k, ctx, icfg, dtype: str, top_k: int,
                    rows=None, return_scores: bool = False):
    """Index lists for prefill.

    idx_q [B,S,Hi,hd], idx_k [B,S,hd] raw storage; ctx [B] live lengths.
    rows: iterable of (b, t) to compute, or None for every row.
    Returns int32 [B,S,top_k] (rows=None) or a dict {(b, t): int32 [top_k]}.
    With return_scores, also a dict {(b, t): float64 scores of blocks < nc(t)}.
    """
    B, S = idx_k.shape[0], idx_k.shape[1]
    r = icfg.compress_ratio
    want = ([(b, t) for b in range(B) for t in range(S)] if rows is None
            else [(int(b), int(t)) for b, t in rows])
    by_b = {}
    for b, t in want:
        by_b.setdefault(b, []).append(t)
    lists, scores = {}, {}
    for b, ts in by_b.items():
        live = min(int(ctx[b]), S)
        nblk = max(live, 0) // r
        kbar = pool_blocks(widen(idx_k[b, : nblk * r], dtype), 0, w_k, icfg, dtype)
        live_ts = [t for t in ts if t < live]
        if live_ts:
            tt = np.asarray(live_ts)
            qhat = prep_queries(widen(idx_q[b, tt], dtype), tt, w_q, icfg)
        for t in ts:
            if t >= live:
                lists[(b, t)] = np.full(top_k, -1, dtype=np.int32)
                continue
            qh = qhat[live_ts.index(t)]
            nc = (t + 1) // r
            s = block_scores(qh, kbar[:nc])
            lists[(b, t)] = expand_list(t, select_blocks(s, icfg.budget), icfg, top_k)
            if return_scores:
                scores[(b, t)] = s
    if rows is None:
        out = np.full((B, S, top_k), -1, dtype=np.int32)
        for (b, t), l in lists.items():
            out[b, t] = l
        lists = out
    return (lists, scores) if return_scores else lists


# ---------------------------------------------------------------------------
# Sparse GQA attention  [Runner: QsaSparsePrefillParams, QsaSparseDecodeParams]
# ---------------------------------------------------------------------------
def attend(q_heads: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * q k^T) v for one KV head.  q_heads [G, D] float64,
    k_rows / v_rows [n, D] float64.  No positional mask."""
    if k_rows.shape[0] == 0:
        return np.zeros_like(q_heads)
    logits = scale * (q_heads @ k_rows.T)                 # [G, n]
    logits -= logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    p /= p.sum(axis=1, keepdims=True)
    return p @ v_rows


def sparse_prefill(q, k, v, indices, ctx, scale: float, dtype: str, rows=None):
    """Sparse prefill attention over index lists.

    q [B,S,Hq,D], k/v [B,S,Hkv,D] storage; indices int32 [B,S,top_k]; ctx [B].
    Query head h reads KV head h // (Hq/Hkv).  Rows at or past ctx are +0.0.
    Returns float64 [B,S,Hq,D] (rows=None) or {(b, t): [Hq, D]}."""
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    sc = f32(scale)
    want = ([(b, t) for b in range(B) for t in range(S)] if rows is None
            else [(int(b), int(t)) for b, t in rows])
    res = {}
    for b, t in want:
        o = np.zeros((Hq, D), dtype=np.float64)
        if t < min(int(ctx[b]), S):
            ids = indices[b, t]
            ids = ids[ids >= 0]
            if ids.size:
                kr = widen(k[b, ids], dtype)             # [n, Hkv, D]
                vr = widen(v[b, ids], dtype)
                qr = widen(q[b, t], dtype)                # [Hq, D]
                for kv in range(Hkv):
                    o[kv * G:(kv + 1) * G] = attend(qr[kv * G:(kv + 1) * G], kr[:, kv], vr[:, kv], sc)
        res[(b, t)] = o
    if rows is None:
        out = np.zeros((B, S, Hq, D), dtype=np.float64)
        for (b, t), o in res.items():
            out[b, t] = o
        return out
    return res


def pool_row(pool, page_table, b: int, plane: int, token: int, page_tokens: int = 128):
    """(flat page, row) of ``token`` of sequence b in plane 0 (K) or 1 (V).
    Plane 1 page ids already include the +numPages offset."""
    return int(page_table[b, plane, token // page_tokens]), token % page_tokens


def sparse_decode(q, pool, page_table, indices, ctx, scale: float, D: int, dtype: str,
                  seqs=None, page_tokens: int = 128):
    """Single-token decode attention reading K/V through the page table.

    q [B,1,Hq,D]; pool [2*numPages,128,Hkv,poolHeadDim]; only columns [0, D)
    are used.  Returns float64 [B,Hq,D] (seqs=None) or {b: [Hq, D]}."""
    B, _, Hq, _ = q.shape
    Hkv = pool.shape[2]
    G = Hq // Hkv
    sc = f32(scale)
    want = range(B) if seqs is None else [int(b) for b in seqs]
    res = {}
    for b in want:
        o = np.zeros((Hq, D), dtype=np.float64)
        if int(ctx[b]) > 0:
            ids = indices[b, 0]
            ids = ids[ids >= 0]
            if ids.size:
                kp = page_table[b, 0, ids // page_tokens]
                vp = page_table[b, 1, ids // page_tokens]
                kr = widen(pool[kp, ids % page_tokens, :, :D], dtype)   # [n, Hkv, D]
                vr = widen(pool[vp, ids % page_tokens, :, :D], dtype)
                qr = widen(q[b, 0], dtype)
                for kv in range(Hkv):
                    o[kv * G:(kv + 1) * G] = attend(qr[kv * G:(kv + 1) * G], kr[:, kv], vr[:, kv], sc)
        res[b] = o
    if seqs is None:
        return np.stack([res[b] for b in range(B)])
    return res


# ---------------------------------------------------------------------------
# Indexer, decode  [Plugin: decode B1/B2/B3 and the KV pool contract]
# ---------------------------------------------------------------------------
def indexer_decode(idx_q, idx_k, w_q, w_k, pool, page_table, ctx, icfg, D: int, dtype: str,
                   top_k: int, seqs=None, page_tokens: int = 128, return_scores: bool = False):
    """One decode step of the indexer for each sequence.

    The indexer state lives in columns [D, D+hd) of KV head 0 of pool rows:
    block g's kbar in the V-row tail of token ratio*g, and, for the trailing
    incomplete block only, each token's raw index key in its K-row tail.

    B1: token p = ctx-1.  If its block stays incomplete (ctx mod ratio != 0)
        its raw key goes to its K-row tail; otherwise block g = ctx/ratio - 1
        is pooled from the raw tails of its first ratio-1 tokens plus the new
        key, and kbar goes to the V-row tail of token ratio*g.
    B2: scores of blocks g < floor(ctx/ratio) from the V-row tails.
    B3: top-``budget`` select and expand, as in prefill, for row p.

    The pool is not modified.  Returns (writes, lists): writes is a list of
    (flat_page, row, values[hd] storage) tail updates, lists is int32
    [B,1,top_k] (seqs=None) or {b: int32 [top_k]}.  With return_scores, also
    {b: float64 block scores}."""
    B = idx_k.shape[0]
    r = icfg.compress_ratio
    hd = icfg.head_dim
    tail = slice(D, D + hd)
    want = range(B) if seqs is None else [int(b) for b in seqs]
    writes, lists, all_scores = [], {}, {}
    for b in want:
        c = int(ctx[b])
        if c <= 0:
            lists[b] = np.full(top_k, -1, dtype=np.int32)
            continue
        p = c - 1
        new_k = widen(idx_k[b, 0], dtype)
        pending = {}
        if c % r != 0:
            pg, row = pool_row(pool, page_table, b, 0, p, page_tokens)
            writes.append((pg, row, narrow(new_k, dtype)))
        else:
            g = c // r - 1
            raw = [widen(pool[pool_row(pool, page_table, b, 0, r * g + j, page_tokens) + (0,)][tail], dtype)
                   for j in range(r - 1)] + [new_k]
            kb = pool_blocks(np.stack(raw), g, w_k, icfg, dtype)[0]
            pg, row = pool_row(pool, page_table, b, 1, r * g, page_tokens)
            writes.append((pg, row, narrow(kb, dtype)))
            pending[g] = kb
        nc = c // r
        kbar = np.empty((nc, hd), dtype=np.float64)
        for g in range(nc):
            if g in pending:
                kbar[g] = pending[g]
            else:
                pg, row = pool_row(pool, page_table, b, 1, r * g, page_tokens)
                kbar[g] = widen(pool[pg, row, 0, tail], dtype)
        qhat = prep_queries(widen(idx_q[b, 0], dtype), p, w_q, icfg)
        s = block_scores(qhat, kbar)
        all_scores[b] = s
        lists[b] = expand_list(p, select_blocks(s, icfg.budget), icfg, top_k)
    if seqs is None:
        lists = np.stack([lists[b] for b in range(B)])[:, None, :]
    return (writes, lists, all_scores) if return_scores else (writes, lists)


def indexer_chunk(idx_q, idx_k, w_q, w_k, pool, page_table, start, ctx, icfg, D: int, dtype: str, top_k: int,
                  page_tokens: int = 128, return_scores: bool = False):
    """The indexer over a chunk of rows that continue the state in the pool
    tails (decode is the chunk of one row).

    idx_q [B,C,Hi,hd], idx_k [B,C,hd] raw storage of the chunk's tokens;
    start [B] past lengths (positions of chunk row 0), ctx [B] total lengths.
    Returns (writes, lists [B,C,top_k]) with writes the tail updates in
    indexer_decode's form: the kbar of every block the chunk completes (V-row
    tail of its first token) and the raw keys of the chunk's tokens in the
    trailing incomplete block (their K-row tails).  The pool is not modified."""
    B, C = idx_k.shape[0], idx_k.shape[1]
    r, hd = icfg.compress_ratio, icfg.head_dim
    tail = slice(D, D + hd)
    writes = []
    lists = np.full((B, C, top_k), -1, dtype=np.int32)
    scores = {}
    for b in range(B):
        P, c = int(start[b]), int(ctx[b])
        if c <= P:
            continue
        raw_of = lambda j: (widen(idx_k[b, j - P], dtype) if j >= P else
                            widen(pool[pool_row(pool, page_table, b, 0, j, page_tokens) + (0,)][tail], dtype))
        nc_all = c // r
        kbar = np.empty((nc_all, hd), dtype=np.float64)
        for g in range(nc_all):
            if r * g + r <= P:           # complete before the chunk: its V-row tail holds kbar
                pg, row = pool_row(pool, page_table, b, 1, r * g, page_tokens)
                kbar[g] = widen(pool[pg, row, 0, tail], dtype)
            else:                        # completed by the chunk: pool it
                kbar[g] = pool_blocks(np.stack([raw_of(r * g + j) for j in range(r)]), g, w_k, icfg, dtype)[0]
                pg, row = pool_row(pool, page_table, b, 1, r * g, page_tokens)
                writes.append((pg, row, narrow(kbar[g], dtype)))
        for j in range(max(P, r * nc_all), c):  # the chunk's tokens of the trailing incomplete block
            pg, row = pool_row(pool, page_table, b, 0, j, page_tokens)
            writes.append((pg, row, np.asarray(idx_k[b, j - P]).copy()))
        for t in range(min(C, c - P)):
            p = P + t
            qhat = prep_queries(widen(idx_q[b, t], dtype), p, w_q, icfg)
            s = block_scores(qhat, kbar[: (p + 1) // r])
            lists[b, t] = expand_list(p, select_blocks(s, icfg.budget), icfg, top_k)
            if return_scores:
                scores[(b, t)] = s
    return (writes, lists, scores) if return_scores else (writes, lists)


def sparse_chunk(q, pool, page_table, indices, start, ctx, scale: float, D: int, dtype: str, page_tokens: int = 128):
    """Sparse attention of chunk rows over the paged pool.  q [B,C,Hq,D];
    indices [B,C,top_k]; row t of sequence b is live while start[b] + t <
    ctx[b], other rows are +0.0.  Returns float64 [B,C,Hq,D]."""
    B, C, Hq, _ = q.shape
    Hkv = pool.shape[2]
    G = Hq // Hkv
    sc = f32(scale)
    out = np.zeros((B, C, Hq, D), dtype=np.float64)
    for b in range(B):
        for t in range(C):
            if int(start[b]) + t >= int(ctx[b]):
                continue
            ids = indices[b, t]
            ids = ids[ids >= 0]
            if not ids.size:
                continue
            kp = page_table[b, 0, ids // page_tokens]
            vp = page_table[b, 1, ids // page_tokens]
            kr = widen(pool[kp, ids % page_tokens, :, :D], dtype)
            vr = widen(pool[vp, ids % page_tokens, :, :D], dtype)
            qr = widen(q[b, t], dtype)
            for kv in range(Hkv):
                out[b, t, kv * G:(kv + 1) * G] = attend(qr[kv * G:(kv + 1) * G], kr[:, kv], vr[:, kv], sc)
    return out


def prefill_state_writes(idx_k, w_k, ctx, page_table, icfg, D: int, dtype: str, page_tokens: int = 128):
    """The indexer state a prefill of each sequence leaves in the pool tails
    for decode to continue from [Plugin: "KV pool contract (widened rows)"]:
    with c = the live length, block g < floor(c/ratio) keeps its kbar (the
    value prefill scores with) in the V-row tail of token ratio*g, and each
    token of the trailing incomplete block ratio*floor(c/ratio) .. c-1 keeps
    its raw index key in its K-row tail.

    idx_k [B,S,hd] raw storage; page_table [B,2,maxPages] (plane 1 pages
    already offset by numPages).  Returns tail updates (flat_page, row,
    values[hd] storage) in the form indexer_decode returns; pages past the
    table or out of range are the caller's to avoid."""
    B, S = idx_k.shape[0], idx_k.shape[1]
    r = icfg.compress_ratio
    writes = []
    for b in range(B):
        c = min(int(ctx[b]), S)
        if c <= 0:
            continue
        nc = c // r
        kbar = pool_blocks(widen(idx_k[b, : nc * r], dtype), 0, w_k, icfg, dtype)
        for g in range(nc):
            pg, row = pool_row(None, page_table, b, 1, r * g, page_tokens)
            writes.append((pg, row, narrow(kbar[g], dtype)))
        for j in range(nc * r, c):
            pg, row = pool_row(None, page_table, b, 0, j, page_tokens)
            writes.append((pg, row, idx_k[b, j].copy()))
    return writes


# ---------------------------------------------------------------------------
# Front end  [Plugin: fused step 1, KV pool contract]
# ---------------------------------------------------------------------------
def rms_norm_gamma(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean_d x_d^2 + eps) * gamma over the last axis; gamma is the
    folded gain (1 + w)."""
    ms = np.mean(np.square(x), axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)


def split_packed_qkv(qkv: np.ndarray, Hq: int, Hkv: int, D: int):
    """[..., (Hq + 2 Hkv) D] -> q [..., Hq, D], k [..., Hkv, D], v [..., Hkv, D]."""
    lead = qkv.shape[:-1]
    assert qkv.shape[-1] == (Hq + 2 * Hkv) * D
    q = qkv[..., : Hq * D].reshape(*lead, Hq, D)
    k = qkv[..., Hq * D: (Hq + Hkv) * D].reshape(*lead, Hkv, D)
    v = qkv[..., (Hq + Hkv) * D:].reshape(*lead, Hkv, D)
    return q, k, v


def front_end(qkv, q_gamma, k_gamma, ctx, Hq: int, Hkv: int, D: int, rot: int, theta: float, eps: float,
              dtype: str, start=None, page_table=None, page_tokens: int = 128):
    """Packed QKV -> (q, k, v, pool_writes).

    qkv [B, S, (Hq+2Hkv) D] storage; q_gamma, k_gamma fp32 [D] (folded 1+w);
    ctx [B] total lengths; start [B] past lengths or None (all 0).
    q [B,S,Hq,D] and k [B,S,Hkv,D]: qk-norm then rope at the row's position,
    rounded once to dtype; v [B,S,Hkv,D]: unchanged.  Every row is computed;
    pool_writes, with a page table, lists for each live row (position <
    ctx[b]) (flat_page, row, 'k' or 'v' plane, values [Hkv, D] storage), the
    leading D columns of that token's K and V pool rows."""
    B, S = qkv.shape[0], qkv.shape[1]
    st = np.zeros(B, dtype=np.int64) if start is None else np.asarray(start, dtype=np.int64)
    x = widen(qkv, dtype)
    q_raw, k_raw, _ = split_packed_qkv(x, Hq, Hkv, D)
    pos = st[:, None] + np.arange(S)[None, :]                         # [B, S]
    eps32, theta32 = f32(eps), f32(theta)
    q = rope(rms_norm_gamma(q_raw, widen(q_gamma, "fp32"), eps32), pos[..., None], rot, theta32)
    k = rope(rms_norm_gamma(k_raw, widen(k_gamma, "fp32"), eps32), pos[..., None], rot, theta32)
    q, k = round_to(q, dtype), round_to(k, dtype)
    writes = []
    if page_table is not None:
        for b in range(B):
            for t in range(S):
                p = int(pos[b, t])
                if p >= int(ctx[b]):
                    continue
                pk, row = pool_row(None, page_table, b, 0, p, page_tokens)
                pv, _ = pool_row(None, page_table, b, 1, p, page_tokens)
                writes.append((pk, row, "k", narrow(k[b, t], dtype)))
                writes.append((pv, row, "v", np.asarray(qkv[b, t, (Hq + Hkv) * D:]).reshape(Hkv, D).copy()))
    v = np.asarray(qkv)[..., (Hq + Hkv) * D:].reshape(B, S, Hkv, D).copy()   # raw V, storage unchanged
    return narrow(q, dtype), narrow(k, dtype), v, writes


def apply_front_end_writes(pool: np.ndarray, writes, D: int) -> None:
    """Apply front_end's pool writes in place: columns [0, D) of every head."""
    for pg, row, _, vals in writes:
        pool[pg, row, :, :D] = vals


def apply_tail_writes(pool: np.ndarray, writes, D: int) -> None:
    """Apply indexer_decode's tail updates to a pool in place (head 0)."""
    for pg, row, vals in writes:
        pool[pg, row, 0, D:D + vals.shape[0]] = vals
