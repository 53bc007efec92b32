"""Seeded synthetic inputs for the QSA hot path.

This module only draws random data and lays it out; it holds none of the
method's arithmetic.  Both the CPU oracle's tests and the GPU path's tests and
bench draw their inputs here, so the two sides always see the same bytes.

Conventions
-----------
* Generator: NumPy ``default_rng(seed)`` (PCG64).
* Activations are drawn as float32 N(0, 1) and rounded to nearest-even into
  the storage dtype.  fp16 is stored as ``np.float16``; bf16 is stored as its
  16-bit pattern in ``np.uint16`` (NumPy has no bfloat16).
* Norm weights are float32 N(0, 0.1^2) (std 0.1), one ``[hd]`` vector for the
  indexer queries and one for the indexer keys.
* Draw order for a prefill workload: Q, K, V, idx_q, idx_k, w_q, w_k, then
  extras.  For a decode workload: q, idx_q, idx_k, w_q, w_k, context lengths,
  page permutation, pool.

The five named workloads follow the shapes of the pages' contract (dense
padded BSND prefill, a 128-token paged pool for decode, a 4 x 128 indexer with
a 512-block budget and compress ratio 4, lists of 2051 ids).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

PAGE_TOKENS = 128


@dataclass(frozen=True)
class IndexerCfg:
    num_heads: int = 4
    head_dim: int = 128
    rot_dim: int = 64
    compress_ratio: int = 4
    budget: int = 512
    rope_theta: float = 1.0e6
    rms_eps: float = 1.0e-6

    @property
    def top_k(self) -> int:
        # budget whole blocks plus at most ratio-1 tail tokens
        return self.budget * self.compress_ratio + self.compress_ratio - 1


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest-even) and return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "fp16":
        return x.astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def normal(rng: np.random.Generator, shape, dtype: str, chunk: int = 1 << 26) -> np.ndarray:
    """float32 N(0,1) rounded into ``dtype`` storage, drawn in chunks."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float16 if dtype == "fp16" else np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = to_storage(rng.standard_normal(e - s, dtype=np.float32), dtype)
    return out.reshape(shape)


def norm_weights(rng: np.random.Generator, hd: int) -> np.ndarray:
    return (rng.standard_normal(hd, dtype=np.float32) * np.float32(0.1)).astype(np.float32)


@dataclass
class PrefillInputs:
    B: int
    S: int
    Hq: int
    Hkv: int
    D: int
    dtype: str
    scale: float
    ctx: np.ndarray            # int32 [B]
    q: np.ndarray              # [B,S,Hq,D]
    k: np.ndarray              # [B,S,Hkv,D]
    v: np.ndarray              # [B,S,Hkv,D]
    idx_q: np.ndarray | None = None   # [B,S,Hi,hd]
    idx_k: np.ndarray | None = None   # [B,S,hd]
    w_q: np.ndarray | None = None     # fp32 [hd]
    w_k: np.ndarray | None = None     # fp32 [hd]
    indices: np.ndarray | None = None # int32 [B,S,top_k] when lists are given
    top_k: int = 0
    icfg: IndexerCfg = field(default_factory=IndexerCfg)


def make_prefill(seed: int, B: int, S: int, Hq: int, Hkv: int, D: int, dtype: str,
                 ctx, scale: float | None = None, icfg: IndexerCfg | None = None,
                 with_indexer: bool = True, rng: np.random.Generator | None = None) -> PrefillInputs:
    icfg = icfg or IndexerCfg()
    rng = rng if rng is not None else np.random.default_rng(seed)
    q = normal(rng, (B, S, Hq, D), dtype)
    k = normal(rng, (B, S, Hkv, D), dtype)
    v = normal(rng, (B, S, Hkv, D), dtype)
    inp = PrefillInputs(B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype,
                        scale=float(np.float32(scale if scale is not None else 1.0 / math.sqrt(D))),
                        ctx=np.asarray(ctx, dtype=np.int32).reshape(B), q=q, k=k, v=v,
                        top_k=icfg.top_k, icfg=icfg)
    if with_indexer:
        hi, hd = icfg.num_heads, icfg.head_dim
        inp.idx_q = normal(rng, (B, S, hi, hd), dtype)
        inp.idx_k = normal(rng, (B, S, hd), dtype)
        inp.w_q = norm_weights(rng, hd)
        inp.w_k = norm_weights(rng, hd)
    return inp


def random_lists(rng: np.random.Generator, B: int, S: int, top_k: int, ctx) -> np.ndarray:
    """Row t lists min(t+1, top_k) distinct ids drawn uniformly from [0, t],
    in drawn (unsorted) order, -1 padded on the right.  Rows at or past the
    live length are all -1."""
    out = np.full((B, S, top_k), -1, dtype=np.int32)
    for b in range(B):
        for t in range(min(S, int(ctx[b]))):
            n = min(t + 1, top_k)
            out[b, t, :n] = rng.choice(t + 1, n, replace=False)
    return out


@dataclass
class DecodeInputs:
    B: int
    Hq: int
    Hkv: int
    D: int
    pool_head_dim: int
    dtype: str
    scale: float
    ctx: np.ndarray            # int32 [B], total length incl. the new token
    num_pages: int             # K pages; the pool holds 2*num_pages
    max_pages: int
    q: np.ndarray              # [B,1,Hq,D]
    idx_q: np.ndarray          # [B,1,Hi,hd]
    idx_k: np.ndarray          # [B,1,hd]
    w_q: np.ndarray
    w_k: np.ndarray
    page_table: np.ndarray     # int32 [B,2,max_pages]; row 1 = row 0 + num_pages
    pool: np.ndarray           # [2*num_pages,128,Hkv,pool_head_dim]
    top_k: int = 0
    icfg: IndexerCfg = field(default_factory=IndexerCfg)


def make_decode(seed: int, ctx=None, B: int = 32, Hq: int = 32, Hkv: int = 4, D: int = 128,
                dtype: str = "fp16", ctx_range=(8192, 65536), max_pages: int = 512,
                scale: float | None = None, icfg: IndexerCfg | None = None) -> DecodeInputs:
    icfg = icfg or IndexerCfg()
    rng = np.random.default_rng(seed)
    hi, hd = icfg.num_heads, icfg.head_dim
    phd = D + hd
    q = normal(rng, (B, 1, Hq, D), dtype)
    idx_q = normal(rng, (B, 1, hi, hd), dtype)
    idx_k = normal(rng, (B, 1, hd), dtype)
    w_q = norm_weights(rng, hd)
    w_k = norm_weights(rng, hd)
    if ctx is None:
        ctx = rng.integers(ctx_range[0], ctx_range[1], size=B, endpoint=True)
    ctx = np.asarray(ctx, dtype=np.int32).reshape(B)
    pages_per = [(int(c) + PAGE_TOKENS - 1) // PAGE_TOKENS for c in ctx]
    assert max(pages_per) <= max_pages
    num_pages = max(1, sum(pages_per))
    perm = rng.permutation(num_pages).astype(np.int32)
    pt = np.full((B, 2, max_pages), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(pages_per):
        pt[b, 0, :n] = perm[off:off + n]
        pt[b, 1, :n] = perm[off:off + n] + num_pages
        off += n
    pool = normal(rng, (2 * num_pages, PAGE_TOKENS, Hkv, phd), dtype)
    return DecodeInputs(B=B, Hq=Hq, Hkv=Hkv, D=D, pool_head_dim=phd, dtype=dtype,
                        scale=float(np.float32(scale if scale is not None else 1.0 / math.sqrt(D))),
                        ctx=ctx, num_pages=num_pages, max_pages=max_pages, q=q, idx_q=idx_q,
                        idx_k=idx_k, w_q=w_q, w_k=w_k, page_table=pt, pool=pool,
                        top_k=icfg.top_k, icfg=icfg)


@dataclass
class FrontEndInputs:
    B: int
    S: int
    Hq: int
    Hkv: int
    D: int
    dtype: str
    rot: int
    ctx: np.ndarray            # int32 [B] total lengths
    start: np.ndarray | None   # int32 [B] past lengths, or None
    qkv: np.ndarray            # [B,S,(Hq+2Hkv)*D]
    q_gamma: np.ndarray        # fp32 [D], 1 + N(0, 0.1^2)
    k_gamma: np.ndarray
    num_pages: int
    max_pages: int
    page_table: np.ndarray     # int32 [B,2,max_pages]
    pool: np.ndarray           # [2*num_pages,128,Hkv,D+128]


def make_front_end(seed: int, B: int, S: int, Hq: int, Hkv: int, D: int, dtype: str, ctx, rot: int,
                   start=None, max_pages: int | None = None, tail: int = 128) -> FrontEndInputs:
    """Packed QKV rows, folded gains 1 + N(0, 0.1^2), and a pool with a
    seeded page permutation holding every position below ctx.  Draw order:
    qkv, q gain, k gain, page permutation, pool."""
    rng = np.random.default_rng(seed)
    qkv = normal(rng, (B, S, (Hq + 2 * Hkv) * D), dtype)
    q_gamma = (1.0 + norm_weights(rng, D)).astype(np.float32)
    k_gamma = (1.0 + norm_weights(rng, D)).astype(np.float32)
    ctx = np.asarray(ctx, dtype=np.int32).reshape(B)
    pages_per = [(int(c) + PAGE_TOKENS - 1) // PAGE_TOKENS for c in ctx]
    max_pages = max_pages or max(1, max(pages_per))
    num_pages = max(1, sum(pages_per))
    perm = rng.permutation(num_pages).astype(np.int32)
    pt = np.full((B, 2, max_pages), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(pages_per):
        pt[b, 0, :n] = perm[off:off + n]
        pt[b, 1, :n] = perm[off:off + n] + num_pages
        off += n
    pool = normal(rng, (2 * num_pages, PAGE_TOKENS, Hkv, D + tail), dtype)
    return FrontEndInputs(B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, rot=rot, ctx=ctx,
                          start=None if start is None else np.asarray(start, dtype=np.int32).reshape(B),
                          qkv=qkv, q_gamma=q_gamma, k_gamma=k_gamma, num_pages=num_pages, max_pages=max_pages,
                          page_table=pt, pool=pool)


# ---------------------------------------------------------------------------
# The five named workloads.  Seed = workload number.
# ---------------------------------------------------------------------------
WORKLOADS = {
    1: "tiny fixed-list sparse prefill: B=1 S=64 Hq=4 Hkv=1 D=64 fp16 topK=16 scale 1/8",
    2: "indexer + sparse prefill: B=1 S=4096 Hq=16 Hkv=2 D=128 fp16 topK=2051",
    3: "long indexer + sparse prefill: B=1 S=32768 Hq=32 Hkv=4 D=128 fp16 topK=2051",
    4: "paged split-K decode: B=32 ctx~U[8192,65536] Hq=32 Hkv=4 D=128 pool_head_dim=256 fp16 topK=2051",
    5: "ragged prefill: B=4 S=16384 ctx={16384,12000,8000,3000} Hq=64 Hkv=4 D=128 bf16 topK=2051",
}


def workload(n: int):
    if n == 1:
        rng = np.random.default_rng(1)
        inp = make_prefill(1, B=1, S=64, Hq=4, Hkv=1, D=64, dtype="fp16", ctx=[64],
                           scale=1.0 / 8.0, with_indexer=False, rng=rng)
        inp.top_k = 16
        inp.indices = random_lists(rng, 1, 64, 16, inp.ctx)
        return inp
    if n == 2:
        return make_prefill(2, B=1, S=4096, Hq=16, Hkv=2, D=128, dtype="fp16", ctx=[4096])
    if n == 3:
        return make_prefill(3, B=1, S=32768, Hq=32, Hkv=4, D=128, dtype="fp16", ctx=[32768])
    if n == 4:
        return make_decode(4)
    if n == 5:
        return make_prefill(5, B=4, S=16384, Hq=64, Hkv=4, D=128, dtype="bf16",
                            ctx=[16384, 12000, 8000, 3000])
    raise ValueError(n)
