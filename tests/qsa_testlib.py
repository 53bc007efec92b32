"""Helpers shared by the GPU parity tests: moving seeded inputs to the device
and the comparison rules between the HIP path and the oracle.

Comparison rules
* Attention output: |gpu - oracle| <= 2e-3 (fp16) or 1e-2 (bf16), or within
  one unit in the last place of the 16-bit dtype at the oracle value (a
  correctly rounded output of magnitude >= 8 (fp16) / >= 4 (bf16) can exceed
  the absolute bound).  Rows past the live length must be +0.0 bit for bit.
* Index lists: same number of valid ids, -1 exactly on the right, the same
  causal tail, whole blocks only; blocks in the symmetric difference of the
  kept sets must sit within a relative margin 1e-5 of the cut:
  |s_b - s*| / s_max < 1e-5 with s* the oracle's budget-th score and s_max its
  largest.  Rows with no more complete blocks than the budget get no
  allowance.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from oracle import qsa_oracle as O

ATTN_TOL = {"fp16": 2e-3, "bf16": 1e-2}
MARGIN = 1e-5


def dev(a: np.ndarray, dtype: str | None = None, device="cuda"):
    """numpy storage array -> device tensor (fp16, bf16 bits, int32, fp32)."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host_f64(t, dtype: str) -> np.ndarray:
    """Device 16-bit tensor -> exact float64 numpy values."""
    t = t.detach().cpu()
    if dtype == "bf16":
        return O.widen(t.view(torch.int16).numpy().view(np.uint16), "bf16")
    return t.numpy().astype(np.float64)


def ulp16(x: np.ndarray, dtype: str) -> np.ndarray:
    p = 11 if dtype == "fp16" else 8
    emin = -14 if dtype == "fp16" else -126
    _, e = np.frexp(np.abs(x))
    return np.ldexp(1.0, np.maximum(e - 1, emin) - (p - 1))


def check_attention(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "") -> dict:
    err = np.abs(got - ref)
    tol = ATTN_TOL[dtype]
    within_tol = err <= tol
    within_ulp = err <= ulp16(ref, dtype)
    ok = within_tol | within_ulp
    if not ok.all():
        i = np.unravel_index(np.argmax(np.where(ok, 0, err)), err.shape)
        raise AssertionError(f"{what}: {int((~ok).sum())} elements out of tolerance; worst at {i}: "
                             f"gpu {got[i]!r} oracle {ref[i]!r} err {err[i]:.3e} (tol {tol})")
    return {"max_err": float(err.max()) if err.size else 0.0, "ulp_clause": int((~within_tol).sum())}


def check_zero_rows(gpu_rows: torch.Tensor, what: str = "") -> None:
    bits = gpu_rows.detach().contiguous().view(torch.int16)
    assert int((bits != 0).sum()) == 0, f"{what}: rows past the live length are not +0.0"


def check_list(got: np.ndarray, ref: np.ndarray, scores: np.ndarray | None, t: int, icfg,
               what: str = "") -> bool:
    """Compare one GPU list with the oracle's.  Returns True when the boundary
    allowance was used."""
    r, budget = icfg.compress_ratio, icfg.budget
    n_ref = int((ref >= 0).sum())
    valid = got >= 0
    n = int(valid.sum())
    assert n == n_ref, f"{what} t={t}: {n} valid ids, oracle {n_ref}"
    assert valid[:n].all() and not valid[n:].any(), f"{what} t={t}: -1 not only on the right"
    if n_ref == 0:          # a row past the live length: all -1 on both sides
        return False
    ids = got[:n].astype(np.int64)
    nc = (t + 1) // r
    tail = np.sort(ids[ids >= r * nc])
    assert np.array_equal(tail, np.arange(r * nc, t + 1)), f"{what} t={t}: wrong causal tail"
    body = np.sort(ids[ids < r * nc])
    assert body.size % r == 0
    blk = body.reshape(-1, r)
    assert np.all(blk == blk[:, :1] + np.arange(r)) and np.all(blk[:, 0] % r == 0), \
        f"{what} t={t}: ids are not whole blocks"
    assert len(set(ids.tolist())) == n, f"{what} t={t}: duplicate ids"
    g_got = set((blk[:, 0] // r).tolist())
    rid = ref[:n_ref].astype(np.int64)
    g_ref = set((rid[rid < r * nc] // r).tolist())
    sym = g_got ^ g_ref
    if not sym:
        return False
    assert nc > budget and scores is not None, f"{what} t={t}: kept blocks differ ({sorted(sym)[:8]})"
    order = np.sort(scores)[::-1]
    s_star, s_max = order[budget - 1], order[0]
    margins = [abs(scores[g] - s_star) / s_max for g in sym]
    assert max(margins) < MARGIN, \
        f"{what} t={t}: swap of blocks {sorted(sym)[:8]} with relative margin {max(margins):.3e}"
    return True


def check_list_invariants_all_rows(lists: np.ndarray, ctx, icfg, what: str = "", row0: int = 0) -> int:
    """Every row of an index-list array [B, S, top_k] against the closed forms
    the method fixes, vectorised: |list(t)| = r*min(nc, budget) + (t+1) mod r,
    -1 exactly on the right, the causal tail {r*nc .. t} present, the rest
    whole aligned blocks of r ids below r*nc, all ids distinct and <= t; rows
    at or past the live length all -1.  Rows below row0 are not checked (a
    chunk's rows start there).  Returns the rows checked."""
    r, budget = icfg.compress_ratio, icfg.budget
    B, S, K = lists.shape
    big = np.iinfo(np.int32).max
    checked = 0
    for b in range(B):
        live = min(int(ctx[b]), S)
        assert np.all(lists[b, live:] == -1), f"{what} b={b}: a row past the live length is not all -1"
        if live <= row0:
            continue
        L = lists[b, row0:live]
        t = np.arange(row0, live)
        nc = (t + 1) // r
        n_exp = r * np.minimum(nc, budget) + (t + 1) % r
        valid = L >= 0
        n = valid.sum(axis=1)
        bad = np.nonzero(n != n_exp)[0]
        assert bad.size == 0, f"{what} b={b}: row {bad[0]} has {n[bad[0]]} ids, expected {n_exp[bad[0]]}"
        right = np.arange(K)[None, :] < n[:, None]
        assert np.array_equal(valid, right), f"{what} b={b}: -1 not only on the right"
        srt = np.sort(np.where(valid, L, big), axis=1)
        # distinct
        dup = (srt[:, 1:] == srt[:, :-1]) & (srt[:, 1:] != big)
        assert not dup.any(), f"{what} b={b}: duplicate ids in row {np.nonzero(dup.any(1))[0][0]}"
        # all ids <= t: the largest valid id is the last one of the sorted valid part
        last = srt[np.arange(t.size), n - 1]
        assert np.all(last <= t), f"{what} b={b}: an id past its row"
        # the tail: the (t+1) mod r largest ids are r*nc .. t
        tl = (t + 1) % r
        for j in range(1, r):
            rows = np.nonzero(tl >= j)[0]
            if rows.size:
                want = t[rows] - (j - 1)
                got = srt[rows, n[rows] - j]
                assert np.array_equal(got, want), f"{what} b={b}: wrong causal tail in row {rows[np.argmax(got != want)]}"
        # the body: whole aligned blocks below r*nc
        nb = n - tl                         # ids in whole blocks
        col = np.arange(K)[None, :]
        body = col < nb[:, None]
        ids = np.where(body, srt, 0)
        first = ids[:, ::r] if r > 1 else ids
        assert np.all((first % r == 0) | ~body[:, ::r]), f"{what} b={b}: a block does not start at a multiple of r"
        for j in range(1, r):
            cj = ids[:, j::r][:, :first.shape[1]]
            mask = body[:, j::r][:, :first.shape[1]]
            assert np.all((cj == first[:, :cj.shape[1]] + j) | ~mask), f"{what} b={b}: ids are not whole blocks"
        assert np.all(np.where(body, srt, -1) < (r * nc)[:, None]), f"{what} b={b}: a block reaches the tail"
        checked += t.size
    return checked


def structured_lists(rng: np.random.Generator, B: int, S: int, ctx, icfg, top_k: int,
                     shuffle: bool = True) -> np.ndarray:
    """Lists with the shape the indexer produces -- min(nc, budget) whole
    blocks drawn at random, the causal tail, -1 padding -- without scoring.
    Seeded synthetic attention input for full-size parity runs."""
    r, budget = icfg.compress_ratio, icfg.budget
    out = np.full((B, S, top_k), -1, dtype=np.int32)
    for b in range(B):
        for t in range(min(int(ctx[b]), S)):
            nc = (t + 1) // r
            if nc <= budget:
                ids = np.arange(t + 1)
            else:
                g = rng.choice(nc, budget, replace=False)
                ids = np.concatenate([(r * g[:, None] + np.arange(r)).reshape(-1), np.arange(r * nc, t + 1)])
            if shuffle:
                ids = rng.permutation(ids)
            out[b, t, :ids.size] = ids
    return out


def sample_rows(B: int, S: int, ctx, n_per_b: int, rng: np.random.Generator):
    """Rows to check at full size: the first rows, rows around the point where
    selection starts (t ~ 2050), the last live rows, a few dead rows and a
    random spread."""
    rows = []
    for b in range(B):
        live = min(int(ctx[b]), S)
        fixed = [0, 1, 2, 3, 4, 5, 2045, 2046, 2047, 2048, 2049, 2050, 2051, 2052, 2053, 2054,
                 live - 3, live - 2, live - 1, live, live + 1, S - 1]
        rnd = rng.integers(0, S, size=n_per_b).tolist()
        rows += [(b, t) for t in sorted(set(x for x in fixed + rnd if 0 <= x < S))]
    return rows


def idx_cfg_struct(icfg):
    import top_indexed_sparse_qsa_amd as q
    return q.indexer_config(icfg.num_heads, icfg.head_dim, icfg.rot_dim, icfg.compress_ratio, icfg.budget,
                            icfg.rope_theta, icfg.rms_eps)


def log(msg: str) -> None:
    print(msg, flush=True)
