"""Chunked prefill over the paged pool (qsa_indexer_chunk + qsa_sparse_chunk,
through the C ABI) against the oracle, and against the library's own one-shot
prefill: a sequence prefilled to P (state handed to the pool tails), then a
chunk of the tokens P .. N-1, selects for those rows what a prefill of N
selects and leaves the tails a prefill of N leaves."""
import numpy as np
import pytest
import torch

import qsa_synth as syn
import qsa_testlib as TL
import top_indexed_sparse_qsa_amd as Q
from oracle import qsa_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("a gpu test ran without a GPU")
    Q.load()
    yield
    torch.cuda.synchronize()


def paged_state(rng, inp, N, max_pages):
    """Pool with the K/V of positions < N (leading columns) through a
    permuted page table; random tails."""
    B, Hkv, D, hd = inp.B, inp.Hkv, inp.D, inp.icfg.head_dim
    pages = (N + 127) // 128
    npg = B * pages
    perm = rng.permutation(npg).astype(np.int32)
    pt = np.full((B, 2, max_pages), -1, dtype=np.int32)
    for b in range(B):
        pt[b, 0, :pages] = perm[b * pages:(b + 1) * pages]
        pt[b, 1, :pages] = pt[b, 0, :pages] + npg
    pool = syn.normal(rng, (2 * npg, 128, Hkv, D + hd), inp.dtype)
    tok = np.arange(N)
    for b in range(B):
        pool[pt[b, 0, tok // 128], tok % 128, :, :D] = inp.k[b, :N]
        pool[pt[b, 1, tok // 128], tok % 128, :, :D] = inp.v[b, :N]
    return pool, pt


def gpu_chunk(inp, pool_dev, pt, P, ctx, C):
    icfg = inp.icfg
    cfg = TL.idx_cfg_struct(icfg)
    B = inp.B
    start = np.full(B, P, dtype=np.int32)
    ws = torch.empty(Q.qsa_indexer_chunk_workspace_bytes(cfg, B, C, pt.shape[-1]), dtype=torch.uint8, device="cuda")
    lists = torch.full((B, C, icfg.top_k), -7, dtype=torch.int32, device="cuda")
    iq = np.ascontiguousarray(inp.idx_q[:, P:P + C])
    ik = np.ascontiguousarray(inp.idx_k[:, P:P + C])
    Q.qsa_indexer_chunk(TL.dev(iq, inp.dtype), TL.dev(ik, inp.dtype), TL.dev(inp.w_q), TL.dev(inp.w_k), pool_dev,
                        TL.dev(pt), TL.dev(start), TL.dev(ctx), lists, ws, cfg, inp.D)
    q = TL.dev(np.ascontiguousarray(inp.q[:, P:P + C]), inp.dtype)
    o = torch.full_like(q, float("nan"))
    Q.qsa_sparse_chunk(q, o, pool_dev, TL.dev(pt), lists, TL.dev(start), TL.dev(ctx), inp.scale, head_dim=inp.D)
    torch.cuda.synchronize()
    return lists, o, start


CASES = [
    dict(P=300, N=377, S=400, budget=8, dtype="fp16", B=2, Hq=8, Hkv=2, D=128),
    dict(P=301, N=390, S=400, budget=8, dtype="bf16", B=1, Hq=16, Hkv=1, D=64),
    dict(P=302, N=303, S=303, budget=5, dtype="fp16", B=2, Hq=4, Hkv=4, D=64),
    dict(P=2040, N=2233, S=2233, budget=512, dtype="bf16", B=1, Hq=8, Hkv=2, D=128),
    dict(P=0, N=150, S=150, budget=8, dtype="fp16", B=1, Hq=2, Hkv=1, D=64),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"P{c['P']}N{c['N']}b{c['budget']}{c['dtype']}")
def test_chunk_matches_oracle_and_one_shot_prefill(case):
    c = dict(case)
    P, N, S, budget = c.pop("P"), c.pop("N"), c.pop("S"), c.pop("budget")
    icfg = syn.IndexerCfg(budget=budget)
    TL.log(f"chunk {case}")
    inp = syn.make_prefill(70 + P, S=S, ctx=[N] * c["B"], icfg=icfg, **c)
    rng = np.random.default_rng(70 + N)
    max_pages = (S + 127) // 128 + 1
    pool, pt = paged_state(rng, inp, N, max_pages)
    start = np.full(inp.B, P, dtype=np.int32)
    ctx = np.full(inp.B, N, dtype=np.int32)
    O.apply_tail_writes(pool, O.prefill_state_writes(inp.idx_k, inp.w_k, start, pt, icfg, inp.D, inp.dtype), inp.D)
    C = N - P + 3                       # three padding rows past the total length
    pool_dev = TL.dev(pool, inp.dtype)
    pad = lambda a: np.concatenate([a, np.zeros_like(a[:, :3])], axis=1) if P + C > S else a
    inp.idx_q, inp.idx_k, inp.q = pad(inp.idx_q), pad(inp.idx_k), pad(inp.q)
    lists, o, _ = gpu_chunk(inp, pool_dev, pt, P, ctx, C)
    got = lists.cpu().numpy()
    # the oracle's chunk: lists (margin rule) and tail writes (bit for bit)
    writes, ref, scores = O.indexer_chunk(inp.idx_q[:, P:P + C], inp.idx_k[:, P:P + C], inp.w_q, inp.w_k, pool, pt,
                                          start, ctx, icfg, inp.D, inp.dtype, icfg.top_k, return_scores=True)
    same = []
    for b in range(inp.B):
        for t in range(C):
            if P + t >= N:
                assert np.all(got[b, t] == -1), f"padding row {t}"
                continue
            if not TL.check_list(got[b, t], ref[b, t], scores.get((b, t)), P + t, icfg, f"chunk b={b}"):
                same.append((b, t))
    expect = pool.copy()
    O.apply_tail_writes(expect, writes, inp.D)
    assert torch.equal(pool_dev.view(torch.int16), TL.dev(expect, inp.dtype).view(torch.int16)), "pool after chunk"
    # attention of the live rows whose lists agree
    ref_o = O.sparse_chunk(inp.q[:, P:P + C], pool, pt, ref, start, ctx, inp.scale, inp.D, inp.dtype)
    got_o = TL.host_f64(o, inp.dtype)
    for (b, t) in same:
        TL.check_attention(got_o[b, t], ref_o[b, t], inp.dtype, f"chunk attention b={b} t={t}")
    for b in range(inp.B):
        TL.check_zero_rows(o[b, N - P:], "chunk padding rows")
    # the library's one-shot prefill of N selects the same, bit for bit
    cfg = TL.idx_cfg_struct(icfg)
    ws = torch.empty(Q.qsa_indexer_prefill_workspace_bytes(cfg, inp.B, S), dtype=torch.uint8, device="cuda")
    one = torch.full((inp.B, S, icfg.top_k), -7, dtype=torch.int32, device="cuda")
    Q.qsa_indexer_prefill(TL.dev(np.ascontiguousarray(inp.idx_q[:, :S]), inp.dtype),
                          TL.dev(np.ascontiguousarray(inp.idx_k[:, :S]), inp.dtype), TL.dev(inp.w_q), TL.dev(inp.w_k),
                          TL.dev(ctx), one, ws, cfg)
    torch.cuda.synchronize()
    one = one.cpu().numpy()
    for b in range(inp.B):
        for t in range(N - P):
            assert np.array_equal(np.sort(got[b, t]), np.sort(one[b, P + t])), f"chunk row {t} vs one-shot row {P + t}"


def test_chunk_long_prefill_tail():
    """A 2048-token chunk at the end of the long prefill (S = 32768, Hq 32,
    Hkv 4, fp16): every row's list passes the closed-form invariants at its
    position, every list matches the oracle's (margin rule), the tails are
    bit-exact, and sampled rows' attention matches."""
    S, P = 32768, 30720
    C = S - P
    TL.log("chunk at the end of the long prefill")
    inp = syn.make_prefill(75, B=1, S=S, Hq=32, Hkv=4, D=128, dtype="fp16", ctx=[S])
    icfg = inp.icfg
    rng = np.random.default_rng(75)
    pool, pt = paged_state(rng, inp, S, S // 128)
    start = np.array([P], dtype=np.int32)
    ctx = np.array([S], dtype=np.int32)
    O.apply_tail_writes(pool, O.prefill_state_writes(inp.idx_k, inp.w_k, start, pt, icfg, inp.D, inp.dtype), inp.D)
    pool_dev = TL.dev(pool, inp.dtype)
    lists, o, _ = gpu_chunk(inp, pool_dev, pt, P, ctx, C)
    got = lists.cpu().numpy()
    full = np.full((1, S, icfg.top_k), -1, dtype=np.int32)
    full[0, P:] = got[0]
    n = TL.check_list_invariants_all_rows(full, ctx, icfg, "long chunk", row0=P)
    TL.log(f"  invariants hold on {n} chunk rows")
    TL.log("  oracle chunk")
    writes, ref, scores = O.indexer_chunk(inp.idx_q[:, P:], inp.idx_k[:, P:], inp.w_q, inp.w_k, pool, pt, start, ctx,
                                          icfg, inp.D, inp.dtype, icfg.top_k, return_scores=True)
    swaps = sum(TL.check_list(got[0, t], ref[0, t], scores[(0, t)], P + t, icfg, "long chunk") for t in range(C))
    TL.log(f"  boundary swaps used: {swaps} of {C}")
    expect = pool.copy()
    O.apply_tail_writes(expect, writes, inp.D)
    assert torch.equal(pool_dev.view(torch.int16), TL.dev(expect, inp.dtype).view(torch.int16)), "pool after chunk"
    rows = sorted(set([0, 1, 2, 3, C - 1] + rng.integers(0, C, 12).tolist()))
    rows = [t for t in rows if np.array_equal(np.sort(got[0, t]), np.sort(ref[0, t]))]
    sub_q = np.ascontiguousarray(inp.q[:, P:][:, rows])
    ref_o = O.sparse_chunk(sub_q, pool, pt, ref[:, rows], np.zeros(1, np.int32), ctx, inp.scale, inp.D, inp.dtype)
    got_o = TL.host_f64(o, inp.dtype)
    for j, t in enumerate(rows):
        TL.check_attention(got_o[0, t], ref_o[0, j], inp.dtype, f"long chunk row {t}")


def test_chunk_ragged_starts():
    """Three sequences whose chunks start and end at different positions (one
    from position 0, one ending a few rows into the chunk, one past a page
    boundary): every list against the oracle (margin rule), the tails bit for
    bit, the attention of rows whose lists agree, the padding rows, and the
    same lists as the one-shot prefill of each sequence."""
    B, S = 3, 900
    start = np.array([100, 0, 641], dtype=np.int32)
    ctx = np.array([700, 351, 900], dtype=np.int32)
    C = int((ctx - start).max()) + 2
    icfg = syn.IndexerCfg(budget=16)
    TL.log(f"chunk ragged starts {start.tolist()} ctx {ctx.tolist()} C={C}")
    inp = syn.make_prefill(77, B=B, S=S, Hq=8, Hkv=2, D=64, dtype="bf16", ctx=ctx, icfg=icfg)
    rng = np.random.default_rng(77)
    max_pages = (S + 127) // 128 + 1
    pool, pt = paged_state(rng, inp, S, max_pages)
    O.apply_tail_writes(pool, O.prefill_state_writes(inp.idx_k, inp.w_k, start, pt, icfg, inp.D, inp.dtype), inp.D)

    def rows_from(a):  # each sequence's C rows from its own start, zero past S
        out = np.zeros((B, C) + a.shape[2:], dtype=a.dtype)
        for b in range(B):
            n = min(C, S - int(start[b]))
            out[b, :n] = a[b, start[b]:start[b] + n]
        return out
    iq, ik, q = rows_from(inp.idx_q), rows_from(inp.idx_k), rows_from(inp.q)
    cfg = TL.idx_cfg_struct(icfg)
    ws = torch.empty(Q.qsa_indexer_chunk_workspace_bytes(cfg, B, C, max_pages), dtype=torch.uint8, device="cuda")
    lists = torch.full((B, C, icfg.top_k), -7, dtype=torch.int32, device="cuda")
    pool_dev = TL.dev(pool, inp.dtype)
    Q.qsa_indexer_chunk(TL.dev(iq, inp.dtype), TL.dev(ik, inp.dtype), TL.dev(inp.w_q), TL.dev(inp.w_k), pool_dev,
                        TL.dev(pt), TL.dev(start), TL.dev(ctx), lists, ws, cfg, inp.D)
    q_dev = TL.dev(q, inp.dtype)
    o = torch.full_like(q_dev, float("nan"))
    Q.qsa_sparse_chunk(q_dev, o, pool_dev, TL.dev(pt), lists, TL.dev(start), TL.dev(ctx), inp.scale, head_dim=inp.D)
    torch.cuda.synchronize()
    got = lists.cpu().numpy()
    writes, ref, scores = O.indexer_chunk(iq, ik, inp.w_q, inp.w_k, pool, pt, start, ctx, icfg, inp.D, inp.dtype,
                                          icfg.top_k, return_scores=True)
    same, swaps = [], 0
    for b in range(B):
        live = int(ctx[b] - start[b])
        for t in range(C):
            if t >= live:
                assert np.all(got[b, t] == -1), f"b={b}: padding row {t}"
                continue
            used = TL.check_list(got[b, t], ref[b, t], scores.get((b, t)), int(start[b]) + t, icfg, f"ragged b={b}")
            swaps += used
            if not used:
                same.append((b, t))
    TL.log(f"  boundary swaps used: {swaps}")
    expect = pool.copy()
    O.apply_tail_writes(expect, writes, inp.D)
    assert torch.equal(pool_dev.view(torch.int16), TL.dev(expect, inp.dtype).view(torch.int16)), "pool after chunk"
    ref_o = O.sparse_chunk(q, pool, pt, ref, start, ctx, inp.scale, inp.D, inp.dtype)
    got_o = TL.host_f64(o, inp.dtype)
    for (b, t) in same:
        TL.check_attention(got_o[b, t], ref_o[b, t], inp.dtype, f"ragged chunk attention b={b} t={t}")
    for b in range(B):
        TL.check_zero_rows(o[b, int(ctx[b] - start[b]):], f"ragged chunk b={b} padding rows")
    # the one-shot prefill of each sequence selects the same lists
    wsp = torch.empty(Q.qsa_indexer_prefill_workspace_bytes(cfg, B, S), dtype=torch.uint8, device="cuda")
    one = torch.full((B, S, icfg.top_k), -7, dtype=torch.int32, device="cuda")
    Q.qsa_indexer_prefill(TL.dev(inp.idx_q, inp.dtype), TL.dev(inp.idx_k, inp.dtype), TL.dev(inp.w_q),
                          TL.dev(inp.w_k), TL.dev(ctx), one, wsp, cfg)
    torch.cuda.synchronize()
    one = one.cpu().numpy()
    for b in range(B):
        for t in range(int(ctx[b] - start[b])):
            assert np.array_equal(np.sort(got[b, t]), np.sort(one[b, start[b] + t])), \
                f"b={b}: chunk row {t} vs one-shot row {start[b] + t}"


def test_chunk_rows_across_select_classes():
    """Chunk rows on both sides of 8192 complete blocks (the pool holds
    longer rows, so the per-row kernel and the workgroup kernel both run over
    the chunk and split its rows): every list against the oracle (margin
    rule), the tails bit for bit, and the one-shot prefill's lists."""
    B, S = 2, 33300
    start = np.array([32700, 32000], dtype=np.int32)
    ctx = np.array([33300, 32800], dtype=np.int32)
    C = int((ctx - start).max()) + 1
    icfg = syn.IndexerCfg()
    TL.log(f"chunk across select classes: starts {start.tolist()} ctx {ctx.tolist()} C={C}")
    inp = syn.make_prefill(78, B=B, S=S, Hq=2, Hkv=1, D=64, dtype="fp16", ctx=ctx, icfg=icfg)
    rng = np.random.default_rng(78)
    max_pages = (S + 127) // 128 + 1
    pool, pt = paged_state(rng, inp, S, max_pages)
    O.apply_tail_writes(pool, O.prefill_state_writes(inp.idx_k, inp.w_k, start, pt, icfg, inp.D, inp.dtype), inp.D)

    def rows_from(a):
        out = np.zeros((B, C) + a.shape[2:], dtype=a.dtype)
        for b in range(B):
            n = min(C, S - int(start[b]))
            out[b, :n] = a[b, start[b]:start[b] + n]
        return out
    iq, ik = rows_from(inp.idx_q), rows_from(inp.idx_k)
    cfg = TL.idx_cfg_struct(icfg)
    ws = torch.empty(Q.qsa_indexer_chunk_workspace_bytes(cfg, B, C, max_pages), dtype=torch.uint8, device="cuda")
    lists = torch.full((B, C, icfg.top_k), -7, dtype=torch.int32, device="cuda")
    pool_dev = TL.dev(pool, inp.dtype)
    Q.qsa_indexer_chunk(TL.dev(iq, inp.dtype), TL.dev(ik, inp.dtype), TL.dev(inp.w_q), TL.dev(inp.w_k), pool_dev,
                        TL.dev(pt), TL.dev(start), TL.dev(ctx), lists, ws, cfg, inp.D)
    torch.cuda.synchronize()
    got = lists.cpu().numpy()
    writes, ref, scores = O.indexer_chunk(iq, ik, inp.w_q, inp.w_k, pool, pt, start, ctx, icfg, inp.D, inp.dtype,
                                          icfg.top_k, return_scores=True)
    swaps, long_rows = 0, 0
    for b in range(B):
        live = int(ctx[b] - start[b])
        for t in range(C):
            if t >= live:
                assert np.all(got[b, t] == -1), f"b={b}: padding row {t}"
                continue
            long_rows += (int(start[b]) + t + 1) // icfg.compress_ratio > 8192
            swaps += TL.check_list(got[b, t], ref[b, t], scores.get((b, t)), int(start[b]) + t, icfg, f"b={b}")
    TL.log(f"  rows past 8192 blocks: {long_rows}; boundary swaps used: {swaps}")
    assert long_rows > 0 and long_rows < int((ctx - start).sum()), "the chunk must span both select classes"
    expect = pool.copy()
    O.apply_tail_writes(expect, writes, inp.D)
    assert torch.equal(pool_dev.view(torch.int16), TL.dev(expect, inp.dtype).view(torch.int16)), "pool after chunk"
    del ws
    wsp = torch.empty(Q.qsa_indexer_prefill_workspace_bytes(cfg, B, S), dtype=torch.uint8, device="cuda")
    one = torch.full((B, S, icfg.top_k), -7, dtype=torch.int32, device="cuda")
    Q.qsa_indexer_prefill(TL.dev(inp.idx_q, inp.dtype), TL.dev(inp.idx_k, inp.dtype), TL.dev(inp.w_q),
                          TL.dev(inp.w_k), TL.dev(ctx), one, wsp, cfg)
    torch.cuda.synchronize()
    one_np = one[:, 32000:].cpu().numpy()
    for b in range(B):
        for t in range(int(ctx[b] - start[b])):
            assert np.array_equal(np.sort(got[b, t]), np.sort(one_np[b, start[b] + t - 32000])), \
                f"b={b}: chunk row {t} vs one-shot row {start[b] + t}"
