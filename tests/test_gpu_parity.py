"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Small cases compare every row; the five named workloads run at full size in
the launch configuration bench.py times and compare sampled rows (the oracle
computes those one by one).  See qsa_testlib for the comparison rules.
"""
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


# ---------------------------------------------------------------------------
# runners (HIP path through the C ABI)
# ---------------------------------------------------------------------------
def gpu_sparse_prefill(inp, indices):
    q, k, v = TL.dev(inp.q, inp.dtype), TL.dev(inp.k, inp.dtype), TL.dev(inp.v, inp.dtype)
    o = torch.full_like(q, float("nan"))
    idx = indices if isinstance(indices, torch.Tensor) else TL.dev(indices)
    Q.qsa_sparse_prefill(q, k, v, o, idx, TL.dev(inp.ctx), inp.scale)
    torch.cuda.synchronize()
    return o


def check_rows_written(o, inp, what):
    """Every live row, not only the sampled ones: written (the output starts
    as NaN), finite, and no larger than its KV head's largest |v| (each
    output row is a convex combination of V rows; 1 % for rounding)."""
    v = TL.dev(inp.v, inp.dtype)
    G = inp.Hq // inp.Hkv
    for b in range(inp.B):
        live = min(int(inp.ctx[b]), inp.S)
        if live <= 0:
            continue
        ob = o[b, :live].float()
        assert torch.isfinite(ob).all(), f"{what}: b={b} has unwritten or non-finite live rows"
        vmax = v[b, :live].float().abs().amax(dim=(0, 2))  # [Hkv]
        omax = ob.abs().view(live, inp.Hkv, G, inp.D).amax(dim=(0, 2, 3))
        assert bool((omax <= vmax * 1.01).all()), f"{what}: b={b} output exceeds max |v|: {omax} vs {vmax}"


def gpu_indexer_prefill(inp, icfg, top_k):
    cfg = TL.idx_cfg_struct(icfg)
    nbytes = Q.qsa_indexer_prefill_workspace_bytes(cfg, inp.B, inp.S)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.full((inp.B, inp.S, top_k), -7, dtype=torch.int32, device="cuda")
    Q.qsa_indexer_prefill(TL.dev(inp.idx_q, inp.dtype), TL.dev(inp.idx_k, inp.dtype), TL.dev(inp.w_q),
                          TL.dev(inp.w_k), TL.dev(inp.ctx), out, ws, cfg)
    torch.cuda.synchronize()
    return out, ws


def kbar_from_workspace(ws, inp, icfg):
    """The kbar region of the prefill workspace: after the queries (two fp16
    scoring pieces per value)."""
    qbytes = inp.B * inp.S * icfg.num_heads * icfg.head_dim * 4
    off = (qbytes + 255) // 256 * 256
    gmax = inp.S // icfg.compress_ratio
    raw = ws[off:off + inp.B * gmax * icfg.head_dim * 2].view(torch.int16).cpu().numpy().view(np.uint16)
    return raw.reshape(inp.B, gmax, icfg.head_dim)       # storage bits; rows past the live blocks are unset


def compare_lists(lists_gpu, inp, icfg, top_k, rows, what):
    ref, scores = O.indexer_prefill(inp.idx_q, inp.idx_k, inp.w_q, inp.w_k, inp.ctx, icfg, inp.dtype,
                                    top_k, rows=rows, return_scores=True)
    swaps, same = 0, []
    for (b, t) in rows:
        used = TL.check_list(lists_gpu[b, t], ref[(b, t)], scores.get((b, t)), t, icfg, what)
        swaps += used
        if not used:
            same.append((b, t))
    return ref, swaps, same


# ---------------------------------------------------------------------------
# sparse prefill on given lists
# ---------------------------------------------------------------------------
PREFILL_CASES = [
    dict(B=2, S=300, Hq=8, Hkv=2, D=128, dtype="fp16", top_k=100, ctx=[300, 177]),
    dict(B=1, S=200, Hq=16, Hkv=1, D=128, dtype="bf16", top_k=200, ctx=[200]),
    dict(B=2, S=130, Hq=4, Hkv=4, D=64, dtype="bf16", top_k=40, ctx=[130, 1]),
    dict(B=1, S=100, Hq=12, Hkv=4, D=128, dtype="fp16", top_k=2051, ctx=[100]),
    dict(B=3, S=70, Hq=6, Hkv=2, D=64, dtype="fp16", top_k=33, ctx=[0, 70, 45]),
    dict(B=2, S=90, Hq=12, Hkv=3, D=128, dtype="fp16", top_k=64, ctx=[90, 61]),
    dict(B=1, S=50, Hq=16, Hkv=16, D=64, dtype="bf16", top_k=50, ctx=[50]),
    dict(B=1, S=77, Hq=16, Hkv=8, D=128, dtype="bf16", top_k=70, ctx=[77]),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: f"B{c['B']}S{c['S']}Hq{c['Hq']}Hkv{c['Hkv']}"
                         f"D{c['D']}{c['dtype']}k{c['top_k']}")
def test_sparse_prefill_small_all_rows(case):
    c = dict(case)
    top_k = c.pop("top_k")
    TL.log(f"sparse_prefill small {case}")
    inp = syn.make_prefill(7, with_indexer=False, **c)
    idx = syn.random_lists(np.random.default_rng(70), inp.B, inp.S, top_k, inp.ctx)
    o = gpu_sparse_prefill(inp, idx)
    ref = O.sparse_prefill(inp.q, inp.k, inp.v, idx, inp.ctx, inp.scale, inp.dtype)
    got = TL.host_f64(o, inp.dtype)
    for b in range(inp.B):
        live = min(int(inp.ctx[b]), inp.S)
        TL.check_attention(got[b, :live], ref[b, :live], inp.dtype, f"b={b}")
        TL.check_zero_rows(o[b, live:], f"b={b}")


def test_sparse_prefill_workload1():
    inp = syn.workload(1)
    TL.log("sparse_prefill workload 1")
    o = gpu_sparse_prefill(inp, inp.indices)
    ref = O.sparse_prefill(inp.q, inp.k, inp.v, inp.indices, inp.ctx, inp.scale, "fp16")
    TL.check_attention(TL.host_f64(o, "fp16"), ref, "fp16", "workload 1")


def test_sparse_prefill_permuted_lists_same_result():
    inp = syn.make_prefill(8, B=1, S=160, Hq=8, Hkv=1, D=128, dtype="fp16", ctx=[160], with_indexer=False)
    rng = np.random.default_rng(80)
    idx = syn.random_lists(rng, 1, 160, 96, inp.ctx)
    perm = idx.copy()
    for t in range(160):
        n = int((idx[0, t] >= 0).sum())
        perm[0, t, :n] = rng.permutation(idx[0, t, :n])
    a = TL.host_f64(gpu_sparse_prefill(inp, idx), "fp16")
    p = TL.host_f64(gpu_sparse_prefill(inp, perm), "fp16")
    ref = O.sparse_prefill(inp.q, inp.k, inp.v, idx, inp.ctx, inp.scale, "fp16")
    TL.check_attention(a, ref, "fp16", "sorted")
    TL.check_attention(p, ref, "fp16", "permuted")


def identity_lists(rng, B, S, ctx, top_k, mode):
    """Lists whose heads are the identity (slot s holds id s), as every row
    gets before the budget fills, plus variants that break the identity at
    various points: "full" identity to min(t, top_k - 1); "tail" identity
    for a row-dependent length, then other distinct ids in random order;
    "mixed" identity rows next to random-order rows in some groups of four
    consecutive rows (one workgroup's rows); "holes" identity with a
    few -1 slots; "dups" one id repeated in every fifth row; "future" a few
    ids past t in free slots of every third row."""
    out = np.full((B, S, top_k), -1, dtype=np.int32)
    for b in range(B):
        for t in range(min(int(ctx[b]), S)):
            n = min(t + 1, top_k)
            # "mixed": two rows of every third group of four rows go random
            odd_one = mode == "mixed" and ((S - 1 - t) // 4) % 3 == 1 and t % 2 == 0
            if mode == "full" or (mode == "mixed" and not odd_one):
                out[b, t, :n] = np.arange(n)
            elif mode == "tail":
                k = min(n, 40 + (t * 7) % 90)
                rest = rng.permutation(np.arange(k, t + 1))[:n - k]
                out[b, t, :k] = np.arange(k)
                out[b, t, k:k + len(rest)] = rest
            elif mode == "mixed":
                out[b, t, :n] = rng.permutation(t + 1)[:n]
            elif mode == "holes":
                out[b, t, :n] = np.arange(n)
                if n > 40:
                    out[b, t, rng.integers(0, n, 3)] = -1
            elif mode == "dups":
                # the contract's ids are distinct; a repeated id counts twice
                # on both sides (the list walk and the oracle)
                out[b, t, :n] = np.arange(n)
                if n > 8 and t % 5 == 0:
                    j, j2 = rng.choice(n, 2, replace=False)
                    out[b, t, j] = out[b, t, j2]
            elif mode == "future":
                # ids past t (outside the causal range) in free slots: both
                # sides use them as listed
                live = min(int(ctx[b]), S)
                out[b, t, :n] = np.arange(n)
                if t % 3 == 0 and n < top_k and t + 1 < live:
                    extra = rng.choice(np.arange(t + 1, live), min(2, top_k - n, live - t - 1), replace=False)
                    out[b, t, n:n + len(extra)] = extra
    return out


IDENTITY_CASES = [
    dict(B=2, S=301, Hq=8, Hkv=2, D=128, dtype="fp16", top_k=300, ctx=[301, 170], mode="full"),
    dict(B=1, S=400, Hq=16, Hkv=4, D=128, dtype="bf16", top_k=2051, ctx=[400], mode="tail"),
    dict(B=2, S=200, Hq=8, Hkv=1, D=128, dtype="fp16", top_k=256, ctx=[200, 131], mode="mixed"),
    dict(B=1, S=260, Hq=8, Hkv=1, D=64, dtype="bf16", top_k=260, ctx=[260], mode="full"),
    dict(B=1, S=150, Hq=6, Hkv=3, D=128, dtype="fp16", top_k=150, ctx=[150], mode="full"),
    dict(B=1, S=330, Hq=8, Hkv=2, D=128, dtype="fp16", top_k=330, ctx=[330], mode="holes"),
    dict(B=1, S=90, Hq=8, Hkv=2, D=128, dtype="fp16", top_k=16, ctx=[90], mode="full"),
    dict(B=1, S=200, Hq=16, Hkv=1, D=128, dtype="bf16", top_k=200, ctx=[200], mode="full"),
    dict(B=1, S=520, Hq=16, Hkv=2, D=128, dtype="fp16", top_k=520, ctx=[515], mode="full"),
    dict(B=1, S=100, Hq=10, Hkv=2, D=128, dtype="bf16", top_k=100, ctx=[100], mode="full"),
    dict(B=2, S=120, Hq=12, Hkv=1, D=64, dtype="fp16", top_k=70, ctx=[120, 50], mode="full"),
    dict(B=1, S=300, Hq=16, Hkv=2, D=128, dtype="fp16", top_k=300, ctx=[300], mode="dups"),
    dict(B=1, S=300, Hq=16, Hkv=2, D=128, dtype="bf16", top_k=200, ctx=[280], mode="future"),
    dict(B=1, S=260, Hq=16, Hkv=1, D=128, dtype="fp16", top_k=260, ctx=[260], mode="dups"),
]


@pytest.mark.parametrize("case", IDENTITY_CASES, ids=lambda c: f"{c['mode']}-B{c['B']}S{c['S']}Hkv{c['Hkv']}"
                         f"D{c['D']}{c['dtype']}k{c['top_k']}")
def test_sparse_prefill_identity_prefix_lists_all_rows(case):
    """Rows before the budget fills whose lists are their whole causal prefix
    run as dense causal tiles (rows x heads packed as MFMA columns, K/V
    staged once per tile), and a tile holding any other list falls back to
    the list walk; every row must match the oracle either way (tiles with
    ragged ends, rows past the live length, dead columns when G is not a
    power of two, G below 4 without tiles)."""
    TL.log(f"sparse_prefill identity lists {case}")
    inp = syn.make_prefill(14, B=case["B"], S=case["S"], Hq=case["Hq"], Hkv=case["Hkv"], D=case["D"],
                           dtype=case["dtype"], ctx=case["ctx"], with_indexer=False)
    lists = identity_lists(np.random.default_rng(14), inp.B, inp.S, inp.ctx, case["top_k"], case["mode"])
    o = gpu_sparse_prefill(inp, lists)
    ref = O.sparse_prefill(inp.q, inp.k, inp.v, lists, inp.ctx, inp.scale, inp.dtype)
    got = TL.host_f64(o, inp.dtype)
    for b in range(inp.B):
        live = min(int(inp.ctx[b]), inp.S)
        for t in range(live):
            TL.check_attention(got[b, t], ref[b, t], inp.dtype, f"b={b} t={t}")
        TL.check_zero_rows(o[b, live:], f"b={b}")


@pytest.mark.parametrize("mode", ["full", "dups"])
def test_sparse_prefill_two_column_tiles_g8(mode):
    """At G = 8 a launch with tiles for two rounds of two per CU (here
    2 x 4 x 132 tiles of 16 rows) runs two 16-column MFMA tiles per wave;
    sampled rows of every tile position (first, last, ragged end) match the
    oracle, with lists the key mask holds and with repeated ids (the tile's
    rows then go to the list walk)."""
    TL.log(f"sparse_prefill two column tiles G=8 {mode}")
    inp = syn.make_prefill(16, B=2, S=2100, Hq=32, Hkv=4, D=128, dtype="fp16", ctx=[2100, 1999], with_indexer=False)
    lists = identity_lists(np.random.default_rng(16), inp.B, inp.S, inp.ctx, 2051, mode)
    o = gpu_sparse_prefill(inp, lists)
    got = TL.host_f64(o, inp.dtype)
    rng = np.random.default_rng(17)
    for b in range(inp.B):
        live = min(int(inp.ctx[b]), inp.S)
        rows = sorted(set([0, 1, 15, 16, 17, live - 1, live - 2, 2047, 2048, 2050, 2051]
                          + list(rng.choice(live, 120, replace=False))))
        rows = [r for r in rows if r < live]
        ref = O.sparse_prefill(inp.q, inp.k, inp.v, lists, inp.ctx, inp.scale, inp.dtype, rows=[(b, r) for r in rows])
        for t in rows:
            TL.check_attention(got[b, t], ref[b, t], inp.dtype, f"b={b} t={t}")
        TL.check_zero_rows(o[b, live:], f"b={b}")


# ---------------------------------------------------------------------------
# indexer prefill
# ---------------------------------------------------------------------------
INDEXER_SMALL = [
    dict(B=2, S=400, dtype="fp16", ctx=[400, 233], icfg=dict(budget=8)),
    dict(B=2, S=257, dtype="bf16", ctx=[257, 96], icfg=dict(budget=5)),
    dict(B=1, S=130, dtype="fp16", ctx=[130], icfg=dict(budget=3, compress_ratio=2, rot_dim=32, num_heads=3)),
    dict(B=1, S=3, dtype="bf16", ctx=[3], icfg=dict(budget=1)),
]


@pytest.mark.parametrize("case", INDEXER_SMALL, ids=lambda c: f"B{c['B']}S{c['S']}{c['dtype']}{c['icfg']}")
def test_indexer_prefill_small_all_rows(case):
    icfg = syn.IndexerCfg(**case["icfg"])
    TL.log(f"indexer_prefill small {case}")
    inp = syn.make_prefill(9, B=case["B"], S=case["S"], Hq=2, Hkv=1, D=64, dtype=case["dtype"], ctx=case["ctx"],
                           icfg=icfg)
    out, ws = gpu_indexer_prefill(inp, icfg, icfg.top_k)
    lists = out.cpu().numpy()
    rows = [(b, t) for b in range(inp.B) for t in range(inp.S)]
    _, swaps, _ = compare_lists(lists, inp, icfg, icfg.top_k, rows, "indexer small")
    TL.log(f"  boundary swaps used: {swaps}")
    # kbar is computed in float64 and rounded once on both sides
    kb = kbar_from_workspace(ws, inp, icfg)
    for b in range(inp.B):
        n = min(int(inp.ctx[b]), inp.S) // icfg.compress_ratio
        ref = O.pool_blocks(O.widen(inp.idx_k[b, :n * icfg.compress_ratio], inp.dtype), 0, inp.w_k, icfg, inp.dtype)
        got = kb[b, :n].view(np.float16) if inp.dtype == "fp16" else kb[b, :n]
        assert np.array_equal(O.widen(got, inp.dtype), ref), "kbar differs from the oracle"


def test_indexer_prefill_budget512_selective_rows():
    icfg = syn.IndexerCfg()
    TL.log("indexer_prefill S=2600 budget 512")
    inp = syn.make_prefill(10, B=1, S=2600, Hq=2, Hkv=1, D=64, dtype="fp16", ctx=[2600])
    out, _ = gpu_indexer_prefill(inp, icfg, icfg.top_k)
    rows = [(0, t) for t in list(range(0, 64)) + list(range(2040, 2600))]
    _, swaps, _ = compare_lists(out.cpu().numpy(), inp, icfg, icfg.top_k, rows, "S2600")
    TL.log(f"  boundary swaps used: {swaps}")


def tie_classes(inp, icfg, classes):
    """Give every token of block g the raw key of class g mod `classes`.  With
    rot_dim 0 the pooled keys of one class are then identical, so a row's
    scores tie exactly inside each class."""
    r = icfg.compress_ratio
    pats = inp.idx_k[0, :classes].copy()
    inp.idx_k[:] = pats[(np.arange(inp.S) // r) % classes][None]


def tie_expectation(t, class_score, classes, icfg):
    """The one list the tie rule allows: classes by score, lower blocks first
    inside the class that straddles the budget."""
    r, budget = icfg.compress_ratio, icfg.budget
    nc = (t + 1) // r
    if nc <= budget:
        return np.arange(t + 1)
    blocks = np.arange(nc)
    order = np.lexsort((blocks, -class_score[blocks % classes]))
    keep = np.sort(order[:budget])
    return np.concatenate([(keep[:, None] * r + np.arange(r)).ravel(), np.arange(r * nc, t + 1)])


def check_tied_rows(lists, inp, icfg, classes, rows, what):
    _, scores = O.indexer_prefill(inp.idx_q, inp.idx_k, inp.w_q, inp.w_k, inp.ctx, icfg, inp.dtype, icfg.top_k,
                                  rows=rows, return_scores=True)
    checked = 0
    for (b, t) in rows:
        got = lists[b, t] if isinstance(lists, np.ndarray) else lists[(b, t)]
        live = min(int(inp.ctx[b]), inp.S)
        if t >= live:
            assert np.all(got == -1), f"{what}: dead row {t}"
            continue
        sc = scores.get((b, t))
        if sc is None or len(sc) == 0:
            exp = np.arange(t + 1)
        else:
            cs = np.array([sc[c] for c in range(min(classes, len(sc)))])
            # classes whose scores sit within 1e-3 of each other could swap by
            # rounding: such rows are left out
            if len(cs) > 1 and np.min(np.diff(np.sort(cs))) <= 1e-3 * max(np.max(cs), 1e-30):
                continue
            exp = tie_expectation(t, cs, len(cs), icfg)
        n = len(exp)
        assert np.array_equal(np.sort(got[:n]), np.sort(exp)), f"{what}: row {t} breaks the tie rule"
        assert np.all(got[n:] == -1), f"{what}: row {t} padding"
        checked += 1
    assert checked >= len(rows) // 2, f"{what}: only {checked} rows had well separated classes"


@pytest.mark.parametrize("classes", [1, 3])
def test_indexer_prefill_exact_ties_wave_select(classes):
    """Exact score ties at the cut: the lowest block indices win."""
    icfg = syn.IndexerCfg(rot_dim=0)
    TL.log(f"indexer_prefill ties classes={classes} S=3000")
    inp = syn.make_prefill(12, B=2, S=3000, Hq=2, Hkv=1, D=64, dtype="fp16", ctx=[3000, 2100], icfg=icfg)
    tie_classes(inp, icfg, classes)
    out, _ = gpu_indexer_prefill(inp, icfg, icfg.top_k)
    rows = [(b, t) for b in range(2) for t in list(range(2040, 2120)) + list(range(2900, 3000))]
    check_tied_rows(out.cpu().numpy(), inp, icfg, classes, rows, f"ties{classes}")


@pytest.mark.parametrize("classes", [0, 3])
def test_indexer_prefill_two_wave_rows(classes):
    """Rows of 4097..8192 complete blocks take the two-wave select (shorter
    rows of the same call take the one-wave kernels); with a budget of 64 and
    three tied classes the cut falls inside the best class, whose equal keys
    sit in both waves."""
    icfg = syn.IndexerCfg(budget=64, rot_dim=0) if classes else syn.IndexerCfg(budget=64)
    S = 17000
    TL.log(f"indexer_prefill two-wave rows S={S} classes={classes}")
    inp = syn.make_prefill(15, B=1, S=S, Hq=2, Hkv=1, D=64, dtype="fp16", ctx=[S], icfg=icfg)
    if classes:
        tie_classes(inp, icfg, classes)
    out, _ = gpu_indexer_prefill(inp, icfg, icfg.top_k)
    rng = np.random.default_rng(15)
    rows = sorted({(0, int(t)) for t in rng.integers(16387, S, 10)} | {(0, 16387), (0, 16386), (0, S - 1),
                                                                         (0, 9000), (0, 300)})
    out_np = out.cpu().numpy()
    lists = {r: out_np[r] for r in rows}
    if classes:
        check_tied_rows(lists, inp, icfg, classes, rows, "two-wave ties")
    else:
        _, swaps, _ = compare_lists(lists, inp, icfg, icfg.top_k, rows, "two-wave rows")
        TL.log(f"  boundary swaps used: {swaps}")


@pytest.mark.parametrize("classes", [0, 7])
def test_indexer_prefill_long_rows_workgroup_select(classes):
    """Rows with more than 8192 complete blocks take the workgroup select."""
    icfg = syn.IndexerCfg(rot_dim=0) if classes else syn.IndexerCfg()
    S = 33100
    TL.log(f"indexer_prefill long rows S={S} classes={classes}")
    inp = syn.make_prefill(13, B=1, S=S, Hq=2, Hkv=1, D=64, dtype="bf16", ctx=[S], icfg=icfg)
    if classes:
        tie_classes(inp, icfg, classes)
    out, _ = gpu_indexer_prefill(inp, icfg, icfg.top_k)
    rng = np.random.default_rng(13)
    rows = sorted({(0, int(t)) for t in rng.integers(2048, S, 10)} | {(0, S - 1), (0, S - 4), (0, 32771)})
    out_np = out.cpu().numpy()
    lists = {r: out_np[r] for r in rows}
    if classes:
        check_tied_rows(lists, inp, icfg, classes, rows, "long ties")
    else:
        _, swaps, _ = compare_lists(lists, inp, icfg, icfg.top_k, rows, "long rows")
        TL.log(f"  boundary swaps used: {swaps}")


RAGGED_BATCHES = [
    # every row: three sequences (B does not divide the eight XCDs' order)
    dict(B=3, S=1300, dtype="fp16", ctx=[1300, 0, 777], budget=12, rows="all"),
    # every row: eight sequences with empty, one-token and near-full lengths
    dict(B=8, S=600, dtype="bf16", ctx=[600, 1, 599, 333, 0, 64, 450, 2], budget=9, rows="all"),
    # sampled rows: the two-wave select class in three sequences
    dict(B=3, S=17000, dtype="fp16", ctx=[17000, 16500, 9000], budget=64, rows=12),
    # sampled rows: 2048 row groups of <= 32 chunks, so scoring takes whole
    # rows per workgroup; ragged lengths across eight sequences
    dict(B=8, S=8192, dtype="bf16", ctx=[8192, 8000, 100, 8192, 5000, 0, 7777, 4096], budget=512, rows=6),
]


@pytest.mark.parametrize("case", RAGGED_BATCHES, ids=lambda c: f"B{c['B']}S{c['S']}{c['dtype']}k{c['budget']}")
def test_indexer_prefill_ragged_batches(case):
    """Batches of several sequences of different lengths: scoring deals row
    groups to the XCDs sequence by sequence and the selects spread rows over
    them; every list (or a sample of rows of every sequence, plus every row's
    closed-form invariants) must match the oracle."""
    icfg = syn.IndexerCfg(budget=case["budget"])
    TL.log(f"indexer_prefill ragged {case}")
    inp = syn.make_prefill(21, B=case["B"], S=case["S"], Hq=2, Hkv=1, D=64, dtype=case["dtype"], ctx=case["ctx"],
                           icfg=icfg)
    out, _ = gpu_indexer_prefill(inp, icfg, icfg.top_k)
    out_np = out.cpu().numpy()
    if case["rows"] == "all":
        rows = [(b, t) for b in range(inp.B) for t in range(inp.S)]
    else:
        rng = np.random.default_rng(21)
        rows = set()
        for b in range(inp.B):
            live = min(int(inp.ctx[b]), inp.S)
            rows |= {(b, int(t)) for t in rng.integers(0, max(live, 1), case["rows"])}
            rows |= {(b, max(live - 1, 0)), (b, inp.S - 1)}
        rows = sorted(rows)
        n_rows = TL.check_list_invariants_all_rows(out_np, inp.ctx, icfg, "ragged")
        TL.log(f"  list invariants hold on all {n_rows} live rows")
    lists = {r: out_np[r] for r in rows}
    _, swaps, _ = compare_lists(lists, inp, icfg, icfg.top_k, rows, "ragged")
    TL.log(f"  rows {len(rows)}, boundary swaps used: {swaps}")


# ---------------------------------------------------------------------------
# the prefill workloads at full size (bench launch configuration)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("wl", [2, 3, 5])
def test_prefill_workload_full_size(wl):
    TL.log(f"prefill workload {wl}: generating")
    inp = syn.workload(wl)
    icfg = inp.icfg
    TL.log(f"prefill workload {wl}: indexer")
    out, _ = gpu_indexer_prefill(inp, icfg, icfg.top_k)
    TL.log(f"prefill workload {wl}: attention")
    o = gpu_sparse_prefill(inp, out)
    rng = np.random.default_rng(100 + wl)
    # workload 2 (the headline one) row by row in full; the larger ones sampled
    rows = ([(b, t) for b in range(inp.B) for t in range(inp.S)] if wl == 2
            else TL.sample_rows(inp.B, inp.S, inp.ctx, 128, rng))
    out_np = out.cpu().numpy()
    n_rows = TL.check_list_invariants_all_rows(out_np, inp.ctx, icfg, f"workload {wl}")
    TL.log(f"prefill workload {wl}: list invariants hold on all {n_rows} live rows")
    TL.log(f"prefill workload {wl}: oracle on {len(rows)} rows")
    lists = {r: out_np[r] for r in rows}
    ref_lists, swaps, same = compare_lists(lists, inp, icfg, icfg.top_k, rows, f"workload {wl}")
    TL.log(f"  boundary swaps used: {swaps} of {len(rows)} rows")
    # attention parity on rows whose lists agree (each side reads its own lists)
    full = np.full((inp.B, inp.S, icfg.top_k), -1, dtype=np.int32)
    for r in same:
        full[r] = ref_lists[r]
    ref_o = O.sparse_prefill(inp.q, inp.k, inp.v, full, inp.ctx, inp.scale, inp.dtype, rows=same)
    TL.log(f"prefill workload {wl}: attention compared on {len(same)} rows")
    for (b, t) in same:
        live = min(int(inp.ctx[b]), inp.S)
        if t < live:
            TL.check_attention(TL.host_f64(o[b, t], inp.dtype), ref_o[(b, t)], inp.dtype,
                               f"workload {wl} b={b} t={t}")
    for b in range(inp.B):
        live = min(int(inp.ctx[b]), inp.S)
        TL.check_zero_rows(o[b, live:], f"workload {wl} b={b}")
    check_rows_written(o, inp, f"workload {wl}")


def test_prefill_reruns_bit_identical():
    """Workload 5 (ragged bf16, G = 16: list tiles and the list walk) three
    times, the lists and the output poisoned between runs: every run gives
    the first run's lists and output bit for bit (fixed reduction orders, no
    order-dependent atomics)."""
    TL.log("prefill reruns: workload 5")
    inp = syn.workload(5)
    icfg = inp.icfg
    cfg = TL.idx_cfg_struct(icfg)
    ws = torch.empty(Q.qsa_indexer_prefill_workspace_bytes(cfg, inp.B, inp.S), dtype=torch.uint8, device="cuda")
    iq, ik = TL.dev(inp.idx_q, inp.dtype), TL.dev(inp.idx_k, inp.dtype)
    wq, wk, ctx = TL.dev(inp.w_q), TL.dev(inp.w_k), TL.dev(inp.ctx)
    q, k, v = TL.dev(inp.q, inp.dtype), TL.dev(inp.k, inp.dtype), TL.dev(inp.v, inp.dtype)
    lists = torch.empty((inp.B, inp.S, icfg.top_k), dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    first = None
    for run in range(3):
        lists.fill_(-7)
        o.view(torch.int16).fill_(0x7e00)
        ws.fill_(0xab)
        Q.qsa_indexer_prefill(iq, ik, wq, wk, ctx, lists, ws, cfg)
        Q.qsa_sparse_prefill(q, k, v, o, lists, ctx, inp.scale)
        torch.cuda.synchronize()
        if first is None:
            first = (lists.clone(), o.clone())
            continue
        assert torch.equal(lists, first[0]), f"run {run}: lists differ"
        assert torch.equal(o.view(torch.int16), first[1].view(torch.int16)), f"run {run}: output differs"
    TL.log("  three runs bit-identical")


@pytest.mark.parametrize("wl", [2, 3, 5])
def test_sparse_prefill_structured_lists_full_size(wl):
    TL.log(f"sparse prefill structured lists workload {wl}")
    inp = syn.workload(wl)
    rng = np.random.default_rng(200 + wl)
    idx = TL.structured_lists(rng, inp.B, inp.S, inp.ctx, inp.icfg, inp.icfg.top_k)
    o = gpu_sparse_prefill(inp, idx)
    rows = ([(0, t) for t in range(inp.S)] if wl == 2 else TL.sample_rows(inp.B, inp.S, inp.ctx, 128, rng))
    ref = O.sparse_prefill(inp.q, inp.k, inp.v, idx, inp.ctx, inp.scale, inp.dtype, rows=rows)
    for (b, t) in rows:
        TL.check_attention(TL.host_f64(o[b, t], inp.dtype), ref[(b, t)], inp.dtype, f"b={b} t={t}")
    check_rows_written(o, inp, f"structured lists workload {wl}")


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------
def gpu_indexer_decode(inp, pool_dev):
    icfg = inp.icfg
    cfg = TL.idx_cfg_struct(icfg)
    ws = torch.empty(Q.qsa_indexer_decode_workspace_bytes(cfg, inp.B, inp.max_pages), dtype=torch.uint8,
                     device="cuda")
    out = torch.full((inp.B, 1, inp.top_k), -7, dtype=torch.int32, device="cuda")
    Q.qsa_indexer_decode(TL.dev(inp.idx_q, inp.dtype), TL.dev(inp.idx_k, inp.dtype), TL.dev(inp.w_q),
                         TL.dev(inp.w_k), pool_dev, TL.dev(inp.page_table), TL.dev(inp.ctx), out, ws, cfg,
                         inp.D)
    torch.cuda.synchronize()
    return out


class DecodeWs:
    def __init__(self, inp):
        self.po = torch.empty(Q.qsa_sparse_decode_partial_o_elems(inp.B, inp.Hkv, inp.D), dtype=torch.float32,
                              device="cuda")
        self.ps = torch.empty(Q.qsa_sparse_decode_partial_stats_elems(inp.B, inp.Hkv), dtype=torch.float32,
                              device="cuda")


def gpu_sparse_decode(inp, pool_dev, lists_dev, ws, num_splits=0):
    q = TL.dev(inp.q, inp.dtype)
    o = torch.full_like(q, float("nan"))
    Q.qsa_sparse_decode(q, o, pool_dev, TL.dev(inp.page_table), lists_dev, TL.dev(inp.ctx), ws.po, ws.ps,
                        inp.scale, head_dim=inp.D, num_splits=num_splits)
    torch.cuda.synchronize()
    return o


def decode_parity(inp, what, splits=(0,)):
    icfg = inp.icfg
    pool_dev = TL.dev(inp.pool, inp.dtype)
    TL.log(f"{what}: indexer decode")
    lists_t = gpu_indexer_decode(inp, pool_dev)
    writes, ref_lists, scores = O.indexer_decode(inp.idx_q, inp.idx_k, inp.w_q, inp.w_k, inp.pool,
                                                 inp.page_table, inp.ctx, icfg, inp.D, inp.dtype, inp.top_k,
                                                 return_scores=True)
    # owned tails bit-exact, everything else bit-unchanged
    expect = TL.dev(inp.pool, inp.dtype)
    for pg, row, vals in writes:
        expect[pg, row, 0, inp.D:inp.D + vals.shape[0]] = TL.dev(vals, inp.dtype)
    assert torch.equal(pool_dev.view(torch.int16), expect.view(torch.int16)), f"{what}: pool differs"
    del expect
    lists = lists_t.cpu().numpy()
    swaps, same = 0, []
    for b in range(inp.B):
        c = int(inp.ctx[b])
        if c <= 0:
            assert np.all(lists[b, 0] == -1)
            continue
        used = TL.check_list(lists[b, 0], ref_lists[b, 0], scores[b], c - 1, icfg, f"{what} b={b}")
        swaps += used
        if not used:
            same.append(b)
    TL.log(f"  boundary swaps used: {swaps} of {inp.B}")
    ref_o = O.sparse_decode(inp.q, inp.pool, inp.page_table, ref_lists, inp.ctx, inp.scale, inp.D, inp.dtype)
    ws = DecodeWs(inp)
    outs = []
    for ns in splits:
        TL.log(f"{what}: sparse decode num_splits={ns}")
        o = gpu_sparse_decode(inp, pool_dev, lists_t, ws, ns)
        got = TL.host_f64(o, inp.dtype)[:, 0]
        for b in same:
            TL.check_attention(got[b], ref_o[b], inp.dtype, f"{what} splits={ns} b={b}")
        for b in range(inp.B):
            if int(inp.ctx[b]) <= 0:
                TL.check_zero_rows(o[b], f"{what} splits={ns} b={b} (empty)")
        outs.append(o)
    return pool_dev, lists_t, ws, outs


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_indexer_prefill_handoff_then_decode_steps(dtype):
    """qsa_indexer_prefill with the pool handoff leaves exactly the oracle's
    tails and touches nothing else in the pool; qsa_indexer_decode steps that
    continue from that state select for the following rows as the oracle's
    prefill of the longer sequences does, and the pool ends with the oracle's
    state (bit for bit)."""
    icfg = syn.IndexerCfg(budget=8)
    S, D, starts = 420, 64, np.array([300, 233], dtype=np.int32)
    TL.log(f"indexer prefill handoff + decode steps {dtype}")
    inp = syn.make_prefill(44, B=2, S=S, Hq=2, Hkv=1, D=D, dtype=dtype, ctx=[S, S], icfg=icfg)
    dec = syn.make_decode(44, ctx=[S, S], B=2, Hq=8, Hkv=2, D=D, dtype=dtype, max_pages=8, icfg=icfg)
    pool_dev, pt_dev = TL.dev(dec.pool, dtype), TL.dev(dec.page_table)
    cfg = TL.idx_cfg_struct(icfg)
    lists = torch.full((2, S, icfg.top_k), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(Q.qsa_indexer_prefill_workspace_bytes(cfg, 2, S), dtype=torch.uint8, device="cuda")
    Q.qsa_indexer_prefill(TL.dev(inp.idx_q, dtype), TL.dev(inp.idx_k, dtype), TL.dev(inp.w_q), TL.dev(inp.w_k),
                          TL.dev(starts), lists, ws, cfg, kv_pool=pool_dev, page_table=pt_dev, head_dim=D)
    torch.cuda.synchronize()
    expect = dec.pool.copy()
    O.apply_tail_writes(expect, O.prefill_state_writes(inp.idx_k, inp.w_k, starts, dec.page_table, icfg, D, dtype),
                        D)
    assert torch.equal(pool_dev.view(torch.int16), TL.dev(expect, dtype).view(torch.int16)), "handoff tails differ"
    steps = 6
    rows = [(b, int(starts[b]) + s) for b in range(2) for s in range(steps)]
    ref, scores = O.indexer_prefill(inp.idx_q, inp.idx_k, inp.w_q, inp.w_k, np.array([S, S]), icfg, dtype,
                                    icfg.top_k, rows=rows, return_scores=True)
    wsd = torch.empty(Q.qsa_indexer_decode_workspace_bytes(cfg, 2, dec.max_pages), dtype=torch.uint8, device="cuda")
    swaps = 0
    for step in range(steps):
        ctx = starts + step + 1
        tok = ctx - 1
        q1 = np.stack([inp.idx_q[b, tok[b]] for b in range(2)])[:, None]
        k1 = np.stack([inp.idx_k[b, tok[b]] for b in range(2)])[:, None]
        out = torch.full((2, 1, icfg.top_k), -7, dtype=torch.int32, device="cuda")
        Q.qsa_indexer_decode(TL.dev(q1, dtype), TL.dev(k1, dtype), TL.dev(inp.w_q), TL.dev(inp.w_k), pool_dev, pt_dev,
                             TL.dev(ctx.astype(np.int32)), out, wsd, cfg, D)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        for b in range(2):
            t = int(tok[b])
            swaps += TL.check_list(got[b, 0], ref[(b, t)], scores[(b, t)], t, icfg, f"step {step} b={b}")
        writes, _ = O.indexer_decode(q1, k1, inp.w_q, inp.w_k, expect, dec.page_table, ctx, icfg, D, dtype,
                                     icfg.top_k)
        O.apply_tail_writes(expect, writes, D)
    TL.log(f"  boundary swaps used: {swaps}")
    assert torch.equal(pool_dev.view(torch.int16), TL.dev(expect, dtype).view(torch.int16)), "pool after decode differs"


DECODE_SMALL = [
    dict(B=6, Hq=32, Hkv=4, D=128, dtype="fp16", ctx=[1, 6, 2052, 3000, 4096, 8191], max_pages=64),
    dict(B=5, Hq=64, Hkv=4, D=128, dtype="bf16", ctx=[2, 7, 2051, 5000, 2049], max_pages=40),
    dict(B=3, Hq=8, Hkv=2, D=64, dtype="fp16", ctx=[0, 2200, 4100], max_pages=33),
]


@pytest.mark.parametrize("case", DECODE_SMALL, ids=lambda c: f"B{c['B']}Hq{c['Hq']}D{c['D']}{c['dtype']}")
def test_decode_small(case):
    TL.log(f"decode small {case}")
    inp = syn.make_decode(11, **case)
    decode_parity(inp, "decode small", splits=(0, 1, 2, 3, 4, 5, 8, 13, 16))


@pytest.mark.parametrize("B", [512, 513])
def test_decode_large_batch(B):
    """Up to 512 sequences the decode scoring deals the batch's tiles out in
    equal ranges over the chip; past that it takes a workgroup per 128
    blocks of each sequence.  Both against the oracle on every row."""
    rng = np.random.default_rng(B)
    ctx = rng.integers(1, 3000, size=B)
    ctx[:8] = [0, 1, 3, 4, 2048, 2051, 2052, 2999]
    inp = syn.make_decode(14, ctx=ctx, B=B, Hq=8, Hkv=2, D=64, dtype="bf16", max_pages=24)
    decode_parity(inp, f"decode batch {B}", splits=(0,))


def test_sparse_decode_largest_page_table():
    """max_pages_per_seq = 4096, the largest the attention boundary accepts:
    the page-table copy in LDS takes the workgroup past 64 KB of LDS.  Lists
    come from the oracle's decode indexer (the indexer itself is limited to
    QSA_MAX_BLOCKS blocks, i.e. 1024 pages at ratio 4)."""
    inp = syn.make_decode(13, ctx=[300, 2052, 9001], B=3, Hq=16, Hkv=2, D=128, dtype="bf16", max_pages=4096)
    _, ref_lists = O.indexer_decode(inp.idx_q, inp.idx_k, inp.w_q, inp.w_k, inp.pool, inp.page_table, inp.ctx,
                                    inp.icfg, inp.D, inp.dtype, inp.top_k)
    pool_dev = TL.dev(inp.pool, inp.dtype)
    ref_o = O.sparse_decode(inp.q, inp.pool, inp.page_table, ref_lists, inp.ctx, inp.scale, inp.D, inp.dtype)
    ws = DecodeWs(inp)
    for ns in (0, 3, 16):
        o = gpu_sparse_decode(inp, pool_dev, TL.dev(ref_lists), ws, ns)
        got = TL.host_f64(o, inp.dtype)[:, 0]
        for b in range(inp.B):
            TL.check_attention(got[b], ref_o[b], inp.dtype, f"max pages splits={ns} b={b}")


def test_decode_default_plan_needs_no_partials():
    """The library's own split plan is one workgroup per (sequence, KV head):
    NULL partial buffers are accepted and the output equals the one computed
    with them, bit for bit."""
    inp = syn.make_decode(12, ctx=[2051, 2052, 9000, 3], B=4, Hq=32, Hkv=4, D=128, dtype="fp16", max_pages=80)
    pool_dev = TL.dev(inp.pool, inp.dtype)
    lists_t = gpu_indexer_decode(inp, pool_dev)
    ws = DecodeWs(inp)
    ref = gpu_sparse_decode(inp, pool_dev, lists_t, ws, 0)
    q = TL.dev(inp.q, inp.dtype)
    o = torch.full_like(q, float("nan"))
    Q.qsa_sparse_decode(q, o, pool_dev, TL.dev(inp.page_table), lists_t, TL.dev(inp.ctx), None, None, inp.scale,
                        head_dim=inp.D)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), ref.view(torch.int16))


def test_decode_workload4_full_size_and_determinism():
    TL.log("decode workload 4: generating")
    inp = syn.workload(4)
    pool_dev, lists_t, ws, outs = decode_parity(inp, "workload 4", splits=(0, 4, 8))
    ref_bits = outs[0].view(torch.int16).clone()
    for i in range(10):
        ws.po.fill_(float("nan"))           # partials need no initial contents
        o = gpu_sparse_decode(inp, pool_dev, lists_t, ws, 0)
        assert torch.equal(o.view(torch.int16), ref_bits), f"rerun {i} differs"
    # the indexer step is idempotent: a second call rewrites the same tails and lists
    again = gpu_indexer_decode(inp, pool_dev)
    assert torch.equal(again, lists_t)
