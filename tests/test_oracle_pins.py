"""Pins of the CPU oracle against things other than itself: library routines
(NumPy / PyTorch casts, torch SDPA), closed forms, brute force on tiny inputs,
invariants the pages state, and hand-worked golden fixtures."""
import cmath
import json
import math
import os

import numpy as np
import pytest
import torch

import qsa_synth as syn
from oracle import qsa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------
def _wide_values(rng, n):
    mag = np.exp2(rng.uniform(-30, 17, n))
    x = mag * rng.choice([-1.0, 1.0], n)
    # exact midpoints between neighbouring fp16 / bf16 values (tie cases)
    h = rng.standard_normal(n // 4).astype(np.float16).astype(np.float64)
    ties16 = h + np.ldexp(1.0, np.frexp(h)[1] - 12)
    b = O.widen(syn.f32_to_bf16_bits(rng.standard_normal(n // 4).astype(np.float32)), "bf16")
    ties_b = b + np.ldexp(1.0, np.frexp(b)[1] - 9)
    return np.concatenate([x, ties16, ties_b, [0.0, -0.0]])


def test_round_to_fp16_matches_numpy_cast():
    x = _wide_values(np.random.default_rng(0), 200000)
    x = x[np.abs(x) < 65504]
    got = O.round_to(x, "fp16")
    ref = x.astype(np.float16).astype(np.float64)
    assert np.array_equal(got, ref)


def test_round_to_fp32_matches_numpy_cast():
    x = _wide_values(np.random.default_rng(1), 200000) * 1e-3
    assert np.array_equal(O.round_to(x, "fp32"), x.astype(np.float32).astype(np.float64))


def test_round_to_bf16_matches_torch_cast():
    # torch casts float32 -> bfloat16 with round-to-nearest-even; for inputs that
    # are exact float32 values this is the single rounding round_to performs.
    x32 = _wide_values(np.random.default_rng(2), 200000).astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_to(x32.astype(np.float64), "bf16"), ref)


def test_widen_narrow_roundtrip_and_generator_rounding():
    rng = np.random.default_rng(3)
    x32 = rng.standard_normal(10000).astype(np.float32)
    bits = syn.f32_to_bf16_bits(x32)
    w = O.widen(bits, "bf16")
    assert np.array_equal(w, torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy())
    assert np.array_equal(O.narrow(w, "bf16"), bits)
    h = x32.astype(np.float16)
    assert np.array_equal(O.narrow(O.widen(h, "fp16"), "fp16"), h)


# ---------------------------------------------------------------------------
# RMSNorm and RoPE
# ---------------------------------------------------------------------------
def test_rms_norm_hand_value():
    y = O.rms_norm(np.array([3.0, 4.0]), np.zeros(2), 0.0)
    ms = (9.0 + 16.0) / 2.0
    assert np.allclose(y, [3.0 / math.sqrt(ms), 4.0 / math.sqrt(ms)], rtol=0, atol=1e-15)


def test_rms_norm_zero_weight_output_rms():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((50, 128))
    eps = 1e-2
    y = O.rms_norm(x, np.zeros(128), eps)
    ms = np.mean(x * x, axis=1)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), np.sqrt(ms / (ms + eps)), rtol=1e-13)


def test_rms_norm_gain_is_one_plus_w():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 128))
    w = rng.standard_normal(128) * 0.1
    assert np.allclose(O.rms_norm(x, w, 1e-6), O.rms_norm(x, np.zeros(128), 1e-6) * (1 + w), rtol=1e-14)
    # with eps = 0 the norm is scale invariant
    assert np.allclose(O.rms_norm(5.0 * x, w, 0.0), O.rms_norm(x, w, 0.0), rtol=1e-13)


def test_rope_position_zero_and_rot_zero_are_identity():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((3, 128))
    assert np.array_equal(O.rope(x, np.zeros(3), 64, 1e6), x)
    assert np.array_equal(O.rope(x, np.arange(3) + 100, 0, 1e6), x)


def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(7)
    x = rng.standard_normal(128)
    rot, theta, pos = 64, 1e6, 12345
    y = O.rope(x, np.array(pos), rot, theta)
    for i in range(rot // 2):
        z = complex(x[i], x[i + rot // 2]) * cmath.exp(1j * pos * theta ** (-2.0 * i / rot))
        assert abs(y[i] - z.real) < 1e-12 and abs(y[i + rot // 2] - z.imag) < 1e-12
    assert np.array_equal(y[rot:], x[rot:])          # dims past rot pass through


def test_rope_relative_position_and_norm():
    rng = np.random.default_rng(8)
    a, b = rng.standard_normal(128), rng.standard_normal(128)
    rot, theta = 64, 1e4
    m, n = 731, 229
    lhs = O.rope(a, np.array(m), rot, theta)[:rot] @ O.rope(b, np.array(n), rot, theta)[:rot]
    rhs = O.rope(a, np.array(m - n), rot, theta)[:rot] @ b[:rot]
    assert abs(lhs - rhs) < 1e-10
    y = O.rope(a, np.array(m), rot, theta)
    h = rot // 2
    assert np.allclose(y[:h] ** 2 + y[h:rot] ** 2, a[:h] ** 2 + a[h:rot] ** 2, rtol=1e-12)


# ---------------------------------------------------------------------------
# block pooling and query prep
# ---------------------------------------------------------------------------
def test_pool_ratio_one_is_per_token_norm_rope():
    icfg = syn.IndexerCfg(compress_ratio=1)
    rng = np.random.default_rng(9)
    k = rng.standard_normal((10, 128)).astype(np.float16)
    w = (rng.standard_normal(128) * 0.1).astype(np.float32)
    got = O.pool_blocks(O.widen(k, "fp16"), 0, w, icfg, "fp16")
    ref = O.round_to(O.rope(O.rms_norm(O.widen(k, "fp16"), w.astype(np.float64), O.f32(1e-6)),
                            np.arange(10), 64, 1e6), "fp16")
    assert np.array_equal(got, ref)


def test_pool_is_mean_then_norm_at_block_start():
    icfg = syn.IndexerCfg()
    rng = np.random.default_rng(10)
    k = rng.standard_normal((12, 128)).astype(np.float16)
    w = (rng.standard_normal(128) * 0.1).astype(np.float32)
    got = O.pool_blocks(O.widen(k, "fp16"), 5, w, icfg, "fp16")     # blocks 5, 6, 7
    for j in range(3):
        mean = O.widen(k[4 * j:4 * j + 4], "fp16").mean(axis=0)
        # a block whose four keys all equal the mean pools to the same kbar
        same = O.pool_blocks(np.tile(mean, (4, 1)), 5 + j, w, icfg, "fp16")[0]
        assert np.array_equal(got[j], same)
        ref = O.round_to(O.rope(O.rms_norm(mean, w.astype(np.float64), O.f32(1e-6)),
                                np.array(4 * (5 + j)), 64, 1e6), "fp16")
        assert np.array_equal(got[j], ref)


def test_pool_divides_by_ratio_before_norm():
    # With a large eps the norm is not scale invariant, so a pooled sum and a
    # pooled mean give different keys.  Constant keys k: mean = k, and with
    # rot = 0 kbar = k / sqrt(mean(k^2) + eps) * (1 + w).
    icfg = syn.IndexerCfg(head_dim=4, rot_dim=0, rms_eps=1.0)
    k = np.tile(np.array([[1.0, -2.0, 0.5, 3.0]], dtype=np.float16), (4, 1))
    w = np.array([0.0, 0.5, -0.25, 0.0], dtype=np.float32)
    got = O.pool_blocks(O.widen(k, "fp16"), 0, w, icfg, "fp16")[0]
    x = np.array([1.0, -2.0, 0.5, 3.0])
    ref = x / math.sqrt((1 + 4 + 0.25 + 9) / 4 + 1.0) * (1 + w.astype(np.float64))
    assert np.array_equal(got, O.round_to(ref, "fp16"))


def test_prep_queries_float32_per_head_at_row_position():
    icfg = syn.IndexerCfg()
    rng = np.random.default_rng(11)
    q = rng.standard_normal((3, 4, 128)).astype(np.float16)
    w = (rng.standard_normal(128) * 0.1).astype(np.float32)
    pos = np.array([0, 17, 4099])
    got = O.prep_queries(O.widen(q, "fp16"), pos, w, icfg)
    for r in range(3):
        for h in range(4):
            ref = O.rope(O.rms_norm(O.widen(q[r, h], "fp16"), w.astype(np.float64), O.f32(1e-6)),
                         np.array(pos[r]), 64, 1e6)
            assert np.array_equal(got[r, h], ref.astype(np.float32).astype(np.float64))


# ---------------------------------------------------------------------------
# scores, selection, lists
# ---------------------------------------------------------------------------
def test_scores_bruteforce_loops():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((4, 16))
    kb = rng.standard_normal((9, 16))
    got = O.block_scores(q, kb)
    for g in range(9):
        tot = 0.0
        for h in range(4):
            d = math.fsum(q[h, i] * kb[g, i] for i in range(16))
            tot += max(d, 0.0)
        assert abs(got[g] - tot / 4.0) < 1e-12


def test_scores_are_nonnegative_and_zero_when_all_dots_negative():
    q = np.ones((4, 8))
    kb = np.vstack([-np.ones(8), np.ones(8)])
    s = O.block_scores(q, kb)
    assert s[0] == 0.0 and s[1] == pytest.approx(4 * 8 / math.sqrt(8))


def test_select_bruteforce_with_ties():
    rng = np.random.default_rng(13)
    for trial in range(200):
        n = int(rng.integers(1, 40))
        budget = int(rng.integers(1, 8))
        s = rng.integers(0, 6, n).astype(np.float64)          # many exact ties
        got = O.select_blocks(s, budget)
        ranked = sorted(range(n), key=lambda g: (-s[g], g))
        assert list(got) == sorted(ranked[:budget])


def test_golden_tiny_indexer():
    gd = _golden("worked_tiny_indexer.json")
    icfg = syn.IndexerCfg(num_heads=1, head_dim=4, rot_dim=0, compress_ratio=2, budget=1,
                          rope_theta=10000.0, rms_eps=0.0)
    k = np.array(gd["idx_k"], dtype=np.float16)
    q = np.array(gd["idx_q_one_head"], dtype=np.float16)[:, None, :]
    w = np.zeros(4, dtype=np.float32)
    assert icfg.top_k == 3
    kb = O.pool_blocks(O.widen(k, "fp16"), 0, w, icfg, "fp16")
    assert np.array_equal(kb, np.array(gd["kbar"], dtype=np.float64))
    lists, scores = O.indexer_prefill(q[None], k[None], w, w, np.array([8]), icfg, "fp16", 3,
                                      return_scores=True)
    assert np.array_equal(lists[0], np.array(gd["lists"]))
    assert np.array_equal(scores[(0, 7)], np.array(gd["scores_row7"], dtype=np.float64))
    icfg2 = syn.IndexerCfg(num_heads=2, head_dim=4, rot_dim=0, compress_ratio=2, budget=1,
                           rope_theta=10000.0, rms_eps=0.0)
    q2 = np.zeros((1, 8, 2, 4), dtype=np.float16)
    q2[0, 7] = np.array(gd["two_head_row7_q"], dtype=np.float16)
    l2, s2 = O.indexer_prefill(q2, k[None], w, w, np.array([8]), icfg2, "fp16", 3,
                               rows=[(0, 7)], return_scores=True)
    assert np.array_equal(s2[(0, 7)], np.array(gd["two_head_row7_scores"], dtype=np.float64))
    assert list(l2[(0, 7)]) == gd["two_head_row7_list"]


def test_page_constants():
    pc = _golden("page_constants.json")
    icfg = syn.IndexerCfg()
    assert icfg.budget == pc["budget_blocks"]["value"]
    assert icfg.compress_ratio == pc["compress_ratio"]["value"]
    assert icfg.top_k == pc["top_k"]["value"] == 512 * 4 + 3
    assert max(O.list_length(t, icfg) for t in range(0, 9000)) == pc["top_k"]["value"]
    assert syn.PAGE_TOKENS == pc["page_tokens"]["value"]


def _check_list_invariants(lst, t, icfg, top_k):
    r = icfg.compress_ratio
    n = int((lst >= 0).sum())
    assert n == O.list_length(t, icfg)
    assert np.all(lst[:n] >= 0) and np.all(lst[n:] == -1)           # -1 only on the right
    ids = lst[:n]
    assert len(set(ids.tolist())) == n and ids.max() <= t            # distinct, causal
    nc = (t + 1) // r
    assert list(ids[n - (t + 1) % r:]) == list(range(r * nc, t + 1)) if (t + 1) % r else True
    blocks = ids[: n - (t + 1) % r].reshape(-1, r)
    assert np.all(blocks == blocks[:, :1] + np.arange(r))            # whole blocks
    assert np.all(blocks[:, 0] % r == 0) and np.all(blocks[:, 0] // r < nc)


def test_lists_closed_forms_full_budget():
    icfg = syn.IndexerCfg()
    inp = syn.make_prefill(21, B=1, S=2600, Hq=2, Hkv=1, D=16, dtype="fp16", ctx=[2600])
    rows = [(0, t) for t in list(range(0, 40)) + list(range(2040, 2060)) + list(range(2560, 2600))]
    lists = O.indexer_prefill(inp.idx_q, inp.idx_k, inp.w_q, inp.w_k, inp.ctx, icfg, "fp16",
                              icfg.top_k, rows=rows)
    for (b, t), lst in lists.items():
        _check_list_invariants(lst, t, icfg, icfg.top_k)
        if t <= 2050:                                   # at most 512 blocks: whole prefix
            assert np.array_equal(lst[: t + 1], np.arange(t + 1))


def test_rows_before_the_first_complete_block():
    # S < ratio: no complete block exists; every row is its causal tail 0..t.
    icfg = syn.IndexerCfg(budget=1)
    inp = syn.make_prefill(23, B=1, S=3, Hq=1, Hkv=1, D=16, dtype="fp16", ctx=[3], icfg=icfg)
    lists = O.indexer_prefill(inp.idx_q, inp.idx_k, inp.w_q, inp.w_k, inp.ctx, icfg, "fp16", icfg.top_k)
    assert lists[0].tolist() == [[0, -1, -1, -1, -1, -1, -1], [0, 1, -1, -1, -1, -1, -1],
                                 [0, 1, 2, -1, -1, -1, -1]]


def test_lists_bruteforce_small_budget():
    icfg = syn.IndexerCfg(budget=3, head_dim=16, rot_dim=8)
    inp = syn.make_prefill(22, B=2, S=60, Hq=2, Hkv=1, D=16, dtype="bf16", ctx=[60, 37], icfg=icfg)
    lists, scores = O.indexer_prefill(inp.idx_q, inp.idx_k, inp.w_q, inp.w_k, inp.ctx, icfg, "bf16",
                                      icfg.top_k, return_scores=True)
    for b in range(2):
        for t in range(60):
            lst = lists[b, t]
            if t >= inp.ctx[b]:
                assert np.all(lst == -1)
                continue
            _check_list_invariants(lst, t, icfg, icfg.top_k)
            s = scores[(b, t)]
            nc = (t + 1) // 4
            ranked = sorted(range(nc), key=lambda g: (-s[g], g))[:3]
            kept = sorted(set(x // 4 for x in lst[lst >= 0] if x < 4 * nc))
            assert kept == sorted(ranked)


# ---------------------------------------------------------------------------
# sparse attention
# ---------------------------------------------------------------------------
def test_attention_full_prefix_equals_causal_sdpa():
    rng = np.random.default_rng(30)
    inp = syn.make_prefill(30, B=2, S=48, Hq=8, Hkv=2, D=32, dtype="fp16", ctx=[48, 48],
                           scale=0.3, with_indexer=False)
    idx = np.full((2, 48, 64), -1, dtype=np.int32)
    for b in range(2):
        for t in range(48):
            idx[b, t, : t + 1] = rng.permutation(t + 1)          # full prefix, unsorted
    got = O.sparse_prefill(inp.q, inp.k, inp.v, idx, inp.ctx, inp.scale, "fp16")
    q = torch.from_numpy(O.widen(inp.q, "fp16")).permute(0, 2, 1, 3)
    k = torch.from_numpy(O.widen(inp.k, "fp16")).permute(0, 2, 1, 3).repeat_interleave(4, dim=1)
    v = torch.from_numpy(O.widen(inp.v, "fp16")).permute(0, 2, 1, 3).repeat_interleave(4, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True,
                                                           scale=O.f32(inp.scale))
    assert np.allclose(got, ref.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-12)


def test_attention_bruteforce_workload1():
    inp = syn.workload(1)
    got = O.sparse_prefill(inp.q, inp.k, inp.v, inp.indices, inp.ctx, inp.scale, "fp16")
    q, k, v = (O.widen(a, "fp16") for a in (inp.q, inp.k, inp.v))
    for t in range(0, 64, 7):
        ids = [int(j) for j in inp.indices[0, t] if j >= 0]
        for h in range(4):
            logits = [0.125 * math.fsum(q[0, t, h, d] * k[0, j, 0, d] for d in range(64)) for j in ids]
            mx = max(logits)
            e = [math.exp(x - mx) for x in logits]
            z = math.fsum(e)
            for d in range(0, 64, 5):
                ref = math.fsum(e[i] * v[0, j, 0, d] for i, j in enumerate(ids)) / z
                assert abs(got[0, t, h, d] - ref) < 1e-12


def test_attention_single_id_returns_that_value_row():
    inp = syn.make_prefill(31, B=1, S=20, Hq=4, Hkv=2, D=16, dtype="bf16", ctx=[20], with_indexer=False)
    idx = np.full((1, 20, 5), -1, dtype=np.int32)
    for t in range(20):
        idx[0, t, 0] = t // 2
    got = O.sparse_prefill(inp.q, inp.k, inp.v, idx, inp.ctx, inp.scale, "bf16")
    v = O.widen(inp.v, "bf16")
    for t in range(20):
        for h in range(4):
            assert np.array_equal(got[0, t, h], v[0, t // 2, h // 2])


def test_attention_permutation_invariant_and_zero_rows():
    rng = np.random.default_rng(32)
    inp = syn.make_prefill(32, B=2, S=30, Hq=4, Hkv=1, D=16, dtype="fp16", ctx=[30, 11],
                           with_indexer=False)
    idx = syn.random_lists(rng, 2, 30, 8, inp.ctx)
    perm = idx.copy()
    for b in range(2):
        for t in range(30):
            n = int((idx[b, t] >= 0).sum())
            perm[b, t, :n] = rng.permutation(idx[b, t, :n])
    a = O.sparse_prefill(inp.q, inp.k, inp.v, idx, inp.ctx, inp.scale, "fp16")
    p = O.sparse_prefill(inp.q, inp.k, inp.v, perm, inp.ctx, inp.scale, "fp16")
    assert np.allclose(a, p, rtol=0, atol=1e-13)
    dead = a[1, 11:]
    assert np.all(dead == 0.0) and not np.any(np.signbit(dead))       # +0.0 exactly
    # a live row whose list is all -1 is +0.0 as well
    idx[0, 5] = -1
    z = O.sparse_prefill(inp.q, inp.k, inp.v, idx, inp.ctx, inp.scale, "fp16", rows=[(0, 5)])
    assert np.all(z[(0, 5)] == 0.0)


def test_attention_uniform_weights_average_values():
    # q = 0 gives equal logits, so the output is the mean of the listed V rows.
    q = np.zeros((1, 3, 1, 2), dtype=np.float16)
    k = np.array([[[[1, 2]], [[3, 4]], [[5, 6]]]], dtype=np.float16)
    v = np.array([[[[1, 2]], [[3, 4]], [[5, 6]]]], dtype=np.float16)
    idx = np.array([[[0, -1], [1, 0], [2, 0]]], dtype=np.int32)
    out = O.sparse_prefill(q, k, v, idx, np.array([3]), 1.0, "fp16")
    assert np.array_equal(out[0, :, 0], np.array([[1, 2], [2, 3], [3, 4]], dtype=np.float64))


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------
def _pool_from_dense(rng, k, v, D, hd, page=128, extra_tail=None):
    """Scatter dense K/V [S,Hkv,D] of one sequence into a paged pool with a
    random page permutation; tails filled with random values."""
    S, Hkv, _ = k.shape
    npg = (S + page - 1) // page + 3                     # a few unused pages
    perm = rng.permutation(npg)
    pool = rng.standard_normal((2 * npg, page, Hkv, D + hd)).astype(k.dtype)
    pt = np.full((1, 2, npg), -1, dtype=np.int32)
    for i in range((S + page - 1) // page):
        pt[0, 0, i] = perm[i]
        pt[0, 1, i] = perm[i] + npg
    for s in range(S):
        pool[pt[0, 0, s // page], s % page, :, :D] = k[s]
        pool[pt[0, 1, s // page], s % page, :, :D] = v[s]
    return pool, pt


def test_decode_paged_equals_dense_prefill_row():
    rng = np.random.default_rng(40)
    S = 300
    inp = syn.make_prefill(40, B=1, S=S, Hq=8, Hkv=2, D=32, dtype="fp16", ctx=[S], with_indexer=False)
    idx = syn.random_lists(rng, 1, S, 40, inp.ctx)
    pool, pt = _pool_from_dense(rng, inp.k[0], inp.v[0], 32, 16)
    for t in (0, 127, 128, 299):
        dense = O.sparse_prefill(inp.q, inp.k, inp.v, idx, inp.ctx, inp.scale, "fp16", rows=[(0, t)])
        dec = O.sparse_decode(inp.q[:, t:t + 1], pool, pt, idx[:, t:t + 1], np.array([t + 1]),
                              inp.scale, 32, "fp16")
        assert np.array_equal(dec[0], dense[(0, t)])


@pytest.mark.parametrize("budget,S,ts", [(6, 120, [3, 30, 61, 62, 63, 64, 101, 119]),
                                         (512, 2070, [2051, 2054, 2068, 2069])])
def test_decode_indexer_continues_prefill_state(budget, S, ts):
    """Seed the pool tails the way the page's tail layout says a finished
    prefix would leave them; the decode step at ctx = t+1 must then produce the
    prefill list of row t, and the compress step must reproduce prefill pooling."""
    icfg = syn.IndexerCfg(budget=budget)
    hd, D, r = icfg.head_dim, 16, icfg.compress_ratio
    inp = syn.make_prefill(41, B=1, S=S, Hq=2, Hkv=2, D=D, dtype="fp16", ctx=[S], icfg=icfg)
    rng = np.random.default_rng(41)
    pool0, pt = _pool_from_dense(rng, inp.k[0], inp.v[0], D, hd)
    kbar = O.pool_blocks(O.widen(inp.idx_k[0, : (S // r) * r], "fp16"), 0, inp.w_k, icfg, "fp16")
    pre = O.indexer_prefill(inp.idx_q, inp.idx_k, inp.w_q, inp.w_k, inp.ctx, icfg, "fp16",
                            icfg.top_k, rows=[(0, t) for t in ts])
    for t in ts:
        pool = pool0.copy()
        c = t + 1
        done = t // r if c % r else c // r - 1            # blocks finished before token t
        for g in range(done):
            pg, row = O.pool_row(pool, pt, 0, 1, r * g)
            pool[pg, row, 0, D:] = O.narrow(kbar[g], "fp16")
        for s in range(r * (t // r), t):                     # raw keys of the open block
            pg, row = O.pool_row(pool, pt, 0, 0, s)
            pool[pg, row, 0, D:] = inp.idx_k[0, s]
        # the oracle's prefill handoff over the first t tokens leaves exactly these tails
        handoff = O.prefill_state_writes(inp.idx_k[:, :t], inp.w_k, np.array([t]), pt, icfg, D, "fp16")
        pool_h = pool0.copy()
        O.apply_tail_writes(pool_h, handoff, D)
        assert np.array_equal(pool_h.view(np.uint16), pool.view(np.uint16))
        writes, lists = O.indexer_decode(inp.idx_q[:, t:t + 1], inp.idx_k[:, t:t + 1], inp.w_q,
                                         inp.w_k, pool, pt, np.array([c]), icfg, D, "fp16",
                                         icfg.top_k)
        assert np.array_equal(lists[0, 0], pre[(0, t)])
        assert len(writes) == 1
        pg, row, vals = writes[0]
        if c % r:
            assert (pg, row) == O.pool_row(pool, pt, 0, 0, t)
            assert np.array_equal(vals, inp.idx_k[0, t])
        else:
            assert (pg, row) == O.pool_row(pool, pt, 0, 1, r * (c // r - 1))
            assert np.array_equal(O.widen(vals, "fp16"), kbar[c // r - 1])


def test_decode_steps_after_prefill_handoff_match_prefill_rows():
    """Multi-step decode from the prefill handoff: after a prefill of c tokens,
    decode steps at c+1, c+2, ... select for rows c, c+1, ... exactly as a
    prefill over the longer sequence does, and the pool then holds the state
    a prefill of the longer sequence would leave."""
    icfg = syn.IndexerCfg(budget=5)
    hd, D, r = icfg.head_dim, 16, icfg.compress_ratio
    S = 90
    inp = syn.make_prefill(43, B=2, S=S, Hq=2, Hkv=2, D=D, dtype="bf16", ctx=[S, S], icfg=icfg)
    rng = np.random.default_rng(43)
    pool, pt = _pool_from_dense(rng, inp.k[0], inp.v[0], D, hd)
    pt = np.concatenate([pt, pt], axis=0)                # both sequences share the layout, own rows differ
    pool = np.concatenate([pool, pool], axis=0)
    npg = pool.shape[0] // 4
    pt[1, 0] = np.where(pt[1, 0] >= 0, pt[1, 0] + 2 * npg, -1)
    pt[1, 1] = np.where(pt[1, 1] >= 0, pt[1, 1] + 2 * npg, -1)
    starts = [61, 70]                                    # prefill lengths: 1 and 2 tokens of an open block
    pre = O.indexer_prefill(inp.idx_q, inp.idx_k, inp.w_q, inp.w_k, inp.ctx, icfg, "bf16", icfg.top_k)
    for b, c0 in enumerate(starts):
        O.apply_tail_writes(pool, [w for w in O.prefill_state_writes(inp.idx_k[b:b + 1, :c0], inp.w_k,
                                                                        np.array([c0]), pt[b:b + 1], icfg, D,
                                                                        "bf16")], D)
    for step in range(9):
        ctx = np.array([c0 + step + 1 for c0 in starts])
        tok = ctx - 1
        q1 = np.stack([inp.idx_q[b, tok[b]] for b in range(2)])[:, None]
        k1 = np.stack([inp.idx_k[b, tok[b]] for b in range(2)])[:, None]
        writes, lists = O.indexer_decode(q1, k1, inp.w_q, inp.w_k, pool, pt, ctx, icfg, D, "bf16", icfg.top_k)
        for b in range(2):
            assert np.array_equal(lists[b, 0], pre[b, tok[b]]), (step, b)
        O.apply_tail_writes(pool, writes, D)
    for b, c0 in enumerate(starts):
        c = c0 + 9
        expect = O.prefill_state_writes(inp.idx_k[b:b + 1, :c], inp.w_k, np.array([c]), pt[b:b + 1], icfg, D, "bf16")
        for pg, row, vals in expect:
            assert np.array_equal(pool[pg, row, 0, D:].view(np.uint16), vals.view(np.uint16))


# ---------------------------------------------------------------------------
# front end [Plugin: fused step 1; KV pool contract]
# ---------------------------------------------------------------------------
def test_front_end_gamma_is_the_folded_one_plus_w():
    """The front end's qk-norm takes the gain already folded (gamma = 1 + w);
    it equals the indexer's RMSNorm*(1+w) on the same w, and gamma = 1 leaves
    an output RMS of sqrt(ms / (ms + eps))."""
    rng = np.random.default_rng(50)
    x = rng.standard_normal((3, 128))
    w = rng.standard_normal(128) * 0.1
    eps = 1e-6
    assert np.allclose(O.rms_norm_gamma(x, 1.0 + w, eps), O.rms_norm(x, w, eps), rtol=0, atol=1e-15)
    y = O.rms_norm_gamma(x, np.ones(128), eps)
    ms = np.mean(x * x, axis=1)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), np.sqrt(ms / (ms + eps)), rtol=1e-14)


def test_front_end_packed_layout():
    """A packed row is Q heads, then K heads, then V heads, D each."""
    Hq, Hkv, D = 3, 2, 4
    row = np.arange((Hq + 2 * Hkv) * D, dtype=np.float64)
    q, k, v = O.split_packed_qkv(row, Hq, Hkv, D)
    for h in range(Hq):
        assert list(q[h]) == [h * D + d for d in range(D)]
    for h in range(Hkv):
        assert list(k[h]) == [(Hq + h) * D + d for d in range(D)]
        assert list(v[h]) == [(Hq + Hkv + h) * D + d for d in range(D)]


def test_front_end_position_zero_is_norm_times_gamma_hand_loop():
    """At position 0 RoPE is the identity: q and k are x / sqrt(mean x^2 + eps)
    * gamma, rounded once; written out with fsum loops.  V is the packed V
    unchanged, bit for bit."""
    rng = np.random.default_rng(51)
    Hq, Hkv, D = 2, 1, 64
    qkv = syn.normal(rng, (1, 1, (Hq + 2 * Hkv) * D), "fp16")
    gq = (1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    gk = (1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    eps = 1e-6
    q, k, v, _ = O.front_end(qkv, gq, gk, [1], Hq, Hkv, D, 32, 1e6, eps, "fp16")
    x = qkv[0, 0].astype(np.float64)
    e32 = float(np.float32(eps))
    for h, (out, g, base) in enumerate([(q[0, 0, 0], gq, 0), (q[0, 0, 1], gq, D), (k[0, 0, 0], gk, Hq * D)]):
        xs = x[base:base + D]
        den = math.sqrt(math.fsum(t * t for t in xs) / D + e32)
        want = np.array([xs[d] / den * float(g[d]) for d in range(D)]).astype(np.float16)
        assert np.array_equal(out, want), f"head {h}"
    assert np.array_equal(v[0, 0, 0], qkv[0, 0, (Hq + Hkv) * D:])


def test_front_end_pool_matches_dense_mirrors_through_permuted_pages():
    """The rows the front end writes to the paged pool (through a permuted
    page table, V pages offset by numPages) are the rows of its dense K/V
    mirrors: decode attention over the pool equals prefill attention over the
    mirrors for the same list.  Tails (columns >= D) and dead rows are not
    written."""
    rng = np.random.default_rng(52)
    B, S, Hq, Hkv, D, hd = 2, 300, 8, 2, 64, 32
    ctx = np.array([300, 171], dtype=np.int32)
    qkv = syn.normal(rng, (B, S, (Hq + 2 * Hkv) * D), "bf16")
    gq = (1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    gk = (1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    pages = [3, 2]
    perm = rng.permutation(sum(pages)).astype(np.int32)
    npg = len(perm)
    pt = np.full((B, 2, 4), -1, dtype=np.int32)
    pt[0, 0, :3], pt[1, 0, :2] = perm[:3], perm[3:5]
    pt[:, 1] = np.where(pt[:, 0] >= 0, pt[:, 0] + npg, -1)
    q, k, v, writes = O.front_end(qkv, gq, gk, ctx, Hq, Hkv, D, 32, 1e6, 1e-6, "bf16", page_table=pt)
    assert len(writes) == 2 * int(ctx.sum())
    pool = syn.normal(rng, (2 * npg, 128, Hkv, D + hd), "bf16")
    before = pool.copy()
    O.apply_front_end_writes(pool, writes, D)
    assert np.array_equal(pool[..., D:], before[..., D:]), "a tail changed"
    for b in range(B):
        t = int(ctx[b]) - 1
        ids = np.sort(rng.choice(t + 1, min(t + 1, 40), replace=False)).astype(np.int32)
        lst = np.full((B, 1, 64), -1, dtype=np.int32)
        lst[b, 0, :ids.size] = ids
        ql = q[:, t:t + 1]
        dec = O.sparse_decode(ql, pool, pt, lst, ctx, 0.125, D, "bf16", seqs=[b])[b]
        full = np.full((B, S, 64), -1, dtype=np.int32)
        full[b, t, :ids.size] = ids
        pre = O.sparse_prefill(q, k, v, full, ctx, 0.125, "bf16", rows=[(b, t)])[(b, t)]
        assert np.allclose(dec, pre, rtol=0, atol=1e-12)


def test_front_end_append_equals_prefill_row():
    """Decode's rope-append of token p (one row, start = p) gives prefill row
    p's q, k and pool rows bit for bit."""
    rng = np.random.default_rng(53)
    B, S, Hq, Hkv, D = 1, 70, 4, 1, 128
    qkv = syn.normal(rng, (B, S, (Hq + 2 * Hkv) * D), "fp16")
    g = (1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    pt = np.array([[[0], [1]]], dtype=np.int32)
    q, k, v, w = O.front_end(qkv, g, g, [S], Hq, Hkv, D, 64, 1e6, 1e-6, "fp16", page_table=pt)
    for p in (0, 1, 37, 69):
        q1, k1, v1, w1 = O.front_end(qkv[:, p:p + 1], g, g, [p + 1], Hq, Hkv, D, 64, 1e6, 1e-6, "fp16",
                                     start=[p], page_table=pt)
        assert np.array_equal(q1[0, 0], q[0, p]) and np.array_equal(k1[0, 0], k[0, p])
        assert np.array_equal(v1[0, 0], v[0, p])
        want = [x for x in w if x[1] == p]
        assert len(w1) == 2 and all(a[:3] == b_[:3] and np.array_equal(a[3], b_[3]) for a, b_ in zip(w1, want))


# ---------------------------------------------------------------------------
# chunked prefill [reading: a chunk row's list is the prefill list of its position]
# ---------------------------------------------------------------------------
def _paged_state(rng, B, N, D, Hkv, hd, dtype, k, v):
    """A pool holding the K/V rows of positions < N of each sequence (columns
    [0, D)) through a permuted page table, random tails elsewhere."""
    pages = (N + 127) // 128
    perm = rng.permutation(B * pages).astype(np.int32)
    npg = B * pages
    pt = np.full((B, 2, pages), -1, dtype=np.int32)
    for b in range(B):
        pt[b, 0] = perm[b * pages:(b + 1) * pages]
        pt[b, 1] = pt[b, 0] + npg
    pool = syn.normal(rng, (2 * npg, 128, Hkv, D + hd), dtype)
    for b in range(B):
        tok = np.arange(N)
        pool[pt[b, 0, tok // 128], tok % 128, :, :D] = k[b, :N]
        pool[pt[b, 1, tok // 128], tok % 128, :, :D] = v[b, :N]
    return pool, pt


@pytest.mark.parametrize("P,N", [(300, 377), (301, 390), (302, 303), (303, 420), (96, 100), (0, 70)])
def test_chunk_equals_unchunked_prefill(P, N):
    """Prefill of P tokens (its state handed to the pool tails), then one
    chunk of the tokens P .. N-1: the chunk's lists are the prefill lists of
    rows P .. N-1 of a one-shot prefill of N tokens, bit for bit; its tail
    writes leave the state a prefill of N leaves; its attention over the pool
    equals the prefill attention of those rows."""
    icfg = syn.IndexerCfg(budget=8)
    rng = np.random.default_rng(60 + P + N)
    B, Hq, Hkv, D, dt = 2, 4, 2, 64, "fp16"
    inp = syn.make_prefill(60, B=B, S=N, Hq=Hq, Hkv=Hkv, D=D, dtype=dt, ctx=[N, N], icfg=icfg)
    ref = O.indexer_prefill(inp.idx_q, inp.idx_k, inp.w_q, inp.w_k, inp.ctx, icfg, dt, icfg.top_k)
    pool, pt = _paged_state(rng, B, N, D, Hkv, icfg.head_dim, dt, inp.k, inp.v)
    start = np.array([P, P], dtype=np.int32)
    O.apply_tail_writes(pool, O.prefill_state_writes(inp.idx_k, inp.w_k, start, pt, icfg, D, dt), D)
    writes, lists = O.indexer_chunk(inp.idx_q[:, P:], inp.idx_k[:, P:], inp.w_q, inp.w_k, pool, pt, start, inp.ctx,
                                    icfg, D, dt, icfg.top_k)
    assert np.array_equal(lists, ref[:, P:])
    after = pool.copy()
    O.apply_tail_writes(after, writes, D)
    want = pool.copy()
    O.apply_tail_writes(want, O.prefill_state_writes(inp.idx_k, inp.w_k, inp.ctx, pt, icfg, D, dt), D)
    # the state a decode continues from: V-row tails of complete blocks and K-row tails of the open block
    r = icfg.compress_ratio
    for b in range(B):
        for g in range(N // r):
            pg, row = O.pool_row(None, pt, b, 1, r * g)
            assert np.array_equal(after[pg, row, 0, D:], want[pg, row, 0, D:]), f"kbar of block {g}"
        for j in range(r * (N // r), N):
            pg, row = O.pool_row(None, pt, b, 0, j)
            assert np.array_equal(after[pg, row, 0, D:], want[pg, row, 0, D:]), f"raw tail of token {j}"
    out = O.sparse_chunk(inp.q[:, P:], pool, pt, lists, start, inp.ctx, inp.scale, D, dt)
    pre = O.sparse_prefill(inp.q, inp.k, inp.v, ref, inp.ctx, inp.scale, dt)
    assert np.allclose(out, pre[:, P:], rtol=0, atol=1e-12)


def test_chunk_of_one_row_is_a_decode_step():
    inp = syn.make_decode(64, ctx=[2052, 9001, 7, 4096], B=4, Hq=8, Hkv=2, D=64, dtype="bf16", max_pages=80)
    w1, l1 = O.indexer_decode(inp.idx_q, inp.idx_k, inp.w_q, inp.w_k, inp.pool, inp.page_table, inp.ctx, inp.icfg,
                              inp.D, inp.dtype, inp.top_k)
    w2, l2 = O.indexer_chunk(inp.idx_q, inp.idx_k, inp.w_q, inp.w_k, inp.pool, inp.page_table, inp.ctx - 1, inp.ctx,
                             inp.icfg, inp.D, inp.dtype, inp.top_k)
    assert np.array_equal(l1, l2)
    key = lambda w: sorted((int(p), int(r), tuple(v.view(np.uint16).tolist())) for p, r, v in w)
    assert key(w1) == key(w2)


def test_chunk_padding_rows():
    """Chunk rows at or past the total length: lists all -1, output +0.0."""
    icfg = syn.IndexerCfg(budget=4)
    inp = syn.make_prefill(65, B=2, S=40, Hq=2, Hkv=1, D=64, dtype="fp16", ctx=[40, 40], icfg=icfg)
    rng = np.random.default_rng(65)
    pool, pt = _paged_state(rng, 2, 40, 64, 1, 128, "fp16", inp.k, inp.v)
    start = np.array([20, 30], dtype=np.int32)
    ctx = np.array([33, 30], dtype=np.int32)       # 13 live rows; none in the second sequence
    O.apply_tail_writes(pool, O.prefill_state_writes(inp.idx_k, inp.w_k, start, pt, icfg, 64, "fp16"), 64)
    _, lists = O.indexer_chunk(inp.idx_q[:, 20:], inp.idx_k[:, 20:], inp.w_q, inp.w_k, pool, pt, start, ctx, icfg,
                               64, "fp16", icfg.top_k)
    assert np.all(lists[0, 13:] == -1) and np.all(lists[1] == -1) and np.all(lists[0, :13, 0] >= 0)
    out = O.sparse_chunk(inp.q[:, 20:], pool, pt, lists, start, ctx, inp.scale, 64, "fp16")
    assert np.all(out[0, 13:] == 0) and np.all(out[1] == 0)
