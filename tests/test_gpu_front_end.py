"""Parity of the fused front end (qsa_qkv_front_end, through the C ABI) with
the oracle: Q, the dense K/V mirrors and the pool's leading head_dim columns
bit for bit (fp64 evaluation, one rounding on both sides), every pool tail
and every row past the live length left bit-unchanged."""
import numpy as np
import pytest
import torch

import qsa_synth as syn
import qsa_testlib as TL
import top_indexed_sparse_qsa_amd as Q
from oracle import qsa_oracle as O

pytestmark = pytest.mark.gpu
THETA, EPS = 1.0e6, 1.0e-6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("a gpu test ran without a GPU")
    Q.load()
    yield
    torch.cuda.synchronize()


def run_gpu(inp, mirrors=True, pool=True):
    qkv = TL.dev(inp.qkv, inp.dtype)
    q = torch.full((inp.B, inp.S, inp.Hq, inp.D), float("nan"), dtype=qkv.dtype, device="cuda")
    k = torch.full((inp.B, inp.S, inp.Hkv, inp.D), float("nan"), dtype=qkv.dtype, device="cuda") if mirrors else None
    v = torch.full_like(k, float("nan")) if mirrors else None
    pool_d = TL.dev(inp.pool, inp.dtype) if pool else None
    Q.qsa_qkv_front_end(qkv, TL.dev(inp.q_gamma), TL.dev(inp.k_gamma), TL.dev(inp.ctx), q, inp.Hq, inp.Hkv, inp.rot,
                        THETA, EPS, k_out=k, v_out=v,
                        start_positions=None if inp.start is None else TL.dev(inp.start),
                        kv_pool=pool_d, page_table=TL.dev(inp.page_table) if pool else None)
    torch.cuda.synchronize()
    return q, k, v, pool_d


def bits(t):
    return t.detach().cpu().view(torch.int16).numpy()


def oracle_bits(a, dtype):
    a = np.ascontiguousarray(a)
    return a.view(np.int16)


CASES = [
    dict(B=2, S=300, Hq=8, Hkv=2, D=128, dtype="fp16", ctx=[300, 171], rot=64),
    dict(B=2, S=200, Hq=16, Hkv=4, D=128, dtype="bf16", ctx=[133, 200], rot=128),
    dict(B=3, S=130, Hq=4, Hkv=4, D=64, dtype="bf16", ctx=[130, 1, 0], rot=34),   # odd half: partners across lanes
    dict(B=2, S=70, Hq=4, Hkv=2, D=128, dtype="fp16", ctx=[70, 33], rot=34),      # odd half, two dims per lane
    dict(B=1, S=257, Hq=12, Hkv=3, D=64, dtype="fp16", ctx=[257], rot=0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c['B']}S{c['S']}Hq{c['Hq']}Hkv{c['Hkv']}D{c['D']}{c['dtype']}rot{c['rot']}")
def test_front_end_small_bit_exact(case):
    TL.log(f"front end {case}")
    inp = syn.make_front_end(61, **case)
    q, k, v, pool = run_gpu(inp)
    rq, rk, rv, writes = O.front_end(inp.qkv, inp.q_gamma, inp.k_gamma, inp.ctx, inp.Hq, inp.Hkv, inp.D, inp.rot,
                                     THETA, EPS, inp.dtype, page_table=inp.page_table)
    assert np.array_equal(bits(q), oracle_bits(rq, inp.dtype)), "q differs"
    assert np.array_equal(bits(k), oracle_bits(rk, inp.dtype)), "k mirror differs"
    assert np.array_equal(bits(v), oracle_bits(rv, inp.dtype)), "v mirror differs"
    expect = inp.pool.copy()
    O.apply_front_end_writes(expect, writes, inp.D)
    assert np.array_equal(bits(pool), oracle_bits(expect, inp.dtype)), "pool differs (columns [0,D) or a tail)"


def test_front_end_decode_append_pool_only():
    """Decode: one new token per sequence at its past length, Q and the pool
    rows only (no mirrors); nothing else in the pool changes."""
    ctx = np.array([1, 129, 4000, 2052], dtype=np.int32)
    inp = syn.make_front_end(62, B=4, S=1, Hq=32, Hkv=4, D=128, dtype="fp16", ctx=ctx, rot=64, start=ctx - 1)
    q, _, _, pool = run_gpu(inp, mirrors=False)
    rq, _, _, writes = O.front_end(inp.qkv, inp.q_gamma, inp.k_gamma, inp.ctx, inp.Hq, inp.Hkv, inp.D, inp.rot,
                                   THETA, EPS, inp.dtype, start=inp.start, page_table=inp.page_table)
    assert np.array_equal(bits(q), oracle_bits(rq, inp.dtype))
    expect = inp.pool.copy()
    O.apply_front_end_writes(expect, writes, inp.D)
    assert len(writes) == 8
    assert np.array_equal(bits(pool), oracle_bits(expect, inp.dtype))


def test_front_end_long_prefill_shape_sampled_rows():
    """The long prefill's shape (S = 32768, Hq 32, Hkv 4, D 128, fp16) in one
    call: sampled rows against the oracle (row by row, each at its own
    position), every other pool row untouched outside the live rows."""
    S = 32768
    inp = syn.make_front_end(63, B=1, S=S, Hq=32, Hkv=4, D=128, dtype="fp16", ctx=[S - 5], rot=64)
    q, k, v, pool = run_gpu(inp)
    rng = np.random.default_rng(63)
    rows = sorted(set([0, 1, 127, 128, 4095, S - 6, S - 5, S - 1] + rng.integers(0, S, 40).tolist()))
    qb, kb, vb = bits(q), bits(k), bits(v)
    for t in rows:
        rq, rk, rv, _ = O.front_end(inp.qkv[:, t:t + 1], inp.q_gamma, inp.k_gamma, inp.ctx, inp.Hq, inp.Hkv, inp.D,
                                    inp.rot, THETA, EPS, inp.dtype, start=[t])
        assert np.array_equal(qb[0, t], oracle_bits(rq[0, 0], inp.dtype)), f"q row {t}"
        assert np.array_equal(kb[0, t], oracle_bits(rk[0, 0], inp.dtype)), f"k row {t}"
        assert np.array_equal(vb[0, t], oracle_bits(rv[0, 0], inp.dtype)), f"v row {t}"
    # the pool holds the mirrors' rows at every live position and nothing changed in the tails
    pool_b = bits(pool)
    before = oracle_bits(inp.pool, inp.dtype)
    assert np.array_equal(pool_b[..., inp.D:], before[..., inp.D:]), "a pool tail changed"
    pt = inp.page_table
    live = S - 5
    tok = np.arange(live)
    kp, vp = pt[0, 0, tok // 128], pt[0, 1, tok // 128]
    assert np.array_equal(pool_b[kp, tok % 128, :, :inp.D], kb[0, :live]), "pool K rows differ from the mirror"
    assert np.array_equal(pool_b[vp, tok % 128, :, :inp.D], vb[0, :live]), "pool V rows differ from the mirror"
    dead = np.arange(live, ((live + 127) // 128) * 128)
    assert np.array_equal(pool_b[pt[0, 0, dead // 128], dead % 128], before[pt[0, 0, dead // 128], dead % 128])
