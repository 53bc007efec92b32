"""qsa_decode_step: the decode indexer and the sparse decode in one call, with
the select (decode B3) fused into the attention kernel.  Its results are the
two separate calls' results bit for bit -- the pool tails, the lists and the
output -- on every path (fused: up to 16384 blocks per row and one workgroup
per (sequence, KV head); otherwise the two calls' own kernels), and the
oracle's through them (checked directly on a small case).
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


class Bufs:
    """Device copies of one decode input (its own pool: B1 writes the tails)."""

    def __init__(self, inp):
        self.cfg = TL.idx_cfg_struct(inp.icfg)
        self.pool = TL.dev(inp.pool, inp.dtype)
        self.pt = TL.dev(inp.page_table)
        self.ctx = TL.dev(inp.ctx)
        self.q = TL.dev(inp.q, inp.dtype)
        self.iq, self.ik = TL.dev(inp.idx_q, inp.dtype), TL.dev(inp.idx_k, inp.dtype)
        self.wq, self.wk = TL.dev(inp.w_q), TL.dev(inp.w_k)
        self.ws = torch.empty(Q.qsa_indexer_decode_workspace_bytes(self.cfg, inp.B, inp.max_pages),
                              dtype=torch.uint8, device="cuda")
        self.po = torch.empty(Q.qsa_sparse_decode_partial_o_elems(inp.B, inp.Hkv, inp.D), dtype=torch.float32,
                              device="cuda")
        self.ps = torch.empty(Q.qsa_sparse_decode_partial_stats_elems(inp.B, inp.Hkv), dtype=torch.float32,
                              device="cuda")
        self.lists = torch.full((inp.B, 1, inp.top_k), -7, dtype=torch.int32, device="cuda")
        self.o = torch.full_like(self.q, float("nan"))


def separate(inp, bb, splits):
    Q.qsa_indexer_decode(bb.iq, bb.ik, bb.wq, bb.wk, bb.pool, bb.pt, bb.ctx, bb.lists, bb.ws, bb.cfg, inp.D)
    Q.qsa_sparse_decode(bb.q, bb.o, bb.pool, bb.pt, bb.lists, bb.ctx, bb.po, bb.ps, inp.scale, head_dim=inp.D,
                        num_splits=splits)
    torch.cuda.synchronize()


def fused(inp, bb, splits):
    Q.qsa_decode_step(bb.iq, bb.ik, bb.wq, bb.wk, bb.q, bb.o, bb.pool, bb.pt, bb.ctx, bb.lists, bb.ws, bb.cfg,
                      inp.scale, partial_o=bb.po, partial_stats=bb.ps, head_dim=inp.D, num_splits=splits)
    torch.cuda.synchronize()


def same_bits(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype != torch.int32 else a,
                       b.view(torch.int16) if b.dtype != torch.int32 else b)


def compare(inp, what, splits=(0,)):
    for ns in splits:
        TL.log(f"{what}: num_splits={ns}")
        ref, got = Bufs(inp), Bufs(inp)
        separate(inp, ref, ns)
        fused(inp, got, ns)
        assert same_bits(got.pool, ref.pool), f"{what} splits={ns}: pool tails differ"
        assert torch.equal(got.lists, ref.lists), f"{what} splits={ns}: lists differ"
        assert same_bits(got.o, ref.o), f"{what} splits={ns}: output differs"


STEP_CASES = [
    dict(B=6, Hq=32, Hkv=4, D=128, dtype="fp16", ctx=[1, 6, 2052, 3000, 4096, 8191], max_pages=64),
    dict(B=5, Hq=64, Hkv=4, D=128, dtype="bf16", ctx=[2, 7, 2051, 5000, 2049], max_pages=40),
    dict(B=3, Hq=8, Hkv=2, D=64, dtype="fp16", ctx=[0, 2200, 4100], max_pages=33),
    # budget / tail boundaries: nc = budget - 1, budget, budget + 1 with each tail length
    dict(B=8, Hq=16, Hkv=2, D=128, dtype="bf16", ctx=[3, 4, 2047, 2048, 2049, 2050, 2051, 2052], max_pages=17),
]


@pytest.mark.parametrize("case", STEP_CASES, ids=lambda c: f"B{c['B']}Hq{c['Hq']}D{c['D']}{c['dtype']}")
def test_decode_step_equals_two_calls(case):
    inp = syn.make_decode(21, **case)
    compare(inp, f"decode step {case['B']}x{case['Hq']}", splits=(0, 1, 3, 8, 13, 16))


@pytest.mark.parametrize("max_pages,ctx", [(256, [32768, 32767, 30001]), (257, [32896, 100, 2052]),
                                            (512, [65536, 65535, 40000]), (513, [65540, 65536, 9000])],
                         ids=lambda v: str(v))
def test_decode_step_row_width_classes(max_pages, ctx):
    """Rows of up to 8192 blocks hold 16 scores per thread, up to 16384 32;
    past 16384 (513 pages) the step runs the two calls' own kernels."""
    inp = syn.make_decode(22, ctx=ctx, B=3, Hq=32, Hkv=4, D=128, dtype="fp16", max_pages=max_pages)
    compare(inp, f"decode step max_pages={max_pages}")


def test_decode_step_small_budget_against_oracle():
    """A small budget (8 blocks, top_k 35) on a short pool, checked against the
    oracle directly: lists by the margin rule, output per row."""
    icfg = syn.IndexerCfg(budget=8)
    inp = syn.make_decode(23, ctx=[0, 1, 5, 33, 34, 35, 36, 200, 511], B=9, Hq=8, Hkv=2, D=64, dtype="fp16",
                          max_pages=4, icfg=icfg)
    compare(inp, "small budget", splits=(0, 2))
    bb = Bufs(inp)
    fused(inp, bb, 0)
    _, ref_lists, scores = O.indexer_decode(inp.idx_q, inp.idx_k, inp.w_q, inp.w_k, inp.pool, inp.page_table,
                                            inp.ctx, icfg, inp.D, inp.dtype, inp.top_k, return_scores=True)
    lists = bb.lists.cpu().numpy()
    ref_o = O.sparse_decode(inp.q, inp.pool, inp.page_table, ref_lists, inp.ctx, inp.scale, inp.D, inp.dtype)
    got = TL.host_f64(bb.o, inp.dtype)[:, 0]
    for b in range(inp.B):
        c = int(inp.ctx[b])
        if c <= 0:
            assert np.all(lists[b, 0] == -1)
            TL.check_zero_rows(bb.o[b], f"small budget b={b} (empty)")
            continue
        swapped = TL.check_list(lists[b, 0], ref_lists[b, 0], scores[b], c - 1, icfg, f"small budget b={b}")
        if not swapped:
            TL.check_attention(got[b], ref_o[b], inp.dtype, f"small budget b={b}")


def test_decode_step_workload4_and_reruns():
    """The decode workload at full size (B=32, ctx ~ U[8192, 65536]): the step
    equals the two calls, and ten more steps on the same state give the same
    bits (the tails a step writes are the ones it read)."""
    TL.log("decode step workload 4: generating")
    inp = syn.workload(4)
    compare(inp, "decode step workload 4", splits=(0,))
    bb = Bufs(inp)
    fused(inp, bb, 0)
    lists0, o0 = bb.lists.clone(), bb.o.clone()
    for i in range(10):
        bb.lists.fill_(-7)
        bb.o.fill_(float("nan"))
        fused(inp, bb, 0)
        assert torch.equal(bb.lists, lists0), f"rerun {i}: lists differ"
        assert same_bits(bb.o, o0), f"rerun {i}: output differs"
