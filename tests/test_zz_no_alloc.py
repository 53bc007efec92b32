"""The allocation-free decode indexer (qsa_indexer_decode_noalloc) against
qsa_indexer_decode with a caller workspace: the same lists and the same pool
bit for bit, on two calls in a row, the second on a smaller input (so the
per-GPU scratch holds the first call's scores when the second one starts)."""
import numpy as np
import pytest
import torch

import qsa_synth as syn
import qsa_testlib as TL
import top_indexed_sparse_qsa_amd as Q

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("a gpu test ran without a GPU")
    Q.load()
    yield
    torch.cuda.synchronize()


def _both(inp):
    cfg = TL.idx_cfg_struct(inp.icfg)
    args = lambda: (TL.dev(inp.idx_q, inp.dtype), TL.dev(inp.idx_k, inp.dtype), TL.dev(inp.w_q), TL.dev(inp.w_k))
    pool_a, pool_b = TL.dev(inp.pool, inp.dtype), TL.dev(inp.pool, inp.dtype)
    pt, ctx = TL.dev(inp.page_table), TL.dev(inp.ctx)
    ws = torch.empty(Q.qsa_indexer_decode_workspace_bytes(cfg, inp.B, inp.max_pages), dtype=torch.uint8,
                     device="cuda")
    la = torch.full((inp.B, 1, inp.top_k), -7, dtype=torch.int32, device="cuda")
    lb = torch.full((inp.B, 1, inp.top_k), -7, dtype=torch.int32, device="cuda")
    Q.qsa_indexer_decode(*args(), pool_a, pt, ctx, la, ws, cfg, inp.D)
    Q.qsa_indexer_decode_noalloc(*args(), pool_b, pt, ctx, lb, cfg, inp.D)
    torch.cuda.synchronize()
    return la, lb, pool_a, pool_b


def test_noalloc_matches_workspace_call_twice_second_smaller():
    cases = [
        syn.make_decode(31, ctx=[1, 6, 2052, 3000, 4096, 8191, 30000, 65535], B=8, Hq=32, Hkv=4, D=128,
                        dtype="fp16", max_pages=512),
        syn.make_decode(32, ctx=[2051, 7, 4100], B=3, Hq=8, Hkv=2, D=64, dtype="bf16", max_pages=40),
    ]
    for i, inp in enumerate(cases):
        TL.log(f"noalloc call {i}: B={inp.B} max_pages={inp.max_pages} {inp.dtype}")
        need = Q.qsa_indexer_decode_workspace_bytes(TL.idx_cfg_struct(inp.icfg), inp.B, inp.max_pages)
        assert need <= Q.QSA_NOALLOC_SCRATCH_BYTES
        la, lb, pa, pb = _both(inp)
        assert torch.equal(la, lb), f"call {i}: lists differ"
        assert torch.equal(pa.view(torch.int16), pb.view(torch.int16)), f"call {i}: pool tails differ"
        assert int((la == -7).sum()) == 0
