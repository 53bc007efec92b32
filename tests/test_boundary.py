"""Host-side tests of the C ABI: the library loads, exports every function the
header declares, sizes workspaces by the documented formulas and rejects bad
arguments with the documented status before any device work.

The argument-rejection tests pass fake (never dereferenced) device addresses;
each case is built to fail validation.  They run without a GPU only."""
import ctypes
import os
import re

import pytest

import top_indexed_sparse_qsa_amd as Q
from top_indexed_sparse_qsa_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libqsa.h")

OK, NULLP, SHAPE, UNSUP, WS, LAUNCH = range(6)
FAKE = 0x7F0000000000          # 256-byte aligned, never dereferenced


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(qsa_[a-z_]+)\s*\(", txt)))


def test_header_and_binding_agree():
    assert _declared() == sorted(Q.EXPORTS)


def test_library_exports_every_declared_function():
    lib = Q.load()
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, f"libqsa.so lacks {missing}"


def test_status_strings():
    for s in range(6):
        assert isinstance(Q.qsa_status_string(s), str) and Q.qsa_status_string(s)
    assert Q.qsa_status_string(99) == "unknown status"


def test_workspace_sizes_follow_layout():
    cfg = Q.indexer_config()
    a = lambda x: (x + 255) // 256 * 256
    # prefill: queries (two fp16 pieces per value) | kbar | fp32 scores with a 16-rounded stride
    B, S = 1, 32768
    g = S // 4
    assert Q.qsa_indexer_prefill_workspace_bytes(cfg, B, S) == \
        a(B * S * 4 * 128 * 4) + a(B * g * 128 * 2) + a(B * S * g * 4)
    B, S = 4, 16383
    g = S // 4
    st = (g + 15) // 16 * 16
    assert Q.qsa_indexer_prefill_workspace_bytes(cfg, B, S) == \
        a(B * S * 4 * 128 * 4) + a(B * g * 128 * 2) + a(B * S * st * 4)
    # decode: one fp32 score row per sequence, stride 128 * max_pages / ratio rounded to 16
    assert Q.qsa_indexer_decode_workspace_bytes(cfg, 32, 512) == a(32 * 16384 * 4)
    assert Q.qsa_indexer_decode_workspace_bytes(cfg, 3, 33) == a(3 * 1056 * 4)
    # workgroup partials: at most QSA_MAX_SPLITS / 8 per (sequence, KV head)
    assert Q.qsa_sparse_decode_partial_o_elems(32, 4, 128) == 32 * 4 * 2 * 16 * 128
    assert Q.qsa_sparse_decode_partial_stats_elems(32, 4) == 32 * 4 * 2 * 2 * 16
    assert Q.qsa_indexer_prefill_workspace_bytes(Q.indexer_config(head_dim=64), 1, 10) == 0
    assert Q.qsa_sparse_decode_partial_o_elems(0, 4, 128) == 0


def test_default_split_plan():
    assert Q.qsa_sparse_decode_default_splits(32, 4, 2051) == 8      # ~1024 waves
    assert Q.qsa_sparse_decode_default_splits(8, 4, 2051) == 8       # one 8-wave workgroup per pair at most
    assert Q.qsa_sparse_decode_default_splits(1, 1, 40) == 2       # never more splits than 32-slot chunks
    assert Q.qsa_sparse_decode_default_splits(4096, 8, 2051) == 1
    assert Q.qsa_sparse_decode_default_splits(0, 4, 2051) == 0


@pytest.fixture
def no_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("argument-rejection cases use fake device addresses; host-only test")


def _prefill(**kw):
    p = L.SparsePrefillParams(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 8, 2, 128, 16, 0.125, 0, None)
    for k, v in kw.items():
        setattr(p, k, v)
    return Q.load().qsa_sparse_prefill(ctypes.byref(p))


def _decode(**kw):
    p = L.SparseDecodeParams(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                             2, 32, 4, 128, 256, 16, 8, 2051, 0, 0.088, 0, None)
    for k, v in kw.items():
        setattr(p, k, v)
    return Q.load().qsa_sparse_decode(ctypes.byref(p))


def _iprefill(**kw):
    cfg = kw.pop("cfg", Q.indexer_config())
    p = L.IndexerPrefillParams(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, 1, 4096, 2051, cfg, 0, None)
    for k, v in kw.items():
        setattr(p, k, v)
    return Q.load().qsa_indexer_prefill(ctypes.byref(p))


def _idecode(**kw):
    cfg = kw.pop("cfg", Q.indexer_config())
    p = L.IndexerDecodeParams(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40,
                              2, 4, 128, 256, 16, 8, 2051, cfg, 0, None)
    for k, v in kw.items():
        setattr(p, k, v)
    return Q.load().qsa_indexer_decode(ctypes.byref(p))


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), NULLP), (dict(indices=None), NULLP), (dict(context_lengths=None), NULLP),
    (dict(dtype=2), UNSUP), (dict(batch=0), SHAPE), (dict(seq_len=0), SHAPE), (dict(top_k=0), SHAPE),
    (dict(num_q_heads=7), SHAPE), (dict(num_q_heads=34), UNSUP), (dict(head_dim=96), UNSUP),
    (dict(num_kv_heads=0), SHAPE), (dict(q=FAKE + 8), SHAPE), (dict(attention_scale=float("inf")), SHAPE),
    (dict(attention_scale=0.0), SHAPE), (dict(attention_scale=-0.125), SHAPE), (dict(attention_scale=float("nan")), SHAPE),
    # 24-bit token-row multiply: ids and row bytes below 2^24
    (dict(seq_len=1 << 24, num_q_heads=1, num_kv_heads=1, head_dim=64), UNSUP),
    (dict(num_q_heads=1 << 16, num_kv_heads=1 << 16, head_dim=128, seq_len=1), UNSUP),
])
def test_sparse_prefill_rejects(no_gpu, kw, status):
    assert _prefill(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(partial_o=None, num_splits=9), NULLP), (dict(page_table=None), NULLP),
    (dict(partial_stats=None, num_splits=16), NULLP), (dict(partial_o=FAKE + 4, num_splits=12), SHAPE),
    (dict(dtype=-1), UNSUP), (dict(batch=0), SHAPE), (dict(num_flat_pages=0), SHAPE),
    (dict(pool_head_dim=120), SHAPE), (dict(pool_head_dim=130), SHAPE), (dict(num_splits=17), SHAPE),
    (dict(num_splits=-1), SHAPE), (dict(max_pages_per_seq=5000), UNSUP), (dict(num_q_heads=33), SHAPE),
    (dict(kv_pool=FAKE + 4), SHAPE), (dict(head_dim=256), UNSUP), (dict(attention_scale=0.0), SHAPE),
])
def test_sparse_decode_rejects(no_gpu, kw, status):
    assert _decode(**kw) == status


def test_sparse_decode_partials_only_needed_past_one_workgroup(no_gpu):
    """With the default plan (at most 8 splits, one workgroup per sequence and
    KV head) the partial buffers are unused and may be NULL; validation of
    the remaining arguments still runs first."""
    assert _decode(partial_o=None, partial_stats=None, num_splits=8, batch=0) == SHAPE
    assert _decode(partial_o=None, partial_stats=None, num_splits=0, head_dim=96) == UNSUP


@pytest.mark.parametrize("kw,status", [
    (dict(workspace=None), NULLP), (dict(q_norm_w=None), NULLP),
    (dict(cfg=Q.indexer_config(num_heads=5)), UNSUP), (dict(cfg=Q.indexer_config(head_dim=64)), UNSUP),
    (dict(cfg=Q.indexer_config(rot_dim=63)), UNSUP), (dict(cfg=Q.indexer_config(compress_ratio=9)), UNSUP),
    (dict(cfg=Q.indexer_config(budget=0)), SHAPE), (dict(cfg=Q.indexer_config(rms_eps=-1.0)), SHAPE),
    (dict(top_k=2050), SHAPE), (dict(seq_len=4 * 32768 + 4), UNSUP), (dict(workspace_bytes=1000), WS),
    (dict(workspace=FAKE + 16), SHAPE), (dict(dtype=3), UNSUP), (dict(batch=0), SHAPE),
])
def test_indexer_prefill_rejects(no_gpu, kw, status):
    assert _iprefill(**kw) == status


HANDOFF = dict(kv_pool=FAKE, page_table=FAKE, num_kv_heads=4, head_dim=128, pool_head_dim=256,
               num_flat_pages=16, max_pages_per_seq=8)


@pytest.mark.parametrize("kw,status", [
    (dict(page_table=None), NULLP), (dict(num_kv_heads=0), SHAPE), (dict(num_flat_pages=0), SHAPE),
    (dict(max_pages_per_seq=0), SHAPE), (dict(pool_head_dim=255), SHAPE), (dict(pool_head_dim=200), SHAPE),
    (dict(head_dim=0), SHAPE), (dict(head_dim=100), SHAPE), (dict(kv_pool=FAKE + 4), SHAPE),
])
def test_indexer_prefill_handoff_rejects(no_gpu, kw, status):
    """The optional pool handoff is checked like qsa_indexer_decode's pool."""
    assert _iprefill(**{**HANDOFF, **kw}) == status


@pytest.mark.parametrize("kw,status", [
    (dict(kv_pool=None), NULLP), (dict(indices=None), NULLP),
    (dict(pool_head_dim=255), SHAPE), (dict(pool_head_dim=200), SHAPE), (dict(top_k=100), SHAPE),
    (dict(max_pages_per_seq=2048), UNSUP), (dict(workspace_bytes=64), WS), (dict(num_kv_heads=0), SHAPE),
    (dict(cfg=Q.indexer_config(num_heads=0)), UNSUP), (dict(batch=1 << 23), UNSUP),
])
def test_indexer_decode_rejects(no_gpu, kw, status):
    assert _idecode(**kw) == status


def _step(ikw=None, akw=None, drop=None):
    """qsa_decode_step on a matching pair of structs, then edited."""
    cfg = Q.indexer_config()
    ip = L.IndexerDecodeParams(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40,
                               2, 4, 128, 256, 16, 8, 2051, cfg, 0, None)
    ap = L.SparseDecodeParams(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                              2, 32, 4, 128, 256, 16, 8, 2051, 0, 0.088, 0, None)
    for k, v in (ikw or {}).items():
        setattr(ip, k, v)
    for k, v in (akw or {}).items():
        setattr(ap, k, v)
    return Q.load().qsa_decode_step(None if drop == "i" else ctypes.byref(ip),
                                    None if drop == "a" else ctypes.byref(ap))


@pytest.mark.parametrize("ikw,akw,status", [
    # each half is validated as its own call would be
    (dict(workspace_bytes=64), {}, WS), (dict(kv_pool=None), {}, NULLP), ({}, dict(num_splits=17), SHAPE),
    ({}, dict(q=None), NULLP), ({}, dict(head_dim=96), UNSUP),
    # and both must describe the same step
    ({}, dict(indices=FAKE + 256), SHAPE), ({}, dict(context_lengths=FAKE + 256), SHAPE),
    ({}, dict(kv_pool=FAKE + 256), SHAPE), ({}, dict(page_table=FAKE + 256), SHAPE),
    ({}, dict(batch=3), SHAPE), ({}, dict(num_kv_heads=2), SHAPE), ({}, dict(top_k=2052), SHAPE),
    ({}, dict(dtype=1), SHAPE), ({}, dict(stream=1), SHAPE), ({}, dict(max_pages_per_seq=4), SHAPE),
    ({}, dict(num_flat_pages=17), SHAPE), (dict(pool_head_dim=264), dict(pool_head_dim=264, head_dim=64), SHAPE),
])
def test_decode_step_rejects(no_gpu, ikw, akw, status):
    assert _step(ikw, akw) == status


def test_decode_step_null_structs(no_gpu):
    assert _step(drop="i") == NULLP
    assert _step(drop="a") == NULLP


def _idecode_noalloc(**kw):
    cfg = kw.pop("cfg", Q.indexer_config())
    p = L.IndexerDecodeParams(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0,
                              2, 4, 128, 256, 16, 8, 2051, cfg, 0, None)
    for k, v in kw.items():
        setattr(p, k, v)
    return Q.load().qsa_indexer_decode_noalloc(ctypes.byref(p))


@pytest.mark.parametrize("kw,status", [
    (dict(kv_pool=None), NULLP), (dict(indices=None), NULLP), (dict(top_k=100), SHAPE),
    (dict(max_pages_per_seq=2048), UNSUP), (dict(cfg=Q.indexer_config(num_heads=0)), UNSUP),
    # the scratch holds batch * stride fp32 scores: 16 MiB, e.g. 256 sequences
    # of 512 pages; 257 of them do not fit
    (dict(batch=257, max_pages_per_seq=512), WS), (dict(batch=129, max_pages_per_seq=1024), WS),
])
def test_indexer_decode_noalloc_rejects(no_gpu, kw, status):
    """The allocation-free variant validates like qsa_indexer_decode, against
    its fixed scratch size, before any HIP call (the caller's workspace
    fields are ignored: here NULL and 0)."""
    assert _idecode_noalloc(**kw) == status


def test_noalloc_scratch_size_covers_the_decode_workload():
    cfg = Q.indexer_config()
    assert Q.qsa_indexer_decode_workspace_bytes(cfg, 256, 512) <= Q.QSA_NOALLOC_SCRATCH_BYTES
    assert Q.qsa_indexer_decode_workspace_bytes(cfg, 257, 512) > Q.QSA_NOALLOC_SCRATCH_BYTES
    hdr = open(HEADER).read()
    assert re.search(r"#define QSA_NOALLOC_SCRATCH_BYTES \(16u << 20\)", hdr)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(L, "_LIB", None)
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "libqsa.so"))
    with pytest.raises(RuntimeError, match="missing"):
        L.load()


def test_bench_counter_figures_follow_kernel_code(tmp_path):
    """The committed HBM counter figures apply while the attention kernel's
    code is unchanged: a comment or whitespace edit keeps the key, a code
    edit changes it."""
    import bench
    src = open(bench.KERNEL_SRCS[0]).read()
    rest = bench.KERNEL_SRCS[1:]
    base = bench.kernel_code_sha256()
    edited = tmp_path / "comments.hip"
    edited.write_text("// a new comment\n" + src.replace("\n", "\n\n", 3) + "\n/* trailing */\n")
    assert bench.kernel_code_sha256([str(edited)] + rest) == base
    changed = tmp_path / "code.hip"
    changed.write_text(src.replace("kTileRangeX2 = QSA_TILE_RANGE_X2", "kTileRangeX2 = QSA_TILE_RANGE_X2 + 1", 1))
    assert bench.kernel_code_sha256([str(changed)] + rest) != base
    # the shared chunk machinery counts too; the decode kernels do not
    assert any(p.endswith("attention_core.h") for p in rest)
    assert not any(p.endswith("decode_attention.hip") for p in bench.KERNEL_SRCS)


def test_product_path_and_oracle_are_separate():
    """The package (binding and HIP sources) never imports or includes the
    oracle, and the oracle never imports the package or its sources: the two
    share only the seeded input generator used by the tests."""
    import ast
    import subprocess
    import sys
    pkg = os.path.join(ROOT, "top_indexed_sparse_qsa_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            path = os.path.join(dirpath, f)
            if f.endswith(".py"):
                tree = ast.parse(open(path).read())
                mods = [a.name for n in ast.walk(tree) if isinstance(n, ast.Import) for a in n.names]
                mods += [n.module or "" for n in ast.walk(tree) if isinstance(n, ast.ImportFrom)]
                assert not [m for m in mods if m.split(".")[0] in ("oracle", "qsa_oracle", "qsa_synth")], path
            elif f.endswith((".hip", ".cpp", ".h")):
                incs = re.findall(r'#include\s+[<"]([^>"]+)[>"]', open(path).read())
                assert not [i for i in incs if "oracle" in i], path
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith(".py"):
            tree = ast.parse(open(os.path.join(ROOT, "oracle", f)).read())
            mods = [a.name for n in ast.walk(tree) if isinstance(n, ast.Import) for a in n.names]
            mods += [n.module or "" for n in ast.walk(tree) if isinstance(n, ast.ImportFrom)]
            assert not [m for m in mods if m.split(".")[0] in ("top_indexed_sparse_qsa_amd", "torch")], f
    # importing the binding and loading the library pulls in no oracle module
    code = ("import sys, top_indexed_sparse_qsa_amd as Q; Q.load(); "
            "print(sorted(m for m in sys.modules if 'oracle' in m))")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, check=True)
    assert out.stdout.strip() == "[]", out.stdout


def _front(**kw):
    p = L.FrontEndParams(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None,
                         1, 64, 8, 2, 128, 64, 0, 0, 0, 1.0e6, 1.0e-6, 0, None)
    for k, v in kw.items():
        setattr(p, k, v)
    return Q.load().qsa_qkv_front_end(ctypes.byref(p))


@pytest.mark.parametrize("kw,status", [
    (dict(qkv=None), NULLP), (dict(q_out=None), NULLP), (dict(k_out=None), NULLP), (dict(q_gamma=None), NULLP),
    (dict(dtype=5), UNSUP), (dict(batch=0), SHAPE), (dict(num_kv_heads=0), SHAPE), (dict(head_dim=96), UNSUP),
    (dict(rot_dim=130), UNSUP), (dict(rot_dim=33), UNSUP), (dict(rope_theta=0.0), SHAPE), (dict(rms_eps=-1.0), SHAPE),
    (dict(q_out=FAKE + 2), SHAPE), (dict(kv_pool=FAKE), NULLP),
    (dict(kv_pool=FAKE, page_table=FAKE, num_flat_pages=4, max_pages_per_seq=2, pool_head_dim=100), SHAPE),
    (dict(kv_pool=FAKE, page_table=FAKE, num_flat_pages=0, max_pages_per_seq=2, pool_head_dim=256), SHAPE),
])
def test_front_end_rejects(no_gpu, kw, status):
    assert _front(**kw) == status


def _ichunk(**kw):
    cfg = kw.pop("cfg", Q.indexer_config())
    p = L.IndexerChunkParams(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40,
                             2, 64, 4, 128, 256, 16, 8, 2051, cfg, 0, None)
    for k, v in kw.items():
        setattr(p, k, v)
    return Q.load().qsa_indexer_chunk(ctypes.byref(p))


def _schunk(**kw):
    p = L.SparseChunkParams(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 64, 32, 4, 128, 256, 16, 8, 2051, 0.088, 0, None)
    for k, v in kw.items():
        setattr(p, k, v)
    return Q.load().qsa_sparse_chunk(ctypes.byref(p))


@pytest.mark.parametrize("kw,status", [
    (dict(start_positions=None), NULLP), (dict(kv_pool=None), NULLP), (dict(workspace=None), NULLP),
    (dict(chunk_len=0), SHAPE), (dict(top_k=2050), SHAPE), (dict(pool_head_dim=200), SHAPE),
    (dict(max_pages_per_seq=2048), UNSUP), (dict(workspace_bytes=100), WS), (dict(workspace=FAKE + 8), SHAPE),
    (dict(cfg=Q.indexer_config(compress_ratio=0)), UNSUP),
])
def test_indexer_chunk_rejects(no_gpu, kw, status):
    assert _ichunk(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(start_positions=None), NULLP), (dict(indices=None), NULLP), (dict(chunk_len=0), SHAPE),
    (dict(num_q_heads=33), SHAPE), (dict(head_dim=96), UNSUP), (dict(max_pages_per_seq=5000), UNSUP),
    (dict(attention_scale=-1.0), SHAPE), (dict(q=FAKE + 4), SHAPE), (dict(pool_head_dim=120), SHAPE),
])
def test_sparse_chunk_rejects(no_gpu, kw, status):
    assert _schunk(**kw) == status


def test_chunk_workspace_follows_layout():
    cfg = Q.indexer_config()
    a = lambda x: (x + 255) // 256 * 256
    B, C, mp = 2, 100, 20
    g = mp * 128 // 4
    assert Q.qsa_indexer_chunk_workspace_bytes(cfg, B, C, mp) == a(B * C * 4 * 128 * 4) + a(B * g * 128 * 2) + \
        a(B * C * g * 4)
    assert Q.qsa_indexer_chunk_workspace_bytes(cfg, 0, C, mp) == 0
