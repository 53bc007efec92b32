"""Benchmark of the QSA hot path on one MI355X.

One step = one prefill pass of the headline workload (the long prefill,
B=1 S=32768 Hq=32 Hkv=4 D=128 fp16 by default): qsa_indexer_prefill
(pooling, query prep, block scoring, top-512 select + expand) followed by
qsa_sparse_prefill over the lists it produced.  Inputs are resident in HBM
before the timed region.  ``value`` is live tokens per second over the wall
clock of the timed steps.

The same JSON line carries, per workload, the same measurement for the other
prefill workloads (``workloads``: the tiny fixed-list one runs attention
only), and the decode pair (qsa_indexer_decode + qsa_sparse_decode) on the
paged workload (``decode``, sequences per second over the wall clock).

Rooflines.  Every ``frac`` is a fraction of a published peak that the
quantity really can reach:
* prefill attention: algorithmic flops (QK^T and PV over the listed keys)
  per second against the dense fp16/bf16 MFMA peak.  The algorithmic bytes
  (every listed K/V row counted once per row) exceed the HBM peak in rate,
  because rows share K/V through the caches, so they are reported as a rate
  of their own (``algorithmic_byte_rate_gbs``), not as a fraction; HBM is
  priced with the bytes the counters saw (``traffic``, from the committed
  rocprofv3 FETCH_SIZE / WRITE_SIZE figures, null once the kernel code has
  changed since they were taken).
* indexer: scoring flops against the MFMA peak.
* decode: algorithmic bytes per step (distinct pool rows, far larger than
  the caches) against HBM.
Kernel durations are HIP-event averages on the launch stream over a loop of
their own (timing-only events, created without the system-scope fence), so
that the wall-clock loop carries no events.

``cpu_baseline`` times the oracle, unchanged, on all host cores (one worker
process per core, single-threaded BLAS each, over a bounded row sample); it
runs before the GPU is touched.
"""
from __future__ import annotations

import argparse
import json
import multiprocessing as mp
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0  # dense fp16 / bf16
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sparse_prefill_traffic.txt")
# the code the prefill attention kernels are built from
KERNEL_SRCS = [os.path.join(ROOT, "top_indexed_sparse_qsa_amd", "csrc", f)
               for f in ("sparse_attention.hip", "attention_core.h", "qsa_device.h")]
METRIC = "sparse prefill tokens/s + decode seqs/s (topK 2051); % HBM roofline"
PREFILL_WORKLOADS = (1, 2, 3, 5)
DECODE_WORKLOAD = 4
HEADLINE = 3
MAX_CPU_WORKERS = 16  # the host share of one GPU on the box
CPU_PREFILL_ROWS = 1536
CPU_DECODE_SEQS = 32
CPU_DECODE_REPS = 6


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--headline", type=int, default=HEADLINE, choices=(2, 3, 5),
                    help="prefill workload whose rate is `value` (default: 3)")
    ap.add_argument("--workloads", default="1,2,3,4,5",
                    help="comma list of workloads to run (4 = decode); the headline always runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-front-end", action="store_true", help="skip the fused front end measurement")
    ap.add_argument("--no-chunk", action="store_true", help="skip the chunked prefill measurement")
    ap.add_argument("--no-ceilings", action="store_true", help="skip measuring the part's ceilings")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (HBM counter calibration)")
    return ap.parse_args()


class HipTimingEvents:
    """HIP events used only for timing, created with hipEventDisableSystemFence.

    A default event performs a system-scope cache writeback and invalidate
    when it is recorded, and the kernels after it pay for that (about 5 us
    per event between these kernels, measured on MI355X); events that only
    measure time do not need it.  They are recorded on the launch stream and
    read after a device synchronize.  The HIP runtime is the one torch
    loaded (libqsa.so resolves to the same library)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        path = "libamdhip64.so"
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        self.ct = ctypes
        self.hip = hip = ctypes.CDLL(path)
        vp = ctypes.c_void_p
        hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
        hip.hipEventRecord.argtypes = [vp, vp]
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        hip.hipEventDestroy.argtypes = [vp]
        self.made = []

    def _ok(self, what, rc):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def create(self):
        ev = self.ct.c_void_p()
        self._ok("hipEventCreateWithFlags", self.hip.hipEventCreateWithFlags(self.ct.byref(ev), self.DISABLE_SYSTEM_FENCE))
        self.made.append(ev)
        return ev

    def record(self, ev, stream):
        self._ok("hipEventRecord", self.hip.hipEventRecord(ev, self.ct.c_void_p(stream.cuda_stream)))

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        self._ok("hipEventElapsedTime", self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b))
        return float(ms.value)

    def destroy_all(self):
        for ev in self.made:
            self.hip.hipEventDestroy(ev)
        self.made = []


def note(msg):
    print(f"# bench: {msg}", file=sys.stderr, flush=True)


def dev(a, dtype=None):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def cfg_struct(Q, icfg):
    return Q.indexer_config(icfg.num_heads, icfg.head_dim, icfg.rot_dim, icfg.compress_ratio, icfg.budget,
                            icfg.rope_theta, icfg.rms_eps)


def timed_loops(step, steps, warmup, stream, torch, n_marks):
    """Wall clock of `steps` calls of step() (no events), then a second loop
    of `steps` calls with timing events at the n_marks points step() offers;
    returns (wall seconds, [per-interval average ms])."""
    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    T = HipTimingEvents()
    evs = [[T.create() for _ in range(n_marks)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step(lambda k, i=i: T.record(evs[i][k], stream))
    torch.cuda.synchronize()
    parts = [float(np.mean([T.elapsed_ms(e[k], e[k + 1]) for e in evs])) for k in range(n_marks - 1)]
    T.destroy_all()
    return wall, parts


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------
def prefill_bench(wl, inp, args, Q, torch):
    e = 2
    stream = torch.cuda.current_stream()
    q, k, v = dev(inp.q, inp.dtype), dev(inp.k, inp.dtype), dev(inp.v, inp.dtype)
    ctx = dev(inp.ctx)
    o = torch.empty_like(q)
    with_indexer = inp.indices is None
    if with_indexer:
        icfg = inp.icfg
        top_k = icfg.top_k
        cfg = cfg_struct(Q, icfg)
        iq, ik = dev(inp.idx_q, inp.dtype), dev(inp.idx_k, inp.dtype)
        wq, wk = dev(inp.w_q), dev(inp.w_k)
        lists = torch.empty((inp.B, inp.S, top_k), dtype=torch.int32, device="cuda")
        ws = torch.empty(Q.qsa_indexer_prefill_workspace_bytes(cfg, inp.B, inp.S), dtype=torch.uint8,
                         device="cuda")
    else:
        top_k = inp.top_k
        lists = dev(inp.indices)

    def step(mark):
        if mark:
            mark(0)
        if with_indexer:
            Q.qsa_indexer_prefill(iq, ik, wq, wk, ctx, lists, ws, cfg, stream=stream)
        if mark:
            mark(1)
        Q.qsa_sparse_prefill(q, k, v, o, lists, ctx, inp.scale, stream=stream)
        if mark:
            mark(2)

    wall, (idx_ms, attn_ms) = timed_loops(step, args.steps, args.warmup, stream, torch, 3)
    live = int(sum(min(int(c), inp.S) for c in inp.ctx))
    dead = inp.B * inp.S - live
    n_entries = int((lists >= 0).sum().item())  # listed ids over all live rows
    attn_bytes = (n_entries * inp.Hkv * 2 * inp.D * e + live * inp.Hq * inp.D * e * 2
                  + live * top_k * 4 + dead * inp.Hq * inp.D * e)
    attn_flops = n_entries * inp.Hq * inp.D * 4  # QK^T and PV per query head: 4 D flops per listed id
    attn_s = attn_ms * 1e-3
    traffic = measured_traffic(wl)
    attention = {
        "kernel": "qsa_sparse_prefill (sparse_prefill_kernel list walk + sparse_prefill_tile_kernel)",
        "bound": "mfma", "achieved": attn_flops / attn_s / 1e12, "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
        "frac": attn_flops / attn_s / 1e12 / MFMA_PEAK_TFLOPS, "traffic": traffic,
        "algorithmic_flops_per_call": attn_flops, "algorithmic_bytes_per_call": attn_bytes,
        "algorithmic_byte_rate_gbs": attn_bytes / attn_s / 1e9,
        "hbm_counter_gbs": traffic / attn_s / 1e9 if traffic else None,
        "hbm_counter_frac": traffic / attn_s / 1e9 / HBM_PEAK_GBS if traffic else None,
        "ms_per_call": attn_ms,
    }
    res = {
        "workload": __import__("qsa_synth").WORKLOADS[wl],
        "value": live * args.steps / wall, "unit": "tokens/s",
        "ms_per_step": wall / args.steps * 1e3, "steps": args.steps,
        "dtype": inp.dtype, "batch": inp.B, "seq_len": inp.S, "live_tokens": live,
        "num_q_heads": inp.Hq, "num_kv_heads": inp.Hkv, "head_dim": inp.D, "top_k": top_k,
        "attention_ms": attn_ms, "attention": attention,
    }
    if with_indexer:
        icfg = inp.icfg
        r = icfg.compress_ratio
        pairs = sum(sum((t + 1) // r for t in range(min(int(c), inp.S))) for c in inp.ctx)
        score_flops = pairs * icfg.num_heads * icfg.head_dim * 2
        res["indexer_ms"] = idx_ms
        res["indexer"] = {"kernel": "qsa_indexer_prefill (prep, MFMA scoring, radix select + expand)",
                          "bound": "mfma", "achieved": score_flops / (idx_ms * 1e-3) / 1e12,
                          "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "frac": score_flops / (idx_ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS,
                          "algorithmic_flops_per_call": score_flops}
    else:
        res["note"] = "fixed lists, attention only; a few microseconds per call: launch-bound, roofline not meaningful"
    del q, k, v, o, lists
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------
def decode_bench(inp, args, Q, torch):
    icfg = inp.icfg
    e = 2
    stream = torch.cuda.current_stream()
    cfg = cfg_struct(Q, icfg)
    pool = dev(inp.pool, inp.dtype)
    pt, ctx = dev(inp.page_table), dev(inp.ctx)
    iq, ik, wq, wk = dev(inp.idx_q, inp.dtype), dev(inp.idx_k, inp.dtype), dev(inp.w_q), dev(inp.w_k)
    q = dev(inp.q, inp.dtype)
    o = torch.empty_like(q)
    lists = torch.empty((inp.B, 1, inp.top_k), dtype=torch.int32, device="cuda")
    ws = torch.empty(Q.qsa_indexer_decode_workspace_bytes(cfg, inp.B, inp.max_pages), dtype=torch.uint8,
                     device="cuda")
    po = torch.empty(Q.qsa_sparse_decode_partial_o_elems(inp.B, inp.Hkv, inp.D), dtype=torch.float32, device="cuda")
    ps = torch.empty(Q.qsa_sparse_decode_partial_stats_elems(inp.B, inp.Hkv), dtype=torch.float32, device="cuda")

    def step(mark):  # one decode step through qsa_decode_step (select fused into the attention kernel)
        if mark:
            mark(0)
        Q.qsa_decode_step(iq, ik, wq, wk, q, o, pool, pt, ctx, lists, ws, cfg, inp.scale, partial_o=po,
                          partial_stats=ps, head_dim=inp.D, stream=stream)
        if mark:
            mark(1)

    def two_calls(mark):  # the same step as qsa_indexer_decode + qsa_sparse_decode
        if mark:
            mark(0)
        Q.qsa_indexer_decode(iq, ik, wq, wk, pool, pt, ctx, lists, ws, cfg, inp.D, stream=stream)
        if mark:
            mark(1)
        Q.qsa_sparse_decode(q, o, pool, pt, lists, ctx, po, ps, inp.scale, head_dim=inp.D, stream=stream)
        if mark:
            mark(2)

    wall2, (idx_ms, attn_ms) = timed_loops(two_calls, args.steps, args.warmup, stream, torch, 3)
    wall, (step_ms,) = timed_loops(step, args.steps, args.warmup, stream, torch, 2)
    n_entries = int((lists >= 0).sum().item())
    nblk = int(sum(int(c) // icfg.compress_ratio for c in inp.ctx))
    attn_bytes = n_entries * inp.Hkv * 2 * inp.D * e + inp.B * (inp.Hq * inp.D * e * 2 + inp.top_k * 4)
    idx_bytes = nblk * icfg.head_dim * e + inp.B * inp.top_k * 4
    step_s = wall / args.steps
    gbs = lambda nbytes, ms: nbytes / (ms * 1e-3) / 1e9
    out = {
        "workload": __import__("qsa_synth").WORKLOADS[DECODE_WORKLOAD],
        "value": inp.B / step_s,
        "unit": "seqs/s",
        "ms_per_step": step_s * 1e3,
        "steps": args.steps,
        "entry_point": "qsa_decode_step",
        "step_gpu_ms": step_ms,
        "algorithmic_bytes_per_step": attn_bytes + idx_bytes,
        "roofline": {"kernel": "one decode step (qsa_decode_step: idx_dec_score_kernel + "
                               "decode_select_attend_kernel)", "bound": "hbm",
                     "achieved": (attn_bytes + idx_bytes) / step_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": (attn_bytes + idx_bytes) / step_s / 1e9 / HBM_PEAK_GBS},
        "two_calls": {
            "ms_per_step": wall2 / args.steps * 1e3,
            "indexer_ms": idx_ms,
            "attention_ms": attn_ms,
            "attention": {"kernel": "qsa_sparse_decode", "bound": "hbm", "achieved": gbs(attn_bytes, attn_ms),
                          "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs(attn_bytes, attn_ms) / HBM_PEAK_GBS,
                          "algorithmic_bytes_per_call": attn_bytes},
            "indexer": {"kernel": "qsa_indexer_decode", "bound": "hbm", "achieved": gbs(idx_bytes, idx_ms),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs(idx_bytes, idx_ms) / HBM_PEAK_GBS,
                        "algorithmic_bytes_per_call": idx_bytes},
        },
        "splits": Q.qsa_sparse_decode_default_splits(inp.B, inp.Hkv, inp.top_k),
    }
    del pool
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------
# front end (packed QKV -> Q, K/V mirrors, pool rows) at the long prefill's shape
# ---------------------------------------------------------------------------
FRONT_END_SHAPE = dict(B=1, S=32768, Hq=32, Hkv=4, D=128, dtype="fp16", ctx=[32768], rot=64)


def front_end_bench(args, Q, torch, syn):
    inp = syn.make_front_end(6, **FRONT_END_SHAPE)
    stream = torch.cuda.current_stream()
    qkv = dev(inp.qkv, inp.dtype)
    gq, gk, ctx = dev(inp.q_gamma), dev(inp.k_gamma), dev(inp.ctx)
    q = torch.empty((inp.B, inp.S, inp.Hq, inp.D), dtype=qkv.dtype, device="cuda")
    k = torch.empty((inp.B, inp.S, inp.Hkv, inp.D), dtype=qkv.dtype, device="cuda")
    v = torch.empty_like(k)
    pool, pt = dev(inp.pool, inp.dtype), dev(inp.page_table)

    def step(mark):
        if mark:
            mark(0)
        Q.qsa_qkv_front_end(qkv, gq, gk, ctx, q, inp.Hq, inp.Hkv, inp.rot, 1.0e6, 1.0e-6, k_out=k, v_out=v,
                            kv_pool=pool, page_table=pt, stream=stream)
        if mark:
            mark(1)

    wall, (ms,) = timed_loops(step, args.steps, args.warmup, stream, torch, 2)
    e = 2
    rows = inp.B * inp.S
    nbytes = rows * ((inp.Hq + 2 * inp.Hkv) * inp.D * e            # packed rows read
                     + inp.Hq * inp.D * e + 2 * inp.Hkv * inp.D * e  # Q and the K/V mirrors written
                     + 2 * inp.Hkv * inp.D * e)                      # pool K/V leading columns written
    out = {"workload": "fused front end at the long prefill's shape: B=1 S=32768 Hq=32 Hkv=4 D=128 fp16 rot 64, "
                       "packed QKV -> Q, dense K/V mirrors, paged pool rows",
           "value": rows / (wall / args.steps), "unit": "tokens/s", "ms_per_step": wall / args.steps * 1e3,
           "ms_per_call": ms,
           "roofline": {"kernel": "front_end_kernel", "bound": "hbm", "achieved": nbytes / (ms * 1e-3) / 1e9,
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                        "algorithmic_bytes_per_call": nbytes}}
    del qkv, q, k, v, pool
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------
# chunked prefill: the long prefill's last 2048 tokens as one chunk over the
# paged pool (the earlier 30720 tokens' K/V and indexer state already there)
# ---------------------------------------------------------------------------
CHUNK_PAST, CHUNK_LEN = 30720, 2048


def chunk_bench(inp, args, Q, torch, syn):
    icfg = inp.icfg
    e = 2
    stream = torch.cuda.current_stream()
    B, S, P, C = inp.B, inp.S, CHUNK_PAST, CHUNK_LEN
    pages = (S + 127) // 128
    rng = np.random.default_rng(8)
    perm = rng.permutation(B * pages).astype(np.int32)
    pt = np.full((B, 2, pages), -1, dtype=np.int32)
    for b in range(B):
        pt[b, 0] = perm[b * pages:(b + 1) * pages]
        pt[b, 1] = pt[b, 0] + B * pages
    ptd = dev(pt)
    # the pool: K/V of every position (leading columns) and the indexer state
    # of the first P tokens in the tails, laid down by the library itself
    pool = torch.zeros((2 * B * pages, 128, inp.Hkv, inp.D + icfg.head_dim), dtype=torch.float16, device="cuda")
    kd, vd = dev(inp.k, inp.dtype), dev(inp.v, inp.dtype)
    tok = torch.arange(S, device="cuda")
    for b in range(B):
        pool[ptd[b, 0, tok // 128].long(), tok % 128, :, :inp.D] = kd[b]
        pool[ptd[b, 1, tok // 128].long(), tok % 128, :, :inp.D] = vd[b]
    del kd, vd
    cfg = cfg_struct(Q, icfg)
    start = dev(np.full(B, P, dtype=np.int32))
    ctx = dev(np.full(B, S, dtype=np.int32))
    iq_all, ik_all = dev(inp.idx_q, inp.dtype), dev(inp.idx_k, inp.dtype)
    wq, wk = dev(inp.w_q), dev(inp.w_k)
    wsp = torch.empty(Q.qsa_indexer_prefill_workspace_bytes(cfg, B, P), dtype=torch.uint8, device="cuda")
    lp = torch.empty((B, P, icfg.top_k), dtype=torch.int32, device="cuda")
    iq_p, ik_p = iq_all[:, :P].contiguous(), ik_all[:, :P].contiguous()
    Q.qsa_indexer_prefill(iq_p, ik_p, wq, wk, start, lp, wsp, cfg,
                          stream=stream, kv_pool=pool, page_table=ptd, head_dim=inp.D)
    torch.cuda.synchronize()

    # the prefill -> decode handoff: the same indexer call without and with
    # the pool (which adds the tail writes); rerunning it rewrites the same
    # tails and lists
    def prefill_pair(mark):
        if mark:
            mark(0)
        Q.qsa_indexer_prefill(iq_p, ik_p, wq, wk, start, lp, wsp, cfg, stream=stream)
        if mark:
            mark(1)
        Q.qsa_indexer_prefill(iq_p, ik_p, wq, wk, start, lp, wsp, cfg,
                              stream=stream, kv_pool=pool, page_table=ptd, head_dim=inp.D)
        if mark:
            mark(2)

    _, (plain_ms, with_pool_ms) = timed_loops(prefill_pair, max(3, args.steps // 4), 1, stream, torch, 3)
    del wsp, lp, iq_p, ik_p
    iq, ik = iq_all[:, P:].contiguous(), ik_all[:, P:].contiguous()
    q = dev(np.ascontiguousarray(inp.q[:, P:]), inp.dtype)
    o = torch.empty_like(q)
    lists = torch.empty((B, C, icfg.top_k), dtype=torch.int32, device="cuda")
    ws = torch.empty(Q.qsa_indexer_chunk_workspace_bytes(cfg, B, C, pages), dtype=torch.uint8, device="cuda")

    def step(mark):
        if mark:
            mark(0)
        Q.qsa_indexer_chunk(iq, ik, wq, wk, pool, ptd, start, ctx, lists, ws, cfg, inp.D, stream=stream)
        if mark:
            mark(1)
        Q.qsa_sparse_chunk(q, o, pool, ptd, lists, start, ctx, inp.scale, head_dim=inp.D, stream=stream)
        if mark:
            mark(2)

    wall, (idx_ms, attn_ms) = timed_loops(step, args.steps, args.warmup, stream, torch, 3)
    n_entries = int((lists >= 0).sum().item())
    attn_flops = n_entries * inp.Hq * inp.D * 4
    out = {"workload": f"chunked prefill over the paged pool: the last {C} tokens of the long prefill (B=1 "
                       f"S=32768 Hq=32 Hkv=4 D=128 fp16) after {P} prefilled ones, topK 2051",
           "value": B * C / (wall / args.steps), "unit": "tokens/s", "ms_per_step": wall / args.steps * 1e3,
           "indexer_ms": idx_ms, "attention_ms": attn_ms,
           "prefill_handoff": {"indexer_prefill_ms": plain_ms, "with_pool_tails_ms": with_pool_ms,
                               "handoff_ms": with_pool_ms - plain_ms,
                               "note": f"qsa_indexer_prefill over the first {P} tokens without and with the "
                                       "pool (the decode indexer's tail state written as well)"},
           "attention": {"kernel": "qsa_sparse_chunk", "bound": "mfma",
                         "achieved": attn_flops / (attn_ms * 1e-3) / 1e12, "peak": MFMA_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": attn_flops / (attn_ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS,
                         "algorithmic_flops_per_call": attn_flops}}
    del pool, q, o, lists, ws, iq_all, ik_all
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------
# measured ceilings of this part (libqsa_ceilings.so, measurement only)
# ---------------------------------------------------------------------------
CEIL_LIB = os.path.join(ROOT, "top_indexed_sparse_qsa_amd", "libqsa_ceilings.so")


def measure_ceilings(torch):
    """HBM streaming read and random 256-byte row gathers from HBM (a 4 GiB
    buffer) and from L2 (a 2 MiB one, resident), each the median of 5 timed
    launches.  (MFMA fractions stay against the published dense peak.)"""
    import ctypes
    if not os.path.exists(CEIL_LIB):
        return None
    lib = ctypes.CDLL(CEIL_LIB)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.qsa_ceiling_stream_read.argtypes = [vp, sz, vp, i32, vp]
    lib.qsa_ceiling_gather_rows.argtypes = [vp, sz, i32, i32, ctypes.c_uint, vp, vp]
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    T = HipTimingEvents()
    out = torch.zeros(4, dtype=torch.int32, device="cuda")

    def med(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        ev = [(T.create(), T.create()) for _ in range(reps)]
        for a, b in ev:
            T.record(a, stream)
            rc = fn()
            T.record(b, stream)
            if rc != 0:
                raise RuntimeError(f"ceiling kernel failed with {rc}")
        torch.cuda.synchronize()
        return float(np.median([T.elapsed_ms(a, b) for a, b in ev])) * 1e-3

    big = torch.ones(4 << 30, dtype=torch.uint8, device="cuda")
    s_stream = med(lambda: lib.qsa_ceiling_stream_read(big.data_ptr(), big.numel(), out.data_ptr(), 1024, sp))
    waves, batches = 16384, 8
    s_gather = med(lambda: lib.qsa_ceiling_gather_rows(big.data_ptr(), big.numel(), waves, batches, 7,
                                                        out.data_ptr(), sp))
    del big
    small = torch.ones(2 << 20, dtype=torch.uint8, device="cuda")
    s_l2 = med(lambda: lib.qsa_ceiling_gather_rows(small.data_ptr(), small.numel(), waves, 4 * batches, 7,
                                                    out.data_ptr(), sp))
    del small
    T.destroy_all()
    torch.cuda.empty_cache()
    return {"hbm_stream_read_gbs": (4 << 30) / s_stream / 1e9,
            "hbm_gather_256B_gbs": waves * batches * 64 * 256 / s_gather / 1e9,
            "l2_gather_256B_gbs": waves * 4 * batches * 64 * 256 / s_l2 / 1e9,
            "note": "measured on this GPU in this run: a streaming read of 4 GiB; random 256-byte rows gathered "
                    "16 to a wave from a 4 GiB buffer (HBM) and from a 2 MiB one (L2-resident)"}


def attach_ceiling_fracs(line, ceil):
    """Each roofline object also gives its fraction of the matching measured
    ceiling (the published-peak fraction stays in `frac`)."""
    if not ceil:
        return
    def prefill(att):
        f = att["algorithmic_byte_rate_gbs"] / ceil["l2_gather_256B_gbs"]
        if f <= 1.0:
            att["frac_of_measured_l2_gather"] = f
        else:  # the listed ids' bytes are not what moves: list tiles stage each key chunk once for many rows
            att["frac_of_measured_l2_gather"] = None
            att["l2_gather_note"] = ("listed-id bytes above the measured L2 gather ceiling: these rows run as list "
                                     "tiles, which stage each 32-key chunk once for all the tile's rows; see the "
                                     "MFMA fraction")
    prefill(line["roofline"])
    for w in line["workloads"].values():
        if "algorithmic_byte_rate_gbs" in w["attention"]:
            prefill(w["attention"])
    dec = line.get("decode")
    if dec:
        for r in (dec["roofline"], dec["two_calls"]["attention"], dec["two_calls"]["indexer"]):
            r["frac_of_measured_hbm_gather"] = r["achieved"] / ceil["hbm_gather_256B_gbs"]
    fe = line.get("front_end")
    if fe:
        fe["roofline"]["frac_of_measured_hbm_stream"] = fe["roofline"]["achieved"] / ceil["hbm_stream_read_gbs"]


# ---------------------------------------------------------------------------
# HBM counter figures
# ---------------------------------------------------------------------------
def kernel_code_sha256(paths=None):
    """sha256 of the prefill attention kernels' sources with their comments
    and blank space removed, so that the counter figures survive comment
    edits but not code changes."""
    import hashlib
    import re
    code = []
    for path in paths or KERNEL_SRCS:
        with open(path) as f:
            text = re.sub(r"//[^\n]*|/\*.*?\*/", "", f.read(), flags=re.S)
        code.append("\n".join(" ".join(line.split()) for line in text.splitlines() if line.strip()))
    return hashlib.sha256("\n\f\n".join(code).encode()).hexdigest()


def measured_traffic(wl):
    """HBM bytes per qsa_sparse_prefill call from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary, if it was taken on this kernel code."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                line = line.strip()
                if line and not line.startswith("#") and "=" in line:
                    k, v = line.split("=", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_code_sha256") != kernel_code_sha256():
            return None
        return int(kv[f"workload{wl}_fetch_bytes"]) + int(kv[f"workload{wl}_write_bytes"])
    except (OSError, KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on every host core (forked workers, before the GPU
# is touched, so no worker holds the device)
# ---------------------------------------------------------------------------
_CPU = {}


def _cpu_prefill_chunk(rows):
    from threadpoolctl import threadpool_limits

    from oracle import qsa_oracle as O
    inp = _CPU["prefill"]
    icfg = inp.icfg
    with threadpool_limits(1):
        lists = O.indexer_prefill(inp.idx_q, inp.idx_k, inp.w_q, inp.w_k, inp.ctx, icfg, inp.dtype, icfg.top_k,
                                  rows=rows)
        O.sparse_prefill(inp.q, inp.k, inp.v, lists, inp.ctx, inp.scale, inp.dtype, rows=rows)
    return len(rows)


def _cpu_decode_chunk(seqs):
    from threadpoolctl import threadpool_limits

    from oracle import qsa_oracle as O
    inp = _CPU["decode"]
    with threadpool_limits(1):
        _, lists = O.indexer_decode(inp.idx_q, inp.idx_k, inp.w_q, inp.w_k, inp.pool, inp.page_table, inp.ctx,
                                    inp.icfg, inp.D, inp.dtype, inp.top_k, seqs=seqs)
        full = np.full((inp.B, 1, inp.top_k), -1, dtype=np.int32)
        for b, l in lists.items():
            full[b, 0] = l
        O.sparse_decode(inp.q, inp.pool, inp.page_table, full, inp.ctx, inp.scale, inp.D, inp.dtype, seqs=seqs)
    return len(seqs)


def _pool_run(fn, chunks, workers):
    ctx = mp.get_context("fork")
    with ctx.Pool(workers) as pool:
        pool.map(abs, range(workers))  # workers up before the clock starts
        t0 = time.perf_counter()
        n = sum(pool.map(fn, chunks, chunksize=1))
        dt = time.perf_counter() - t0
    return n, dt


def cpu_workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, MAX_CPU_WORKERS))


def cpu_baseline_prefill(inp, workers):
    rng = np.random.default_rng(7)
    live = [(b, int(t)) for b in range(inp.B) for t in range(min(int(inp.ctx[b]), inp.S))]
    pick = rng.choice(len(live), min(CPU_PREFILL_ROWS, len(live)), replace=False)
    rows = [live[i] for i in np.sort(pick)]
    chunks = [rows[i::workers] for i in range(workers)]
    _CPU["prefill"] = inp
    n, dt = _pool_run(_cpu_prefill_chunk, [c for c in chunks if c], workers)
    _CPU.pop("prefill")
    return {"value": n / dt, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": f"{n} live rows drawn uniformly from the workload (indexer + attention per row), "
                      f"rate = rows / wall time of {workers} single-threaded worker processes",
            "seconds": dt, "cpu": platform.processor() or platform.machine()}


def cpu_baseline_decode(inp, workers):
    seqs = list(range(min(CPU_DECODE_SEQS, inp.B))) * CPU_DECODE_REPS
    chunks = [seqs[i::workers] for i in range(workers)]
    _CPU["decode"] = inp
    n, dt = _pool_run(_cpu_decode_chunk, [c for c in chunks if c], workers)
    _CPU.pop("decode")
    return {"value": n / dt, "unit": "seqs/s", "cores": min(workers, n), "kind": "oracle",
            "sample": f"all {min(CPU_DECODE_SEQS, inp.B)} sequences of one decode step, {CPU_DECODE_REPS} times "
                      f"(indexer decode + sparse decode), spread over single-threaded worker processes",
            "seconds": dt, "cpu": platform.processor() or platform.machine()}


# ---------------------------------------------------------------------------
def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the QSA hot path is single-GPU work here "
              "(sharding is described, not built); rerun with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import qsa_synth as syn

    run = sorted({int(x) for x in args.workloads.split(",") if x.strip()} | {args.headline})
    inputs = {}

    def inp_of(wl):
        if wl not in inputs:
            note(f"generating workload {wl}")
            inputs[wl] = syn.workload(wl)
        return inputs[wl]

    cpu, cpu_dec = None, None
    if not args.no_cpu_baseline:
        workers = cpu_workers()
        note(f"cpu baseline (oracle), prefill workload {args.headline}, {workers} workers")
        cpu = cpu_baseline_prefill(inp_of(args.headline), workers)
        if DECODE_WORKLOAD in run:
            note(f"cpu baseline (oracle), decode workload {DECODE_WORKLOAD}")
            cpu_dec = cpu_baseline_decode(inp_of(DECODE_WORKLOAD), workers)

    import torch

    import top_indexed_sparse_qsa_amd as Q
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    Q.load()
    results = {}
    chunk = None
    order = [args.headline] + [w for w in run if w != args.headline]
    for wl in order:
        inp = inp_of(wl)
        note(f"workload {wl}")
        if wl == DECODE_WORKLOAD:
            results[wl] = decode_bench(inp, args, Q, torch)
        else:
            results[wl] = prefill_bench(wl, inp, args, Q, torch)
        note(f"workload {wl}: {results[wl]['ms_per_step']:.4f} ms/step")
        if wl == 3 and not args.no_chunk:
            note("chunked prefill")
            chunk = chunk_bench(inp, args, Q, torch, syn)
            note(f"chunked prefill: {chunk['ms_per_step']:.4f} ms/step")
        inputs.pop(wl, None)
    fe = None
    if not args.no_front_end:
        note("front end")
        fe = front_end_bench(args, Q, torch, syn)
        note(f"front end: {fe['ms_per_call']:.4f} ms/call")
    ceil = None
    if not args.no_ceilings:
        note("measured ceilings")
        ceil = measure_ceilings(torch)
    copy_gbs = None
    n = 1 << 30
    a = torch.empty(n // 2, dtype=torch.float16, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(10):
        b.copy_(a)
    torch.cuda.synchronize()
    copy_gbs = 2 * n * 10 / (time.perf_counter() - t0) / 1e9
    if args.calib_copy:
        torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
    del a, b

    head = results[args.headline]
    dec = results.get(DECODE_WORKLOAD)
    if dec is not None:
        dec["cpu_baseline"] = cpu_dec
    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": {"workload": head["workload"], "batch": head["batch"], "seq_len": head["seq_len"],
                   "live_tokens": head["live_tokens"], "num_q_heads": head["num_q_heads"],
                   "num_kv_heads": head["num_kv_heads"], "head_dim": head["head_dim"], "top_k": head["top_k"],
                   "parallelism": "none"},
        "parts_ms": {"indexer_prefill": head.get("indexer_ms"), "sparse_prefill": head["attention_ms"]},
        "roofline": head["attention"],
        "cpu_baseline": cpu,
        "workloads": {str(w): r for w, r in results.items() if w not in (args.headline, DECODE_WORKLOAD)},
        "decode": dec,
        "front_end": fe,
        "chunk": chunk,
        "hbm_copy_gbs": copy_gbs,
        "ceilings": ceil,
    }
    attach_ceiling_fracs(line, ceil)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
