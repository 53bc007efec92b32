"""Benchmark of the QSA hot path on one MI355X.

One step = one prefill pass of the chosen workload: qsa_indexer_prefill
(pooling, query prep, block scoring, top-512 select + expand) followed by
qsa_sparse_prefill over the lists it produced.  Inputs are resident in HBM
before the timed region.  The decode pair (qsa_indexer_decode +
qsa_sparse_decode) on the paged workload is timed the same way and reported
in the "decode" object of the same JSON line.

Prints ONE JSON line.  The roofline object covers the dominant call
(qsa_sparse_prefill: its tile and row kernels): algorithmic bytes per call /
its average duration measured with HIP events on the launch stream (timing-only
events, created without the system-scope fence), against
HBM, and the algorithmic flops (QK^T and PV over the listed keys) against
the dense fp16/bf16 MFMA peak.  cpu_baseline times the CPU oracle on the
same workload.
"""
from __future__ import annotations

import argparse
import json
import math
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
KERNEL_SRC = os.path.join(ROOT, "top_indexed_sparse_qsa_amd", "csrc", "sparse_attention.hip")
METRIC = "sparse prefill tokens/s + decode seqs/s (topK 2051); % HBM roofline"
PREFILL_WORKLOADS = (2, 3, 5)
TIMING_EVERY = 5  # prefill steps between timed (event-bracketed) steps
DECODE_WORKLOAD = 4


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2, choices=PREFILL_WORKLOADS,
                    help="prefill workload timed as the step (default: 2)")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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


def dev(a, dtype=None):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def cfg_struct(Q, icfg):
    return Q.indexer_config(icfg.num_heads, icfg.head_dim, icfg.rot_dim, icfg.compress_ratio, icfg.budget,
                            icfg.rope_theta, icfg.rms_eps)


def prefill_bench(args, Q, syn, torch):
    inp = syn.workload(args.workload)
    icfg = inp.icfg
    e = 2
    cfg = cfg_struct(Q, icfg)
    q, k, v = dev(inp.q, inp.dtype), dev(inp.k, inp.dtype), dev(inp.v, inp.dtype)
    iq, ik = dev(inp.idx_q, inp.dtype), dev(inp.idx_k, inp.dtype)
    wq, wk, ctx = dev(inp.w_q), dev(inp.w_k), dev(inp.ctx)
    o = torch.empty_like(q)
    lists = torch.empty((inp.B, inp.S, icfg.top_k), dtype=torch.int32, device="cuda")
    ws = torch.empty(Q.qsa_indexer_prefill_workspace_bytes(cfg, inp.B, inp.S), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    T = HipTimingEvents()

    def step(ev=None):
        if ev:
            T.record(ev[0], stream)
        Q.qsa_indexer_prefill(iq, ik, wq, wk, ctx, lists, ws, cfg, stream=stream)
        if ev:
            T.record(ev[1], stream)
        Q.qsa_sparse_prefill(q, k, v, o, lists, ctx, inp.scale, stream=stream)
        if ev:
            T.record(ev[2], stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Timing events on every TIMING_EVERY-th step of the timed region only:
    # each recorded event still costs the kernels after it ~2 us, which the
    # path itself does not have.
    sampled = list(range(0, args.steps, TIMING_EVERY))
    evs = {i: [T.create() for _ in range(3)] for i in sampled}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs.get(i))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    idx_ms = [T.elapsed_ms(a, b) for a, b, _ in evs.values()]
    attn_ms = [T.elapsed_ms(b, c) for _, b, c in evs.values()]
    T.destroy_all()

    live = int(sum(min(int(c), inp.S) for c in inp.ctx))
    dead = inp.B * inp.S - live
    n_entries = int((lists >= 0).sum().item())          # listed ids over all live rows
    attn_bytes = (n_entries * inp.Hkv * 2 * inp.D * e + live * inp.Hq * inp.D * e * 2
                  + live * icfg.top_k * 4 + dead * inp.Hq * inp.D * e)
    attn_avg = float(np.mean(attn_ms)) * 1e-3
    idx_avg = float(np.mean(idx_ms)) * 1e-3
    achieved = attn_bytes / attn_avg / 1e9
    # QK^T and PV over the listed keys, per query head: 2 * D + 2 * D flops per id
    attn_flops = n_entries * inp.Hq * inp.D * 4
    res = {
        "inp": inp, "live": live, "wall": wall,
        "ms_per_step": wall / args.steps * 1e3,
        "indexer_ms": idx_avg * 1e3, "attention_ms": attn_avg * 1e3,
        "attn_bytes": attn_bytes, "achieved_gbs": achieved, "n_entries": n_entries,
        "attn_flops": attn_flops, "achieved_tflops": attn_flops / attn_avg / 1e12,
    }
    del q, k, v, iq, ik, o, lists, ws
    torch.cuda.empty_cache()
    return res


def decode_bench(args, Q, syn, torch):
    inp = syn.workload(DECODE_WORKLOAD)
    icfg = inp.icfg
    e = 2
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
    stream = torch.cuda.current_stream()
    T = HipTimingEvents()

    def step(ev=None):
        if ev:
            T.record(ev[0], stream)
        Q.qsa_indexer_decode(iq, ik, wq, wk, pool, pt, ctx, lists, ws, cfg, inp.D, stream=stream)
        if ev:
            T.record(ev[1], stream)
        Q.qsa_sparse_decode(q, o, pool, pt, lists, ctx, po, ps, inp.scale, head_dim=inp.D, stream=stream)
        if ev:
            T.record(ev[2], stream)

    steps = max(args.steps, 50)
    for _ in range(max(args.warmup, 5)):
        step()
    torch.cuda.synchronize()
    evs = [[T.create() for _ in range(3)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    idx_ms = float(np.median([T.elapsed_ms(a, b) for a, b, _ in evs]))
    attn_ms = float(np.median([T.elapsed_ms(b, c) for _, b, c in evs]))
    T.destroy_all()
    n_entries = int((lists >= 0).sum().item())
    nblk = int(sum(int(c) // icfg.compress_ratio for c in inp.ctx))
    attn_bytes = n_entries * inp.Hkv * 2 * inp.D * e + inp.B * (inp.Hq * inp.D * e * 2 + inp.top_k * 4)
    idx_bytes = nblk * icfg.head_dim * e + inp.B * inp.top_k * 4
    step_ms = idx_ms + attn_ms
    out = {
        "workload": syn.WORKLOADS[DECODE_WORKLOAD],
        "value": inp.B / (step_ms * 1e-3),
        "unit": "seqs/s",
        "ms_per_step": step_ms,
        "wall_ms_per_step": wall / steps * 1e3,
        "indexer_ms": idx_ms,
        "attention_ms": attn_ms,
        "steps": steps,
        "algorithmic_bytes_per_step": attn_bytes + idx_bytes,
        "hbm_frac_step": (attn_bytes + idx_bytes) / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "attention_gbs": attn_bytes / (attn_ms * 1e-3) / 1e9,
        "splits": Q.qsa_sparse_decode_default_splits(inp.B, inp.Hkv, inp.top_k),
    }
    del pool
    torch.cuda.empty_cache()
    return out


def kernel_code_sha256(path=None):
    """sha256 of the attention kernel source with its comments and blank
    space removed, so that the counter figures survive comment edits but
    not code changes."""
    import hashlib
    import re
    with open(path or KERNEL_SRC) as f:
        text = re.sub(r"//[^\n]*|/\*.*?\*/", "", f.read(), flags=re.S)
    code = "\n".join(" ".join(line.split()) for line in text.splitlines() if line.strip())
    return hashlib.sha256(code.encode()).hexdigest()


def measured_traffic(wl):
    """HBM bytes per sparse_prefill launch from the committed rocprofv3
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


def cpu_baseline(wl):
    """The oracle, unchanged, on the same workload (single thread)."""
    import qsa_synth as syn
    from threadpoolctl import threadpool_limits

    from oracle import qsa_oracle as O
    inp = syn.workload(wl)
    icfg = inp.icfg
    if wl == 2:
        rows = None
        n_rows = inp.B * inp.S
        sample = "all 4096 rows of the workload (indexer + attention)"
    else:
        rng = np.random.default_rng(7)
        rows = [(b, int(t)) for b in range(inp.B) for t in rng.integers(0, min(int(inp.ctx[b]), inp.S), 256)]
        n_rows = len(rows)
        sample = f"{n_rows} random live rows (indexer + attention), extrapolated per row"
    with threadpool_limits(1):
        t0 = time.perf_counter()
        lists = O.indexer_prefill(inp.idx_q, inp.idx_k, inp.w_q, inp.w_k, inp.ctx, icfg, inp.dtype, icfg.top_k,
                                  rows=rows)
        if rows is not None:
            full = np.full((inp.B, inp.S, icfg.top_k), -1, dtype=np.int32)
            for r, l in lists.items():
                full[r] = l
            lists = full
        O.sparse_prefill(inp.q, inp.k, inp.v, lists, inp.ctx, inp.scale, inp.dtype, rows=rows)
        dt = time.perf_counter() - t0
    live_rows = n_rows if rows is not None else int(sum(min(int(c), inp.S) for c in inp.ctx))
    return {"value": live_rows / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": sample, "seconds": dt, "cpu": platform.processor() or platform.machine()}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the QSA hot path is single-GPU work here "
              "(sharding is described, not built); rerun with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    import qsa_synth as syn
    import top_indexed_sparse_qsa_amd as Q
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    Q.load()
    print(f"# bench: prefill workload {args.workload}", file=sys.stderr, flush=True)
    pf = prefill_bench(args, Q, syn, torch)
    print(f"# bench: prefill {pf['ms_per_step']:.3f} ms/step", file=sys.stderr, flush=True)
    dec = None
    if not args.no_decode:
        print("# bench: decode workload 4", file=sys.stderr, flush=True)
        dec = decode_bench(args, Q, syn, torch)
        print(f"# bench: decode {dec['ms_per_step']:.4f} ms/step", file=sys.stderr, flush=True)
    if args.calib_copy:
        n = 1 << 30
        a = torch.empty(n // 2, dtype=torch.float16, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        del a, b
    cpu = None
    if not args.no_cpu_baseline:
        print("# bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(args.workload)

    inp = pf["inp"]
    value = pf["live"] * args.steps / pf["wall"]
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pf["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": inp.dtype,
        "data": "synthetic",
        "config": {"workload": syn.WORKLOADS[args.workload], "batch": inp.B, "seq_len": inp.S,
                   "live_tokens": pf["live"], "num_q_heads": inp.Hq, "num_kv_heads": inp.Hkv,
                   "head_dim": inp.D, "top_k": inp.icfg.top_k, "parallelism": "none"},
        "parts_ms": {"indexer_prefill": pf["indexer_ms"], "sparse_prefill": pf["attention_ms"],
                     "timed_steps": len(range(0, args.steps, TIMING_EVERY))},
        "roofline": {"bound": "hbm", "kernel": "qsa_sparse_prefill: sparse_prefill_tile_kernel + sparse_prefill_kernel",
                     "achieved": pf["achieved_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": pf["achieved_gbs"] / HBM_PEAK_GBS, "traffic": measured_traffic(args.workload),
                     "algorithmic_bytes_per_call": pf["attn_bytes"],
                     "mfma": {"achieved": pf["achieved_tflops"], "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                              "frac": pf["achieved_tflops"] / MFMA_PEAK_TFLOPS,
                              "algorithmic_flops_per_call": pf["attn_flops"]}},
        "cpu_baseline": cpu,
        "decode": dec,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
