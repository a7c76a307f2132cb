#!/usr/bin/env python3
"""Benchmark of the paged-attention decode step on one MI355X.

One step = one pass of the whole decode path (block-table gather, scores, online
softmax, V product, and for the split-context mode the log-sum-exp merge of the
partitions: inside the partition launch when each (sequence, KV head) is run by the
waves of one workgroup, else by a second launch) over the whole synthetic batch. Inputs are resident in HBM before timing starts. So that
every step reads its K/V from HBM and not from the 256 MB Infinity Cache or the L2s,
the benchmark keeps R identical replicas of the K and V pools (R x pool >= 2 GiB) and
step i reads replica i mod R, as a decode over many layers does.

The headline line is the largest single-GPU batch: 8 sequences x 32768 tokens (fp16,
32 heads, head_dim 128, 32-token blocks, ~4.3 GB of K/V), split into 512-token
partitions whose states are merged by log-sum-exp (the pages' second, split-context
kernel for long text). Beside it: the same batch in single-pass mode, the other three
measured batches (LLaMA-7B serving shape, shared 500-token prefix, 50/30/20 % length mix
with fp8 KV) in their default modes, the device's plain streaming-read rate for the same
load shape, and the fp64 CPU oracle on a bounded sample (one thread and all host cores).

Prints ONE JSON line. `value` = unique K/V bytes per step / wall time per step.
`roofline.achieved` = compulsory bytes per step (unique K/V, q, out, used table entries,
lengths) / GPU time per step, where the GPU time is measured by two HIP events recorded
on the launch stream around the timed steps (divided by their count).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3] [--mode auto]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD published peak
MFMA16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 / bf16 matrix peak, AMD published
EXTEND_METRIC = "paged extend (chunked prefill) attention TFLOP/s, causal algorithmic flops"
METRIC = "paged-attn decode KV GB/s read and % of MI355X HBM peak; seqs·tokens/s"
HEADLINE_CONFIG = 3
DEFAULT_MODE = {0: "direct", 1: "direct", 2: "direct", 3: "partitioned", 4: "ordered",
                "llama7b_fp16_bs128": "direct", "shared_prefix_bf16_bs256": "direct",
                "long_ctx_fp16_bs512": "ordered", "mixed_fp8_bs256": "ordered",
                "llama70b_gqa8_bf16": "ordered", "d256_gqa2_bf16": "direct",
                "shared_prefix_long_bf16": "grouped"}
SUB_CONFIGS = (1, 2, 4)
KERNEL_SOURCES = ["pagedattention_block_table_amd/csrc/pa_decode_impl.h",
                  "pagedattention_block_table_amd/csrc/pa_mfma_decode.h",
                  "pagedattention_block_table_amd/csrc/pa_group_decode.h",
                  "pagedattention_block_table_amd/csrc/pa_api.hip"]
KV_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1}
IO_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str, mode: str):
    """HBM bytes per step measured by rocprofv3 counters, if recorded for this exact
    kernel source (profiles/traffic_<workload>_<mode>.md), else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}_{mode}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"source_sha:\s*([0-9a-f]+)", text)
    m_val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_val or m_hash.group(1) != source_hash():
        return None
    return float(m_val.group(1))


def compulsory_bytes(b, kv_unique: int) -> int:
    """Bytes every step must move at least: unique K/V, q, out, used table entries, lengths."""
    sp = b.spec
    nblk = sum((int(L) + sp.block_size - 1) // sp.block_size for L in b.context_lens)
    return kv_unique + 2 * b.q.size * IO_BYTES[sp.io_dtype] + 4 * nblk + 4 * b.num_seqs


# ----------------------------------------------------------------------------------
# CPU baseline: the fp64 oracle as it stands, on whole (sequence, KV head) units
# ----------------------------------------------------------------------------------

_CPU_BATCH = None  # the batch the forked oracle workers read (inherited, never copied)


def _unit_order(b):
    sp = b.spec
    units = [(s, g) for g in range(sp.num_kv_heads) for s in range(sp.num_seqs)]
    n = len(units)
    # interleave so that a short sample still spans sequences and heads
    return [units[(i * 7919) % n] for i in range(n)] if n % 7919 else units


def _oracle_units(args):
    """Worker body: oracle units wid, wid + nw, ... of the interleaved order until
    `seconds` have passed; returns (K/V bytes, tokens, units, seconds)."""
    wid, nw, seconds = args
    from threadpoolctl import threadpool_limits

    import oracle

    b = _CPU_BATCH
    sp = b.spec
    G = sp.num_heads // sp.num_kv_heads
    e = KV_BYTES[sp.kv_dtype]
    order = _unit_order(b)
    n = len(order)
    done = nbytes = tokens = 0
    i = wid
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            s, g = order[i % n]
            oracle.decode_batch(b, pairs=[(s, g * G + j) for j in range(G)])
            L = int(b.context_lens[s])
            nbytes += 2 * L * sp.head_dim * e
            tokens += L
            done += 1
            i += nw
            dt = time.perf_counter() - t0
            if dt >= seconds:
                break
    return nbytes, tokens, done, dt


def cpu_baseline(b, seconds: float):
    """The fp64 oracle on whole (sequence, KV head) units of the same batch, cycling over
    the batch until `seconds` of work: once on one thread, once on all host cores the
    process may use (at most 16; forked worker processes, one oracle unit at a time each).
    Runs before the GPU is initialised, so the fork is safe."""
    import multiprocessing as mp

    global _CPU_BATCH
    _CPU_BATCH = b
    sp = b.spec
    G = sp.num_heads // sp.num_kv_heads
    n_units = sp.num_seqs * sp.num_kv_heads
    one = _oracle_units((0, 1, seconds))
    affinity = len(os.sched_getaffinity(0))
    nw = max(1, min(16, affinity))
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(nw) as pool:
        parts = pool.map(_oracle_units, [(w, nw, seconds) for w in range(nw)])
    wall = time.perf_counter() - t0
    dt = max(p[3] for p in parts)
    nbytes = sum(p[0] for p in parts)
    tokens = sum(p[1] for p in parts)
    units = sum(p[2] for p in parts)
    _CPU_BATCH = None
    return {"value": round(nbytes / dt / 1e9, 6), "unit": "GB/s", "cores": nw, "kind": "oracle",
            "sample": f"{units} (sequence, KV head) units of {sp.name} ({n_units} per batch, cycled in an "
                      f"interleaved order), all {G} query heads each, fp64 numpy oracle, {nw} worker "
                      f"processes with one BLAS thread each, {dt:.1f} s (pool wall {wall:.1f} s)",
            "seq_tokens_per_s": round(tokens / dt, 3),
            "single_thread": {"value": round(one[0] / one[3] / 1e9, 6), "unit": "GB/s", "cores": 1,
                              "sample": f"{one[2]} units, {one[3]:.1f} s",
                              "seq_tokens_per_s": round(one[1] / one[3], 3)},
            "host_cpus": os.cpu_count(), "affinity_cpus": affinity, "host_ram_gb": _host_ram_gb()}


def _host_ram_gb():
    try:
        import psutil
        return round(psutil.virtual_memory().total / 2**30, 1)
    except Exception:  # psutil missing: not reported
        return None


# ----------------------------------------------------------------------------------
# GPU timing
# ----------------------------------------------------------------------------------

def dev_t(torch, x, dt):
    import numpy as np
    if dt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


class DeviceBatch:
    """One workload on the device: q, tables, lengths, out, and R replicas of the pools."""

    def __init__(self, torch, b, replica_bytes: float):
        import oracle
        sp = b.spec
        self.b = b
        self.q = dev_t(torch, b.q, sp.io_dtype)
        self.bt = torch.from_numpy(b.block_tables).cuda()
        self.cl = torch.from_numpy(b.context_lens).cuda()
        k0 = dev_t(torch, b.k_pool, sp.kv_dtype)
        v0 = dev_t(torch, b.v_pool, sp.kv_dtype)
        pool_bytes = k0.numel() * k0.element_size() * 2
        self.R = max(2, int(math.ceil(replica_bytes / pool_bytes)))
        self.ks = [k0] + [k0.clone() for _ in range(self.R - 1)]
        self.vs = [v0] + [v0.clone() for _ in range(self.R - 1)]
        self.pool_bytes = pool_bytes
        self.out = torch.empty_like(self.q)
        self.kv_unique = oracle.kv_unique_bytes(b.block_tables, b.context_lens, sp.block_size,
                                                sp.num_kv_heads, sp.head_dim, KV_BYTES[sp.kv_dtype])
        self.kv_logical = int(b.context_lens.sum()) * sp.num_kv_heads * sp.head_dim * KV_BYTES[sp.kv_dtype] * 2
        self.algo = compulsory_bytes(b, self.kv_unique)

    def plan(self, pa, mode, P, workgroups, stream, workspace=None):
        b = self.b
        kw = dict(scale=float(b.scale), k_scale=float(b.k_scale), v_scale=float(b.v_scale),
                  out=self.out, stream=stream, workspace=workspace)
        if mode == "direct":
            kw.pop("workspace")
            return pa.DecodePlan(self.q, self.ks[0], self.vs[0], self.bt, self.cl, **kw)
        if mode == "balanced":
            return pa.DecodePlan(self.q, self.ks[0], self.vs[0], self.bt, self.cl, balanced=True,
                                 num_workgroups=workgroups, **kw)
        if mode == "ordered":
            return pa.DecodePlan(self.q, self.ks[0], self.vs[0], self.bt, self.cl, ordered=True, **kw)
        if mode == "grouped":
            return pa.DecodePlan(self.q, self.ks[0], self.vs[0], self.bt, self.cl, grouped=True,
                                 num_splits=workgroups, **kw)
        return pa.DecodePlan(self.q, self.ks[0], self.vs[0], self.bt, self.cl,
                             max_context_len=max(b.max_context_len, 1), partition_size=P, **kw)

    def release(self):
        del self.ks, self.vs


def time_steps(torch, step, warmup: int, K: int, stream):
    """Warm up, then time K steps back to back: wall time between synchronizations, and
    GPU time from two HIP events recorded on the launch stream around the K steps.
    Returns (wall ms per step, GPU ms per step)."""
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(K):
        step(warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / K
    return wall, e0.elapsed_time(e1) / K


def measure_decode(torch, pa, db: DeviceBatch, mode: str, P: int, steps: int, warmup: int,
                   workgroups: int = 0, graph: bool = False):
    """Time one decode mode on a device batch; returns a result dict."""
    b = db.b
    sp = b.spec
    stream = torch.cuda.current_stream()
    plan = db.plan(pa, mode, P, workgroups, stream)
    calls = [plan.bound(db.ks[r], db.vs[r]) for r in range(db.R)]

    def step(i):
        rc = calls[i % db.R]()
        if rc != 0:
            raise pa.PagedAttentionError("decode", rc)

    wall_ms, gpu_ms = time_steps(torch, step, warmup, steps, stream)
    sum_l = int(b.context_lens.sum())
    r = {"workload": sp.name, "mode": mode,
         "partition_size": P if mode == "partitioned" else None,
         "us_per_step": round(wall_ms * 1e3, 3), "gpu_us_per_step": round(gpu_ms * 1e3, 3),
         "kv_unique_bytes": db.kv_unique, "algorithmic_bytes": db.algo,
         "GB_per_s": round(db.kv_unique / (wall_ms * 1e-3) / 1e9, 2),
         "pct_of_hbm_peak": round(100.0 * db.kv_unique / (wall_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
         "roofline_frac": round(db.algo / (gpu_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
         "seq_tokens_per_s": round(sum_l / (wall_ms * 1e-3), 1),
         "traffic": read_traffic(sp.name, mode)}
    if graph:
        r["graph_replay"] = graph_replay(torch, pa, db, mode, P, workgroups, steps)
    return r


def graph_replay(torch, pa, db: DeviceBatch, mode, P, workgroups, steps):
    """The same steps captured once into a HIP graph (R launches, one per replica) and
    replayed: what a caller that captures its decode loop sees. Workspaces are made before
    the capture, so the graph holds the decode kernels only."""
    b = db.b
    try:
        ws = None
        if mode == "balanced":
            ws = pa.balanced_workspace(db.q, db.ks[0], workgroups)
        elif mode == "ordered":
            ws = pa.ordered_workspace(db.q)
        elif mode == "grouped":
            ws = pa.grouped_workspace(db.q, db.ks[0], workgroups)
        elif mode == "partitioned":
            sp = b.spec
            need = pa.pa_partitioned_workspace_bytes(sp.num_seqs, sp.num_heads, sp.head_dim,
                                                     max(b.max_context_len, 1), P)
            ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            gplan = db.plan(pa, mode, P, workgroups, torch.cuda.current_stream(), workspace=ws)
            for r in range(db.R):
                gplan(db.ks[r], db.vs[r])
        reps = max(1, steps // db.R)
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / (reps * db.R)
        del g
        return {"us_per_step": round(ms * 1e3, 3), "GB_per_s": round(db.kv_unique / (ms * 1e-3) / 1e9, 2)}
    except Exception as exc:  # graph capture unavailable: report the eager numbers only
        log(f"[bench] graph replay skipped: {exc}")
        return None


def measure_append(torch, pa, db: DeviceBatch, steps: int):
    """The write that precedes each decode step: one new token's K/V per sequence, stored
    (quantised for fp8) into its block, timed on its own. The rows go to the slot of each
    sequence's last cached token, so the pool keeps its shape."""
    b = db.b
    sp = b.spec
    stream = torch.cuda.current_stream()
    gen = torch.Generator(device="cuda").manual_seed(7)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[sp.io_dtype]
    kn = torch.randn((sp.num_seqs, sp.num_kv_heads, sp.head_dim), generator=gen, device="cuda").to(tdt)
    vn = torch.randn((sp.num_seqs, sp.num_kv_heads, sp.head_dim), generator=gen, device="cuda").to(tdt)
    sid = torch.arange(sp.num_seqs, dtype=torch.int32, device="cuda")
    pos = torch.clamp(db.cl - 1, min=0)
    k0, v0 = db.ks[0], db.vs[0]

    def step(i):
        pa.pa_append_kv(kn, vn, sid, pos, db.bt, k0, v0, k_scale=float(b.k_scale), v_scale=float(b.v_scale),
                        stream=stream)

    _, gpu_ms = time_steps(torch, step, 3, steps, stream)
    nbytes = sp.num_seqs * (sp.num_kv_heads * sp.head_dim * 2 * (IO_BYTES[sp.io_dtype] + KV_BYTES[sp.kv_dtype]) + 12)
    return {"us_per_launch": round(gpu_ms * 1e3, 3), "bytes_per_launch": nbytes,
            "GB_per_s": round(nbytes / (gpu_ms * 1e-3) / 1e9, 2)}


def stream_read_ceiling(torch, pa, sizes, replica_bytes: float, steps: int):
    """Plain streaming read (pa_debug_stream_read: 16-byte loads, 1 KiB per wave
    instruction, nothing else) of buffers of the given sizes, cold like the decode steps
    (replicas cycled, >= 2 GiB in all). Every (load kind, loads per thread, grid) triple of
    a small sweep is timed with events over `steps` launches; the best is the ceiling for
    that size (also reported per load kind: plain and non-temporal)."""
    stream = torch.cuda.current_stream()
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    out = {}
    for label, nbytes in sizes:
        run_b = 16 * 16 * 256  # multiple of every unroll's run
        nbytes = nbytes // run_b * run_b
        R = max(2, int(math.ceil(replica_bytes / nbytes)))
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(R)]
        for t in bufs:
            t.fill_(1)
        best = None
        best_kind = {}
        sweep = []
        for nt in (0, 1):
            for unroll in (4, 8, 16):
                for wgs in (0, 2048, 4096, 8192):
                    def step(i, unroll=unroll, wgs=wgs, nt=nt):
                        rc = pa._lib.lib().pa_debug_stream_read(bufs[i % R].data_ptr(), nbytes, unroll, wgs, nt,
                                                                sink.data_ptr(), stream.cuda_stream)
                        if rc != 0:
                            raise pa.PagedAttentionError("pa_debug_stream_read", rc)
                    _, gpu_ms = time_steps(torch, step, 3, steps, stream)
                    gbs = nbytes / (gpu_ms * 1e-3) / 1e9
                    sweep.append(("nt" if nt else "plain", unroll, wgs, round(gpu_ms * 1e3, 2), round(gbs, 1)))
                    if best is None or gbs > best[3]:
                        best = (unroll, wgs, gpu_ms, gbs, nt)
                    kind = "nontemporal" if nt else "plain"
                    if kind not in best_kind or gbs > best_kind[kind]["GB_per_s"]:
                        best_kind[kind] = {"GB_per_s": round(gbs, 1), "us": round(gpu_ms * 1e3, 2)}
        out[label] = {"bytes": nbytes, "GB_per_s": round(best[3], 1),
                      "pct_of_hbm_peak": round(100 * best[3] / HBM_PEAK_GBS, 2),
                      "us": round(best[2] * 1e3, 2), "unroll": best[0], "workgroups": best[1] or "one pass",
                      "loads": "nontemporal" if best[4] else "plain", "by_load_kind": best_kind,
                      "sweep_kind_unroll_wgs_us_GBps": sweep}
        log(f"[bench] stream read {label}: best {best[3]:.0f} GB/s ({best[2] * 1e3:.1f} us, "
            f"{'non-temporal' if best[4] else 'plain'} loads, unroll {best[0]}, wgs {best[1] or 'one pass'}); "
            f"plain {best_kind['plain']['GB_per_s']:.0f} GB/s")
        del bufs
    return out


# ----------------------------------------------------------------------------------
# extend
# ----------------------------------------------------------------------------------

def extend_flops(e) -> int:
    """4 * D flops per (query row, head, key it attends to): 2D for q.k, 2D for p*v."""
    sp = e.base.spec
    total = 0
    for s in range(e.base.num_seqs):
        L = int(e.base.context_lens[s])
        Q = int(e.query_start_loc[s + 1] - e.query_start_loc[s])
        # new token i attends to L - Q + i + 1 keys
        total += sum(max(0, L - Q + i + 1) for i in range(Q))
    return 4 * sp.head_dim * sp.num_heads * total


def extend_cpu_baseline(e, seconds: float):
    """The fp64 extend oracle (as it stands) on whole (sequence, KV head) units, cycled
    until `seconds` of work, one thread; reported in TFLOP/s of the same flop count."""
    from threadpoolctl import threadpool_limits

    from oracle import extend as ext_oracle

    b = e.base
    sp = b.spec
    G = sp.num_heads // sp.num_kv_heads
    units = [(s, g) for g in range(sp.num_kv_heads) for s in range(sp.num_seqs)
             if e.query_start_loc[s + 1] > e.query_start_loc[s]]
    n = len(units)
    order = [units[(i * 7919) % n] for i in range(n)] if n % 7919 else units
    done = flops = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            s, g = order[done % n]
            lo, hi = int(e.query_start_loc[s]), int(e.query_start_loc[s + 1])
            rows = [(t, h) for t in range(lo, hi) for h in range(g * G, (g + 1) * G)]
            ext_oracle.paged_extend(e.q, b.k_pool, b.v_pool, b.block_tables, b.context_lens,
                                    e.query_start_loc, b.scale, sp.num_kv_heads, sp.io_dtype, sp.kv_dtype,
                                    float(b.k_scale), float(b.v_scale), rows=rows)
            L, Q = int(b.context_lens[s]), hi - lo
            flops += 4 * sp.head_dim * G * sum(max(0, L - Q + i + 1) for i in range(Q))
            done += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 9), "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} (sequence, KV head) units of {sp.name} ({n} per batch, cycled), all new "
                      f"tokens and {G} query heads each, fp64 numpy oracle on 1 thread, {dt:.1f} s"}


def bench_extend(args, name):
    """One step = one pa_extend call over the whole chunked-prefill batch."""
    from pagedattention_block_table_amd import workloads as W

    spec, ql = W.EXTEND[name]
    t0 = time.time()
    e = W.make_extend_batch(spec, ql)
    cpu = None if args.no_cpu_baseline else extend_cpu_baseline(e, args.cpu_seconds)

    import torch

    import oracle
    import pagedattention_block_table_amd as pa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(3)
    pa._lib.lib()  # fail loudly if the HIP library is missing
    b = e.base
    sp = b.spec
    flops = extend_flops(e)
    kv_unique = oracle.kv_unique_bytes(b.block_tables, b.context_lens, sp.block_size, sp.num_kv_heads,
                                       sp.head_dim, KV_BYTES[sp.kv_dtype])
    log(f"[bench] extend workload {sp.name}: S={sp.num_seqs} H={sp.num_heads} Hkv={sp.num_kv_heads} "
        f"D={sp.head_dim} BS={sp.block_size} kv={sp.kv_dtype} T={e.num_tokens} "
        f"sumL={int(b.context_lens.sum())} flops={flops / 1e9:.1f} G (generated in {time.time() - t0:.1f}s)")
    q = dev_t(torch, e.q, sp.io_dtype)
    out = torch.empty_like(q)
    bt = torch.from_numpy(b.block_tables).cuda()
    cl = torch.from_numpy(b.context_lens).cuda()
    qsl = torch.from_numpy(e.query_start_loc).cuda()
    k0 = dev_t(torch, b.k_pool, sp.kv_dtype)
    v0 = dev_t(torch, b.v_pool, sp.kv_dtype)
    pool_bytes = k0.numel() * k0.element_size() * 2
    R = max(2, int(math.ceil(args.replica_bytes / pool_bytes)))
    ks = [k0] + [k0.clone() for _ in range(R - 1)]
    vs = [v0] + [v0.clone() for _ in range(R - 1)]
    stream = torch.cuda.current_stream()
    mq = e.max_query_len

    def step(i):
        pa.pa_extend(q, ks[i % R], vs[i % R], bt, cl, qsl, mq, scale=float(b.scale), k_scale=float(b.k_scale),
                     v_scale=float(b.v_scale), out=out, stream=stream)

    K = args.steps
    wall_ms, gpu_ms = time_steps(torch, step, args.warmup, K, stream)
    value = flops / (wall_ms * 1e-3) / 1e12
    achieved = flops / (gpu_ms * 1e-3) / 1e12
    res = {
        "metric": EXTEND_METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(wall_ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": sp.io_dtype, "data": "synthetic",
        "config": {"workload": sp.name, "num_seqs": sp.num_seqs, "num_heads": sp.num_heads,
                   "num_kv_heads": sp.num_kv_heads, "head_dim": sp.head_dim, "block_size": sp.block_size,
                   "io_dtype": sp.io_dtype, "kv_dtype": sp.kv_dtype, "accumulate": "f32",
                   "new_tokens": e.num_tokens, "max_query_len": mq,
                   "sum_context_len": int(b.context_lens.sum()), "kv_unique_bytes": kv_unique,
                   "kv_replicas": R},
        "kv_GB_per_s": round(kv_unique / (wall_ms * 1e-3) / 1e9, 2),
        "new_tokens_per_s": round(e.num_tokens / (wall_ms * 1e-3), 1),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": MFMA16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel_ms": round(gpu_ms, 6), "algorithmic_flops_per_launch": flops},
        "cpu_baseline": dict(cpu, gpu_over_oracle=round(value / cpu["value"], 1)) if cpu else cpu,
    }
    log(f"[bench] {wall_ms * 1e3:.2f} us/step wall, {gpu_ms * 1e3:.2f} us/step GPU (events): "
        f"{value:.1f} TFLOP/s, {res['kv_GB_per_s']:.0f} GB/s unique KV, mfma frac {achieved / MFMA16_PEAK_TFLOPS:.3f}")
    del ks, vs
    print(json.dumps(res), flush=True)


# ----------------------------------------------------------------------------------
# main
# ----------------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=HEADLINE_CONFIG)
    ap.add_argument("--workload", default="",
                    help="a named variant of a config (larger blocks) or an extend workload "
                         "(extend_*), instead of --config")
    ap.add_argument("--mode", default="auto", choices=["auto", "direct", "partitioned", "balanced", "ordered",
                                                    "grouped"])
    ap.add_argument("--partition-size", type=int, default=0)
    ap.add_argument("--workgroups", type=int, default=0,
                    help="balanced mode: workgroup count; grouped mode: splits per group "
                         "(0 = library default)")
    ap.add_argument("--replica-bytes", type=float, default=2 * 2**30)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sub", action="store_true",
                    help="headline workload only: skip the other batches, the single-pass mode of the "
                         "headline batch and the streaming-read ceiling")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration for rocprofv3)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    from pagedattention_block_table_amd import workloads as W

    if args.workload in W.EXTEND:
        bench_extend(args, args.workload)
        return

    cfg = args.workload or args.config
    mode = DEFAULT_MODE[cfg] if args.mode == "auto" else args.mode
    t0 = time.time()
    b = W.make_batch(W.VARIANTS[cfg] if args.workload else cfg)
    sp = b.spec
    log(f"[bench] workload {sp.name}: S={sp.num_seqs} H={sp.num_heads} Hkv={sp.num_kv_heads} "
        f"D={sp.head_dim} BS={sp.block_size} kv={sp.kv_dtype} sumL={int(b.context_lens.sum())} "
        f"(generated in {time.time() - t0:.1f}s)")
    # the oracle runs first, before anything initialises the GPU (its workers are forked)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(b, args.cpu_seconds)
        log(f"[bench] cpu oracle: {cpu['value']:.3f} GB/s on {cpu['cores']} cores, "
            f"{cpu['single_thread']['value']:.3f} GB/s on one")

    import torch

    import pagedattention_block_table_amd as pa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(3)
    pa._lib.lib()  # fail loudly if the HIP library is missing

    P = args.partition_size or sp.partition_size or 512
    db = DeviceBatch(torch, b, args.replica_bytes)
    log(f"[bench] mode={mode} P={P if mode == 'partitioned' else '-'} replicas={db.R} "
        f"(pool {db.pool_bytes / 1e6:.1f} MB each), KV unique {db.kv_unique / 1e6:.2f} MB")

    if args.calibrate_copy:
        src = torch.empty(2**30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    head = measure_decode(torch, pa, db, mode, P, args.steps, args.warmup, args.workgroups, graph=True)
    log(f"[bench] {sp.name} {mode}: {head['us_per_step']:.2f} us/step wall, {head['gpu_us_per_step']:.2f} us/step "
        f"GPU: {head['GB_per_s']:.1f} GB/s KV, roofline frac {head['roofline_frac']:.4f}")
    app = measure_append(torch, pa, db, args.steps) if sp.io_dtype in IO_BYTES else None

    alt = {}
    subs = {}
    ceiling = None
    if not args.no_sub:
        for m in ("direct", "partitioned"):
            if m != mode:
                r = measure_decode(torch, pa, db, m, P, args.steps, args.warmup)
                alt[m] = {k: r[k] for k in ("mode", "partition_size", "us_per_step", "gpu_us_per_step",
                                            "GB_per_s", "pct_of_hbm_peak", "roofline_frac", "traffic")}
                log(f"[bench] {sp.name} {m}: {r['us_per_step']:.2f} us/step, frac {r['roofline_frac']:.4f}")
    replicas = db.R
    db.release()
    del db
    torch.cuda.empty_cache()

    if not args.no_sub and not args.workload:
        for c in SUB_CONFIGS:
            if c == cfg:
                continue
            bc = W.make_batch(c)
            dbc = DeviceBatch(torch, bc, args.replica_bytes)
            mc = DEFAULT_MODE[c]
            r = measure_decode(torch, pa, dbc, mc, bc.spec.partition_size or 512, args.steps, args.warmup)
            subs[bc.spec.name] = r
            log(f"[bench] {bc.spec.name} {mc}: {r['us_per_step']:.2f} us/step wall, {r['gpu_us_per_step']:.2f} GPU, "
                f"{r['GB_per_s']:.1f} GB/s, frac {r['roofline_frac']:.4f}")
            dbc.release()
            del dbc, bc
            torch.cuda.empty_cache()
    if not args.no_sub:
        sizes = [("131MB", 131 * 10**6), ("1GB", 10**9), ("4.3GB", 2**32)]
        ceiling = stream_read_ceiling(torch, pa, sizes, args.replica_bytes, max(20, args.steps // 4))

    wall_ms = head["us_per_step"] * 1e-3
    gpu_ms = head["gpu_us_per_step"] * 1e-3
    value = head["kv_unique_bytes"] / (wall_ms * 1e-3) / 1e9
    achieved = head["algorithmic_bytes"] / (gpu_ms * 1e-3) / 1e9
    sum_l = int(b.context_lens.sum())
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": sp.name, "mode": mode,
                   "partition_size": P if mode == "partitioned" else None,
                   "workgroups": (args.workgroups or "library default") if mode == "balanced" else None,
                   "splits": (args.workgroups or "library default") if mode == "grouped" else None,
                   "num_seqs": sp.num_seqs, "num_heads": sp.num_heads,
                   "num_kv_heads": sp.num_kv_heads, "head_dim": sp.head_dim,
                   "block_size": sp.block_size, "io_dtype": sp.io_dtype, "kv_dtype": sp.kv_dtype,
                   "accumulate": "f32", "sum_context_len": sum_l,
                   "max_context_len": b.max_context_len, "pool_blocks": b.num_blocks,
                   "kv_unique_bytes": head["kv_unique_bytes"], "kv_logical_bytes": sum_l * sp.num_kv_heads
                   * sp.head_dim * KV_BYTES[sp.kv_dtype] * 2, "kv_replicas": replicas},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "seq_tokens_per_s": round(sum_l / (wall_ms * 1e-3), 1),
        "seqs_per_s": round(sp.num_seqs / (wall_ms * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": head["traffic"],
                     "kernel_ms": round(gpu_ms, 6),
                     "algorithmic_bytes_per_launch": head["algorithmic_bytes"],
                     "timing": "HIP events on the launch stream around the timed steps; one step = "
                               + ("the split-context launch with the log-sum-exp merge of the partitions "
                                  "(inside it when every (sequence, KV head) is run by one workgroup, "
                                  "else a second launch)"
                                  if mode == "partitioned" else "the decode launch(es) of the mode")},
        "cpu_baseline": dict(cpu, gpu_over_oracle=round(value / cpu["value"], 1)) if cpu else cpu,
        "alt_modes": alt or None,
        "configs": subs or None,
        "stream_read_ceiling": ceiling,
        "append_kv": app,
        "graph_replay": head.get("graph_replay"),
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
