#!/usr/bin/env python3
"""Benchmark of the paged-attention decode step on one MI355X.

One step = one decode call (all kernels of the path) over the whole synthetic batch of
the chosen workload. Inputs are resident in HBM before timing starts. So that every
step reads its K/V from HBM and not from the 256 MB Infinity Cache or the L2s, the
benchmark keeps R identical replicas of the K and V pools (R x pool >= 2 GiB) and step i
reads replica i mod R, as a decode over many layers does.

Prints ONE JSON line: KV GB/s (unique K/V bytes per step / time per step), % of the
8 TB/s HBM peak, seq*tokens/s, the roofline of the decode kernel (its duration from
HIP events on the launch stream) and the fp64 CPU oracle timed on a bounded sample.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1] [--mode auto]
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
DEFAULT_MODE = {0: "direct", 1: "direct", 2: "direct", 3: "direct", 4: "ordered",
                "llama7b_fp16_bs128": "direct", "shared_prefix_bf16_bs256": "direct",
                "long_ctx_fp16_bs512": "ordered", "mixed_fp8_bs256": "ordered",
                "llama70b_gqa8_bf16": "ordered", "d256_gqa2_bf16": "direct"}
KERNEL_SOURCES = ["pagedattention_block_table_amd/csrc/pa_decode_impl.h",
                  "pagedattention_block_table_amd/csrc/pa_mfma_decode.h",
                  "pagedattention_block_table_amd/csrc/pa_api.hip"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str, mode: str):
    """HBM bytes per launch measured by rocprofv3 counters, if recorded for this exact
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
    """Bytes every launch must move at least: unique K/V, q, out, used table entries, lengths."""
    sp = b.spec
    io = {"f32": 4, "f16": 2, "bf16": 2}[sp.io_dtype]
    nblk = sum((int(L) + sp.block_size - 1) // sp.block_size for L in b.context_lens)
    return kv_unique + 2 * b.q.size * io + 4 * nblk + 4 * b.num_seqs


def cpu_baseline(b, seconds: float):
    """Time the fp64 oracle (as it stands) on whole (sequence, KV head) units of the same
    batch, cycling over the batch in a fixed interleaved order until `seconds` of work;
    report KV GB/s."""
    from threadpoolctl import threadpool_limits

    import oracle

    sp = b.spec
    G = sp.num_heads // sp.num_kv_heads
    e = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1}[sp.kv_dtype]
    units = [(s, g) for g in range(sp.num_kv_heads) for s in range(sp.num_seqs)]
    # interleave so that a short sample still spans sequences and heads
    n = len(units)
    order = [units[(i * 7919) % n] for i in range(n)] if n % 7919 else units
    done = 0
    nbytes = 0
    tokens = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            s, g = order[done % n]
            oracle.decode_batch(b, pairs=[(s, g * G + i) for i in range(G)])
            L = int(b.context_lens[s])
            nbytes += 2 * L * sp.head_dim * e
            tokens += L
            done += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = time.perf_counter() - t0
    return {"value": round(nbytes / dt / 1e9, 6), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} (sequence, KV head) units of {sp.name} ({n} per batch, cycled), all "
                      f"{G} query heads each, fp64 numpy oracle on 1 thread, {dt:.1f} s",
            "seq_tokens_per_s": round(tokens / dt, 3)}


def extend_flops(e) -> int:
    """4 * D flops per (query row, head, key it attends to): 2D for q.k, 2D for p*v."""
    sp = e.base.spec
    total = 0
    for s in range(e.base.num_seqs):
        L = int(e.base.context_lens[s])
        Q = int(e.query_start_loc[s + 1] - e.query_start_loc[s])
        # new token i attends to L - Q + i + 1 keys
        keys = sum(max(0, L - Q + i + 1) for i in range(Q))
        total += keys
    return 4 * sp.head_dim * sp.num_heads * total


def extend_cpu_baseline(e, seconds: float):
    """The fp64 extend oracle (as it stands) on whole (sequence, KV head) units, cycled
    until `seconds` of work; reported in TFLOP/s of the same flop count."""
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
    import numpy as np
    import torch

    import oracle
    import pagedattention_block_table_amd as pa
    from pagedattention_block_table_amd import workloads as W

    spec, ql = W.EXTEND[name]
    t0 = time.time()
    e = W.make_extend_batch(spec, ql)
    b = e.base
    sp = b.spec
    flops = extend_flops(e)
    kv_e = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1}[sp.kv_dtype]
    kv_unique = oracle.kv_unique_bytes(b.block_tables, b.context_lens, sp.block_size, sp.num_kv_heads,
                                       sp.head_dim, kv_e)
    log(f"[bench] extend workload {sp.name}: S={sp.num_seqs} H={sp.num_heads} Hkv={sp.num_kv_heads} "
        f"D={sp.head_dim} BS={sp.block_size} kv={sp.kv_dtype} T={e.num_tokens} "
        f"sumL={int(b.context_lens.sum())} flops={flops / 1e9:.1f} G (generated in {time.time() - t0:.1f}s)")

    def dev_t(x, dt):
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()

    q = dev_t(e.q, sp.io_dtype)
    out = torch.empty_like(q)
    bt = torch.from_numpy(b.block_tables).cuda()
    cl = torch.from_numpy(b.context_lens).cuda()
    qsl = torch.from_numpy(e.query_start_loc).cuda()
    k0 = dev_t(b.k_pool, sp.kv_dtype)
    v0 = dev_t(b.v_pool, sp.kv_dtype)
    pool_bytes = k0.numel() * k0.element_size() * 2
    R = max(2, int(math.ceil(args.replica_bytes / pool_bytes)))
    ks = [k0] + [k0.clone() for _ in range(R - 1)]
    vs = [v0] + [v0.clone() for _ in range(R - 1)]
    stream = torch.cuda.current_stream()
    mq = e.max_query_len

    def step(i):
        pa.pa_extend(q, ks[i % R], vs[i % R], bt, cl, qsl, mq, scale=float(b.scale), k_scale=float(b.k_scale),
                     v_scale=float(b.v_scale), out=out, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    t_wall = time.perf_counter()
    for i in range(K):
        step(args.warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_per_step = wall * 1e3 / K
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        starts[i].record(stream)
        step(args.warmup + K + i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    durs_ms = [s_.elapsed_time(e_) for s_, e_ in zip(starts, ends)]
    kern_ms = float(np.mean(durs_ms))
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kern_ms * 1e-3) / 1e12
    res = {
        "metric": EXTEND_METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": sp.io_dtype, "data": "synthetic",
        "config": {"workload": sp.name, "num_seqs": sp.num_seqs, "num_heads": sp.num_heads,
                   "num_kv_heads": sp.num_kv_heads, "head_dim": sp.head_dim, "block_size": sp.block_size,
                   "io_dtype": sp.io_dtype, "kv_dtype": sp.kv_dtype, "accumulate": "f32",
                   "new_tokens": e.num_tokens, "max_query_len": mq,
                   "sum_context_len": int(b.context_lens.sum()), "kv_unique_bytes": kv_unique,
                   "kv_replicas": R},
        "kv_GB_per_s": round(kv_unique / (ms_per_step * 1e-3) / 1e9, 2),
        "new_tokens_per_s": round(e.num_tokens / (ms_per_step * 1e-3), 1),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": MFMA16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel_ms": round(kern_ms, 6), "algorithmic_flops_per_launch": flops,
                     "p10_p90_ms": [round(float(np.percentile(durs_ms, 10)), 6),
                                    round(float(np.percentile(durs_ms, 90)), 6)]},
        "cpu_baseline": None,
    }
    log(f"[bench] {ms_per_step * 1e3:.2f} us/step wall, {kern_ms * 1e3:.2f} us/launch (events): "
        f"{value:.1f} TFLOP/s, {res['kv_GB_per_s']:.0f} GB/s unique KV, mfma frac {achieved / MFMA16_PEAK_TFLOPS:.3f}")
    del ks, vs
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = extend_cpu_baseline(e, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=1)
    ap.add_argument("--workload", default="",
                    help="a named variant of a config (larger blocks) or an extend workload "
                         "(extend_*), instead of --config")
    ap.add_argument("--mode", default="auto", choices=["auto", "direct", "partitioned", "balanced", "ordered"])
    ap.add_argument("--partition-size", type=int, default=0)
    ap.add_argument("--workgroups", type=int, default=0,
                    help="balanced mode: workgroup count (0 = library default)")
    ap.add_argument("--replica-bytes", type=float, default=2 * 2**30)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration for rocprofv3)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import pagedattention_block_table_amd as pa
    from pagedattention_block_table_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(3)
    pa._lib.lib()  # fail loudly if the HIP library is missing
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

    import oracle
    e = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1}[sp.kv_dtype]
    kv_unique = oracle.kv_unique_bytes(b.block_tables, b.context_lens, sp.block_size,
                                       sp.num_kv_heads, sp.head_dim, e)
    kv_logical = int(b.context_lens.sum()) * sp.num_kv_heads * sp.head_dim * e * 2
    algo_bytes = compulsory_bytes(b, kv_unique)

    def dev_t(x, dt):
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()

    q = dev_t(b.q, sp.io_dtype)
    bt = torch.from_numpy(b.block_tables).cuda()
    cl = torch.from_numpy(b.context_lens).cuda()
    k0 = dev_t(b.k_pool, sp.kv_dtype)
    v0 = dev_t(b.v_pool, sp.kv_dtype)
    pool_bytes = k0.numel() * k0.element_size() * 2
    R = max(2, int(math.ceil(args.replica_bytes / pool_bytes)))
    ks = [k0] + [k0.clone() for _ in range(R - 1)]
    vs = [v0] + [v0.clone() for _ in range(R - 1)]
    out = torch.empty_like(q)
    P = args.partition_size or sp.partition_size or 512
    maxL = max(b.max_context_len, 1)
    ws = None
    if mode == "partitioned":
        need = pa.pa_partitioned_workspace_bytes(sp.num_seqs, sp.num_heads, sp.head_dim, maxL, P)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    log(f"[bench] mode={mode} P={P if mode == 'partitioned' else '-'} replicas={R} "
        f"(pool {pool_bytes / 1e6:.1f} MB each), KV unique {kv_unique / 1e6:.2f} MB")

    kw = dict(scale=float(b.scale), k_scale=float(b.k_scale), v_scale=float(b.v_scale),
              out=out, stream=stream)
    if mode == "direct":
        plan = pa.DecodePlan(q, k0, v0, bt, cl, **kw)
    elif mode == "balanced":
        plan = pa.DecodePlan(q, k0, v0, bt, cl, balanced=True, num_workgroups=args.workgroups, **kw)
    elif mode == "ordered":
        plan = pa.DecodePlan(q, k0, v0, bt, cl, ordered=True, **kw)
    else:
        plan = pa.DecodePlan(q, k0, v0, bt, cl, max_context_len=maxL, partition_size=P,
                             workspace=ws, **kw)

    calls = [plan.bound(ks[r], vs[r]) for r in range(R)]

    def step(i):
        rc = calls[i % R]()
        if rc != 0:
            raise pa.PagedAttentionError("decode", rc)

    if args.calibrate_copy:
        src = torch.empty(2**30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    K = args.steps
    # timed region: K steps back to back, bracketed by synchronizations (the throughput)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(K):
        step(args.warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_per_step = wall * 1e3 / K
    # kernel duration: the same K steps again, each bracketed by HIP events on the launch
    # stream (recording events costs host time, so this pass is kept out of the throughput)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        starts[i].record(stream)
        step(args.warmup + K + i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    durs_ms = [s.elapsed_time(e_) for s, e_ in zip(starts, ends)]
    kern_ms = float(np.mean(durs_ms))

    # the same steps replayed from one HIP graph (R captured launches, one per replica):
    # what a caller that captures its decode loop gets, without per-launch host work.
    # Workspaces are made before the capture, so the graph holds the decode kernels only.
    graph_ms = None
    try:
        gws = (pa.balanced_workspace(q, k0, args.workgroups) if mode == "balanced"
               else pa.ordered_workspace(q) if mode == "ordered" else ws)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            gkw = dict(kw, stream=torch.cuda.current_stream())
            if mode == "direct":
                gplan = pa.DecodePlan(q, k0, v0, bt, cl, **gkw)
            elif mode == "balanced":
                gplan = pa.DecodePlan(q, k0, v0, bt, cl, balanced=True, num_workgroups=args.workgroups,
                                      workspace=gws, **gkw)
            elif mode == "ordered":
                gplan = pa.DecodePlan(q, k0, v0, bt, cl, ordered=True, workspace=gws, **gkw)
            else:
                gplan = pa.DecodePlan(q, k0, v0, bt, cl, max_context_len=maxL, partition_size=P,
                                      workspace=gws, **gkw)
            for r in range(R):
                gplan(ks[r], vs[r])
        reps = max(1, K // R)
        graph.replay()
        torch.cuda.synchronize()
        t_g = time.perf_counter()
        for _ in range(reps):
            graph.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t_g) * 1e3 / (reps * R)
        del graph
    except Exception as exc:  # graph capture unavailable: report the eager numbers only
        log(f"[bench] graph replay skipped: {exc}")

    # the write that precedes each decode step: one new token's K/V per sequence, stored
    # (quantised for fp8) into its block. Timed on its own; the appended rows go to the slot
    # of each sequence's last cached token, so the pool keeps its shape and cost is the same.
    app = None
    if sp.io_dtype in ("f32", "f16", "bf16"):
        gen = torch.Generator(device="cuda").manual_seed(7)
        tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[sp.io_dtype]
        kn = torch.randn((sp.num_seqs, sp.num_kv_heads, sp.head_dim), generator=gen, device="cuda").to(tdt)
        vn = torch.randn((sp.num_seqs, sp.num_kv_heads, sp.head_dim), generator=gen, device="cuda").to(tdt)
        sid = torch.arange(sp.num_seqs, dtype=torch.int32, device="cuda")
        pos = torch.clamp(cl - 1, min=0)
        appk = [torch.cuda.Event(enable_timing=True) for _ in range(2 * K)]
        for i in range(3):
            pa.pa_append_kv(kn, vn, sid, pos, bt, k0, v0, k_scale=float(b.k_scale), v_scale=float(b.v_scale))
        torch.cuda.synchronize()
        for i in range(K):
            appk[2 * i].record(stream)
            pa.pa_append_kv(kn, vn, sid, pos, bt, k0, v0, k_scale=float(b.k_scale), v_scale=float(b.v_scale))
            appk[2 * i + 1].record(stream)
        torch.cuda.synchronize()
        app_ms = float(np.mean([appk[2 * i].elapsed_time(appk[2 * i + 1]) for i in range(K)]))
        io_b = {"f32": 4, "f16": 2, "bf16": 2}[sp.io_dtype]
        app_bytes = sp.num_seqs * (sp.num_kv_heads * sp.head_dim * 2 * (io_b + e) + 12)
        app = {"us_per_launch": round(app_ms * 1e3, 3), "bytes_per_launch": app_bytes,
               "GB_per_s": round(app_bytes / (app_ms * 1e-3) / 1e9, 2)}

    value = kv_unique / (ms_per_step * 1e-3) / 1e9
    achieved = algo_bytes / (kern_ms * 1e-3) / 1e9
    traffic = read_traffic(sp.name, mode)
    sum_l = int(b.context_lens.sum())
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": sp.name, "mode": mode,
                   "partition_size": P if mode == "partitioned" else None,
                   "workgroups": (args.workgroups or "library default") if mode == "balanced" else None,
                   "num_seqs": sp.num_seqs, "num_heads": sp.num_heads,
                   "num_kv_heads": sp.num_kv_heads, "head_dim": sp.head_dim,
                   "block_size": sp.block_size, "io_dtype": sp.io_dtype, "kv_dtype": sp.kv_dtype,
                   "accumulate": "f32", "sum_context_len": sum_l,
                   "max_context_len": b.max_context_len, "pool_blocks": b.num_blocks,
                   "kv_unique_bytes": kv_unique, "kv_logical_bytes": kv_logical,
                   "kv_replicas": R},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "seq_tokens_per_s": round(sum_l / (ms_per_step * 1e-3), 1),
        "seqs_per_s": round(sp.num_seqs / (ms_per_step * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel_ms": round(kern_ms, 6),
                     "algorithmic_bytes_per_launch": algo_bytes,
                     "p10_p90_ms": [round(float(np.percentile(durs_ms, 10)), 6),
                                    round(float(np.percentile(durs_ms, 90)), 6)]},
        "cpu_baseline": None,
        "append_kv": app,
        "graph_replay": None if graph_ms is None else {
            "ms_per_step": round(graph_ms, 6),
            "GB_per_s": round(kv_unique / (graph_ms * 1e-3) / 1e9, 2)},
    }
    log(f"[bench] {ms_per_step * 1e3:.2f} us/step wall, {kern_ms * 1e3:.2f} us/launch (events): "
        f"{value:.1f} GB/s KV, roofline frac {achieved / HBM_PEAK_GBS:.3f}")
    del ks, vs
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(b, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
