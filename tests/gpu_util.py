"""Helpers for the GPU tests: move a generated batch to the device, run the HIP path,
and compare with the fp64 oracle."""
import sys

import numpy as np

import pagedattention_block_table_amd as pa

# max |GPU - oracle| allowed, by KV storage dtype. fp16 / bf16 / fp8 values are the
# stated requirement for this decode path. fp32 (not covered there) gets the same 4e-3
# bar and, separately, a bar derived from fp32 arithmetic (see F32_DERIVED).
TOL = {"f32": 4e-3, "f16": 4e-3, "bf16": 4e-3, "fp8_e4m3": 1.5e-2}
# fp32 storage, fp32 accumulation: per-score error <= ~D * 2^-24 * |q||k| ~ 1e-5 for the
# N(0,1) inputs used, times |V| <= ~4, plus exp2 (2 ulp) and output rounding; 1e-4 bounds it.
F32_DERIVED = 1e-4


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(b, device="cuda"):
    import torch

    def conv(x, dt):
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(x)).to(device)

    sp = b.spec
    return dict(q=conv(b.q, sp.io_dtype), k_pool=conv(b.k_pool, sp.kv_dtype),
                v_pool=conv(b.v_pool, sp.kv_dtype),
                block_tables=torch.from_numpy(b.block_tables).to(device),
                context_lens=torch.from_numpy(b.context_lens).to(device))


def run(b, dev, mode="direct", partition_size=None, stream=None, num_workgroups=0, workspace=None):
    """HIP decode of a batch; returns the output tensor (io dtype, on the device).
    mode: "direct" (pa_decode), "partitioned" (partition_size), "balanced"
    (num_workgroups, 0 = library default), "ordered" (pa_decode_ordered) or "grouped"
    (pa_decode_grouped, num_workgroups = number of splits, 0 = library default)."""
    kw = dict(scale=float(b.scale), k_scale=float(b.k_scale), v_scale=float(b.v_scale), stream=stream)
    if mode == "grouped":
        return pa.pa_decode_grouped(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_tables"],
                                    dev["context_lens"], num_splits=num_workgroups,
                                    workspace=workspace, **kw)
    if mode == "direct":
        return pa.pa_decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_tables"],
                            dev["context_lens"], **kw)
    if mode == "ordered":
        return pa.pa_decode_ordered(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_tables"],
                                    dev["context_lens"], workspace=workspace, **kw)
    if mode == "balanced":
        return pa.pa_decode_balanced(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_tables"],
                                     dev["context_lens"], num_workgroups=num_workgroups,
                                     workspace=workspace, **kw)
    P = partition_size if partition_size is not None else (b.spec.partition_size or 512)
    return pa.pa_decode_partitioned(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_tables"],
                                    dev["context_lens"], max(b.max_context_len, 1),
                                    partition_size=P, **kw)


def to_f64(t):
    import torch
    return t.to(torch.float64).cpu().numpy()


# significand bits of each io format, for the half-ulp output-rounding allowance
IO_PRECISION = {"f32": 24, "f16": 11, "bf16": 8}


def half_ulp(io, x):
    """Half a unit in the last place of the io format at |x| (normal range)."""
    _, ex = np.frexp(np.abs(x))
    return np.ldexp(1.0, ex - 1 - IO_PRECISION[io])


def check_against_oracle(b, got, pairs=None, tol=None, io_rounding=False):
    """Element-wise comparison of the GPU output with the oracle on (s, h) pairs.

    The bar is the stated max |delta|. With io_rounding, each element may in addition
    differ by the half ulp that rounding the exact result to the io format costs: the
    stated bars are below that half ulp once |out| >= 1 in bf16 (|out| >= 8 in f16),
    which only the short-context edge cases reach."""
    import oracle
    sp = b.spec
    ref = oracle.decode_batch(b, pairs=pairs)
    if pairs is None:
        pairs = [(s, h) for s in range(sp.num_seqs) for h in range(sp.num_heads)]
    idx_s = np.array([p[0] for p in pairs])
    idx_h = np.array([p[1] for p in pairs])
    g = got[idx_s, idx_h]
    r = ref[idx_s, idx_h]
    assert np.isfinite(g).all(), "non-finite GPU output"
    bar = TOL[sp.kv_dtype] if tol is None else tol
    d = np.abs(g - r)
    err = float(d.max()) if g.size else 0.0
    allow = bar + (half_ulp(sp.io_dtype, r) if io_rounding else 0.0)
    worst = float((d - allow).max()) if g.size else -1.0
    assert worst <= 0, f"{sp.name}: max |gpu - oracle| = {err:.3e} exceeds bar {bar:.1e}" + (
        " + half ulp" if io_rounding else "")
    return err
