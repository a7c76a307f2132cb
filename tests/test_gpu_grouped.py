"""GPU parity of the grouped (shared-prefix) decode against the fp64 oracle (MI355X).

pa_decode_grouped reads a physical block once for all sequences of a group that map
the same logical chunk to it. Its result must equal the oracle's attention over every
sequence's own block table, whatever is shared; the instrumented build counts the loads
per physical block so that the read-once claim is checked, not assumed. Expected values
come only from oracle/.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import pagedattention_block_table_amd as pa
from pagedattention_block_table_amd import workloads as W

from gpu_util import TOL, check_against_oracle, log, run, to_device, to_f64

pytestmark = pytest.mark.gpu

SPLITS = (1, 2, 3, 7, 0)


@pytest.fixture(scope="module", autouse=True)
def _native_library():
    pa._lib.lib()


def _group_size(b):
    return 16 // (b.spec.num_heads // b.spec.num_kv_heads)


def _expected_block_reads(b):
    """Loads of 16 cached rows per (physical block, KV head) when each group of 16 / G
    consecutive sequences reads a block once per 16-token chunk position that any of its
    members maps to it. Derived from the block tables alone."""
    sp = b.spec
    NG = _group_size(b)
    reads = np.zeros((b.num_blocks, sp.num_kv_heads), dtype=np.int64)
    S = b.num_seqs
    for s0 in range(0, S, NG):
        members = range(s0, min(s0 + NG, S))
        Lmax = max(int(b.context_lens[i]) for i in members)
        for c in range((Lmax + 15) // 16):
            ids = {int(b.block_tables[i, (16 * c) // sp.block_size]) for i in members
                   if 16 * c < int(b.context_lens[i])}
            for bid in ids:
                reads[bid, :] += 1
    return reads


def _raw_u8(a):
    return np.ascontiguousarray(a).view(np.uint8)


def _trace_grouped(b, splits):
    import torch
    sp = b.spec
    dev = to_device(b)
    maxL = max(b.max_context_len, 1)
    out, kr, vr, counts, breads = pa.pa_debug_trace_grouped(
        dev["q"], dev["k_pool"], dev["v_pool"], dev["block_tables"], dev["context_lens"], maxL,
        scale=float(b.scale), num_splits=splits, k_scale=float(b.k_scale), v_scale=float(b.v_scale))
    plain = run(b, dev, "grouped", num_workgroups=splits)
    torch.cuda.synchronize()
    assert torch.equal(out, plain)
    counts = counts.cpu().numpy()
    kr, vr = kr.cpu(), vr.cpu()
    if sp.kv_dtype == "bf16":
        kr, vr = kr.view(torch.int16), vr.view(torch.int16)
    kr, vr = kr.numpy(), vr.numpy()
    for s in range(sp.num_seqs):
        L = int(b.context_lens[s])
        for g in range(sp.num_kv_heads):
            assert (counts[s, g, :L] == 1).all(), (s, g)
            assert (counts[s, g, L:] == 0).all(), (s, g)
            ek = oracle.gather(b.k_pool, b.block_tables[s], L, g)
            ev = oracle.gather(b.v_pool, b.block_tables[s], L, g)
            np.testing.assert_array_equal(_raw_u8(kr[s, g, :L]), _raw_u8(ek))
            np.testing.assert_array_equal(_raw_u8(vr[s, g, :L]), _raw_u8(ev))
    got = breads.cpu().numpy().astype(np.int64)
    np.testing.assert_array_equal(got, _expected_block_reads(b))
    return to_f64(out), got


def _with_tables(b, block_tables, context_lens, name):
    """The same pools under other block tables and lengths (the oracle reads whatever
    the tables say)."""
    spec = b.spec.replace(name=name, num_seqs=int(context_lens.shape[0]))
    return dataclasses.replace(b, spec=spec, block_tables=np.ascontiguousarray(block_tables, dtype=np.int32),
                               context_lens=np.ascontiguousarray(context_lens, dtype=np.int32),
                               q=np.ascontiguousarray(b.q[:context_lens.shape[0]]),
                               logical_k=None, logical_v=None)


@pytest.mark.parametrize("splits", SPLITS)
@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_grouped_small_parity(cfg, splits):
    """Every small workload through pa_decode_grouped (shapes the grouped kernel does not
    take run the single-pass kernel) against the oracle."""
    b = W.make_batch(W.small_variant(cfg))
    log(f"[grouped] cfg={cfg} {b.spec.name} splits={splits}")
    got = to_f64(run(b, to_device(b), "grouped", num_workgroups=splits))
    check_against_oracle(b, got)


@pytest.mark.parametrize("splits", (1, 2, 5))
def test_shared_prefix_read_once_per_group(splits):
    """Shared prefix blocks are loaded once per group of 16 / G sequences and KV head,
    private blocks once per sequence; every position is consumed once per sequence with
    the bytes of the oracle's gather, and the output matches the oracle."""
    b = W.make_batch(W.small_variant(2))
    log(f"[grouped-trace] {b.spec.name} splits={splits}")
    got, reads = _trace_grouped(b, splits)
    check_against_oracle(b, got)
    NG = _group_size(b)
    ngroups = (b.num_seqs + NG - 1) // NG
    per_block = b.spec.block_size // 16
    shared = b.shared_blocks
    assert shared.size > 0
    assert (reads[shared] == ngroups * per_block).all()
    # a private block is loaded at most once per 16-token chunk (fewer when it is a
    # sequence's partly filled last block)
    private = np.setdiff1d(np.unique(b.block_tables[b.block_tables >= 0]), shared)
    assert (reads[private] >= 1).all() and (reads[private] <= per_block).all()
    unused = np.setdiff1d(np.arange(b.num_blocks), np.unique(b.block_tables[b.block_tables >= 0]))
    assert (reads[unused] == 0).all()


@pytest.mark.parametrize("splits", (1, 3, 0))
def test_grouped_bitwise_under_sharing_and_placement(splits):
    """The grouped kernel's order of arithmetic follows logical positions only: private
    copies of the shared prefix, another placement and another block size (>= 16) give
    the same bits."""
    import torch
    b = W.make_batch(W.small_variant(2), keep_logical=True)
    log(f"[grouped-bitwise] splits={splits}")
    base = run(b, to_device(b), "grouped", num_workgroups=splits)
    variants = [W.repage(b, unshare=True, seed=7), W.repage(b, seed=5)]
    for bs in (16, 32, 64, 256):
        variants.append(W.repage(b, block_size=bs, seed=bs))
    for v in variants:
        got = run(v, to_device(v), "grouped", num_workgroups=splits)
        torch.cuda.synchronize()
        assert torch.equal(got, base), (v.spec.block_size, v.num_blocks)


def test_grouped_agrees_with_single_pass():
    b = W.make_batch(W.small_variant(2))
    dev = to_device(b)
    d = to_f64(run(b, dev, "direct"))
    for splits in SPLITS:
        g = to_f64(run(b, dev, "grouped", num_workgroups=splits))
        assert np.abs(d - g).max() <= TOL[b.spec.kv_dtype]


GROUP_SHAPES = [("bf16", "bf16", 4, 128, 16), ("f16", "f16", 2, 128, 32), ("bf16", "fp8_e4m3", 8, 128, 16),
                ("f16", "fp8_e4m3", 4, 128, 64), ("bf16", "bf16", 8, 64, 16), ("f16", "f16", 4, 64, 256)]


@pytest.mark.parametrize("io,kv,G,D,BS", GROUP_SHAPES, ids=[f"{a}-{b}-g{c}-d{d}-bs{e}" for a, b, c, d, e in
                                                             GROUP_SHAPES])
def test_grouped_edges(io, kv, G, D, BS):
    """Shapes of the grouped kernel: ragged lengths around 16-token chunks and blocks, a
    partial last group, forks that share their partly filled last block at different
    lengths, sharing between non-adjacent sequences, and empty contexts."""
    Hkv = 2
    prefix = 2 * BS + 5
    lens = tuple(prefix + d for d in (0, 1, 11, BS - 5, BS - 4, 2 * BS - 6, 3 * BS + 12, 300, 3))
    spec = W.Spec(f"grouped_{io}_{kv}_{G}_{D}_{BS}", len(lens), Hkv * G, Hkv, D, BS, io, kv,
                  ("fixed", lens), shared_prefix=prefix, seed=7000 + G + D + BS)
    b = W.make_batch(spec)
    bt = b.block_tables.copy()
    cl = b.context_lens.copy()
    # sequence 1 becomes a fork of sequence 0 (same table, shorter: the last block is shared
    # partly filled); sequence 5 takes sequence 2's whole table at its own, shorter length
    bt[1] = bt[0]
    cl[1] = cl[0] - 3
    bt[5] = bt[2]
    cl[5] = min(cl[5], cl[2])
    forked = _with_tables(b, bt, cl, spec.name + "_forks")
    # ragged batch with empty contexts, no sharing
    edge = W.make_batch(W.Spec(spec.name + "_edge", 11, Hkv * G, Hkv, D, BS, io, kv,
                               ("fixed", (0, 1, 2, 15, 16, 17, 31, 32, 33, 0, 100)), seed=7100 + G))
    for batch in (b, forked, edge):
        dev = to_device(batch)
        for splits in (1, 2, 4, 0):
            log(f"[grouped-edge] {batch.spec.name} splits={splits}")
            got = to_f64(run(batch, dev, "grouped", num_workgroups=splits))
            check_against_oracle(batch, got, io_rounding=True)
            zero = batch.context_lens == 0
            assert (got[zero] == 0).all()
    _trace_grouped(forked, 3)


@pytest.mark.parametrize("io,kv,G,D,BS", [("f32", "f32", 4, 64, 16), ("bf16", "bf16", 1, 128, 16),
                                          ("f16", "f16", 4, 128, 8), ("bf16", "bf16", 2, 256, 16)])
def test_grouped_other_shapes_run_single_pass(io, kv, G, D, BS):
    """Shapes outside the grouped kernel (fp32, one head per KV head, 8-token blocks,
    head_dim 256) take pa_decode's kernel: the same bits as pa_decode."""
    import torch
    spec = W.Spec(f"grouped_fallback_{io}_{G}_{D}_{BS}", 5, 2 * G, 2, D, BS, io, kv,
                  ("fixed", (0, 1, 40, 100, 333)), seed=7200 + G + D)
    b = W.make_batch(spec)
    dev = to_device(b)
    got = run(b, dev, "grouped", num_workgroups=3)
    ref = run(b, dev, "direct")
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    assert pa.pa_grouped_workspace_bytes(5, 2 * G, 2, D, 3) == (0 if G == 1 else 5 * 2 * G * 3 * (D + 2) * 4)


def test_grouped_workspace_errors():
    import torch
    b = W.make_batch(W.small_variant(2))
    dev = to_device(b)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(pa.PagedAttentionError):
        run(b, dev, "grouped", num_workgroups=4, workspace=small)
    with pytest.raises(pa.PagedAttentionError):
        run(b, dev, "grouped", num_workgroups=-1)
