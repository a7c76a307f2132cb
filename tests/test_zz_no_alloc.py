"""The allocation-free split-context decode (pa_decode_partitioned_noalloc): its partition
states live in the library's static device scratch. Through the C ABI it must give the
bits of pa_decode_partitioned (same kernels, caller workspace) and meet the oracle's bar,
on two calls in a row, the second with a smaller batch (the scratch keeps the first
call's contents), and it must refuse requests larger than the scratch."""
import ctypes

import pytest

import pagedattention_block_table_amd as pa
from pagedattention_block_table_amd import _lib
from pagedattention_block_table_amd import workloads as W

from gpu_util import check_against_oracle, log, to_device, to_f64

pytestmark = pytest.mark.gpu


def _noalloc_raw(b, dev, out, P):
    """The entry point called through ctypes with plain pointers; returns the status."""
    import torch
    sp = b.spec
    L = _lib.lib()
    return L.pa_decode_partitioned_noalloc(
        dev["q"].data_ptr(), dev["k_pool"].data_ptr(), dev["v_pool"].data_ptr(),
        dev["block_tables"].data_ptr(), dev["context_lens"].data_ptr(), sp.num_seqs,
        b.block_tables.shape[1], b.num_blocks, sp.num_heads, sp.num_kv_heads, sp.head_dim,
        sp.block_size, ctypes.c_float(float(b.scale)), _lib.dtype_code(dev["q"]),
        _lib.dtype_code(dev["k_pool"]), ctypes.c_float(float(b.k_scale)), ctypes.c_float(float(b.v_scale)),
        max(b.max_context_len, 1), P, out.data_ptr(), torch.cuda.current_stream().cuda_stream)


def _reference(b, dev, P):
    return pa.pa_decode_partitioned(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_tables"],
                                    dev["context_lens"], max(b.max_context_len, 1), scale=float(b.scale),
                                    partition_size=P, k_scale=float(b.k_scale), v_scale=float(b.v_scale))


def test_noalloc_matches_workspace_path_two_calls_second_smaller():
    import torch
    big = W.make_batch(W.small_variant(4))          # fp8 KV, GQA 4, mixed lengths
    small = W.make_batch(W.Spec("noalloc_small", 3, 8, 2, 128, 16, "f16", "f16",
                                ("fixed", (1, 40, 17)), seed=91))
    for b, P in ((big, 64), (small, 16)):
        log(f"[noalloc] {b.spec.name} S={b.num_seqs} maxL={b.max_context_len} P={P}")
        dev = to_device(b)
        out = torch.full_like(dev["q"], float("nan"))
        assert _noalloc_raw(b, dev, out, P) == _lib.PA_OK
        ref = _reference(b, dev, P)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        check_against_oracle(b, to_f64(out), io_rounding=True)


def test_noalloc_full_size_long_context():
    """The 8 x 32768-token batch at 512-token partitions fits the scratch (8.5 MB): sampled
    rows against the oracle and every row against the workspace path."""
    import torch
    b = W.make_batch(3)
    P = 512
    log(f"[noalloc] {b.spec.name} full size P={P}")
    dev = to_device(b)
    out = torch.empty_like(dev["q"])
    assert _noalloc_raw(b, dev, out, P) == _lib.PA_OK
    ref = _reference(b, dev, P)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    pairs = [(s, h) for s in range(b.num_seqs) for h in (0, 13, 31)]
    check_against_oracle(b, to_f64(out), pairs=pairs)


def test_noalloc_refuses_more_than_the_scratch():
    import torch
    b = W.make_batch(W.small_variant(1))
    dev = to_device(b)
    sp = b.spec
    out = torch.empty_like(dev["q"])
    L = _lib.lib()
    # a bound on the context length whose partition states exceed 16 MiB
    maxL = 1 << 20
    assert _lib.pa_partitioned_workspace_bytes(sp.num_seqs, sp.num_heads, sp.head_dim, maxL, sp.block_size) \
        > _lib.PA_NOALLOC_SCRATCH_BYTES
    rc = L.pa_decode_partitioned_noalloc(
        dev["q"].data_ptr(), dev["k_pool"].data_ptr(), dev["v_pool"].data_ptr(),
        dev["block_tables"].data_ptr(), dev["context_lens"].data_ptr(), sp.num_seqs,
        b.block_tables.shape[1], b.num_blocks, sp.num_heads, sp.num_kv_heads, sp.head_dim, sp.block_size,
        ctypes.c_float(float(b.scale)), _lib.dtype_code(dev["q"]), _lib.dtype_code(dev["k_pool"]),
        ctypes.c_float(1.0), ctypes.c_float(1.0), maxL, sp.block_size, out.data_ptr(),
        torch.cuda.current_stream().cuda_stream)
    assert rc == _lib.PA_ERR_SCRATCH
    assert "scratch" in _lib.pa_status_str(rc)
