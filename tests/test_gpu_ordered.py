"""GPU tests of the longest-first decode (pa_decode_ordered): parity with the fp64
oracle, and bit-identical output to pa_decode (the same per-unit kernels run; only the
dispatch order differs), on batches that mix short and long contexts."""
import numpy as np
import pytest

import pagedattention_block_table_amd as pa
from pagedattention_block_table_amd import workloads as W

from gpu_util import check_against_oracle, log, run, to_device, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _native_library():
    pa._lib.lib()


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_ordered_small_parity_and_bitwise(cfg):
    import torch
    b = W.make_batch(W.small_variant(cfg))
    log(f"[ordered] cfg={cfg} {b.spec.name} lens={b.context_lens.tolist()[:8]}")
    dev = to_device(b)
    got = run(b, dev, "ordered")
    ref = run(b, dev, "direct")
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    check_against_oracle(b, to_f64(got))


# Mixed lengths with 8 KV heads (one KV head per XCD share, rank-major dispatch) and with
# 4 and 12 KV heads (shares that are not whole KV heads), including empty sequences.
@pytest.mark.parametrize("H,Hkv", [(32, 8), (8, 4), (24, 12)])
def test_ordered_mixed_lengths(H, Hkv):
    import torch
    sp = W.Spec(f"ordered_mix_{Hkv}", 37, H, Hkv, 128, 16, "bf16", "bf16",
                ("choice", (0, 1, 17, 128, 700, 1500), (0.05, 0.1, 0.15, 0.3, 0.25, 0.15)), seed=77)
    b = W.make_batch(sp)
    log(f"[ordered-mix] H={H} Hkv={Hkv} lens={b.context_lens.tolist()}")
    dev = to_device(b)
    ws = pa.ordered_workspace(dev["q"])
    outs = [run(b, dev, "ordered", workspace=ws) for _ in range(2)]  # workspace reused
    ref = run(b, dev, "direct")
    torch.cuda.synchronize()
    assert torch.equal(outs[0], ref) and torch.equal(outs[1], ref)
    check_against_oracle(b, to_f64(outs[0]))


def test_ordered_needs_no_workspace():
    """The decode launch derives the order itself: a NULL workspace is accepted through the
    C ABI and gives the bits of pa_decode."""
    import ctypes

    import torch
    from pagedattention_block_table_amd import _lib
    b = W.make_batch(W.small_variant(4))
    dev = to_device(b)
    sp = b.spec
    assert pa.pa_ordered_workspace_bytes(b.num_seqs) == 0
    out = torch.empty_like(dev["q"])
    rc = _lib.lib().pa_decode_ordered(
        dev["q"].data_ptr(), dev["k_pool"].data_ptr(), dev["v_pool"].data_ptr(), dev["block_tables"].data_ptr(),
        dev["context_lens"].data_ptr(), sp.num_seqs, b.block_tables.shape[1], b.num_blocks, sp.num_heads,
        sp.num_kv_heads, sp.head_dim, sp.block_size, ctypes.c_float(float(b.scale)), _lib.dtype_code(dev["q"]),
        _lib.dtype_code(dev["k_pool"]), ctypes.c_float(float(b.k_scale)), ctypes.c_float(float(b.v_scale)),
        None, 0, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == _lib.PA_OK
    ref = run(b, dev, "direct")
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("S", [1, 63, 64, 65, 300])
def test_ordered_rank_selection_edges(S):
    """Batch sizes around the 64-sequence steps of the in-launch selection, all lengths in
    one class and spread over many, each (sequence, KV head) computed exactly once (bits of
    pa_decode)."""
    import torch
    for kind in (("const", 100), ("choice", (1, 16, 17, 100, 1000, 3000), (0.1, 0.1, 0.2, 0.2, 0.2, 0.2))):
        sp = W.Spec(f"ordered_edges_{S}", S, 8, 2, 64, 16, "f16", "f16", kind, seed=300 + S)
        b = W.make_batch(sp)
        dev = to_device(b)
        got = run(b, dev, "ordered")
        ref = run(b, dev, "direct")
        torch.cuda.synchronize()
        assert torch.equal(got, ref), (S, kind[0])


@pytest.mark.parametrize("S", [2047, 2048, 2049, 4100])
def test_ordered_large_batches(S):
    """Batch sizes at and past the 2048 sequences that take the longest-first dispatch
    (larger batches keep the index order), with one length class and with several: each
    (sequence, KV head) computed exactly once (bits of pa_decode)."""
    import torch
    for kind in (("const", 16), ("choice", (1, 7, 16, 17, 40, 100), (0.1, 0.1, 0.3, 0.2, 0.2, 0.1))):
        sp = W.Spec(f"ordered_large_{S}", S, 4, 1, 64, 16, "f16", "f16", kind, seed=700 + S % 97)
        b = W.make_batch(sp)
        dev = to_device(b)
        log(f"[ordered-large] S={S} {kind[0]} sumL={int(b.context_lens.sum())}")
        got = run(b, dev, "ordered")
        ref = run(b, dev, "direct")
        torch.cuda.synchronize()
        assert torch.equal(got, ref), (S, kind[0])
