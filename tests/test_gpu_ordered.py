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


def test_ordered_workspace_errors():
    import torch
    b = W.make_batch(W.small_variant(4))
    dev = to_device(b)
    need = pa.pa_ordered_workspace_bytes(b.num_seqs)
    assert need >= 4 * b.num_seqs and need % 256 == 0
    small = torch.empty(need - 256 if need > 256 else 4, dtype=torch.uint8, device="cuda")
    with pytest.raises(pa.PagedAttentionError):
        run(b, dev, "ordered", workspace=small)
