"""The path under HIP graph capture: an append followed by a balanced decode (whose
workspace counters must be back at zero after every call) and an extend, captured once
and replayed several times with eager work and synchronizations in between; every replay
must give the eager results bit for bit."""
import numpy as np
import pytest

import pagedattention_block_table_amd as pa
from pagedattention_block_table_amd import workloads as W

from gpu_util import log, to_device

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    import torch
    b = W.make_batch(W.small_variant(2))                 # bf16, GQA 4, shared prefix
    sp = b.spec
    dev = to_device(b)
    S, Hkv, D, BS = sp.num_seqs, sp.num_kv_heads, sp.head_dim, sp.block_size
    # one new token per sequence goes to the slot of its last cached token, so the tables
    # need no new block and every replay writes the same bytes
    pos = torch.clamp(dev["context_lens"] - 1, min=0)
    sid = torch.arange(S, dtype=torch.int32, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(11)
    kn = torch.randn((S, Hkv, D), generator=g, device="cuda").to(torch.bfloat16)
    vn = torch.randn((S, Hkv, D), generator=g, device="cuda").to(torch.bfloat16)
    ws = pa.balanced_workspace(dev["q"], dev["k_pool"])
    out = torch.empty_like(dev["q"])
    e = W.make_extend_batch(W.small_extend("extend_gqa_bf16_bs256")[0], W.small_extend("extend_gqa_bf16_bs256")[1])
    edev = to_device(e.base)
    eq = torch.from_numpy(np.ascontiguousarray(e.q).view(np.int16)).view(torch.bfloat16).cuda()
    eqsl = torch.from_numpy(e.query_start_loc).cuda()
    eout = torch.empty_like(eq)

    def step(stream):
        pa.pa_append_kv(kn, vn, sid, pos, dev["block_tables"], dev["k_pool"], dev["v_pool"], stream=stream)
        pa.pa_decode_balanced(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_tables"], dev["context_lens"],
                              scale=float(b.scale), workspace=ws, out=out, stream=stream)
        pa.pa_extend(eq, edev["k_pool"], edev["v_pool"], edev["block_tables"], edev["context_lens"], eqsl,
                     e.max_query_len, scale=float(e.base.scale), out=eout, stream=stream)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(side)                                         # eager reference (and warm-up)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref, eref = out.clone(), eout.clone()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(torch.cuda.current_stream())
    for r in range(4):
        out.zero_()
        eout.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        log(f"[graph] replay {r}")
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), r
        assert torch.equal(eout.view(torch.int16), eref.view(torch.int16)), r
        # eager work between replays
        step(torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), r


def test_graph_replays_ordered_decode():
    """The longest-first decode (one launch that derives its order in LDS) under graph
    capture, on a mixed-length fp8 batch: every replay, with eager work in between, is
    bit-identical to the eager call."""
    import torch
    b = W.make_batch(W.small_variant(4))
    dev = to_device(b)
    kw = dict(scale=float(b.scale), k_scale=float(b.k_scale), v_scale=float(b.v_scale))
    out = torch.empty_like(dev["q"])

    def step(stream):
        pa.pa_decode_ordered(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_tables"], dev["context_lens"],
                             out=out, stream=stream, **kw)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(torch.cuda.current_stream())
    for r in range(4):
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        log(f"[graph-ordered] replay {r}")
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), r
        step(torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), r
