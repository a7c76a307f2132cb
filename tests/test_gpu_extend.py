"""GPU parity of the extend / prefill kernel (pa_extend) with the fp64 oracle
(oracle/extend.py), through the C ABI."""
import numpy as np
import pytest

from oracle import extend as ext_oracle
import pagedattention_block_table_amd as pa
from pagedattention_block_table_amd import workloads as W

from gpu_util import TOL, half_ulp, log, to_device, to_f64

pytestmark = pytest.mark.gpu


def _dev_q(e):
    import torch
    sp = e.base.spec
    if sp.io_dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(e.q).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(e.q)).cuda()


def run_extend(e, dev=None):
    import torch
    b = e.base
    dev = dev or to_device(b)
    qsl = torch.from_numpy(e.query_start_loc).cuda()
    return pa.pa_extend(_dev_q(e), dev["k_pool"], dev["v_pool"], dev["block_tables"], dev["context_lens"],
                        qsl, max(e.max_query_len, 0), scale=float(b.scale), k_scale=float(b.k_scale),
                        v_scale=float(b.v_scale))


def oracle_extend(e, rows=None):
    b = e.base
    sp = b.spec
    return ext_oracle.paged_extend(e.q, b.k_pool, b.v_pool, b.block_tables, b.context_lens,
                                   e.query_start_loc, b.scale, sp.num_kv_heads, sp.io_dtype, sp.kv_dtype,
                                   float(b.k_scale), float(b.v_scale), rows=rows)


def check(e, got, rows=None):
    """max |GPU - oracle| within the bar of the KV dtype, plus, per element, the half ulp
    that rounding the exact value to the io format costs: early tokens of a prefill
    attend to a handful of keys, so their outputs are close to single V rows, of size up
    to about 4, where that half ulp (bf16: 2^-7) exceeds the bar by itself."""
    ref = oracle_extend(e, rows)
    if rows is not None:
        idx = tuple(np.asarray(rows).T)
        got, ref = got[idx], ref[idx]
    assert np.isfinite(got).all()
    d = np.abs(got - ref)
    err = float(d.max()) if ref.size else 0.0
    allow = TOL[e.base.spec.kv_dtype] + half_ulp(e.base.spec.io_dtype, ref)
    assert ref.size == 0 or float((d - allow).max()) <= 0, err
    return err


@pytest.mark.parametrize("name", sorted(W.EXTEND))
def test_small_extend(name):
    sp, ql = W.small_extend(name)
    e = W.make_extend_batch(sp, ql)
    log(f"[extend] {sp.name} L={e.base.context_lens.tolist()} Q={e.query_lens.tolist()}")
    got = to_f64(run_extend(e))
    log(f"  max|err|={check(e, got):.3e}")


EDGE_L = (1, 16, 17, 64, 65, 100, 200, 300, 7, 40)
EDGE_Q = (1, 16, 17, 64, 65, 1, 133, 0, 7, 3)


@pytest.mark.parametrize("io,kv", [("f16", "f16"), ("bf16", "bf16"), ("f16", "fp8_e4m3"), ("bf16", "fp8_e4m3")])
@pytest.mark.parametrize("D,BS,G", [(64, 16, 1), (128, 8, 2), (128, 16, 4), (64, 32, 8), (128, 256, 8),
                                    (128, 512, 1)])
def test_extend_edge_shapes(io, kv, D, BS, G):
    """Query tiles cut at every boundary (Q around 16, 64), whole-context prefill, Q = 0
    and Q = 1, contexts inside one key chunk and across many, every group size."""
    if kv == "fp8_e4m3" and D == 64 and BS == 8:
        pytest.skip("unsupported geometry")
    Hkv = 2
    spec = W.Spec(f"ext_edge_{io}_{kv}_{D}_{BS}_{G}", len(EDGE_L), Hkv * G, Hkv, D, BS, io, kv,
                  ("fixed", EDGE_L), seed=7000 + D + BS + G)
    e = W.make_extend_batch(spec, ("fixed", EDGE_Q))
    log(f"[extend-edge] {spec.name}")
    check(e, to_f64(run_extend(e)))


def test_extend_rows_without_keys_are_zero():
    """Q > L is outside the contract: the rows at negative positions come out as zeros,
    the others as the oracle says."""
    import torch
    spec = W.Spec("ext_q_gt_l", 2, 4, 2, 64, 16, "f16", "f16", ("fixed", (5, 3)), seed=9)
    e = W.make_extend_batch(spec, ("fixed", (5, 3)))
    b = e.base
    qsl = np.array([0, 8, 11], np.int32)     # sequence 0 claims 8 new tokens of 5
    q = np.concatenate([e.q, e.q[:3]])
    e2 = W.ExtendBatch(base=b, query_start_loc=qsl, q=q)
    dev = to_device(b)
    got = to_f64(pa.pa_extend(torch.from_numpy(q).cuda(), dev["k_pool"], dev["v_pool"], dev["block_tables"],
                              dev["context_lens"], torch.from_numpy(qsl).cuda(), 8, scale=float(b.scale)))
    assert (got[:3] == 0).all()
    check(e2, got)


def test_extend_matches_decode_for_one_token():
    """Q = 1 everywhere: the extend kernel and the decode kernel agree within the bar."""
    b = W.make_batch(W.small_variant(2))
    e = W.ExtendBatch(base=b, query_start_loc=np.arange(b.num_seqs + 1, dtype=np.int32), q=b.q)
    dev = to_device(b)
    got = to_f64(run_extend(e, dev))
    dec = to_f64(pa.pa_decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_tables"],
                              dev["context_lens"], scale=float(b.scale)))
    assert np.abs(got - dec).max() <= 2 * TOL["bf16"]
    check(e, got)


def test_extend_placement_invariance_bitwise():
    """The same logical sequences under another physical placement and block size give the
    same bits (the key walk depends only on logical positions)."""
    import torch
    sp, ql = W.small_extend("extend_llama7b_fp16")
    e = W.make_extend_batch(sp, ql, keep_logical=True)
    base = run_extend(e)
    for bs, seed in ((16, 4), (8, 5), (128, 6)):
        nb = W.repage(e.base, block_size=bs, seed=seed)
        got = run_extend(W.ExtendBatch(base=nb, query_start_loc=e.query_start_loc, q=e.q))
        torch.cuda.synchronize()
        assert torch.equal(got, base), bs


SHORT_SHAPES = [("f16", "f16", 2, 128, 16), ("bf16", "bf16", 4, 128, 32), ("bf16", "fp8_e4m3", 4, 128, 16),
                ("f16", "fp8_e4m3", 8, 128, 256), ("bf16", "bf16", 8, 64, 16), ("f16", "f16", 4, 64, 64)]


@pytest.mark.parametrize("io,kv,G,D,BS", SHORT_SHAPES, ids=[f"{a}-{b}-g{c}-d{d}-bs{e}" for a, b, c, d, e in
                                                             SHORT_SHAPES])
def test_extend_short_queries(io, kv, G, D, BS):
    """Queries of at most 16 / G new tokens (several tokens checked at once) run on the
    grouped decode kernel, one row per (new token, head) with its own causal end; longer
    ones in the same call on the extend kernels. Query lengths around that cut, contexts
    inside one block and across many; against the oracle, and the same bits under another
    placement and block size."""
    import torch
    NG = 16 // G
    Hkv = 2
    lens = (1, 2, NG, NG + 1, 17, 40, 333, 1000, 2500, 64, 5)
    qls = (1, 2, NG, NG + 1, max(1, NG - 1), 1, NG, NG + 1, 2, 40, NG)
    spec = W.Spec(f"ext_short_{io}_{kv}_{G}_{D}_{BS}", len(lens), Hkv * G, Hkv, D, BS, io, kv,
                  ("fixed", lens), seed=7300 + G + D + BS)
    e = W.make_extend_batch(spec, ("fixed", qls), keep_logical=True)
    log(f"[extend-short] {spec.name} Q={e.query_lens.tolist()}")
    base = run_extend(e)
    check(e, to_f64(base))
    for bs, seed in ((16, 3), (64, 4)):
        nb = W.repage(e.base, block_size=bs, seed=seed)
        got = run_extend(W.ExtendBatch(base=nb, query_start_loc=e.query_start_loc, q=e.q))
        torch.cuda.synchronize()
        assert torch.equal(got, base), bs


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(W.EXTEND))
def test_full_extend_sampled(name):
    """Full-size extend workloads, checked on sampled rows (every sequence, first, middle
    and last new token, a few heads) and for finiteness everywhere."""
    spec, ql = W.EXTEND[name]
    e = W.make_extend_batch(spec, ql)
    log(f"[extend-full] {name} T={e.num_tokens}")
    got = to_f64(run_extend(e))
    assert np.isfinite(got).all()
    rows = []
    for s in range(e.base.num_seqs):
        lo, hi = int(e.query_start_loc[s]), int(e.query_start_loc[s + 1])
        if hi == lo:
            continue
        for t in sorted({lo, (lo + hi) // 2, hi - 1}):
            rows += [(t, h) for h in (0, 13, spec.num_heads - 1)]
    log(f"  max|err|={check(e, got, rows):.3e} over {len(rows)} rows")
