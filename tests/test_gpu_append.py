"""GPU parity of the KV append kernel against the CPU oracle (oracle/kv_append.py), through
the C ABI: the whole pools must be byte-identical after the append, and decoding the
extended contexts must match the fp64 oracle."""
import numpy as np
import pytest

import oracle
from oracle import kv_append
import pagedattention_block_table_amd as pa
from pagedattention_block_table_amd import workloads as W

from gpu_util import check_against_oracle, log, run, to_device, to_f64

pytestmark = pytest.mark.gpu

NP_IO = {"f32": np.float32, "f16": np.float16}


def _io_tensor(x_f32, io):
    """float32 values -> torch tensor of the io dtype on the GPU (bf16 by RNE bits)."""
    import torch
    if io == "bf16":
        bits = kv_append.bf16_encode(x_f32)
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x_f32.astype(NP_IO[io]))).cuda()


def _io_storage(x_f32, io):
    if io == "bf16":
        return kv_append.bf16_encode(x_f32)
    return x_f32.astype(NP_IO[io])


def _append_case(b, seed, tokens_per_seq=1):
    """New tokens at positions L, L+1, ... of every sequence; tables get a free block
    wherever a token starts a new block. Returns (k_new, v_new, seq_ids, positions, tables)."""
    sp = b.spec
    rng = np.random.default_rng(seed)
    tables = b.block_tables.copy()
    used = set(tables[tables >= 0].tolist())
    free = [x for x in range(b.num_blocks) if x not in used]
    rng.shuffle(free)
    seq_ids, pos = [], []
    for s in range(sp.num_seqs):
        L = int(b.context_lens[s])
        for i in range(tokens_per_seq):
            p = L + i
            if p // sp.block_size >= tables.shape[1]:
                tables = np.concatenate([tables, np.full((tables.shape[0], 1), -1, np.int32)], axis=1)
            if p % sp.block_size == 0 or tables[s, p // sp.block_size] < 0:
                tables[s, p // sp.block_size] = free.pop()
            seq_ids.append(s)
            pos.append(p)
    T = len(seq_ids)
    k_new = (rng.standard_normal((T, sp.num_kv_heads, sp.head_dim)) * 1.5).astype(np.float32)
    v_new = rng.standard_normal((T, sp.num_kv_heads, sp.head_dim)).astype(np.float32)
    return (k_new, v_new, np.asarray(seq_ids, np.int32), np.asarray(pos, np.int32),
            np.ascontiguousarray(tables))


def _raw(t):
    import torch
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.cpu().numpy().view(np.uint8)


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("tps", [1, 3], ids=["decode", "extend3"])
def test_append_pools_bit_exact(cfg, tps):
    b = W.make_batch(W.small_variant(cfg))
    log(f"[append] cfg={cfg} {b.spec.name} tokens/seq={tps}")
    _append_check(b, 100 + cfg, tps)


@pytest.mark.parametrize("cfg,BS", [(1, 64), (2, 128), (4, 256), (3, 512)])
def test_append_large_blocks(cfg, BS):
    b = W.repage(W.make_batch(W.small_variant(cfg), keep_logical=True), block_size=BS, seed=3)
    log(f"[append] cfg={cfg} BS={BS}")
    _append_check(b, 200 + cfg, 2)


def _append_check(b, seed, tps):
    import torch
    sp = b.spec
    k_new, v_new, seq, pos, tables = _append_case(b, seed, tps)
    dev = to_device(b)
    kn = _io_tensor(k_new, sp.io_dtype)
    vn = _io_tensor(v_new, sp.io_dtype)
    bt = torch.from_numpy(tables).cuda()
    pa.pa_append_kv(kn, vn, torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(), bt,
                    dev["k_pool"], dev["v_pool"], k_scale=float(b.k_scale), v_scale=float(b.v_scale))
    torch.cuda.synchronize()
    ek, ev = kv_append.append_kv(b.k_pool, b.v_pool, tables, seq, pos, _io_storage(k_new, sp.io_dtype),
                                 _io_storage(v_new, sp.io_dtype), sp.io_dtype, sp.kv_dtype,
                                 float(b.k_scale), float(b.v_scale))
    np.testing.assert_array_equal(_raw(dev["k_pool"]), np.ascontiguousarray(ek).view(np.uint8))
    np.testing.assert_array_equal(_raw(dev["v_pool"]), np.ascontiguousarray(ev).view(np.uint8))

    # decode the extended contexts against the fp64 oracle on the oracle's pools
    lens = (b.context_lens + tps).astype(np.int32)
    b2 = W.PagedBatch(spec=sp, context_lens=lens, block_tables=tables, q=b.q, k_pool=ek, v_pool=ev,
                      scale=b.scale, k_scale=b.k_scale, v_scale=b.v_scale, num_blocks=b.num_blocks,
                      shared_blocks=b.shared_blocks)
    dev["block_tables"] = bt
    dev["context_lens"] = torch.from_numpy(lens).cuda()
    got = to_f64(run(b2, dev, "direct"))
    check_against_oracle(b2, got, io_rounding=True)


@pytest.mark.parametrize("io", ["f32", "f16", "bf16"])
def test_append_fp8_quantiser_edge_values(io):
    """Every tie midpoint of e4m3 (both signs), its neighbours, saturation, NaN and signed
    zero go through the kernel's fp8 path and must give the oracle's codes."""
    import torch
    vals = sorted({kv_append._fp8_value(c) for c in range(0x7F)})
    mids = np.array([(a + c) / 2 for a, c in zip(vals, vals[1:])], dtype=np.float32)
    x = np.concatenate([mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf),
                        np.array(vals, np.float32), -np.array(vals, np.float32),
                        np.array([448.0, 449.0, 470.0, 1e6, -1e6, np.inf, -np.inf, np.nan, 0.0, -0.0],
                                 np.float32)])
    if io != "f32":
        # the kernel reads io-typed rows: round first so both sides see the same inputs
        x = kv_append.decode_src(_io_storage(x, io), io)
    D, Hkv = 128, 1
    n = int(np.ceil(x.size / D)) * D
    rows = np.zeros(n, np.float32)
    rows[:x.size] = x
    T = n // D
    k_new = rows.reshape(T, Hkv, D)
    BS = 16
    nb = (T + BS - 1) // BS
    kp = torch.zeros((nb, Hkv, BS, D), dtype=torch.uint8, device="cuda")
    vp = torch.zeros_like(kp)
    tables = np.arange(nb, dtype=np.int32)[None]
    seq = np.zeros(T, np.int32)
    pos = np.arange(T, dtype=np.int32)
    kn = _io_tensor(k_new, io)
    pa.pa_append_kv(kn, kn, torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(),
                    torch.from_numpy(tables).cuda(), kp, vp, k_scale=1.0, v_scale=0.5)
    torch.cuda.synchronize()
    got_k = kp.cpu().numpy().reshape(-1)[:x.size]
    got_v = vp.cpu().numpy().reshape(-1)[:x.size]
    for got, scale in ((got_k, 1.0), (got_v, 0.5)):
        ref = kv_append.encode(x, "fp8_e4m3", scale)
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, [(float(x[i]), int(got[i]), int(ref[i])) for i in bad[:10]]


def test_append_skips_out_of_range_tokens():
    """A token whose sequence, position or table entry lies outside the contract writes
    nothing (and the rest of the batch is still written)."""
    import torch
    Hkv, D, BS, nb = 2, 64, 8, 4
    kp = torch.zeros((nb, Hkv, BS, D), dtype=torch.float16, device="cuda")
    vp = torch.zeros_like(kp)
    tables = torch.tensor([[0, 1], [2, 9]], dtype=torch.int32, device="cuda")  # 9 is outside the pool
    seq = torch.tensor([0, 1, 5, 0, 1], dtype=torch.int32, device="cuda")
    pos = torch.tensor([3, 9, 0, 16, 2], dtype=torch.int32, device="cuda")
    kn = torch.ones((5, Hkv, D), dtype=torch.float16, device="cuda")
    pa.pa_append_kv(kn, kn, seq, pos, tables, kp, vp)
    torch.cuda.synchronize()
    k = kp.cpu().numpy()
    assert (k[0, :, 3] == 1).all() and (k[2, :, 2] == 1).all()
    k[0, :, 3] = 0
    k[2, :, 2] = 0
    assert (k == 0).all()
