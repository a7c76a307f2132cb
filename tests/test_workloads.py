"""Seeded generator and pager: structure, determinism, sentinels (no GPU)."""
import numpy as np
import pytest

from pagedattention_block_table_amd import workloads as W


def _used_positions(b):
    bs = b.spec.block_size
    used = set()
    for s, L in enumerate(b.context_lens):
        for t in range(int(L)):
            used.add((int(b.block_tables[s, t // bs]), t % bs))
    return used


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_structure(cfg):
    b = W.make_batch(W.small_variant(cfg))
    sp = b.spec
    nblk = (b.context_lens + sp.block_size - 1) // sp.block_size
    ids = []
    for s in range(sp.num_seqs):
        row = b.block_tables[s]
        assert (row[:nblk[s]] >= 0).all() and (row[:nblk[s]] < b.num_blocks).all()
        assert (row[nblk[s]:] == -1).all()
        ids.extend(row[:nblk[s]].tolist())
    shared = set(b.shared_blocks.tolist())
    private = [i for i in ids if i not in shared]
    assert len(private) == len(set(private)), "a private block is used twice"
    if sp.shared_prefix:
        n_sh = sp.shared_prefix // sp.block_size
        assert len(shared) == n_sh
        assert (b.block_tables[:, :n_sh] == b.block_tables[0, :n_sh]).all()


@pytest.mark.parametrize("cfg", [0, 2, 4])
def test_unused_slots_hold_nan(cfg):
    b = W.make_batch(W.small_variant(cfg))
    used = _used_positions(b)
    mask = np.zeros(b.k_pool.shape[0] * b.k_pool.shape[2], dtype=bool)
    bs = b.spec.block_size
    for blk, slot in used:
        mask[blk * bs + slot] = True
    mask = mask.reshape(b.k_pool.shape[0], bs)
    kv = b.spec.kv_dtype
    for pool in (b.k_pool, b.v_pool):
        unused = pool.transpose(0, 2, 1, 3)[~mask]
        if kv == "f32":
            assert np.isnan(unused).all()
        else:
            assert (unused == W.NAN_BITS[kv]).all()
        if kv == "f32":
            assert np.isfinite(pool.transpose(0, 2, 1, 3)[mask]).all()


def test_deterministic_and_thread_independent():
    a = W.make_batch(W.small_variant(4), threads=1)
    b = W.make_batch(W.small_variant(4), threads=7)
    for f in ("context_lens", "block_tables", "q", "k_pool", "v_pool"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    assert a.k_scale == b.k_scale and a.v_scale == b.v_scale


def test_config_recipes():
    b0 = W.make_batch(0)
    assert b0.context_lens.tolist() == [1, 17, 33, 100] and b0.num_blocks == 32
    assert b0.block_tables.shape == (4, 7)
    b1 = W.make_batch(1)
    assert ((b1.context_lens >= 78 + 156) & (b1.context_lens <= 178 + 356)).all()
    assert b1.num_blocks == int(np.ceil(1.2 * ((b1.context_lens + 15) // 16).sum()))
    b2 = W.make_batch(2)
    assert b2.num_blocks == 2495 and len(b2.shared_blocks) == 31
    assert b2.block_tables.shape == (64, 63)


def test_fp8_scale_is_amax_over_448():
    b = W.make_batch(W.small_variant(4), keep_logical=True)
    # the largest code magnitude in use is 448 (0x7E / 0xFE) in both pools
    for lg in (b.logical_k, b.logical_v):
        codes = np.concatenate([x.reshape(-1) for x in lg])
        assert (codes & 0x7F).max() == 0x7E


def test_spikes_present():
    sp = W.small_variant(3)
    b = W.make_batch(sp, keep_logical=True)
    k = b.logical_k[0].astype(np.float32)
    # every element of a spiked position was shifted by +4 before rounding
    row_means = k.reshape(k.shape[0], -1).mean(axis=1)
    assert (row_means > 3.0).sum() == int(np.ceil(0.01 * b.context_lens[0]))
