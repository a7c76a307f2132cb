"""Pins of the extend oracle (oracle/extend.py) to things other than itself: closed forms
of causal attention, an independently written dense fp64 attention on the unpaged
sequences, the decode oracle (pinned on its own) at every prefix, special cases and
invariances. Planted mistakes must each fail at least one pin. CPU only."""
import numpy as np
import pytest

from oracle import extend, pa_oracle
from pagedattention_block_table_amd import workloads as W

torch = pytest.importorskip("torch")


def _args(e):
    b = e.base
    sp = b.spec
    return (e.q, b.k_pool, b.v_pool, b.block_tables, b.context_lens, e.query_start_loc, b.scale,
            sp.num_kv_heads, sp.io_dtype, sp.kv_dtype, float(b.k_scale), float(b.v_scale))


def _f32_batch(lens, qlens, H=4, Hkv=2, D=16, BS=4, seed=0):
    spec = W.Spec("pin", len(lens), H, Hkv, D, BS, "f32", "f32", ("fixed", tuple(lens)), seed=seed)
    return W.make_extend_batch(spec, ("fixed", tuple(qlens)), keep_logical=True)


def _with_kv(e, k_logical, v_logical):
    """The same tables and queries with new logical K/V rows (f32 pools)."""
    b = e.base
    kp = np.full_like(b.k_pool, np.nan)
    vp = np.full_like(b.v_pool, np.nan)
    BS = b.spec.block_size
    for s, L in enumerate(b.context_lens):
        for t in range(int(L)):
            kp[b.block_tables[s][t // BS], :, t % BS] = k_logical[s][t]
            vp[b.block_tables[s][t // BS], :, t % BS] = v_logical[s][t]
    nb = W.dataclasses.replace(b, k_pool=kp, v_pool=vp, logical_k=k_logical, logical_v=v_logical)
    return W.ExtendBatch(base=nb, query_start_loc=e.query_start_loc, q=e.q)


# ----------------------------------------------------------------------------------
# pins; each takes the function under test (the oracle, or a planted mistake)
# ----------------------------------------------------------------------------------

def pin_dense_causal_attention(f):
    """Against a separately written torch float64 attention over the unpaged rows, with
    the causal mask as a matrix (keys at or before each query's position)."""
    for sp, ql in [W.small_extend(n) for n in W.EXTEND] + [(None, None)]:
        if sp is None:
            e = _f32_batch((9, 17, 5), (9, 3, 5), H=8, Hkv=2, D=32, BS=4, seed=3)
        else:
            e = W.make_extend_batch(sp, ql, keep_logical=True)
        b = e.base
        s_ = b.spec
        out = f(*_args(e))
        G = s_.num_heads // s_.num_kv_heads
        for s in range(b.num_seqs):
            L = int(b.context_lens[s])
            lo, hi = int(e.query_start_loc[s]), int(e.query_start_loc[s + 1])
            Q = hi - lo
            if Q == 0:
                continue
            K = torch.from_numpy(pa_oracle.decode(b.logical_k[s], s_.kv_dtype, float(b.k_scale)))
            V = torch.from_numpy(pa_oracle.decode(b.logical_v[s], s_.kv_dtype, float(b.v_scale)))
            q = torch.from_numpy(pa_oracle.decode(e.q[lo:hi], s_.io_dtype))          # [Q][H][D]
            pos = torch.arange(L - Q, L).unsqueeze(1)                                  # [Q][1]
            allowed = torch.arange(L).unsqueeze(0) <= pos                              # [Q][L]
            for h in range(s_.num_heads):
                g = h // G
                z = (q[:, h, :] @ K[:, g, :].T) * float(np.float32(b.scale))
                z = z.masked_fill(~allowed, float("-inf"))
                ref = torch.softmax(z, dim=1) @ V[:, g, :]
                np.testing.assert_allclose(out[lo:hi, h], ref.numpy(), rtol=0, atol=1e-12)


def pin_prefill_first_token_is_its_value(f):
    """In a prefill of the whole context the first token sees only itself: V[0] exactly."""
    e = _f32_batch((7, 1, 12), (7, 1, 12))
    out = f(*_args(e))
    b = e.base
    for s in range(3):
        row = int(e.query_start_loc[s])
        for h in range(4):
            np.testing.assert_array_equal(out[row, h], b.logical_v[s][0, h // 2].astype(np.float64))


def pin_equal_keys_give_prefix_means(f):
    """All keys equal: query i averages V over positions 0 .. L-Q+i, which fixes the
    causal boundary of every row."""
    e = _f32_batch((10, 6), (4, 6), D=8, BS=4, seed=5)
    b = e.base
    one = np.ones((1, 2, 8), np.float32)
    ks = [np.repeat(one, int(L), axis=0) for L in b.context_lens]
    e2 = _with_kv(e, ks, b.logical_v)
    out = f(*_args(e2))
    for s, L in enumerate(b.context_lens):
        L = int(L)
        lo, hi = int(e.query_start_loc[s]), int(e.query_start_loc[s + 1])
        for i in range(hi - lo):
            p = L - (hi - lo) + i
            for h in range(4):
                mean = b.logical_v[s][:p + 1, h // 2].astype(np.float64).mean(axis=0)
                np.testing.assert_allclose(out[lo + i, h], mean, rtol=0, atol=1e-13)


def pin_every_prefix_is_a_decode(f):
    """Query i of an extend equals the (separately pinned) decode oracle run on the same
    sequence cut to its first p+1 tokens."""
    sp, ql = W.small_extend("extend_gqa_bf16_bs256")
    e = W.make_extend_batch(sp, ql)
    b = e.base
    out = f(*_args(e))
    for s in range(b.num_seqs):
        L = int(b.context_lens[s])
        lo, hi = int(e.query_start_loc[s]), int(e.query_start_loc[s + 1])
        for i in list(range(min(3, hi - lo))) + [hi - lo - 1]:
            p = L - (hi - lo) + i
            dec = pa_oracle.paged_decode(e.q[lo + i][None], b.k_pool, b.v_pool, b.block_tables[s][None],
                                         np.array([p + 1]), b.scale, sp.num_kv_heads, sp.io_dtype,
                                         sp.kv_dtype, float(b.k_scale), float(b.v_scale))
            np.testing.assert_array_equal(out[lo + i], dec[0])


def pin_one_query_is_decode(f):
    """Q = 1 everywhere is exactly one decode step."""
    spec = W.small_variant(4)
    e = W.make_extend_batch(spec, ("const", 1))
    b = e.base
    out = f(*_args(e))
    dec = pa_oracle.paged_decode(e.q, b.k_pool, b.v_pool, b.block_tables, b.context_lens, b.scale,
                                 spec.num_kv_heads, spec.io_dtype, spec.kv_dtype, float(b.k_scale),
                                 float(b.v_scale))
    np.testing.assert_array_equal(out, dec)


def pin_placement_and_block_size_invariance(f):
    """Outputs depend on logical positions only: new placement, block sizes 8 / 64."""
    sp, ql = W.small_extend("extend_llama7b_fp16")
    e = W.make_extend_batch(sp, ql, keep_logical=True)
    ref = f(*_args(e))
    for bs, seed in ((16, 1), (8, 2), (64, 3)):
        nb = W.repage(e.base, block_size=bs, seed=seed)
        got = f(*_args(W.ExtendBatch(base=nb, query_start_loc=e.query_start_loc, q=e.q)))
        np.testing.assert_array_equal(got, ref)


def pin_queries_without_keys_are_zero(f):
    """Q > L (outside the contract): rows whose position would be negative are zeros,
    the rest attend normally; Q = 0 sequences own no rows."""
    e = _f32_batch((3, 4), (3, 0))
    b = e.base
    qsl = np.array([0, 5, 5], np.int32)
    q = np.concatenate([e.q, e.q[:2]])
    out = f(q, b.k_pool, b.v_pool, b.block_tables, b.context_lens, qsl, b.scale, 2, "f32", "f32")
    assert (out[:2] == 0).all()
    np.testing.assert_array_equal(out[2, 0], b.logical_v[0][0, 0].astype(np.float64))


PINS = [pin_dense_causal_attention, pin_prefill_first_token_is_its_value,
        pin_equal_keys_give_prefix_means, pin_every_prefix_is_a_decode, pin_one_query_is_decode,
        pin_placement_and_block_size_invariance, pin_queries_without_keys_are_zero]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(extend.paged_extend)


# ----------------------------------------------------------------------------------
# planted mistakes: a parameterised restatement whose defaults are the definition
# ----------------------------------------------------------------------------------

def _variant(causal_shift=0, causal=True, head_of=lambda h, G, Hkv: h // G,
             first_pos=lambda L, Q: L - Q, q_of=lambda lo, i, Q: lo + i, scale_pow=1):
    def f(q, kp, vp, bt, lens, qsl, scale, Hkv, io, kv, ks=1.0, vs=1.0):
        T, H, D = q.shape
        G = H // Hkv
        out = np.full((T, H, D), np.nan)
        for s in range(len(qsl) - 1):
            L = int(lens[s])
            lo, Q = int(qsl[s]), int(qsl[s + 1] - qsl[s])
            KV = {g: (pa_oracle.decode(pa_oracle.gather(kp, bt[s], L, g), kv, ks),
                      pa_oracle.decode(pa_oracle.gather(vp, bt[s], L, g), kv, vs)) for g in range(Hkv)}
            for i in range(Q):
                p = first_pos(L, Q) + i + causal_shift
                n = max(0, min(p + 1, L)) if causal else L
                for h in range(H):
                    K, V = (x[:n] for x in KV[head_of(h, G, Hkv)])
                    if first_pos(L, Q) + i < 0:
                        out[lo + i, h] = 0.0
                    else:
                        qv = pa_oracle.decode(q[q_of(lo, i, Q), h], io)
                        out[lo + i, h] = pa_oracle.attend(qv, K, V, float(np.float32(scale)) ** scale_pow)
        return out
    return f


MUTANTS = {
    "sees_one_future_token": _variant(causal_shift=1),
    "misses_its_own_token": _variant(causal_shift=-1),
    "not_causal": _variant(causal=False),
    "new_tokens_at_front": _variant(first_pos=lambda L, Q: 0),
    "interleaved_heads": _variant(head_of=lambda h, G, Hkv: h % Hkv),
    "scale_squared": _variant(scale_pow=2),
    "queries_reversed": _variant(q_of=lambda lo, i, Q: lo + Q - 1 - i),
}


def test_restatement_passes_pins():
    f = _variant()
    for pin in PINS:
        pin(f)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_extend_mutant_is_caught(name):
    for pin in PINS:
        try:
            pin(MUTANTS[name])
        except (AssertionError, IndexError, ValueError):
            return
    raise AssertionError(f"mutant {name} passed every pin")
