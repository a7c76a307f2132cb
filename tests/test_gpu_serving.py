"""The block manager, the append and copy kernels and the decode kernels together: a small
serving loop with a shared system prompt (prefix caching), beam forks with copy-on-write,
sequences that finish and free their blocks, and decode steps. Every decode is compared
with dense fp64 attention over each sequence's logical rows (no block tables involved),
and at the end every sequence's cached rows, read through its table, must equal the rows
written for it, byte for byte."""
import zlib

import numpy as np
import pytest

from oracle import kv_append, pa_oracle
import pagedattention_block_table_amd as pa

from gpu_util import log

pytestmark = pytest.mark.gpu

H, HKV, D, BS, NB = 8, 2, 128, 16, 160
TOL = {"f16": 4e-3, "fp8_e4m3": 1.5e-2}


def _row(tokens):
    """The K and V rows of the last token of a prefix: a deterministic function of the
    whole prefix, as a model's would be, so shared prefixes hold identical rows."""
    rng = np.random.default_rng(zlib.crc32(np.asarray(tokens, np.int32).tobytes()))
    return rng.standard_normal((2, HKV, D)).astype(np.float32)


class Loop:
    def __init__(self, kv, seed):
        import torch
        self.torch = torch
        self.kv = kv
        self.rng = np.random.default_rng(seed)
        self.bm = pa.BlockManager(NB, BS, prefix_caching=True)
        pool_dtype = torch.float16 if kv == "f16" else torch.uint8
        # stale contents are NaN (fp8: 0x7F) so a wrong table entry cannot go unnoticed
        if kv == "f16":
            self.kp = torch.full((NB, HKV, BS, D), float("nan"), dtype=pool_dtype, device="cuda")
        else:
            self.kp = torch.full((NB, HKV, BS, D), 0x7F, dtype=pool_dtype, device="cuda")
        self.vp = self.kp.clone()
        self.ks, self.vs = (1.0, 1.0) if kv == "f16" else (4.5 / 448, 4.25 / 448)
        self.tokens = {}       # handle -> token ids
        self.rows = {}         # handle -> list of [2][HKV][D] float32 rows (in f16 precision)

    def _write(self, items):
        """items: (handle, position) pairs whose rows go into the pools now."""
        if not items:
            return
        torch = self.torch
        hs = sorted({h for h, _ in items})
        idx = {h: i for i, h in enumerate(hs)}
        mb = max((self.bm.context_len(h) + BS - 1) // BS for h in hs)
        tables, _ = self.bm.export(hs, mb)
        kn = np.stack([self.rows[h][p][0] for h, p in items])
        vn = np.stack([self.rows[h][p][1] for h, p in items])
        seq = np.asarray([idx[h] for h, _ in items], np.int32)
        pos = np.asarray([p for _, p in items], np.int32)
        pa.pa_append_kv(torch.from_numpy(kn.astype(np.float16)).cuda(),
                        torch.from_numpy(vn.astype(np.float16)).cuda(),
                        torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(),
                        torch.from_numpy(tables).cuda(), self.kp, self.vp,
                        k_scale=self.ks, v_scale=self.vs)

    def add(self, tokens, prefill_check=False):
        h, cached = self.bm.add_sequence(tokens)
        self.tokens[h] = list(tokens)
        self.rows[h] = [_row(tokens[:p + 1]).astype(np.float16).astype(np.float32) for p in range(len(tokens))]
        self._write([(h, p) for p in range(cached, len(tokens))])
        if prefill_check:
            self.check_prefill(h, cached)
        return h, cached

    def check_prefill(self, h, cached):
        """Prefill of the uncached tokens with pa_extend (the cached prefix is only read):
        each new token attends causally over the whole sequence so far."""
        torch = self.torch
        L = len(self.tokens[h])
        Q = L - cached
        if Q == 0:
            return
        tables, lens = self.bm.export([h], (L + BS - 1) // BS)
        q = self.rng.standard_normal((Q, H, D)).astype(np.float16)
        scale = float(np.float32(1 / np.sqrt(D)))
        out = pa.pa_extend(torch.from_numpy(q).cuda(), self.kp, self.vp, torch.from_numpy(tables).cuda(),
                           torch.from_numpy(lens).cuda(),
                           torch.tensor([0, Q], dtype=torch.int32, device="cuda"), Q, scale=scale,
                           k_scale=self.ks, v_scale=self.vs)
        got = out.double().cpu().numpy()
        R = np.stack(self.rows[h])
        G = H // HKV
        worst = 0.0
        for g in range(HKV):
            K = self._stored_value(R[:, 0, g], self.ks)
            V = self._stored_value(R[:, 1, g], self.vs)
            for i in range(Q):
                p = cached + i
                for hh in range(g * G, (g + 1) * G):
                    ref = pa_oracle.attend(q[i, hh].astype(np.float64), K[:p + 1], V[:p + 1], np.float64(scale))
                    # the first tokens see few keys: allow the f16 rounding of |out| up to ~4
                    worst = max(worst, float(np.abs(got[i, hh] - ref).max()))
        assert worst <= TOL[self.kv] + 2.0 ** -10, worst

    def fork(self, h):
        c = self.bm.fork(h)
        self.tokens[c] = list(self.tokens[h])
        self.rows[c] = list(self.rows[h])
        return c

    def free(self, h):
        self.bm.free_sequence(h)
        del self.tokens[h], self.rows[h]

    def step(self):
        """One decode step: every live sequence gets one token; copies before writes."""
        torch = self.torch
        copies, items = [], []
        for h in sorted(self.tokens):
            tok = int(self.rng.integers(0, 50))
            slot, src, dst = self.bm.append_token(h, tok)
            p = len(self.tokens[h])
            self.tokens[h].append(tok)
            self.rows[h].append(_row(self.tokens[h]).astype(np.float16).astype(np.float32))
            table = self.bm.block_table(h)
            assert slot == table[p // BS] * BS + p % BS
            if src >= 0:
                copies.append((src, dst))
            items.append((h, p))
        if copies:
            pa.pa_copy_blocks(self.kp, self.vp, torch.tensor(copies, dtype=torch.int32, device="cuda"))
        self._write(items)
        return len(copies)

    def _expected_storage(self, x, scale):
        if self.kv == "f16":
            return x.astype(np.float16)
        return kv_append.encode(x, "fp8_e4m3", scale)

    def _stored_value(self, x, scale):
        if self.kv == "f16":
            return x.astype(np.float64)
        return pa_oracle.decode(kv_append.encode(x, "fp8_e4m3", scale), "fp8_e4m3", scale)

    def check_decode(self):
        torch = self.torch
        hs = sorted(self.tokens)
        mb = max((self.bm.context_len(h) + BS - 1) // BS for h in hs)
        tables, lens = self.bm.export(hs, mb)
        q = self.rng.standard_normal((len(hs), H, D)).astype(np.float16)
        scale = float(np.float32(1 / np.sqrt(D)))
        out = pa.pa_decode(torch.from_numpy(q).cuda(), self.kp, self.vp, torch.from_numpy(tables).cuda(),
                           torch.from_numpy(lens).cuda(), scale=scale, k_scale=self.ks, v_scale=self.vs)
        got = out.double().cpu().numpy()
        worst = 0.0
        G = H // HKV
        for i, h in enumerate(hs):
            R = np.stack(self.rows[h])                     # [L][2][HKV][D]
            for g in range(HKV):
                K = self._stored_value(R[:, 0, g], self.ks)
                V = self._stored_value(R[:, 1, g], self.vs)
                for hh in range(g * G, (g + 1) * G):
                    ref = pa_oracle.attend(q[i, hh].astype(np.float64), K, V, np.float64(scale))
                    worst = max(worst, float(np.abs(got[i, hh] - ref).max()))
        assert worst <= TOL[self.kv], worst
        return worst

    def check_pools(self):
        kp = self.kp.view(self.torch.uint8).cpu().numpy()
        vp = self.vp.view(self.torch.uint8).cpu().numpy()
        e = 2 if self.kv == "f16" else 1
        kp = kp.reshape(NB, HKV, BS, D * e)
        vp = vp.reshape(NB, HKV, BS, D * e)
        for h in sorted(self.tokens):
            R = np.stack(self.rows[h])
            table = np.asarray(self.bm.block_table(h), np.int32)
            for g in range(HKV):
                for pool, j, sc in ((kp, 0, self.ks), (vp, 1, self.vs)):
                    got = pa_oracle.gather(pool, table, len(R), g)
                    want = np.ascontiguousarray(self._expected_storage(R[:, j, g], sc)).view(np.uint8)
                    np.testing.assert_array_equal(got, want.reshape(len(R), D * e))


@pytest.mark.parametrize("kv", ["f16", "fp8_e4m3"])
def test_serving_loop(kv):
    log(f"[serving] kv={kv}")
    lp = Loop(kv, seed=7)
    system = list(range(100, 140))                           # 40 tokens: 2 full blocks + 8
    handles = []
    for r in range(5):
        suffix = lp.rng.integers(0, 50, int(lp.rng.integers(3, 30))).tolist()
        h, cached = lp.add(system + suffix, prefill_check=r < 3)
        assert cached == (0 if r == 0 else 32)
        handles.append(h)
    log(f"[serving] prefill decode err {lp.check_decode():.2e}")
    beams = [lp.fork(handles[0]), lp.fork(handles[0]), lp.fork(handles[2])]
    total_copies = 0
    for t in range(24):
        total_copies += lp.step()
        if t == 7:
            lp.free(handles[1])
            lp.free(beams[1])
            lp.add(system + [7, 7, 7])
        if t == 15:
            lp.free(handles[3])
            lp.add(system + lp.rng.integers(0, 50, 20).tolist())
        if t in (0, 8, 16, 23):
            log(f"[serving] step {t} decode err {lp.check_decode():.2e}")
    assert total_copies >= 3                                  # every fork copied its partial block
    lp.check_pools()
    lp.bm.close()


def test_copy_blocks_direct():
    """pa_copy_blocks copies whole blocks of K and V (every byte, whatever their fill) and
    skips pairs with an id outside the pool or src == dst."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(3)
    kp = torch.randn((12, 2, 16, 64), generator=g, device="cuda").to(torch.bfloat16)
    vp = torch.randn((12, 2, 16, 64), generator=g, device="cuda").to(torch.bfloat16)
    k0, v0 = kp.clone(), vp.clone()
    pairs = torch.tensor([[1, 5], [2, 2], [3, 12], [-1, 4], [7, 0]], dtype=torch.int32, device="cuda")
    pa.pa_copy_blocks(kp, vp, pairs)
    torch.cuda.synchronize()
    want_k, want_v = k0.clone(), v0.clone()
    want_k[5], want_v[5] = k0[1], v0[1]
    want_k[0], want_v[0] = k0[7], v0[7]
    assert torch.equal(kp.view(torch.int16), want_k.view(torch.int16))
    assert torch.equal(vp.view(torch.int16), want_v.view(torch.int16))
