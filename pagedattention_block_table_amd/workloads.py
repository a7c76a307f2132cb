"""Seeded synthetic inputs for paged decode: lengths, K/V/q values, block placement.

This module is the only code that both the fp64 oracle (``oracle/``) and the HIP
path receive their inputs from. It draws random numbers, rounds them to the
storage dtype and writes them into a paged pool; it holds none of the attention
arithmetic.

Pages cited (by title):
  [P1] "突破GPU内存瓶颈：vLLM与PagedAttention技术深度解析" (ocdem.com/news/957472)
  [P2] "为什么vLLM能实现24倍推理加速" / vLLM architecture deep-dive (lshu.cn/news/246877)
  [P3] "内存优化：KV Cache管理、PagedAttention原理与内存池配置" (5688vip.com)

Storage model ([P1] §2 block table; [P3] figure "static allocation vs paged"):
  * K and V live in two pools of shape [num_blocks][num_kv_heads][block_size][head_dim].
  * block_tables[s][j] names the physical block that holds logical block j of
    sequence s (tokens j*block_size ... j*block_size+block_size-1).
  * Rows past a sequence's last block are padded with -1; they are never read.
  * Every pool slot that no sequence uses (the tail of a partial last block and
    every unreferenced block) holds NaN (fp8: code 0x7F), so an over-read shows.

Storage dtypes as numpy arrays:
  f32 -> float32, f16 -> float16, bf16 -> uint16 bit patterns, fp8_e4m3 -> uint8 codes
  (OCP e4m3 "fn": bias 7, max 448, NaN 0x7F/0xFF, no infinities).

Seeding: ``np.random.SeedSequence(spec.seed)`` is split into independent child
streams (structure, q, prefix, then K and V of each sequence), so that per-sequence
tensors can be drawn on several threads and still give the same bytes.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import math
import os
from typing import Optional, Sequence

import numpy as np

DTYPES = ("f32", "f16", "bf16", "fp8_e4m3")
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1}
NP_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "fp8_e4m3": np.uint8}
# Quiet-NaN bit patterns used as sentinels in unused pool slots.
NAN_BITS = {"f16": 0x7E00, "bf16": 0x7FC0, "fp8_e4m3": 0x7F}
FP8_E4M3_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Spec:
    """Shape and value recipe of one synthetic decode batch.

    lengths is one of
      ("fixed", (L0, L1, ...))
      ("uniform_sum", ((a0, b0), (a1, b1), ...))  -- sum of independent integer U[a, b] draws
      ("choice", (values...), (probs...))         -- i.i.d. categorical per sequence
      ("const", L)
    """

    name: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    io_dtype: str
    kv_dtype: str
    lengths: tuple
    shared_prefix: int = 0          # tokens of identical prefix; its full blocks are shared
    spike_frac: float = 0.0         # fraction of positions whose K gets +spike_value
    spike_value: float = 4.0
    pool_blocks: Optional[int] = None  # explicit pool size; else ceil(pool_factor * used)
    pool_factor: float = 1.2
    partition_size: int = 0         # 0: single-pass decode; else split-context size
    seed: int = 1000

    def replace(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)


# The five workloads. Shapes stand in for the pages' serving scenarios; values are N(0,1).
CONFIGS = {
    # Tiny paged decode, fp32; 32-block pool, random placement, no sharing.
    0: Spec("tiny_fp32", 4, 4, 4, 64, 16, "f32", "f32", ("fixed", (1, 17, 33, 100)),
            pool_blocks=32, seed=1000),
    # LLaMA-7B-shaped layer, fp16; 20 requests, prompt U[78,178] + generated U[156,356]
    # ([P1] §3 serving test: input 128±50, output 256±100 tokens).
    1: Spec("llama7b_fp16", 20, 32, 32, 128, 16, "f16", "f16",
            ("uniform_sum", ((78, 178), (156, 356))), seed=1001),
    # Shared system prompt, bf16, GQA 32/8; 64 x 1000-token histories with a 500-token
    # common prefix ([P3] "prefix caching" case).
    2: Spec("shared_prefix_bf16", 64, 32, 8, 128, 16, "bf16", "bf16", ("const", 1000),
            shared_prefix=500, seed=1002),
    # Long context, fp16, block 32, 8 x 32768 tokens in an exactly-filled 8192-block pool;
    # 1% of positions get +4 on every K element; 512-token partitions + LSE merge.
    3: Spec("long_ctx_fp16", 8, 32, 32, 128, 32, "f16", "f16", ("const", 32768),
            spike_frac=0.01, pool_blocks=8192, partition_size=512, seed=1003),
    # Mixed lengths 50/30/20 % of 128/1K/8K ([P2] §5.3 stress-test mix), fp8-e4m3 KV with
    # per-tensor fp32 scales, bf16 q/out, GQA 32/8.
    4: Spec("mixed_fp8", 256, 32, 8, 128, 16, "bf16", "fp8_e4m3",
            ("choice", (128, 1024, 8192), (0.5, 0.3, 0.2)), partition_size=512, seed=1004),
}


# The same workloads with the larger blocks of [P2] §3.1–§3.2 (256 by default, 128 for
# short and 512 for long texts); pools keep the same token capacity.
VARIANTS = {
    "llama7b_fp16_bs128": CONFIGS[1].replace(name="llama7b_fp16_bs128", block_size=128),
    "shared_prefix_bf16_bs256": CONFIGS[2].replace(name="shared_prefix_bf16_bs256", block_size=256),
    "long_ctx_fp16_bs512": CONFIGS[3].replace(name="long_ctx_fp16_bs512", block_size=512, pool_blocks=512),
    "mixed_fp8_bs256": CONFIGS[4].replace(name="mixed_fp8_bs256", block_size=256),
    # a larger query group: the LLaMA-2-70B attention shape ([P2] §1 benchmarks that model),
    # 64 query heads over 8 KV heads, bf16, 64 requests of 1K-3K cached tokens
    "llama70b_gqa8_bf16": Spec("llama70b_gqa8_bf16", 64, 64, 8, 128, 16, "bf16", "bf16",
                               ("uniform_sum", ((1024, 3072),)), seed=1005),
    # head_dim 256 (16 query heads over 8 KV heads, bf16, 32 requests of 0.5K-2K tokens)
    "d256_gqa2_bf16": Spec("d256_gqa2_bf16", 32, 16, 8, 256, 16, "bf16", "bf16",
                           ("uniform_sum", ((512, 2048),)), seed=1006),
    # the prefix-caching shape with a long shared prompt: 64 requests share an 8000-token
    # prefix (~33 MB of K/V, more than the chip's L2) and hold 500 private tokens each
    "shared_prefix_long_bf16": CONFIGS[2].replace(name="shared_prefix_long_bf16", lengths=("const", 8500),
                                                  shared_prefix=8000, seed=1007),
}


@dataclasses.dataclass
class PagedBatch:
    spec: Spec
    context_lens: np.ndarray        # int32 [S]
    block_tables: np.ndarray        # int32 [S][max_blocks_per_seq], -1 padded
    q: np.ndarray                   # io storage [S][H][D]
    k_pool: np.ndarray              # kv storage [NB][Hkv][BS][D]
    v_pool: np.ndarray
    scale: np.float32
    k_scale: np.float32
    v_scale: np.float32
    num_blocks: int
    shared_blocks: np.ndarray       # int32 physical ids shared by every table (may be empty)
    logical_k: Optional[list] = None  # per sequence, kv storage [L][Hkv][D] (keep_logical)
    logical_v: Optional[list] = None

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.context_lens.size else 0


# ----------------------------------------------------------------------------------
# storage rounding (data preparation, not part of the decode arithmetic)
# ----------------------------------------------------------------------------------

def to_storage(x: np.ndarray, dtype: str, quant_scale: Optional[np.float32] = None) -> np.ndarray:
    """Round float32 values to a storage dtype (round-to-nearest-even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    import torch  # library rounding for bf16 / fp8

    t = torch.from_numpy(x)
    if dtype == "bf16":
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if dtype == "fp8_e4m3":
        assert quant_scale is not None
        y = x / np.float32(quant_scale)
        return torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    raise ValueError(dtype)


def nan_fill(shape, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.full(shape, np.nan, dtype=np.float32)
    return np.full(shape, NAN_BITS[dtype], dtype=NP_STORAGE[dtype])


# ----------------------------------------------------------------------------------
# generator
# ----------------------------------------------------------------------------------

def _draw_lengths(spec: Spec, rng: np.random.Generator) -> np.ndarray:
    kind = spec.lengths[0]
    S = spec.num_seqs
    if kind == "fixed":
        L = np.asarray(spec.lengths[1], dtype=np.int64)
        assert L.shape == (S,)
    elif kind == "const":
        L = np.full(S, int(spec.lengths[1]), dtype=np.int64)
    elif kind == "uniform_sum":
        L = np.zeros(S, dtype=np.int64)
        for a, b in spec.lengths[1]:
            L += rng.integers(a, b + 1, size=S)
    elif kind == "choice":
        vals = np.asarray(spec.lengths[1], dtype=np.int64)
        L = rng.choice(vals, size=S, p=np.asarray(spec.lengths[2], dtype=np.float64))
    else:
        raise ValueError(kind)
    return L.astype(np.int32)


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def _tile(logical: np.ndarray, nblk: int, bs: int, fill) -> np.ndarray:
    """[L][Hkv][D] -> [nblk][Hkv][BS][D], padding the tail slots with `fill`."""
    L, hkv, d = logical.shape
    pad = np.empty((nblk * bs, hkv, d), dtype=logical.dtype)
    pad[:L] = logical
    pad[L:] = fill
    return np.ascontiguousarray(pad.reshape(nblk, bs, hkv, d).transpose(0, 2, 1, 3))


def _workers() -> int:
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


def make_batch(spec, keep_logical: bool = False, threads: Optional[int] = None) -> PagedBatch:
    """Build one seeded decode batch.

    Draw order (fixed): lengths, spike positions, placement permutation from the
    structure stream; q from its own stream; prefix K then V from the prefix stream;
    K then V of sequence s from that sequence's stream.
    """
    if isinstance(spec, int):
        spec = CONFIGS[spec]
    S, H, Hkv, D, BS = spec.num_seqs, spec.num_heads, spec.num_kv_heads, spec.head_dim, spec.block_size
    assert H % Hkv == 0 and spec.io_dtype in DTYPES[:3] and spec.kv_dtype in DTYPES
    ss = np.random.SeedSequence(spec.seed)
    kids = ss.spawn(3 + 2 * S)
    rng_struct = np.random.default_rng(kids[0])
    rng_q = np.random.default_rng(kids[1])
    rng_prefix = np.random.default_rng(kids[2])

    lens = _draw_lengths(spec, rng_struct)
    nblk = (lens.astype(np.int64) + BS - 1) // BS
    P = int(spec.shared_prefix)
    if P:
        assert (lens >= P).all()
    n_shared = P // BS  # full prefix blocks are shared; a partial prefix block stays private

    spikes = [None] * S
    if spec.spike_frac > 0:
        for s in range(S):
            L = int(lens[s])
            n = int(math.ceil(spec.spike_frac * L))
            spikes[s] = np.sort(rng_struct.choice(L, size=n, replace=False))

    used = int(n_shared + (nblk - n_shared).sum()) if P else int(nblk.sum())
    NB = int(spec.pool_blocks) if spec.pool_blocks is not None else max(1, int(math.ceil(spec.pool_factor * used)))
    assert NB >= used, (NB, used)
    perm = rng_struct.permutation(NB).astype(np.int32)
    shared_ids = perm[:n_shared]
    max_blocks = int(nblk.max()) if S else 0
    bt = np.full((S, max(max_blocks, 1)), -1, dtype=np.int32)
    cur = n_shared
    for s in range(S):
        bt[s, :n_shared] = shared_ids
        k = int(nblk[s]) - n_shared
        bt[s, n_shared:n_shared + k] = perm[cur:cur + k]
        cur += k

    q32 = _normal(rng_q, (S, H, D))
    q = to_storage(q32, spec.io_dtype)

    kvd = spec.kv_dtype
    fp8 = kvd == "fp8_e4m3"
    k_pool = nan_fill((NB, Hkv, BS, D), kvd)
    v_pool = nan_fill((NB, Hkv, BS, D), kvd)
    scale = np.float32(1.0 / math.sqrt(D))

    prefix_k = prefix_v = None
    if P:
        prefix_k = _normal(rng_prefix, (P, Hkv, D))
        prefix_v = _normal(rng_prefix, (P, Hkv, D))

    def logical_f32(s):
        r = np.random.default_rng(kids[3 + 2 * s])
        L = int(lens[s])
        k = _normal(r, (L - P, Hkv, D))
        r2 = np.random.default_rng(kids[4 + 2 * s])
        v = _normal(r2, (L - P, Hkv, D))
        if P:
            k = np.concatenate([prefix_k, k], axis=0)
            v = np.concatenate([prefix_v, v], axis=0)
        if spikes[s] is not None:
            k[spikes[s]] += np.float32(spec.spike_value)
        return k, v

    nthreads = threads or _workers()
    k_scale = v_scale = np.float32(1.0)
    if fp8:
        # Per-tensor scales over every used K (resp. V) value: amax / 448, in fp32.
        with _cf.ThreadPoolExecutor(nthreads) as ex:
            f32 = list(ex.map(logical_f32, range(S)))
        kmax = max((float(np.abs(k).max()) for k, _ in f32 if k.size), default=1.0)
        vmax = max((float(np.abs(v).max()) for _, v in f32 if v.size), default=1.0)
        k_scale = np.float32(np.float32(kmax) / np.float32(FP8_E4M3_MAX))
        v_scale = np.float32(np.float32(vmax) / np.float32(FP8_E4M3_MAX))
        get = lambda s: f32[s]
    else:
        get = logical_f32

    fill = k_pool.reshape(-1)[:1].copy()  # NaN sentinel in storage form
    logical_k = [None] * S if keep_logical else None
    logical_v = [None] * S if keep_logical else None

    def page(s):
        k, v = get(s)
        ks = to_storage(k, kvd, k_scale if fp8 else None)
        vs = to_storage(v, kvd, v_scale if fp8 else None)
        if keep_logical:
            logical_k[s], logical_v[s] = ks, vs
        nb = int(nblk[s])
        ids = bt[s, :nb]
        kt = _tile(ks, nb, BS, fill[0])
        vt = _tile(vs, nb, BS, fill[0])
        if s == 0 and n_shared:
            k_pool[ids[:n_shared]] = kt[:n_shared]
            v_pool[ids[:n_shared]] = vt[:n_shared]
        k_pool[ids[n_shared:]] = kt[n_shared:]
        v_pool[ids[n_shared:]] = vt[n_shared:]
        if fp8:
            f32[s] = None

    if S:
        page(0)  # writes the shared prefix blocks once
    with _cf.ThreadPoolExecutor(nthreads) as ex:
        list(ex.map(page, range(1, S)))

    return PagedBatch(spec=spec, context_lens=lens, block_tables=bt, q=q, k_pool=k_pool,
                      v_pool=v_pool, scale=scale, k_scale=k_scale, v_scale=v_scale,
                      num_blocks=NB, shared_blocks=shared_ids.copy(),
                      logical_k=logical_k, logical_v=logical_v)


def repage(batch: PagedBatch, block_size: Optional[int] = None, seed: int = 0,
           unshare: bool = False, pool_blocks: Optional[int] = None) -> PagedBatch:
    """Same logical K/V, new physical placement (and optionally a new block size).

    Requires ``keep_logical``. With ``unshare`` every sequence gets private copies of
    the shared prefix blocks. Used by the placement / block-size / sharing invariants.
    """
    assert batch.logical_k is not None, "make_batch(..., keep_logical=True) first"
    spec = batch.spec
    BS = block_size or spec.block_size
    S, Hkv, D = batch.num_seqs, spec.num_kv_heads, spec.head_dim
    lens = batch.context_lens
    nblk = (lens.astype(np.int64) + BS - 1) // BS
    n_shared = 0 if unshare else (spec.shared_prefix // BS)
    used = int(n_shared + (nblk - n_shared).sum()) if n_shared else int(nblk.sum())
    NB = pool_blocks or int(math.ceil(1.25 * used)) + 3
    rng = np.random.default_rng(seed)
    perm = rng.permutation(NB).astype(np.int32)
    bt = np.full((S, max(int(nblk.max()), 1)), -1, dtype=np.int32)
    shared_ids = perm[:n_shared]
    cur = n_shared
    for s in range(S):
        bt[s, :n_shared] = shared_ids
        k = int(nblk[s]) - n_shared
        bt[s, n_shared:n_shared + k] = perm[cur:cur + k]
        cur += k
    kvd = spec.kv_dtype
    k_pool = nan_fill((NB, Hkv, BS, D), kvd)
    v_pool = nan_fill((NB, Hkv, BS, D), kvd)
    fill = k_pool.reshape(-1)[0]
    for s in range(S):
        nb = int(nblk[s])
        ids = bt[s, :nb]
        k_pool[ids] = _tile(batch.logical_k[s], nb, BS, fill)
        v_pool[ids] = _tile(batch.logical_v[s], nb, BS, fill)
    new_spec = spec.replace(block_size=BS, shared_prefix=0 if unshare else spec.shared_prefix)
    return dataclasses.replace(batch, spec=new_spec, block_tables=bt, k_pool=k_pool,
                               v_pool=v_pool, num_blocks=NB, shared_blocks=shared_ids.copy())


def small_variant(cfg: int) -> Spec:
    """A reduced copy of a workload that the fp64 oracle finishes in seconds, with the
    same dtypes and structure (sharing, spikes, length mix) and ragged tails."""
    base = CONFIGS[cfg]
    if cfg == 0:
        return base
    if cfg == 1:
        return base.replace(name="llama7b_fp16_small", num_seqs=5, seed=2001)
    if cfg == 2:
        return base.replace(name="shared_prefix_bf16_small", num_seqs=6, lengths=("const", 300),
                            shared_prefix=150, seed=2002)
    if cfg == 3:
        return base.replace(name="long_ctx_fp16_small", num_seqs=2, num_heads=4, num_kv_heads=4,
                            lengths=("fixed", (3000, 2333)), pool_blocks=None, seed=2003)
    if cfg == 4:
        return base.replace(name="mixed_fp8_small", num_seqs=12,
                            lengths=("choice", (128, 1024, 2049), (0.5, 0.3, 0.2)), seed=2004)
    raise ValueError(cfg)


# ----------------------------------------------------------------------------------
# several new query tokens per sequence (prefill / extend over the paged cache)
# ----------------------------------------------------------------------------------

@dataclasses.dataclass
class ExtendBatch:
    """A decode-style batch (pools, tables, context lengths that count the new tokens)
    plus the new tokens' queries: sequence s owns rows query_start_loc[s] ..
    query_start_loc[s+1]-1 of q, the last Q_s positions of its context."""
    base: PagedBatch
    query_start_loc: np.ndarray     # int32 [S+1]
    q: np.ndarray                   # io storage [T][H][D]

    @property
    def query_lens(self) -> np.ndarray:
        return np.diff(self.query_start_loc).astype(np.int32)

    @property
    def max_query_len(self) -> int:
        ql = self.query_lens
        return int(ql.max()) if ql.size else 0

    @property
    def num_tokens(self) -> int:
        return int(self.query_start_loc[-1])


def _draw_query_lens(kind: tuple, lens: np.ndarray, rng: np.random.Generator) -> np.ndarray:
    S = lens.shape[0]
    if kind[0] == "const":
        Q = np.full(S, int(kind[1]), dtype=np.int64)
    elif kind[0] == "fixed":
        Q = np.asarray(kind[1], dtype=np.int64)
        assert Q.shape == (S,)
    elif kind[0] == "all":
        Q = lens.astype(np.int64)                       # prefill of the whole context
    elif kind[0] == "choice":
        Q = rng.choice(np.asarray(kind[1], dtype=np.int64), size=S,
                       p=np.asarray(kind[2], dtype=np.float64))
    else:
        raise ValueError(kind)
    return np.minimum(Q, lens).astype(np.int32)


def make_extend_batch(spec, query_lens: tuple, keep_logical: bool = False) -> ExtendBatch:
    """Seeded extend batch: make_batch(spec) for the cache, then, from a stream of its
    own, the query lengths (clamped to the context lengths) and the queries."""
    base = make_batch(spec, keep_logical=keep_logical)
    sp = base.spec
    rng = np.random.default_rng(np.random.SeedSequence([sp.seed, 7919]))
    Q = _draw_query_lens(query_lens, base.context_lens, rng)
    qsl = np.zeros(Q.size + 1, dtype=np.int32)
    np.cumsum(Q, out=qsl[1:])
    q32 = _normal(rng, (int(qsl[-1]), sp.num_heads, sp.head_dim))
    return ExtendBatch(base=base, query_start_loc=qsl, q=to_storage(q32, sp.io_dtype))


# Extend workloads: a chunked-prefill step of 8192 new tokens ([P2] §3.1 sets
# max_num_batched_tokens to 8192; §2.1 names prefill and extend) over cached contexts of
# up to 3.5K tokens, in the LLaMA-7B layer shape and in GQA bf16 with [P2]'s 256-token
# blocks; and a mixed fp8 batch whose query lengths range from a few tokens (several
# tokens checked at once) to a 512-token chunk.
EXTEND = {
    "extend_llama7b_fp16": (Spec("extend_llama7b_fp16", 16, 32, 32, 128, 16, "f16", "f16",
                                 ("uniform_sum", ((512, 512), (0, 3584))), seed=1101),
                            ("const", 512)),
    "extend_gqa_bf16_bs256": (Spec("extend_gqa_bf16_bs256", 16, 32, 8, 128, 256, "bf16", "bf16",
                                   ("uniform_sum", ((512, 512), (0, 3584))), seed=1102),
                              ("const", 512)),
    "extend_mixed_fp8": (Spec("extend_mixed_fp8", 64, 32, 8, 128, 16, "bf16", "fp8_e4m3",
                              ("uniform_sum", ((512, 512), (0, 3584))), seed=1103),
                         ("choice", (4, 64, 512), (0.5, 0.3, 0.2))),
}


def small_extend(name: str):
    """A reduced extend workload the fp64 oracle finishes in seconds (same dtypes, group
    and block sizes; ragged query and context lengths)."""
    spec, ql = EXTEND[name]
    small = spec.replace(name=spec.name + "_small", num_seqs=4,
                         lengths=("fixed", (70, 300, 41, 520)), seed=spec.seed + 1000)
    if ql[0] == "const":
        ql = ("fixed", (70, 37, 41, 200))    # one pure prefill, one whole-context prefill
    else:
        ql = ("fixed", (4, 64, 1, 130))
    return small, ql
