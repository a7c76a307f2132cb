"""fp64 CPU oracle for paged-attention decode over a block table.

TEST INFRASTRUCTURE ONLY. Only tests, the smoke check and the benchmark's CPU
baseline leg may import this module. The product path (the HIP library and its
Python binding) never calls it, and this module imports nothing from the product.

It is the plain definition written out, in float64, slowly and obviously:

  For sequence s with context length L, query head h and its KV head g:
    K_s[t] = k_pool[ block_tables[s][t // BS] ][g][t % BS][:]     t = 0 .. L-1
    V_s[t] = v_pool[ same ]
    z_t    = scale * sum_d q[s][h][d] * K_s[t][d]
    out    = sum_t softmax(z)_t * V_s[t]

Pages cited (by title):
  [P1] "突破GPU内存瓶颈：vLLM与PagedAttention技术深度解析" (ocdem.com)
  [P2] vLLM 24x speed-up / architecture deep-dive (lshu.cn)
  [P3] "内存优化：KV Cache管理、PagedAttention原理与内存池配置" (5688vip.com)

Sources of each step:
  * block table: logical block j of a sequence lives in physical block
    block_tables[s][j]; blocks are fixed-size and non-contiguous
    ([P1] §2 block-table example; [P3] paged-pool figure and "PagedAttention
    principle" section).
  * only the last block of a sequence may be partly filled ([P1] §2).
  * scores are q.K^T divided by sqrt(head_dim) ([P2] §1.1 code fragment).
  * decode attends from the current token's query over ALL cached K/V ([P3] "core
    principle" section). The pages do not write softmax and the V product; the
    plainest reading, standard scaled-dot-product attention, is used.
  * FP8 KV cache ([P2] §4.2 mixed-precision table). The pages name only "FP8"; this
    oracle reads the OCP e4m3 format (1 sign, 4 exponent bits with bias 7, 3
    mantissa bits, no infinities, NaN = S.1111.111, max 448) and dequantizes as
    code_value * per-tensor scale.
  * KV-cache size = 2 x layers x heads x head_dim x seq_len x batch x dtype_bytes
    ([P3] "key parameters at a glance" paragraph).

Readings where the pages are silent:
  * grouped-query heads: query head h uses KV head h // (H / Hkv).
  * context length 0 gives an all-zero output.
  * pool layout [num_blocks][num_kv_heads][block_size][head_dim] for K and V.

Pins (tests/test_oracle.py, run without a GPU): the page-printed KV-size value,
the block-table mappings printed on [P1] §2 and in [P3]'s figure, closed forms of
softmax attention (L = 1, L = 2, equal keys, dominant key, shift invariance,
linearity in V), brute-force unpaged attention on tiny inputs, invariance under
placement / block size / sharing, the LSE-merge identity, and the fp8 / bf16
decode tables against torch's own conversions for every code.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

# ----------------------------------------------------------------------------------
# storage decoding (exact widening to float64)
# ----------------------------------------------------------------------------------


def fp8_e4m3_value(code: int) -> float:
    """Value of one OCP e4m3 code, from the format's definition."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:  # subnormal: 0.man x 2^(1 - bias)
        return sign * (man / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


FP8_E4M3_TABLE = np.array([fp8_e4m3_value(c) for c in range(256)], dtype=np.float64)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 is the top half of an IEEE float32: shift the 16 bits up and reinterpret."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # NaN patterns stay NaN
        return u32.view(np.float32).astype(np.float64)


def decode(arr: np.ndarray, dtype: str, scale: float = 1.0) -> np.ndarray:
    """Storage array -> float64 values (fp8: table value times the per-tensor scale)."""
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(arr, dtype=np.float16).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(arr)
    if dtype == "fp8_e4m3":
        return FP8_E4M3_TABLE[np.asarray(arr, dtype=np.uint8)] * np.float64(np.float32(scale))
    raise ValueError(dtype)


# ----------------------------------------------------------------------------------
# block-table gather
# ----------------------------------------------------------------------------------


def gather(pool: np.ndarray, table_row: np.ndarray, context_len: int, kv_head: int) -> np.ndarray:
    """Raw storage rows K_s[0..L-1] of one sequence and KV head, read through its table.

    pool is [num_blocks][num_kv_heads][block_size][head_dim]. Token t sits in logical
    block t // BS at slot t % BS; its physical block is table_row[t // BS].
    """
    nb_pool, _, bs, d = pool.shape
    out = np.empty((context_len, d), dtype=pool.dtype)
    t = 0
    j = 0
    while t < context_len:
        b = int(table_row[j])
        if not (0 <= b < nb_pool):
            raise IndexError(f"block table entry {b} at logical block {j} outside pool of {nb_pool}")
        n = min(bs, context_len - t)
        out[t:t + n] = pool[b, kv_head, :n, :]
        t += n
        j += 1
    return out


# ----------------------------------------------------------------------------------
# attention (two-pass softmax in float64)
# ----------------------------------------------------------------------------------


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * K q) weighted sum of V rows; zeros when there are no keys."""
    q = np.asarray(q, dtype=np.float64)
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    z = np.float64(scale) * (K @ q)
    m = z.max()
    w = np.exp(z - m)
    return (w @ V) / w.sum()


def paged_decode(q, k_pool, v_pool, block_tables, context_lens, scale,
                 num_kv_heads: int, io_dtype: str, kv_dtype: str,
                 k_scale: float = 1.0, v_scale: float = 1.0,
                 pairs: Optional[Iterable[Tuple[int, int]]] = None) -> np.ndarray:
    """Oracle output [S][H][D] in float64 (rows not in ``pairs`` are left NaN).

    q is [S][H][D] in io storage; pools and tables as described in the module doc.
    ``pairs`` restricts the work to a list of (sequence, query head).
    """
    S, H, D = q.shape
    G = H // num_kv_heads
    assert G * num_kv_heads == H
    out = np.full((S, H, D), np.nan, dtype=np.float64)
    if pairs is None:
        pairs = [(s, h) for s in range(S) for h in range(H)]
    by_unit = {}
    for s, h in pairs:
        by_unit.setdefault((int(s), int(h) // G), []).append(int(h))
    for (s, g), heads in sorted(by_unit.items()):
        L = int(context_lens[s])
        K = decode(gather(k_pool, block_tables[s], L, g), kv_dtype, k_scale)
        V = decode(gather(v_pool, block_tables[s], L, g), kv_dtype, v_scale)
        for h in heads:
            out[s, h] = attend(decode(q[s, h], io_dtype), K, V, float(np.float32(scale)))
    return out


def decode_batch(batch, pairs=None) -> np.ndarray:
    """paged_decode on a workload object with the generator's field names."""
    sp = batch.spec
    return paged_decode(batch.q, batch.k_pool, batch.v_pool, batch.block_tables,
                        batch.context_lens, batch.scale, sp.num_kv_heads, sp.io_dtype,
                        sp.kv_dtype, batch.k_scale, batch.v_scale, pairs=pairs)


# ----------------------------------------------------------------------------------
# split-context partial states and their log-sum-exp merge
# ----------------------------------------------------------------------------------


def partial_state(q, K, V, scale, lo: int, hi: int):
    """(m, l, o) over keys lo..hi-1: running max, sum of exp(z - m), unnormalised output.

    This is the state a split-context pass keeps for one partition ([P2] §3.3 and §4.1
    recommend the second-version kernel for long text; the pages give no algorithm, so
    the usual max/sum/partial-output split is used).
    """
    z = np.float64(scale) * (K[lo:hi] @ np.asarray(q, dtype=np.float64))
    m = z.max()
    w = np.exp(z - m)
    return m, w.sum(), w @ V[lo:hi]


def lse_merge(ms: Sequence[float], ls: Sequence[float], os_: Sequence[np.ndarray]) -> np.ndarray:
    """Combine partition states: rescale each by exp(m_p - max m) and normalise once."""
    ms = np.asarray(ms, dtype=np.float64)
    M = ms.max()
    w = np.exp(ms - M)
    num = sum(wp * op for wp, op in zip(w, os_))
    den = float(np.dot(w, np.asarray(ls, dtype=np.float64)))
    return num / den


# ----------------------------------------------------------------------------------
# byte accounting
# ----------------------------------------------------------------------------------


def kv_cache_bytes(num_layers: int, num_heads: int, head_dim: int, seq_len: int,
                   batch: int, dtype_bytes: int) -> int:
    """KV-cache size: K and V, for every layer, head, dim, position and request ([P3])."""
    return 2 * num_layers * num_heads * head_dim * seq_len * batch * dtype_bytes


def kv_unique_bytes(block_tables, context_lens, block_size: int, num_kv_heads: int,
                    head_dim: int, elem_bytes: int) -> int:
    """Bytes of K and V a decode step must read at least once: distinct physical
    (block, slot) positions that some sequence consumes, times heads, dims, 2."""
    seen = set()
    for s, L in enumerate(np.asarray(context_lens)):
        L = int(L)
        for j in range((L + block_size - 1) // block_size):
            n = min(block_size, L - j * block_size)
            b = int(block_tables[s][j])
            for slot in range(n):
                seen.add((b, slot))
    return len(seen) * num_kv_heads * head_dim * elem_bytes * 2
