"""fp64 CPU oracle for paged attention with several new query tokens per sequence
(prefill / extend over a paged KV cache).

TEST INFRASTRUCTURE ONLY. Only tests, the smoke check and the benchmark's CPU baseline
leg may import this module; the product path never calls it.

Pages cited (by title):
  [P2] vLLM 24x speed-up / architecture deep-dive (lshu.cn), §2.1: the execution engine
       runs prefill (the prompt), decode (generation) and extend (long texts); §2.2: the
       attention metadata carries block tables, context lengths and query lengths.
  [P3] "内存优化：KV Cache管理、PagedAttention原理与内存池配置": tokens attend over the
       cached keys and values of their request.

The plain definition, written out. Sequence s has context_lens[s] = L cached tokens,
counting its new ones, and Q = query_start_loc[s+1] - query_start_loc[s] new tokens:
the last Q of the L. New token i (0 <= i < Q) sits at position p = L - Q + i and its
query for head h is q[query_start_loc[s] + i][h]. It attends over the keys and values
at positions 0 .. p of its own sequence (all cached tokens before it and itself, never
later ones):
    K_s[t] = k_pool[ block_tables[s][t // BS] ][g][t % BS][:],  g = h // (H / Hkv)
    out[query_start_loc[s] + i][h] = softmax(scale * K_s[0..p] q) V_s[0..p]

Readings where the pages are silent (the plainest ones, stated here and in the library
header): the new tokens are the last Q of the context, their K/V are already in the
cache, attention is causal among them, the queries are packed in one [T][H][D] array
with offsets query_start_loc (the query lengths of the metadata are its differences),
and a query with no key (p < 0, i.e. Q > L) gives zeros.
"""
from __future__ import annotations

import numpy as np

from .pa_oracle import attend, decode, gather


def paged_extend(q, k_pool, v_pool, block_tables, context_lens, query_start_loc, scale,
                 num_kv_heads: int, io_dtype: str, kv_dtype: str,
                 k_scale: float = 1.0, v_scale: float = 1.0, rows=None) -> np.ndarray:
    """Oracle output [T][H][D] in float64; ``rows`` optionally restricts the work to a
    list of (query token index into q, head) pairs (other rows are NaN)."""
    T, H, D = q.shape
    G = H // num_kv_heads
    assert G * num_kv_heads == H
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    S = qsl.size - 1
    out = np.full((T, H, D), np.nan, dtype=np.float64)
    want = None if rows is None else {(int(t), int(h)) for t, h in rows}
    sc = float(np.float32(scale))
    for s in range(S):
        L = int(context_lens[s])
        Q = int(qsl[s + 1] - qsl[s])
        if Q == 0:
            continue
        for g in range(num_kv_heads):
            heads = [h for h in range(g * G, (g + 1) * G)]
            todo = [(int(qsl[s]) + i, h) for i in range(Q) for h in heads
                    if want is None or (int(qsl[s]) + i, h) in want]
            if not todo:
                continue
            K = decode(gather(k_pool, block_tables[s], L, g), kv_dtype, k_scale)
            V = decode(gather(v_pool, block_tables[s], L, g), kv_dtype, v_scale)
            for tok, h in todo:
                p = L - Q + (tok - int(qsl[s]))
                if p < 0:
                    out[tok, h] = 0.0
                    continue
                out[tok, h] = attend(decode(q[tok, h], io_dtype), K[:p + 1], V[:p + 1], sc)
    return out
