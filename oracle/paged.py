"""Paged-KV decode oracle in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Efficient attention & KV cache" (section 2.5, and the interview question on what PagedAttention
changes in the attention kernel): the cache lives in fixed-size blocks, a per-sequence block table
names the physical block of each logical block, and attention gathers the blocks through the
table. The result is attention over the gathered contiguous keys, so the oracle gathers first
(plain indexing, block by block in logical order) and then applies the dense definition of
``oracle.attention.dense_head`` to the one query row of each head.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from .attention import _f64, _kv_head, dense_head


def gather_sequence(k_cache, v_cache, table_row, seq_len: int, kv_head: int):
    """Contiguous K, V [seq_len, d] of one sequence and kv head.

    k_cache, v_cache: [num_blocks, Hkv, block_size, d]; table_row: physical block of each logical
    block; position p is row p % block_size of block table_row[p // block_size].
    """
    k_cache, v_cache = np.asarray(k_cache), np.asarray(v_cache)
    bs = k_cache.shape[2]
    n = -(-int(seq_len) // bs)
    ks = [k_cache[int(table_row[i]), kv_head] for i in range(n)]
    vs = [v_cache[int(table_row[i]), kv_head] for i in range(n)]
    if not ks:
        d = k_cache.shape[3]
        return np.zeros((0, d)), np.zeros((0, d))
    return _f64(np.concatenate(ks))[:seq_len], _f64(np.concatenate(vs))[:seq_len]


def paged_decode(Q, k_cache, v_cache, block_table, seq_lens, scale: Optional[float] = None):
    """Decode over a paged cache: Q [B, Hq, d] (one token per sequence) -> O [B, Hq, d], LSE [B, Hq].

    Query head h of sequence b attends to positions 0 .. seq_lens[b]-1 of kv head h / (Hq/Hkv),
    no mask. A sequence of length 0 has no defined softmax; this oracle returns O = 0 and
    LSE = -inf for it, the library's documented output.
    """
    Q = np.asarray(Q)
    B, Hq, d = Q.shape
    Hkv = np.asarray(k_cache).shape[1]
    O = np.zeros((B, Hq, d))
    L = np.full((B, Hq), -np.inf)
    for b in range(B):
        n = int(seq_lens[b])
        if n <= 0:
            continue
        for g in range(Hkv):
            k, v = gather_sequence(k_cache, v_cache, block_table[b], n, g)
            heads = [h for h in range(Hq) if _kv_head(h, Hq, Hkv) == g]
            o, lse = dense_head(Q[b, heads], k, v, False, scale)
            O[b, heads] = o
            L[b, heads] = lse
    return O, L


__all__ = ["gather_sequence", "paged_decode"]
