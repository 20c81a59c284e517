"""Packed variable-length attention oracle in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"4.2 FlashAttention I: IO-Awareness & The Online Softmax" (section "Practical use: you almost never
write this yourself") packs documents back to back without padding and passes cumulative sequence
offsets so that no score between two documents is formed; "Efficient attention & KV cache"
(section 4) names the same document masks for training. Each document is therefore plain
attention on its own slices: the oracle cuts the packed tensors at the offsets and applies
``oracle.attention.dense_head`` per document and head.

Rows that see no key (a causal document with fewer keys than queries, or a document with no keys)
have no defined softmax; the oracle returns O = 0 and LSE = -inf for them, the library's
documented output.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from .attention import _kv_head, dense_head
from .backward import tiled_backward_head


def varlen_attention(Q, K, V, cu_q, cu_k, causal: bool, scale: Optional[float] = None,
                     window: Optional[int] = None):
    """Q [total_q, Hq, d], K, V [total_k, Hkv, d], cu_q / cu_k cumulative lengths (n + 1).

    Returns O [total_q, Hq, d] and LSE [Hq, total_q].
    """
    Q, K, V = np.asarray(Q), np.asarray(K), np.asarray(V)
    total_q, Hq, d = Q.shape
    Hkv = K.shape[1]
    O = np.zeros((total_q, Hq, d))
    L = np.full((Hq, total_q), -np.inf)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        tq, tk = q1 - q0, k1 - k0
        if tq <= 0 or tk <= 0:
            continue
        # rows that see at least one key: all, or under the causal mask those at positions >= 0
        first = max(0, tq - tk) if causal else 0
        rows = np.arange(first, tq)
        if rows.size == 0:
            continue
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            o, lse = dense_head(Q[q0:q1, h], K[k0:k1, g], V[k0:k1, g], causal, scale, rows=rows,
                                window=window)
            O[q0 + rows, h] = o
            L[h, q0 + rows] = lse
    return O, L


def varlen_backward(Q, K, V, O, LSE, dO, cu_q, cu_k, causal: bool, scale: Optional[float] = None,
                    window: Optional[int] = None):
    """Gradients of ``varlen_attention``: each document through ``tiled_backward_head`` (the
    pages' backward from O and L) on its slices; a kv head's dK, dV add over its query heads.

    O, dO: [total_q, Hq, d]; LSE: [Hq, total_q]. Rows that see no key are left out of their
    document's problem (their dQ is 0 and they add nothing to dK, dV).
    Returns (dQ [total_q, Hq, d], dK [total_k, Hkv, d], dV [total_k, Hkv, d]).
    """
    Q, K, V, O, LSE, dO = (np.asarray(x) for x in (Q, K, V, O, LSE, dO))
    total_q, Hq, d = Q.shape
    total_k, Hkv = K.shape[0], K.shape[1]
    dQ = np.zeros((total_q, Hq, d))
    dK = np.zeros((total_k, Hkv, d))
    dV = np.zeros((total_k, Hkv, d))
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        tq, tk = q1 - q0, k1 - k0
        if tq <= 0 or tk <= 0:
            continue
        first = max(0, tq - tk) if causal else 0
        r0 = q0 + first
        if r0 >= q1:
            continue
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            gq, gk, gv = tiled_backward_head(Q[r0:q1, h], K[k0:k1, g], V[k0:k1, g], O[r0:q1, h],
                                             LSE[h, r0:q1], dO[r0:q1, h], causal, scale,
                                             window=window)
            dQ[r0:q1, h] = gq
            dK[k0:k1, g] += gk
            dV[k0:k1, g] += gv
    return dQ, dK, dV


__all__ = ["varlen_attention", "varlen_backward"]
