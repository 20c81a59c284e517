"""Work and traffic accounting for attention, written from the pages' formulas.

TEST INFRASTRUCTURE ONLY (see the package docstring). The benchmark keeps its own metric
formulas; tests check the two agree.
"""

from __future__ import annotations

import math


def attention_flops(B: int, H: int, Tq: int, Tk: int, d: int, causal: bool) -> float:
    """Matmul FLOPs of one forward: 4 B H Tq Tk d (QK^T and PV, 2 FLOPs per multiply-add).

    "Attention from scratch + roofline" (section "FLOPs / bytes / arithmetic intensity") counts
    4 B H T^2 D; its exercise 3 halves the count under a causal mask, the convention the
    prefill TFLOP/s figure uses.
    """
    f = 4.0 * B * H * Tq * Tk * d
    return f / 2.0 if causal else f


def visible_pairs(Tq: int, Tk: int, causal: bool, window: int = 0) -> int:
    """Number of (query, key) pairs a mask leaves visible (bottom-right causal alignment).

    ``window`` > 0 (causal only) keeps the last ``window`` positions of each row.
    """
    if not causal:
        return Tq * Tk
    off = Tk - Tq
    # row i sees keys 0..i+off, or only the last `window` of them
    n = 0
    for i in range(Tq):
        seen = min(Tk, i + off + 1)
        n += min(seen, window) if window > 0 else seen
    return n


def attention_flops_exact(B: int, H: int, Tq: int, Tk: int, d: int, causal: bool,
                          window: int = 0) -> float:
    """4 d FLOPs for every visible (query, key) pair: the work a perfect mask skip leaves."""
    return 4.0 * d * B * H * visible_pairs(Tq, Tk, causal, window)


def window_cache_bytes(layers: int, kv_heads: int, head_dim: int, window: int,
                       dtype_bytes: int = 2) -> int:
    """KV-cache bytes of one sequence under a rolling window of ``window`` positions.

    Per token and layer the cache holds one key and one value vector per kv head; a rolling
    window caps the tokens held ("Efficient attention & KV cache", section 2.3 and exercise 1
    of section 7).
    """
    return 2 * layers * kv_heads * head_dim * dtype_bytes * window


def attention_bytes(B: int, H: int, T: int, d: int, dtype_bytes: int = 2) -> int:
    """Q + K + V + O bytes, the traffic model of "Attention from scratch + roofline"."""
    return dtype_bytes * B * H * d * (T + 2 * T + T)


def arithmetic_intensity(B: int, H: int, T: int, d: int, dtype_bytes: int = 2) -> float:
    return attention_flops(B, H, T, T, d, False) / attention_bytes(B, H, T, d, dtype_bytes)


def decode_intensity(B: int, Hq: int, Hkv: int, d: int, Tk: int, dtype_bytes: int = 2) -> float:
    """FLOPs per byte of one decode step (one query token per head).

    The notebook's decode intensity counts FLOPs with the KV head count, exact for MHA; its
    exercise 1 raises intensity by the group size under GQA. Here FLOPs use the query heads and
    bytes the kv heads (K and V) plus Q and O.
    """
    flops = 4.0 * B * Hq * Tk * d
    byts = dtype_bytes * B * d * (2 * Hkv * Tk + 2 * Hq)
    return flops / byts


def decode_bytes(B: int, Hq: int, Hkv: int, Tk: int, d: int, dtype_bytes: int = 2) -> int:
    """Algorithmic bytes of one decode step: K and V read once, Q read, O written, fp32 LSE."""
    return (2 * B * Hkv * Tk * d + 2 * B * Hq * d) * dtype_bytes + 4 * B * Hq


def prefill_compulsory_bytes(B: int, Hq: int, Hkv: int, Tq: int, Tk: int, d: int,
                             dtype_bytes: int = 2) -> int:
    """Q read, K and V read once, O written, fp32 LSE written."""
    return (2 * B * Hq * Tq * d + 2 * B * Hkv * Tk * d) * dtype_bytes + 4 * B * Hq * Tq


def logical_access_model(seq_len: int, num_heads: int = 32, head_dim: int = 128,
                         bytes_per_elem: int = 2, block_q: int = 128) -> dict:
    """The access-count model of the lab on "Explain tiled attention and verify its output".

    Standard attention: Q, K, V, O once plus S and P written and read (4 T^2 per head).
    Causal tiled loop with query blocks outside and no cache reuse: Q and O once, and each query
    block reads the K and V rows up to the end of its block. Values in MB (1e6 bytes), rounded
    to two decimals as that page prints them.
    """
    qkvo = 4 * num_heads * seq_len * head_dim * bytes_per_elem
    nxn = 4 * num_heads * seq_len * seq_len * bytes_per_elem
    kv_rows = sum(min(seq_len, s + block_q) for s in range(0, seq_len, block_q))
    tiled = (2 * num_heads * seq_len * head_dim
             + 2 * num_heads * kv_rows * head_dim) * bytes_per_elem
    return {
        "standard_qkv_o_mb": round(qkvo / 1e6, 2),
        "standard_nxn_matrix_hbm_mb": round(nxn / 1e6, 2),
        "standard_total_hbm_mb": round((qkvo + nxn) / 1e6, 2),
        "tiled_logical_access_mb_no_cache_reuse": round(tiled / 1e6, 2),
        "qkvo_compulsory_bytes_mb": round(qkvo / 1e6, 2),
        "num_q_blocks": math.ceil(seq_len / block_q),
    }


def score_matrix_bytes(N: int, dtype_bytes: int = 2) -> int:
    """Bytes of one head's N x N score matrix."""
    return N * N * dtype_bytes


def saved_output_bytes(N: int, d: int, dtype_bytes: int = 2, lse_bytes: int = 4) -> int:
    """Bytes of what the fused forward keeps: O (N x d) and the per-row statistic L (N)."""
    return N * d * dtype_bytes + N * lse_bytes
