"""Attention backward oracle: gradients of the forward pass in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

With S = scale * Q K^T (masked entries -inf), P = softmax_row(S), O = P V and an upstream
gradient dO, the chain rule gives ("4.2 FlashAttention I: IO-Awareness & The Online Softmax",
section "The backward pass: recomputation instead of storage"):
    dV = P^T dO,   dP = dO V^T,   D_i = sum_c dO_ic O_ic  (= sum_j P_ij dP_ij),
    dS = P * (dP - D[:, None]),   dQ = scale * dS K,   dK = scale * dS^T Q.
With grouped kv heads the gradients of a kv head add over the query heads that read it.
Masks and the kv-head mapping follow ``oracle.attention`` (bottom-right causal alignment,
optional sliding window).
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from .attention import _check_window, _default_scale, _f64, _kv_head


def _mask(Tq: int, Tk: int, causal: bool, window: Optional[int]) -> np.ndarray:
    """Boolean [Tq, Tk]: True where the key is hidden from the query."""
    if not causal:
        return np.zeros((Tq, Tk), dtype=bool)
    pos = np.arange(Tq)[:, None] + (Tk - Tq)
    cols = np.arange(Tk)[None, :]
    hide = cols > pos
    if window is not None:
        hide = hide | (cols <= pos - int(window))
    return hide


def dense_backward_head(q, k, v, do, causal: bool, scale: Optional[float] = None,
                        window: Optional[int] = None):
    """Gradients of one head by the definition: P materialised, then the chain rule above.

    q: [Tq, d]; k, v: [Tk, d]; do: [Tq, d]. Returns (dQ, dK, dV, O, LSE, D).
    """
    _check_window(causal, window)
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    Tq, d = q.shape
    Tk = k.shape[0]
    sc = _default_scale(d, scale)
    S = sc * (q @ k.T)
    S = np.where(_mask(Tq, Tk, causal, window), -np.inf, S)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    den = E.sum(axis=1, keepdims=True)
    P = E / den
    O = P @ v
    lse = m[:, 0] + np.log(den[:, 0])
    dV = P.T @ do
    dP = do @ v.T
    D = np.sum(do * O, axis=1)
    dS = P * (dP - D[:, None])
    dQ = sc * (dS @ k)
    dK = sc * (dS.T @ q)
    return dQ, dK, dV, O, lse, D


def dense_backward(Q, K, V, dO, causal: bool, scale: Optional[float] = None,
                   window: Optional[int] = None):
    """``dense_backward_head`` over [B, Hq, Tq, d] with grouped kv heads.

    Returns (dQ [B, Hq, Tq, d], dK [B, Hkv, Tk, d], dV [B, Hkv, Tk, d]).
    """
    Q, K, V, dO = np.asarray(Q), np.asarray(K), np.asarray(V), np.asarray(dO)
    B, Hq, Tq, d = Q.shape
    Hkv, Tk = K.shape[1], K.shape[2]
    dQ = np.zeros((B, Hq, Tq, d))
    dK = np.zeros((B, Hkv, Tk, d))
    dV = np.zeros((B, Hkv, Tk, d))
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            gq, gk, gv, *_ = dense_backward_head(Q[b, h], K[b, g], V[b, g], dO[b, h], causal,
                                                 scale, window)
            dQ[b, h] = gq
            dK[b, g] += gk
            dV[b, g] += gv
    return dQ, dK, dV


def tiled_backward_head(q, k, v, o, lse, do, causal: bool, scale: Optional[float] = None,
                        block_q: int = 32, block_kv: int = 32, window: Optional[int] = None):
    """The pages' block backward: P recomputed tile by tile from the saved LSE.

    Steps of ``flash_attention_backward`` on "4.2 FlashAttention I" (section "The backward
    pass"): D = rowsum(dO * O) up front; for each query block and each key block that holds a
    visible key, S = scale * Q_i K_j^T (masked), P = exp(S - L_i), dV_j += P^T dO_i,
    dP = dO_i V_j^T, dS = P * (dP - D_i), dQ_i += scale * dS K_j, dK_j += scale * dS^T Q_i.
    o and lse are the forward outputs of this head. Returns (dQ, dK, dV).
    """
    _check_window(causal, window)
    q, k, v, o, lse, do = (_f64(x) for x in (q, k, v, o, lse, do))
    Tq, d = q.shape
    Tk = k.shape[0]
    sc = _default_scale(d, scale)
    dQ, dK, dV = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    D = np.sum(do * o, axis=1)
    for i0 in range(0, Tq, block_q):
        i1 = min(i0 + block_q, Tq)
        for j0 in range(0, Tk, block_kv):
            j1 = min(j0 + block_kv, Tk)
            hide = _mask(Tq, Tk, causal, window)[i0:i1, j0:j1]
            if hide.all():
                continue
            S = np.where(hide, -np.inf, sc * (q[i0:i1] @ k[j0:j1].T))
            P = np.exp(S - lse[i0:i1, None])
            dV[j0:j1] += P.T @ do[i0:i1]
            dP = do[i0:i1] @ v[j0:j1].T
            dS = P * (dP - D[i0:i1, None])
            dQ[i0:i1] += sc * (dS @ k[j0:j1])
            dK[j0:j1] += sc * (dS.T @ q[i0:i1])
    return dQ, dK, dV


def tiled_backward(Q, K, V, O, LSE, dO, causal: bool, scale: Optional[float] = None,
                   block_q: int = 64, block_kv: int = 64, window: Optional[int] = None):
    """``tiled_backward_head`` over [B, Hq, Tq, d] with grouped kv heads, from given O and LSE.

    This is the backward as the pages define its interface: (Q, K, V, O, L, dO) in, gradients
    out, with P recomputed from L. A kv head's dK and dV add over the query heads that read it.
    Returns (dQ [B, Hq, Tq, d], dK [B, Hkv, Tk, d], dV [B, Hkv, Tk, d]).
    """
    Q, K, V, O, LSE, dO = (np.asarray(x) for x in (Q, K, V, O, LSE, dO))
    B, Hq, Tq, d = Q.shape
    Hkv, Tk = K.shape[1], K.shape[2]
    dQ = np.zeros((B, Hq, Tq, d))
    dK = np.zeros((B, Hkv, Tk, d))
    dV = np.zeros((B, Hkv, Tk, d))
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            gq, gk, gv = tiled_backward_head(Q[b, h], K[b, g], V[b, g], O[b, h], LSE[b, h],
                                             dO[b, h], causal, scale, block_q, block_kv, window)
            dQ[b, h] = gq
            dK[b, g] += gk
            dV[b, g] += gv
    return dQ, dK, dV


def loss_gradient_fd(q, k, v, do, causal: bool, which: str, idx, scale: Optional[float] = None,
                     eps: float = 1e-5, window: Optional[int] = None) -> float:
    """Central difference of sum(dO * O) with respect to one element of q, k or v.

    The gradient check of "4.2 FlashAttention I" (section "The backward pass"): perturb one
    input element by +-eps, evaluate the forward by the definition, difference the scalar.
    """
    from .attention import dense_head

    args = {"q": _f64(q).copy(), "k": _f64(k).copy(), "v": _f64(v).copy()}
    x = args[which]
    orig = x[idx]
    x[idx] = orig + eps
    fp = float(np.sum(_f64(do) * dense_head(args["q"], args["k"], args["v"], causal, scale,
                                             window=window)[0]))
    x[idx] = orig - eps
    fm = float(np.sum(_f64(do) * dense_head(args["q"], args["k"], args["v"], causal, scale,
                                             window=window)[0]))
    x[idx] = orig
    return (fp - fm) / (2 * eps)


def backward_rows(q, k, v, do, rows, causal: bool, scale: Optional[float] = None,
                  window: Optional[int] = None) -> np.ndarray:
    """dQ of the given query rows of one head, each row by the definition.

    For row i: P_i and O_i from ``dense_head`` (the materialised softmax row), D_i = dO_i . O_i,
    dP_i = dO_i V^T, dS_i = P_i * (dP_i - D_i), dQ_i = scale * dS_i K (the chain rule of
    ``dense_backward_head``, one row at a time). Returns [len(rows), d].
    """
    from .attention import dense_head

    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    sc = _default_scale(q.shape[1], scale)
    idx = np.asarray(rows, dtype=np.int64)
    O, _, P = dense_head(q, k, v, causal, scale, rows=idx, return_p=True, window=window)
    D = np.sum(do[idx] * O, axis=1)
    dP = do[idx] @ v.T
    dS = P * (dP - D[:, None])
    return sc * (dS @ k)


def backward_cols(q, k, v, do, keys, causal: bool, scale: Optional[float] = None,
                  window: Optional[int] = None, row_chunk: int = 1024):
    """dK and dV of the given keys of one (query) head, by recomputation from L.

    O and L of every query row come from ``dense_head`` (row chunks of ``row_chunk`` only bound
    the memory; each row is the definition). Then, as in the pages' backward (P_ij = exp(S_ij -
    L_i), "Efficient attention & KV cache", section 2.2), for the key columns j:
    P_:j = exp(scale Q k_j - L) (0 where masked), dV_j = P_:j^T dO, dP_:j = dO v_j,
    dS_:j = P_:j * (dP_:j - D), dK_j = scale dS_:j^T Q, with D = rowsum(dO * O).
    Returns (dK [len(keys), d], dV [len(keys), d]) of this query head alone; a kv head's
    gradient is the sum over the query heads that read it.

    Under a causal mask a row at position i + Tk - Tq sees key j only if j <= i + Tk - Tq, so the
    rows before the first one that sees the smallest requested key have P = 0 in every requested
    column and add nothing to the sums: they are left out (O and L are computed for the rest).
    """
    from .attention import dense_head

    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    Tq, d = q.shape
    Tk = k.shape[0]
    sc = _default_scale(d, scale)
    kk = np.asarray(keys, dtype=np.int64)
    first = max(0, int(kk.min()) - (Tk - Tq)) if (causal and kk.size) else 0
    O = np.zeros((Tq, d))
    L = np.zeros(Tq)
    for r0 in range(first, Tq, row_chunk):
        rr = np.arange(r0, min(r0 + row_chunk, Tq))
        O[rr], L[rr] = dense_head(q, k, v, causal, scale, rows=rr, window=window)
    D = np.sum(do * O, axis=1)
    hide = _mask(Tq, Tk, causal, window)[:, kk]
    hide[:first] = True
    P = np.where(hide, 0.0, np.exp(np.where(hide, 0.0, sc * (q @ k[kk].T)) - L[:, None]))
    dV = P.T @ do
    dS = P * (do @ v[kk].T - D[:, None])
    dK = sc * (dS.T @ q)
    return dK, dV


def backward_flops(B: int, Hq: int, Tq: int, Tk: int, d: int, causal: bool) -> float:
    """Matmul FLOPs of the backward's five products (S, dP, dV, dK, dQ): 10 B Hq Tq Tk d, halved
    under a causal mask (the forward's convention for its two products, 4 B H T^2 d)."""
    f = 10.0 * B * Hq * Tq * Tk * d
    return f / 2.0 if causal else f


__all__ = ["dense_backward_head", "dense_backward", "tiled_backward_head", "tiled_backward",
           "loss_gradient_fd",
           "backward_rows", "backward_cols", "backward_flops"]

