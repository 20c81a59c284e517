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


def backward_flops(B: int, Hq: int, Tq: int, Tk: int, d: int, causal: bool) -> float:
    """Matmul FLOPs of the backward's five products (S, dP, dV, dK, dQ): 10 B Hq Tq Tk d, halved
    under a causal mask (the forward's convention for its two products, 4 B H T^2 d)."""
    f = 10.0 * B * Hq * Tq * Tk * d
    return f / 2.0 if causal else f


__all__ = ["dense_backward_head", "dense_backward", "tiled_backward_head", "loss_gradient_fd",
           "backward_flops"]

