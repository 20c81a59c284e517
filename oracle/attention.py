"""Attention oracle: the plain definition in float64, a tiled online-softmax path and 1-D units.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

Conventions (the readings of the pages that the GPU library follows too):
  * layout [B, H, T, d]; K and V carry Hkv heads and query head h reads kv head h // (Hq // Hkv)
    ("enable_gqa" in "SDPA and FlashAttention's tiling", section "The tiled sketch, in Python");
  * ``scale`` multiplies the dot products before the softmax; callers pass 1/sqrt(d) by default;
  * causal masking is bottom-right aligned: query row i sits at absolute position i + (Tk - Tq)
    and sees keys j <= i + Tk - Tq. For Tq == Tk this is the usual lower triangle used on every
    page; for Tq == 1 it sees every key, as a decode step over a KV cache does
    ("Efficient attention & KV cache", section 1);
  * a sliding window of width W keeps, of the causal keys, only the last W positions: query i
    at position p = i + Tk - Tq sees keys p - W < j <= p (exercise 4 of "4.2 FlashAttention I";
    exercise 2 of "Efficient attention & KV cache", section 7). A window implies causal; W >= p+1
    for every row is plain causal attention;
  * LSE is the natural log-sum-exp of the scaled, masked scores of a row: m + log(l)
    ("4.2 FlashAttention I", FlashAttention forward section; "Efficient attention & KV cache",
    section 3).
"""

from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _default_scale(d: int, scale: Optional[float]) -> float:
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def _check_window(causal: bool, window: Optional[int]) -> None:
    if window is None:
        return
    if not causal:
        raise ValueError("a sliding window is a causal mask: pass causal=True")
    if int(window) < 1:
        raise ValueError("window must be >= 1")


# --------------------------------------------------------------------------------------------
# The definition, materialising S and P.
# --------------------------------------------------------------------------------------------

def dense_head(q, k, v, causal: bool, scale: Optional[float] = None,
               rows: Optional[Sequence[int]] = None, return_p: bool = False,
               window: Optional[int] = None):
    """Exact attention for one head, with the full score and probability rows materialised.

    Follows the reference attention of "4.2 FlashAttention I" (sections "The memory bottleneck"
    and the verification after the forward pass), "Attention from scratch + roofline" (section
    "Naive attention, matched against SDPA") and ``standard_attention`` of "Efficient attention &
    KV cache" (section 3): S = scale * q k^T, masked entries -inf, row max subtracted before the
    exponential, P = exp(S - m) / sum, O = P v; plus LSE = m + log(sum).

    q: [Tq, d]; k, v: [Tk, d]. ``rows`` restricts the computation to those query rows (their
    positions are still their indices in 0..Tq-1), which is how single outputs of a large problem
    are checked one by one. ``window`` (with ``causal``) also hides keys at or before p - W, the
    materialised reference of exercise 4 of "4.2 FlashAttention I". Returns (O [n, d],
    LSE [n]) and P [n, Tk] when ``return_p``.
    """
    _check_window(causal, window)
    q, k, v = _f64(q), _f64(k), _f64(v)
    Tq, d = q.shape
    Tk = k.shape[0]
    if Tk < 1:
        raise ValueError("softmax over an empty key set is undefined")
    sc = _default_scale(d, scale)
    idx = np.arange(Tq) if rows is None else np.asarray(rows, dtype=np.int64)
    S = sc * (q[idx] @ k.T)                                   # [n, Tk]
    if causal:
        off = Tk - Tq
        cols = np.arange(Tk)[None, :]
        pos = idx[:, None] + off
        hidden = cols > pos
        if window is not None:
            hidden = hidden | (cols <= pos - int(window))
        S = np.where(hidden, -np.inf, S)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    den = E.sum(axis=1, keepdims=True)
    P = E / den
    O = P @ v
    lse = m[:, 0] + np.log(den[:, 0])
    if return_p:
        return O, lse, P
    return O, lse


def _kv_head(h: int, Hq: int, Hkv: int) -> int:
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (Hq // Hkv)


def dense_attention(Q, K, V, causal: bool, scale: Optional[float] = None,
                    window: Optional[int] = None):
    """The definition over a whole [B, Hq, Tq, d] problem, head by head (float64).

    Returns O [B, Hq, Tq, d] and LSE [B, Hq, Tq].
    """
    Q, K, V = np.asarray(Q), np.asarray(K), np.asarray(V)
    B, Hq, Tq, d = Q.shape
    Hkv = K.shape[1]
    O = np.empty((B, Hq, Tq, d), np.float64)
    L = np.empty((B, Hq, Tq), np.float64)
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            O[b, h], L[b, h] = dense_head(Q[b, h], K[b, g], V[b, g], causal, scale,
                                          window=window)
    return O, L


def brute_attention(q, k, v, causal: bool, scale: Optional[float] = None,
                    subtract_max: bool = True, window: Optional[int] = None):
    """Scalar pure-Python attention for tiny inputs (lists of rows), one row at a time.

    The same computation as ``standard_attention`` in the lab on "Explain tiled attention and
    verify its output" (section "Read lab.py"), with rows limited to their visible keys. With
    ``subtract_max=False`` the exponentials are taken of the raw scores, which overflows
    (``OverflowError``) for large logits, the failure that page's tests provoke.
    ``window`` keeps only keys p - W < j <= p of a row at position p.
    Returns (O as a list of rows, LSE as a list).
    """
    _check_window(causal, window)
    Tq, Tk = len(q), len(k)
    d = len(q[0])
    sc = _default_scale(d, scale)
    out, lse = [], []
    for i in range(Tq):
        last = i + (Tk - Tq) if causal else Tk - 1
        first = last - int(window) + 1 if window is not None else 0
        scores = []
        for j in range(Tk):
            if j > last or j < first:
                continue
            acc = 0.0
            for c in range(d):
                acc += float(q[i][c]) * float(k[j][c])
            scores.append((j, acc * sc))
        m = max(s for _, s in scores) if subtract_max else 0.0
        weights = [(j, math.exp(s - m)) for j, s in scores]
        total = sum(w for _, w in weights)
        row = [0.0] * d
        for j, w in weights:
            for c in range(d):
                row[c] += (w / total) * float(v[j][c])
        out.append(row)
        lse.append(m + math.log(total))
    return out, lse


# --------------------------------------------------------------------------------------------
# Tiled online-softmax path (the algorithm the kernels implement), float64.
# --------------------------------------------------------------------------------------------

def tiled_head(q, k, v, causal: bool, scale: Optional[float] = None, block_q: int = 32,
               block_kv: int = 32, rescale: bool = True, stats: Optional[dict] = None,
               window: Optional[int] = None):
    """Tiled forward of one head: query blocks outside, key/value blocks inside, online softmax.

    Steps in the order of the forward pass on "4.2 FlashAttention I" (section "FlashAttention
    forward: tiling + online softmax fused into one pass") and ``flash_attention_forward`` on
    "Efficient attention & KV cache" (section 3):
      for each query block, start from m = -inf, l = 0, acc = 0; for each key block that holds
      at least one visible key (causal: stop once the block starts past the block's last query
      position), form the masked score tile, m' = max(m, rowmax), alpha = exp(m - m') (0 while
      m is still -inf), P = exp(S - m'), l = alpha*l + rowsum(P), acc = alpha*acc + P V, m = m';
      finish with O = acc / l and LSE = m + log(l).
    Rows whose running max is still -inf use 0 as the exponent base, the guard of that page.
    ``rescale=False`` drops the rescale of the accumulator (not of l), the planted fault of the
    lab on "Explain tiled attention and verify its output". ``stats`` (a dict) receives the
    number of (query block, key block) tiles visited.
    With ``window`` the key loop also skips the blocks that end before the window of the block's
    first query starts, and the tile mask adds the window's left edge: the two-sided skip of
    exercise 4 of "4.2 FlashAttention I".
    """
    _check_window(causal, window)
    q, k, v = _f64(q), _f64(k), _f64(v)
    Tq, d = q.shape
    Tk = k.shape[0]
    sc = _default_scale(d, scale)
    off = Tk - Tq
    O = np.zeros((Tq, d))
    L = np.zeros(Tq)
    visited = 0
    for i0 in range(0, Tq, block_q):
        i1 = min(i0 + block_q, Tq)
        qi = q[i0:i1]
        m = np.full(i1 - i0, -np.inf)
        l = np.zeros(i1 - i0)
        acc = np.zeros((i1 - i0, d))
        kv_end = min(Tk, i1 + off) if causal else Tk
        # first key any row of the block may see: the window's left edge of the first row
        kv_beg = max(0, i0 + off - int(window) + 1) if window is not None else 0
        for j0 in range(0, kv_end, block_kv):
            j1 = min(j0 + block_kv, Tk)
            if j1 <= kv_beg:
                continue
            visited += 1
            S = sc * (qi @ k[j0:j1].T)
            if causal:
                pos = np.arange(i0, i1)[:, None] + off
                cols = np.arange(j0, j1)[None, :]
                hide = cols > pos
                if window is not None:
                    hide = hide | (cols <= pos - int(window))
                S = np.where(hide, -np.inf, S)
            m_new = np.maximum(m, S.max(axis=1))
            base = np.where(np.isneginf(m_new), 0.0, m_new)
            alpha = np.where(np.isneginf(m), 0.0, np.exp(m - base))
            P = np.exp(S - base[:, None])
            l = alpha * l + P.sum(axis=1)
            acc = (alpha[:, None] if rescale else 1.0) * acc + P @ v[j0:j1]
            m = m_new
        safe = np.where(l == 0.0, 1.0, l)
        O[i0:i1] = acc / safe[:, None]
        L[i0:i1] = m + np.log(safe)
    if stats is not None:
        stats["tiles_visited"] = stats.get("tiles_visited", 0) + visited
    return O, L


def tiled_attention(Q, K, V, causal: bool, scale: Optional[float] = None, block_q: int = 32,
                    block_kv: int = 32, rescale: bool = True, stats: Optional[dict] = None,
                    window: Optional[int] = None):
    """``tiled_head`` over a whole [B, Hq, Tq, d] problem with grouped kv heads."""
    Q, K, V = np.asarray(Q), np.asarray(K), np.asarray(V)
    B, Hq, Tq, d = Q.shape
    Hkv = K.shape[1]
    O = np.empty((B, Hq, Tq, d))
    L = np.empty((B, Hq, Tq))
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            O[b, h], L[b, h] = tiled_head(Q[b, h], K[b, g], V[b, g], causal, scale,
                                          block_q, block_kv, rescale, stats, window)
    return O, L


# --------------------------------------------------------------------------------------------
# Merging results computed over disjoint key sets (the split-K decode combine).
# --------------------------------------------------------------------------------------------

def merge_partials(o_parts, lse_parts):
    """Combine attention results over disjoint key subsets into the result over their union.

    Each part s holds O_s (normalised over its own keys) and LSE_s. Because the running maximum
    can be any value without changing the final ratio ("Efficient attention & KV cache",
    section 2.1), the union is LSE = log sum_s exp(LSE_s) and O = sum_s exp(LSE_s - LSE) O_s.
    A part over no keys has LSE_s = -inf and contributes nothing.
    o_parts: [S, ..., d]; lse_parts: [S, ...]. Returns (O, LSE).
    """
    o_parts, lse_parts = _f64(o_parts), _f64(lse_parts)
    top = lse_parts.max(axis=0)
    base = np.where(np.isneginf(top), 0.0, top)
    w = np.exp(lse_parts - base)
    tot = w.sum(axis=0)
    lse = base + np.log(tot)
    o = (w[..., None] * o_parts).sum(axis=0) / tot[..., None]
    return o, lse


# --------------------------------------------------------------------------------------------
# One-dimensional units of the recurrence.
# --------------------------------------------------------------------------------------------

def _block_rebases(z: np.ndarray, width: int):
    """Walk the 1-D logits z in blocks of ``width``: for each block [lo, hi) yield (lo, hi, top,
    rescale), where top is the running maximum once the block is included and rescale =
    exp(previous top - top) is the factor every sum gathered over earlier blocks is multiplied
    by (0 before any block, when nothing has been gathered). This is the correction factor of
    "4.2 FlashAttention I" (section "The key idea: a running max and a correction factor")."""
    top = -math.inf
    for lo in range(0, z.shape[0], width):
        hi = min(lo + width, z.shape[0])
        new_top = max(top, float(z[lo:hi].max()))
        yield lo, hi, new_top, (math.exp(top - new_top) if top > -math.inf else 0.0)
        top = new_top


def stream_weighted_sum(logits, values, width: int = 4):
    """sum_i softmax(logits)_i values[i], gathered in one pass over blocks of ``width`` logits.

    The streaming weighted sum of "4.2 FlashAttention I" (section "A from-scratch implementation
    and a correctness proof"): the normaliser and the weighted sum are both rescaled by the
    correction factor whenever the running maximum grows, and divided once at the end.
    """
    z, vals = _f64(logits), _f64(values)
    norm, acc = 0.0, np.zeros(vals.shape[1])
    for lo, hi, top, rescale in _block_rebases(z, width):
        w = np.exp(z[lo:hi] - top)
        norm = rescale * norm + w.sum()
        acc = rescale * acc + w @ vals[lo:hi]
    return acc / norm


def stream_softmax(logits, width: int):
    """softmax of a 1-D vector whose maximum and normaliser are gathered in one pass over
    blocks of ``width`` entries ("Efficient attention & KV cache", section 3), then applied."""
    z = _f64(logits)
    norm, top = 0.0, -math.inf
    for lo, hi, top, rescale in _block_rebases(z, width):
        norm = rescale * norm + np.exp(z[lo:hi] - top).sum()
    return np.exp(z - top) / norm


def online_logsumexp_trace(x, block_size: int) -> List[Tuple[float, float, float]]:
    """The (running max, correction factor, normaliser) after each block, for hand traces.

    Exercise 2 of "4.2 FlashAttention I" streams [3, 1, 6, 2] in blocks of two; the final
    log-sum-exp is the running max plus the log of the normaliser.
    """
    z = _f64(x)
    norm, trace = 0.0, []
    for lo, hi, top, rescale in _block_rebases(z, block_size):
        norm = rescale * norm + float(np.exp(z[lo:hi] - top).sum())
        trace.append((top, rescale, norm))
    return trace
