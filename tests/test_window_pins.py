"""Pins of the oracle's sliding-window mask to facts outside itself (CPU only).

A sliding window of width W keeps, for a query at position p (bottom-right alignment,
p = i + Tk - Tq), the keys p - W < j <= p (exercise 4 of "4.2 FlashAttention I"; exercise 2 of
"Efficient attention & KV cache", section 7). The pins: scalar brute force, the reduction of each
row to plain attention over a sliced key range, the two limits (W = 1 and W >= p + 1), the tiled
path with its two-sided block skip, torch's float64 attention with an explicit mask, and the
cache sizes the pages print for a rolling window.
"""

import json
import os

import numpy as np
import pytest

import oracle
from oracle import accounting

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


@pytest.mark.parametrize("Tq,Tk", [(4, 4), (6, 9), (1, 7), (9, 9)])
@pytest.mark.parametrize("W", [1, 2, 3, 5, 20])
def test_window_dense_equals_scalar_brute_force(Tq, Tk, W):
    q, k, v = _rand((Tq, 2), 1), _rand((Tk, 2), 2), _rand((Tk, 2), 3)
    O, L = oracle.dense_head(q, k, v, True, window=W)
    Ob, Lb = oracle.brute_attention(q.tolist(), k.tolist(), v.tolist(), True, window=W)
    assert np.max(np.abs(O - np.array(Ob))) <= 1e-15
    assert np.max(np.abs(L - np.array(Lb))) <= 1e-14


@pytest.mark.parametrize("Tq,Tk,W", [(40, 40, 7), (25, 60, 13), (1, 50, 16), (33, 33, 1)])
def test_window_row_equals_plain_attention_over_sliced_keys(Tq, Tk, W):
    # Row i sees exactly keys max(0, p - W + 1) .. p: non-causal attention of that one query over
    # that slice is the definition with no mask at all.
    d = 8
    q, k, v = _rand((Tq, d), 4), _rand((Tk, d), 5), _rand((Tk, d), 6)
    O, L = oracle.dense_head(q, k, v, True, scale=0.3, window=W)
    off = Tk - Tq
    for i in range(Tq):
        p = i + off
        lo = max(0, p - W + 1)
        Oi, Li = oracle.dense_head(q[i:i + 1], k[lo:p + 1], v[lo:p + 1], False, scale=0.3)
        assert np.max(np.abs(O[i] - Oi[0])) <= 1e-14
        assert abs(L[i] - Li[0]) <= 1e-13


def test_window_of_one_returns_the_row_own_value():
    T, d = 12, 5
    q, k, v = _rand((T, d), 7), _rand((T, d), 8), _rand((T, d), 9)
    O, L = oracle.dense_head(q, k, v, True, scale=0.5, window=1)
    assert np.array_equal(O, v)
    assert np.allclose(L, 0.5 * np.sum(q * k, axis=1), rtol=0, atol=1e-15)


@pytest.mark.parametrize("Tq,Tk", [(30, 30), (10, 30)])
def test_window_covering_every_key_is_causal(Tq, Tk):
    q, k, v = _rand((Tq, 6), 10), _rand((Tk, 6), 11), _rand((Tk, 6), 12)
    Oc, Lc = oracle.dense_head(q, k, v, True)
    for W in (Tk, Tk + 5):
        Ow, Lw = oracle.dense_head(q, k, v, True, window=W)
        assert np.array_equal(Oc, Ow) and np.array_equal(Lc, Lw)
    # one short of covering the last row's keys changes the last row only when Tq == Tk
    Ow, _ = oracle.dense_head(q, k, v, True, window=Tk - 1)
    assert np.max(np.abs(Ow[-1] - Oc[-1])) > 1e-6


def test_decode_window_is_attention_over_the_last_w_keys():
    Tk, d, W = 57, 8, 19
    q, k, v = _rand((1, d), 13), _rand((Tk, d), 14), _rand((Tk, d), 15)
    O, L = oracle.dense_head(q, k, v, True, window=W)
    Or, Lr = oracle.dense_head(q, k[Tk - W:], v[Tk - W:], False)
    assert np.max(np.abs(O - Or)) <= 1e-15 and np.max(np.abs(L - Lr)) <= 1e-14


@pytest.mark.parametrize("block", [1, 7, 32, 128])
@pytest.mark.parametrize("W", [1, 24, 64, 1000])
def test_window_tiled_equals_dense_across_block_sizes(block, W):
    T, d = 150, 16
    q, k, v = _rand((T, d), 16), _rand((T, d), 17), _rand((T, d), 18)
    Od, Ld = oracle.dense_head(q, k, v, True, window=W)
    Ot, Lt = oracle.tiled_head(q, k, v, True, block_q=block, block_kv=block, window=W)
    assert np.max(np.abs(Ot - Od)) <= 1e-12 and np.max(np.abs(Lt - Ld)) <= 1e-12


def test_window_pages_exercise_setup():
    # Exercise 4 of "4.2 FlashAttention I": N = 100, d = 16, W = 24, 32x32 tiles, seed 7;
    # the tiled result agrees with the materialised reference to round-off.
    rng = np.random.default_rng(7)
    N, d, W = 100, 16, 24
    Q = rng.normal(size=(N, d)); K = rng.normal(size=(N, d)); V = rng.normal(size=(N, d))
    Ot, _ = oracle.tiled_head(Q, K, V, True, block_q=32, block_kv=32, window=W)
    Od, _ = oracle.dense_head(Q, K, V, True, window=W)
    assert np.max(np.abs(Ot - Od)) < 1e-13


@pytest.mark.parametrize("T,block,W", [(100, 32, 24), (256, 16, 40), (64, 8, 8), (97, 10, 3)])
def test_window_tile_skip_visits_exactly_the_band(T, block, W):
    # Count, independently, the (query block, key block) pairs holding at least one visible pair.
    expect = 0
    for i0 in range(0, T, block):
        i1 = min(i0 + block, T)
        for j0 in range(0, T, block):
            j1 = min(j0 + block, T)
            if any(j0 <= j < j1 and i - W < j <= i for i in range(i0, i1) for j in range(j0, j1)):
                expect += 1
    stats = {}
    z = np.zeros((T, 2))
    oracle.tiled_head(z, z, z, True, block_q=block, block_kv=block, stats=stats, window=W)
    assert stats["tiles_visited"] == expect


@pytest.mark.parametrize("Tq,Tk,W", [(64, 64, 10), (20, 64, 33)])
def test_window_against_torch_sdpa_fp64_with_explicit_mask(Tq, Tk, W):
    torch = pytest.importorskip("torch")
    B, H, d = 2, 3, 16
    rng = np.random.default_rng(21)
    Q, K, V = (rng.standard_normal((B, H, T, d)) for T in (Tq, Tk, Tk))
    O, L = oracle.dense_attention(Q, K, V, True, window=W)
    pos = np.arange(Tq)[:, None] + (Tk - Tq)
    cols = np.arange(Tk)[None, :]
    keep = torch.from_numpy((cols <= pos) & (cols > pos - W))
    tq, tk, tv = (torch.from_numpy(x) for x in (Q, K, V))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=keep)
    s = (tq @ tk.transpose(-1, -2)) / np.sqrt(d)
    lse = torch.logsumexp(s.masked_fill(~keep, float("-inf")), dim=-1)
    assert np.max(np.abs(O - ref.numpy())) <= 1e-12
    assert np.max(np.abs(L - lse.numpy())) <= 1e-12


def test_window_argument_checks():
    z = np.zeros((3, 2))
    with pytest.raises(ValueError):
        oracle.dense_head(z, z, z, False, window=2)
    with pytest.raises(ValueError):
        oracle.dense_head(z, z, z, True, window=0)


def test_visible_pairs_with_window_brute_force():
    for Tq, Tk, W in [(10, 10, 3), (4, 9, 5), (1, 8, 2), (7, 7, 100)]:
        off = Tk - Tq
        n = sum(1 for i in range(Tq) for j in range(Tk) if i + off - W < j <= i + off)
        assert accounting.visible_pairs(Tq, Tk, True, W) == n


def test_rolling_window_cache_sizes_printed_on_the_pages():
    with open(os.path.join(GOLDEN, "window_cache_exercise.json")) as f:
        g = json.load(f)
    per_token = accounting.window_cache_bytes(g["layers"], g["kv_heads"], g["head_dim"], 1,
                                              g["dtype_bytes"])
    assert per_token == g["printed"]["bytes_per_token"]
    assert accounting.window_cache_bytes(g["layers"], g["kv_heads"], g["head_dim"], g["window"],
                                         g["dtype_bytes"]) == g["printed"]["cache_bytes_per_sequence"]
