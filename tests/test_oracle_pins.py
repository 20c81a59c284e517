"""Pins of the CPU oracle to facts outside itself (CPU only).

Each test ties an oracle function to a value the pages print, a closed form, an invariant, a
library routine or brute force, so that a dropped term, a wrong sign or index, or a transposed
operand in the oracle fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from tests.inputs import lab_qkv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------- brute force on the toy size

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_dense_equals_scalar_brute_force_t4_d2(causal, seed):
    # T = 4, d = 2 is the toy size of "Efficient attention & KV cache", section 1.
    q, k, v = _rand((4, 2), seed), _rand((4, 2), seed + 10), _rand((4, 2), seed + 20)
    O, L = oracle.dense_head(q, k, v, causal)
    Ob, Lb = oracle.brute_attention(q.tolist(), k.tolist(), v.tolist(), causal)
    assert np.max(np.abs(O - np.array(Ob))) <= 1e-15
    assert np.max(np.abs(L - np.array(Lb))) <= 1e-15


@pytest.mark.parametrize("Tq,Tk", [(1, 5), (3, 5), (5, 5)])
def test_dense_equals_brute_force_rectangular_bottom_right(Tq, Tk):
    q, k, v = _rand((Tq, 3), 5), _rand((Tk, 3), 6), _rand((Tk, 3), 7)
    O, L = oracle.dense_head(q, k, v, True, scale=0.7)
    Ob, Lb = oracle.brute_attention(q.tolist(), k.tolist(), v.tolist(), True, scale=0.7)
    assert np.max(np.abs(O - np.array(Ob))) <= 1e-15
    assert np.max(np.abs(L - np.array(Lb))) <= 1e-14


# ---------------------------------------------------------------- the lab's recorded example

def test_lab_recorded_example_values():
    g = _golden("lab_recorded_result.json")
    gen = g["generator"]
    q, k, v = lab_qkv(gen["seq_len"], gen["head_dim"], gen["seed"])
    Od, _, P = oracle.dense_head(q, k, v, True, return_p=True)
    stats = {}
    Ot, _ = oracle.tiled_head(q, k, v, True, block_q=g["block_q"], block_kv=g["block_kv"],
                              stats=stats)
    half_ulp = 0.5 * 10 ** -g["printed_decimals"]
    for O in (Od, Ot):
        assert np.max(np.abs(O[0, :4] - g["sample_row0_first4"])) <= half_ulp + 1e-12
        assert np.max(np.abs(O[-1, :4] - g["sample_last_row_first4"])) <= half_ulp + 1e-12
    # the page's dense/tiled difference is 1.388e-16; ours must be of the same (round-off) order
    assert np.max(np.abs(Od - Ot)) < 1e-12
    # retained elements: every visible score plus its probability
    visible = int(np.count_nonzero(P))
    assert 2 * visible == g["standard_materialized_elements"]
    assert stats["tiles_visited"] == g["flash_tiles_visited"]
    assert g["block_q"] * g["block_kv"] == g["flash_sram_tile_elements"]


def test_lab_tile_sweep_matches_dense():
    g = _golden("lab_checks.json")["tile_sweep"]
    q, k, v = lab_qkv(g["seq_len"], g["head_dim"], g["seed"])
    Od, Ld = oracle.dense_head(q, k, v, g["causal"])
    for bq, bkv in g["blocks"]:
        Ot, Lt = oracle.tiled_head(q, k, v, g["causal"], block_q=bq, block_kv=bkv)
        assert np.max(np.abs(Od - Ot)) < g["max_abs_diff_below"]
        assert np.max(np.abs(Ld - Lt)) < g["max_abs_diff_below"]


def test_lab_overflow_case():
    g = _golden("lab_checks.json")["overflow"]
    q, k, v = g["q"], g["k"], g["v"]
    with pytest.raises(OverflowError):
        oracle.brute_attention(q, k, v, g["causal"], subtract_max=False)
    Od, Ld = oracle.dense_head(q, k, v, g["causal"])
    Ot, Lt = oracle.tiled_head(q, k, v, g["causal"], block_q=g["block_q"], block_kv=g["block_kv"])
    assert np.max(np.abs(Od - Ot)) < g["max_abs_diff_below"]
    # closed form: scores 1000/sqrt2 and 2000/sqrt2, so the weight of key 0 is exp(-1000/sqrt2)
    gap = 1000.0 / math.sqrt(2.0)
    w0 = math.exp(-gap) / (1.0 + math.exp(-gap))
    for O, L in ((Od, Ld), (Ot, Lt)):
        assert O[:, 0] == pytest.approx([w0, w0], rel=1e-12)
        assert O[:, 1] == pytest.approx([1.0, 1.0], abs=1e-300)
        assert L == pytest.approx([2000.0 / math.sqrt(2.0)] * 2, rel=1e-15)


def test_lab_mutation_is_caught():
    g = _golden("lab_checks.json")["mutation"]
    q, k, v = lab_qkv(g["seq_len"], g["head_dim"], g["seed"])
    k[-1] = g["last_key_value"]
    Od, _ = oracle.dense_head(q, k, v, g["causal"])
    good, _ = oracle.tiled_head(q, k, v, g["causal"], block_q=g["block_q"], block_kv=g["block_kv"])
    bad, _ = oracle.tiled_head(q, k, v, g["causal"], block_q=g["block_q"], block_kv=g["block_kv"],
                               rescale=False)
    assert np.max(np.abs(Od - good)) < g["correct_below"]
    assert np.max(np.abs(Od - bad)) > g["faulty_above"]


# ---------------------------------------------------------------- 1-D recurrence

def test_online_softmax_exercise_hand_trace():
    g = _golden("online_softmax_exercise.json")
    h = g["hand_trace_from_printed_constants"]
    tol = g["tolerance"]
    tr = oracle.online_logsumexp_trace(g["x"], g["block_size"])
    assert tr[0][0] == h["after_block_1"]["m"]
    assert abs(tr[0][2] - h["after_block_1"]["l"]) < tol
    assert abs(tr[1][1] - h["block_2_alpha"]["value"]) < tol
    assert tr[1][0] == h["after_block_2"]["m"]
    assert abs(tr[1][2] - h["after_block_2"]["l"]) < tol
    assert abs(tr[1][2] - h["two_pass_l"]["value"]) < tol
    assert abs(tr[1][0] + math.log(tr[1][2]) - h["logsumexp"]["value"]) < tol


def test_online_weighted_sum_against_library_softmax():
    from scipy.special import softmax

    # the chapter's own check: N = 37, d = 8, logits N(0, 5), blocks of 4
    rng = np.random.default_rng(0)
    x = rng.normal(0, 5, size=37)
    V = rng.normal(0, 1, size=(37, 8))
    ref = softmax(x) @ V
    for bs in (1, 4, 5, 37, 64):
        assert np.max(np.abs(oracle.stream_weighted_sum(x, V, bs) - ref)) < 1e-14


@pytest.mark.parametrize("chunk", [1, 3, 16, 100])
def test_online_softmax_against_torch_softmax(chunk):
    import torch

    x = np.random.default_rng(3).normal(0, 20, size=100)   # scores scaled up to stress the max
    ref = torch.softmax(torch.from_numpy(x), dim=0).numpy()
    assert np.max(np.abs(oracle.stream_softmax(x, chunk) - ref)) < 1e-15


# ---------------------------------------------------------------- closed forms and invariants

def test_rows_of_p_sum_to_one():
    q, k, v = _rand((50, 16), 1), _rand((70, 16), 2), _rand((70, 16), 3)
    for causal in (False, True):
        _, _, P = oracle.dense_head(q, k, v, causal, return_p=True)
        assert np.max(np.abs(P.sum(axis=1) - 1.0)) <= 1e-14


def test_reconstruction_from_lse_is_normalised():
    # exercise 5 of "4.2 FlashAttention I": P_ij = exp(S_ij - L_i) sums to one over visible keys
    q, k, v = _rand((40, 8), 4), _rand((40, 8), 5), _rand((40, 8), 6)
    sc = 1 / math.sqrt(8)
    _, L = oracle.dense_head(q, k, v, True)
    S = sc * q @ k.T
    S[np.triu_indices(40, 1)] = -np.inf
    assert np.max(np.abs(np.exp(S - L[:, None]).sum(axis=1) - 1.0)) <= 1e-14


def test_causal_row_zero_is_first_value():
    q, k, v = _rand((30, 8), 7), _rand((30, 8), 8), _rand((30, 8), 9)
    O, L = oracle.dense_head(q, k, v, True)
    assert np.array_equal(O[0], v[0])
    assert L[0] == pytest.approx((q[0] @ k[0]) / math.sqrt(8), rel=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_give_prefix_means(causal):
    T = 25
    k, v = _rand((T, 8), 10), _rand((T, 8), 11)
    q = np.zeros((T, 8))
    O, L = oracle.dense_head(q, k, v, causal)
    if causal:
        counts = np.arange(1, T + 1)
        expect = np.cumsum(v, axis=0) / counts[:, None]
        expect_l = np.log(counts)
    else:
        expect = np.broadcast_to(v.mean(axis=0), v.shape)
        expect_l = np.full(T, math.log(T))
    assert np.max(np.abs(O - expect)) <= 1e-15
    assert np.max(np.abs(L - expect_l)) <= 1e-15
    # a zero scale is the same computation as zero queries
    O0, L0 = oracle.dense_head(_rand((T, 8), 12), k, v, causal, scale=0.0)
    assert np.max(np.abs(O0 - expect)) <= 1e-15
    assert np.max(np.abs(L0 - expect_l)) <= 1e-15


def test_single_key():
    q, k, v = _rand((1, 16), 13), _rand((1, 16), 14), _rand((1, 16), 15)
    for causal in (False, True):
        O, L = oracle.dense_head(q, k, v, causal)
        assert np.array_equal(O[0], v[0])
        assert L[0] == pytest.approx((q[0] @ k[0]) / 4.0, rel=1e-15)


def test_key_shift_invariance():
    q, k, v = _rand((20, 8), 16), _rand((33, 8), 17), _rand((33, 8), 18)
    w = _rand((8,), 19)
    sc = 0.3
    for causal in (False, True):
        O, L = oracle.dense_head(q, k, v, causal, scale=sc)
        O2, L2 = oracle.dense_head(q, k + w, v, causal, scale=sc)
        assert np.max(np.abs(O - O2)) <= 1e-12
        assert np.max(np.abs(L2 - (L + sc * q @ w))) <= 1e-12


def test_key_permutation_invariance_noncausal():
    q, k, v = _rand((20, 8), 20), _rand((33, 8), 21, 4.0), _rand((33, 8), 22)
    perm = np.random.default_rng(23).permutation(33)
    O, L = oracle.dense_head(q, k, v, False)
    O2, L2 = oracle.dense_head(q, k[perm], v[perm], False)
    assert np.max(np.abs(O - O2)) <= 1e-12
    assert np.max(np.abs(L - L2)) <= 1e-12
    Ot, Lt = oracle.tiled_head(q, k[perm], v[perm], False, block_q=7, block_kv=5)
    assert np.max(np.abs(O - Ot)) <= 1e-12
    assert np.max(np.abs(L - Lt)) <= 1e-12


def test_gqa_equals_mha_on_repeated_kv():
    B, Hq, Hkv, T, d = 2, 8, 2, 19, 8
    Q, K, V = _rand((B, Hq, T, d), 24), _rand((B, Hkv, T, d), 25), _rand((B, Hkv, T, d), 26)
    O, L = oracle.dense_attention(Q, K, V, True)
    Kr, Vr = np.repeat(K, Hq // Hkv, axis=1), np.repeat(V, Hq // Hkv, axis=1)
    Om, Lm = oracle.dense_attention(Q, Kr, Vr, True)
    assert np.array_equal(O, Om) and np.array_equal(L, Lm)


def test_causal_single_query_equals_noncausal():
    q, k, v = _rand((1, 16), 27), _rand((40, 16), 28), _rand((40, 16), 29)
    Oc, Lc = oracle.dense_head(q, k, v, True)
    On, Ln = oracle.dense_head(q, k, v, False)
    assert np.array_equal(Oc, On) and np.array_equal(Lc, Ln)


def test_rows_subset_equals_full():
    q, k, v = _rand((45, 8), 30), _rand((60, 8), 31), _rand((60, 8), 32)
    rows = [0, 3, 17, 44]
    for causal in (False, True):
        O, L = oracle.dense_head(q, k, v, causal)
        Os, Ls = oracle.dense_head(q, k, v, causal, rows=rows)
        assert np.array_equal(O[rows], Os) and np.array_equal(L[rows], Ls)


# ---------------------------------------------------------------- library special case

def _torch_reference(Q, K, V, causal, scale):
    import torch
    import torch.nn.functional as F

    Qt, Kt, Vt = (torch.from_numpy(x) for x in (Q, K, V))
    Tq, Tk = Q.shape[-2], K.shape[-2]
    gqa = Q.shape[1] != K.shape[1]
    # torch's is_causal is aligned top-left; build the bottom-right mask explicitly
    mask = None
    if causal:
        mask = torch.ones(Tq, Tk, dtype=torch.bool).tril(diagonal=Tk - Tq)
    O = F.scaled_dot_product_attention(Qt, Kt, Vt, attn_mask=mask, scale=scale, enable_gqa=gqa)
    Kr = Kt.repeat_interleave(Q.shape[1] // K.shape[1], dim=1)
    S = scale * (Qt @ Kr.transpose(-2, -1))
    if causal:
        S = S.masked_fill(~mask, float("-inf"))
    return O.numpy(), torch.logsumexp(S, dim=-1).numpy()


@pytest.mark.parametrize("shape", [(2, 4, 4, 37, 37, 16), (1, 8, 2, 5, 41, 32), (2, 6, 3, 64, 64, 8)])
@pytest.mark.parametrize("causal", [False, True])
def test_dense_against_torch_sdpa_fp64(shape, causal):
    B, Hq, Hkv, Tq, Tk, d = shape
    Q, K, V = _rand((B, Hq, Tq, d), 33), _rand((B, Hkv, Tk, d), 34), _rand((B, Hkv, Tk, d), 35)
    sc = 1 / math.sqrt(d)
    O, L = oracle.dense_attention(Q, K, V, causal, sc)
    Or, Lr = _torch_reference(Q, K, V, causal, sc)
    assert np.max(np.abs(O - Or)) <= 1e-12
    assert np.max(np.abs(L - Lr)) <= 1e-12


# ---------------------------------------------------------------- tiled path == definition

@pytest.mark.parametrize("block", [1, 7, 32, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_tiled_equals_dense_across_block_sizes(block, causal):
    T, d = 300, 64
    q, k, v = _rand((T, d), 36), _rand((T, d), 37), _rand((T, d), 38)
    Od, Ld = oracle.dense_head(q, k, v, causal)
    for bq, bkv in ((block, block), (block, 32), (32, block)):
        Ot, Lt = oracle.tiled_head(q, k, v, causal, block_q=bq, block_kv=bkv)
        assert np.max(np.abs(Od - Ot)) <= 1e-12
        assert np.max(np.abs(Ld - Lt)) <= 1e-12


@pytest.mark.parametrize("Tq,Tk", [(1, 300), (13, 300), (300, 300), (64, 65)])
def test_tiled_equals_dense_rectangular_and_gqa(Tq, Tk):
    B, Hq, Hkv, d = 1, 4, 2, 16
    Q, K, V = _rand((B, Hq, Tq, d), 39), _rand((B, Hkv, Tk, d), 40, 3.0), _rand((B, Hkv, Tk, d), 41)
    for causal in (False, True):
        Od, Ld = oracle.dense_attention(Q, K, V, causal)
        Ot, Lt = oracle.tiled_attention(Q, K, V, causal, block_q=7, block_kv=19)
        assert np.max(np.abs(Od - Ot)) <= 1e-12
        assert np.max(np.abs(Ld - Lt)) <= 1e-12


def test_tiled_causal_visits_lower_triangle_of_tiles():
    # square causal with equal blocks visits n(n+1)/2 tiles (4 blocks -> 10, as the lab records)
    for T, b in ((64, 16), (100, 32), (33, 8)):
        stats = {}
        z = np.zeros((T, 4))
        oracle.tiled_head(z, z, z, True, block_q=b, block_kv=b, stats=stats)
        n = -(-T // b)
        assert stats["tiles_visited"] == n * (n + 1) // 2


def test_large_logit_spikes_need_the_rescale():
    # "Forgetting the rescale" in "Efficient attention & KV cache", section 4: scores scaled up
    q, k, v = _rand((64, 16), 42, 5.0), _rand((64, 16), 43, 5.0), _rand((64, 16), 44)
    Od, _ = oracle.dense_head(q, k, v, True)
    good, _ = oracle.tiled_head(q, k, v, True, block_q=16, block_kv=16)
    bad, _ = oracle.tiled_head(q, k, v, True, block_q=16, block_kv=16, rescale=False)
    assert np.max(np.abs(Od - good)) <= 1e-12
    assert np.max(np.abs(Od - bad)) > 0.1


# ---------------------------------------------------------------- split merge (decode combine)

def test_merge_of_key_splits_equals_whole():
    q, k, v = _rand((3, 16), 45), _rand((100, 16), 46), _rand((100, 16), 47)
    Od, Ld = oracle.dense_head(q, k, v, False)
    for cuts in ([0, 100], [0, 50, 100], [0, 1, 37, 38, 99, 100]):
        parts = [oracle.dense_head(q, k[a:b], v[a:b], False) for a, b in zip(cuts[:-1], cuts[1:])]
        Om, Lm = oracle.merge_partials(np.stack([p[0] for p in parts]),
                                       np.stack([p[1] for p in parts]))
        assert np.max(np.abs(Od - Om)) <= 1e-14
        assert np.max(np.abs(Ld - Lm)) <= 1e-13


def test_merge_ignores_empty_parts():
    o = np.stack([np.ones((2, 4)), np.zeros((2, 4))])
    lse = np.array([[0.5, -1.0], [-np.inf, -np.inf]])
    Om, Lm = oracle.merge_partials(o, lse)
    assert np.array_equal(Om, np.ones((2, 4)))
    assert np.array_equal(Lm, lse[0])
