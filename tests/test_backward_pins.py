"""Pins of the backward oracle (CPU only): finite differences, torch float64 autograd, the
pages' tiled backward, closed forms and invariants of the gradients."""

import numpy as np
import pytest

import oracle


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def test_pages_gradient_check():
    # "4.2 FlashAttention I", section "The backward pass": seed 2, N = 48, d = 8, causal,
    # 16 x 16 tiles; central differences of sum(dO * O) agree to about 1e-7.
    rng = np.random.default_rng(2)
    N, d = 48, 8
    Q = rng.normal(size=(N, d)); K = rng.normal(size=(N, d)); V = rng.normal(size=(N, d))
    O, L = oracle.tiled_head(Q, K, V, True, block_q=16, block_kv=16)
    dO = rng.normal(size=(N, d))
    dQ, dK, dV = oracle.tiled_backward_head(Q, K, V, O, L, dO, True, block_q=16, block_kv=16)
    err = max(abs(oracle.loss_gradient_fd(Q, K, V, dO, True, "q", (3, 2)) - dQ[3, 2]),
              abs(oracle.loss_gradient_fd(Q, K, V, dO, True, "k", (5, 1)) - dK[5, 1]),
              abs(oracle.loss_gradient_fd(Q, K, V, dO, True, "v", (7, 4)) - dV[7, 4]))
    assert err < 1e-6


@pytest.mark.parametrize("causal,window", [(False, None), (True, None), (True, 5)])
@pytest.mark.parametrize("Tq,Tk", [(12, 12), (7, 15)])
def test_dense_backward_against_finite_differences(causal, window, Tq, Tk):
    if causal and Tq > Tk:
        pytest.skip("causal needs Tq <= Tk")
    d = 6
    q, k, v, do = _rand((Tq, d), 1), _rand((Tk, d), 2), _rand((Tk, d), 3), _rand((Tq, d), 4)
    dQ, dK, dV, *_ = oracle.dense_backward_head(q, k, v, do, causal, 0.6, window)
    rng = np.random.default_rng(5)
    for which, g, shape in (("q", dQ, (Tq, d)), ("k", dK, (Tk, d)), ("v", dV, (Tk, d))):
        for _ in range(6):
            idx = (int(rng.integers(shape[0])), int(rng.integers(shape[1])))
            fd = oracle.loss_gradient_fd(q, k, v, do, causal, which, idx, 0.6, window=window)
            assert abs(fd - g[idx]) < 1e-7, (which, idx)


@pytest.mark.parametrize("causal", [False, True])
def test_dense_backward_against_torch_autograd_fp64(causal):
    torch = pytest.importorskip("torch")
    B, Hq, Hkv, Tq, Tk, d = 2, 4, 2, 20, 33, 8
    rng = np.random.default_rng(6)
    Q = rng.standard_normal((B, Hq, Tq, d)); K = rng.standard_normal((B, Hkv, Tk, d))
    V = rng.standard_normal((B, Hkv, Tk, d)); dO = rng.standard_normal((B, Hq, Tq, d))
    dQ, dK, dV = oracle.dense_backward(Q, K, V, dO, causal, 0.35)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
    mask = None
    if causal:  # torch's is_causal is top-left; pass the bottom-right mask explicitly
        pos = np.arange(Tq)[:, None] + (Tk - Tq)
        mask = torch.from_numpy(np.arange(Tk)[None, :] <= pos)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.35,
                                                         enable_gqa=True)
    o.backward(torch.from_numpy(dO))
    for mine, t in ((dQ, tq), (dK, tk), (dV, tv)):
        assert np.max(np.abs(mine - t.grad.numpy())) <= 1e-12


@pytest.mark.parametrize("block", [1, 7, 16, 64])
@pytest.mark.parametrize("causal,window", [(False, None), (True, None), (True, 9)])
def test_tiled_backward_equals_dense(block, causal, window):
    T, d = 70, 8
    q, k, v, do = _rand((T, d), 7), _rand((T, d), 8), _rand((T, d), 9), _rand((T, d), 10)
    dQ, dK, dV, O, L, _ = oracle.dense_backward_head(q, k, v, do, causal, None, window)
    tQ, tK, tV = oracle.tiled_backward_head(q, k, v, O, L, do, causal, None, block, block, window)
    for a, b in ((dQ, tQ), (dK, tK), (dV, tV)):
        assert np.max(np.abs(a - b)) <= 1e-12


def test_d_is_the_row_sum_of_p_times_dp():
    Tq, Tk, d = 9, 13, 5
    q, k, v, do = _rand((Tq, d), 11), _rand((Tk, d), 12), _rand((Tk, d), 13), _rand((Tq, d), 14)
    _, _, _, _, _, D = oracle.dense_backward_head(q, k, v, do, True)
    _, _, P = oracle.dense_head(q, k, v, True, return_p=True)
    assert np.max(np.abs(D - np.sum(P * (do @ v.T), axis=1))) <= 1e-13


def test_single_key_closed_forms():
    # one key: P = 1 whatever the scores, so dQ = dK = 0 and dV = sum of the dO rows
    q, k, v, do = _rand((5, 4), 15), _rand((1, 4), 16), _rand((1, 4), 17), _rand((5, 4), 18)
    dQ, dK, dV, *_ = oracle.dense_backward_head(q, k, v, do, False)
    assert np.max(np.abs(dQ)) <= 1e-15 and np.max(np.abs(dK)) <= 1e-15
    assert np.max(np.abs(dV[0] - do.sum(axis=0))) <= 1e-14
    # causal row 0 sees one key: its dQ row is 0
    q, k, v, do = _rand((6, 4), 19), _rand((6, 4), 20), _rand((6, 4), 21), _rand((6, 4), 22)
    dQ, *_ = oracle.dense_backward_head(q, k, v, do, True)
    assert np.max(np.abs(dQ[0])) <= 1e-15


@pytest.mark.parametrize("causal", [False, True])
def test_key_gradients_sum_to_zero(causal):
    # every row of dS sums to 0 (softmax is invariant to adding a constant to a row's scores),
    # so sum_j dK_j = scale * sum_i q_i * sum_j dS_ij = 0
    q, k, v, do = _rand((11, 6), 23), _rand((11, 6), 24), _rand((11, 6), 25), _rand((11, 6), 26)
    _, dK, *_ = oracle.dense_backward_head(q, k, v, do, causal)
    assert np.max(np.abs(dK.sum(axis=0))) <= 1e-13


def test_backward_flops_convention():
    assert oracle.backward_flops(1, 32, 8192, 8192, 128, True) == 10 * 32 * 8192 ** 2 * 128 / 2
    assert oracle.backward_flops(2, 4, 100, 50, 64, False) == 10 * 2 * 4 * 100 * 50 * 64


@pytest.mark.parametrize("causal,window", [(False, None), (True, None), (True, 6)])
@pytest.mark.parametrize("Tq,Tk", [(40, 40), (23, 57)])
def test_sampled_rows_and_columns_equal_dense(causal, window, Tq, Tk):
    # The sampled forms used at large sizes agree with the dense backward on every row / key.
    d = 8
    q, k, v, do = _rand((Tq, d), 21), _rand((Tk, d), 22), _rand((Tk, d), 23), _rand((Tq, d), 24)
    dQ, dK, dV, *_ = oracle.dense_backward_head(q, k, v, do, causal, 0.45, window)
    rows = list(range(Tq))
    assert np.max(np.abs(oracle.backward_rows(q, k, v, do, rows, causal, 0.45, window) - dQ)) \
        <= 1e-12
    # the second set holds late keys only, so a causal column sum starts past row 0
    for keys in ([0, 1, Tk // 3, Tk - 2, Tk - 1], [Tk - 9, Tk - 4, Tk - 1]):
        sK, sV = oracle.backward_cols(q, k, v, do, keys, causal, 0.45, window, row_chunk=7)
        assert np.max(np.abs(sK - dK[keys])) <= 1e-12
        assert np.max(np.abs(sV - dV[keys])) <= 1e-12


def test_sampled_columns_against_finite_differences():
    # An independent pin of the column form: central differences of sum(dO * O).
    Tq, Tk, d = 11, 19, 5
    q, k, v, do = _rand((Tq, d), 31), _rand((Tk, d), 32), _rand((Tk, d), 33), _rand((Tq, d), 34)
    sK, sV = oracle.backward_cols(q, k, v, do, [2, 17], True, 0.8, 9, row_chunk=4)
    for i, j in enumerate([2, 17]):
        for c in (0, 3):
            assert abs(oracle.loss_gradient_fd(q, k, v, do, True, "k", (j, c), 0.8, window=9)
                       - sK[i, c]) < 1e-7
            assert abs(oracle.loss_gradient_fd(q, k, v, do, True, "v", (j, c), 0.8, window=9)
                       - sV[i, c]) < 1e-7
    sQ = oracle.backward_rows(q, k, v, do, [0, 10], True, 0.8, 9)
    for i, r in enumerate([0, 10]):
        assert abs(oracle.loss_gradient_fd(q, k, v, do, True, "q", (r, 1), 0.8, window=9)
                   - sQ[i, 1]) < 1e-7


@pytest.mark.parametrize("causal,window", [(False, None), (True, None), (True, 4)])
def test_batched_tiled_backward_equals_dense_with_gqa(causal, window):
    B, Hq, Hkv, Tq, Tk, d = 2, 6, 2, 19, 30, 4
    rng = np.random.default_rng(41)
    Q = rng.standard_normal((B, Hq, Tq, d)); K = rng.standard_normal((B, Hkv, Tk, d))
    V = rng.standard_normal((B, Hkv, Tk, d)); dO = rng.standard_normal((B, Hq, Tq, d))
    O, L = oracle.dense_attention(Q, K, V, causal, 0.7, window=window)
    ref = oracle.dense_backward(Q, K, V, dO, causal, 0.7, window)
    got = oracle.tiled_backward(Q, K, V, O, L, dO, causal, 0.7, 8, 5, window)
    for a, b in zip(got, ref):
        assert np.max(np.abs(a - b)) <= 1e-12
