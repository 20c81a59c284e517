"""Pins of the packed variable-length oracle (CPU only)."""

import numpy as np
import pytest

import oracle
from tests import inputs
from tests.inputs import AttnConfig


def _cfg(Hq=4, Hkv=2, d=8, seed=3):
    return AttnConfig("varlen pin", B=1, Hq=Hq, Hkv=Hkv, Tq=1, Tk=1, d=d, dtype="f32",
                      causal=True, dist="normal", seed=seed)


def test_one_document_is_plain_attention():
    cfg = _cfg()
    Q, K, V, cq, ck = inputs.make_packed(cfg, [37])
    for causal in (False, True):
        O, L = oracle.varlen_attention(Q, K, V, cq, ck, causal, 0.4)
        o, l = oracle.dense_attention(Q.transpose(1, 0, 2)[None], K.transpose(1, 0, 2)[None],
                                      V.transpose(1, 0, 2)[None], causal, 0.4)
        assert np.max(np.abs(O - o[0].transpose(1, 0, 2))) <= 1e-13
        assert np.max(np.abs(L - l[0])) <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_packed_equals_block_diagonal_mask_in_torch(causal):
    # An independent route: the whole packed sequence through float64 torch SDPA with a
    # block-diagonal (and, if causal, per-document bottom-right triangular) boolean mask.
    torch = pytest.importorskip("torch")
    cfg = _cfg(Hq=4, Hkv=4)
    lq, lk = [5, 1, 12, 7], [5, 3, 12, 9]
    if causal:
        lq, lk = [5, 1, 12, 7], [5, 1, 15, 9]
    Q, K, V, cq, ck = inputs.make_packed(cfg, lq, lk)
    O, L = oracle.varlen_attention(Q, K, V, cq, ck, causal, 0.6)
    tq, tk = int(cq[-1]), int(ck[-1])
    allow = np.zeros((tq, tk), bool)
    for b in range(len(lq)):
        for i in range(lq[b]):
            for j in range(lk[b]):
                if not causal or j <= i + lk[b] - lq[b]:
                    allow[cq[b] + i, ck[b] + j] = True
    q = torch.tensor(Q.transpose(1, 0, 2), dtype=torch.float64)
    k = torch.tensor(K.transpose(1, 0, 2), dtype=torch.float64)
    v = torch.tensor(V.transpose(1, 0, 2), dtype=torch.float64)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=torch.from_numpy(allow),
                                                         scale=0.6)
    s = (q @ k.transpose(1, 2)) * 0.6
    lse = torch.logsumexp(s.masked_fill(~torch.from_numpy(allow), float("-inf")), dim=-1)
    assert np.max(np.abs(O - o.numpy().transpose(1, 0, 2))) <= 1e-12
    assert np.max(np.abs(L - lse.numpy())) <= 1e-12


def test_documents_do_not_see_each_other():
    cfg = _cfg()
    Q, K, V, cq, ck = inputs.make_packed(cfg, [9, 14, 6])
    O, L = oracle.varlen_attention(Q, K, V, cq, ck, True)
    K2, V2 = K.copy(), V.copy()
    K2[ck[1]:ck[2]] += 3.0
    V2[ck[1]:ck[2]] -= 1.0
    O2, L2 = oracle.varlen_attention(Q, K2, V2, cq, ck, True)
    for b in (0, 2):
        assert np.array_equal(O[cq[b]:cq[b + 1]], O2[cq[b]:cq[b + 1]])
        assert np.array_equal(L[:, cq[b]:cq[b + 1]], L2[:, cq[b]:cq[b + 1]])
    assert not np.array_equal(O[cq[1]:cq[2]], O2[cq[1]:cq[2]])


def test_rows_without_keys_and_window():
    cfg = _cfg(Hq=2, Hkv=1)
    # document 0 causal with 6 queries and 4 keys: its first two rows see nothing;
    # document 1 has no keys at all
    Q, K, V, cq, ck = inputs.make_packed(cfg, [6, 3, 4], [4, 0, 4])
    O, L = oracle.varlen_attention(Q, K, V, cq, ck, True)
    assert not O[0:2].any() and np.all(np.isneginf(L[:, 0:2]))
    assert not O[6:9].any() and np.all(np.isneginf(L[:, 6:9]))
    assert np.all(np.isfinite(L[:, 2:6])) and np.all(np.isfinite(L[:, 9:]))
    # row 2 of document 0 sits at position 0: it returns v_0
    assert np.allclose(O[2, 0], V[0, 0], rtol=0, atol=0)
    # a window of 1 returns each row's own value
    Q, K, V, cq, ck = inputs.make_packed(cfg, [5, 7])
    O, _ = oracle.varlen_attention(Q, K, V, cq, ck, True, window=1)
    assert np.array_equal(O[:, 0], V[:, 0].astype(np.float64))


def _packed_grad(cfg, cq):
    rng = np.random.default_rng(cfg.seed + 100)
    return rng.standard_normal((int(cq[-1]), cfg.Hq, cfg.d))


@pytest.mark.parametrize("causal,window", [(False, None), (True, None), (True, 4)])
def test_packed_backward_equals_dense_per_document(causal, window):
    cfg = _cfg(Hq=4, Hkv=2, d=6)
    lq, lk = [9, 1, 14], ([9, 1, 14] if causal else [12, 3, 5])
    Q, K, V, cq, ck = inputs.make_packed(cfg, lq, lk)
    dO = _packed_grad(cfg, cq)
    O, L = oracle.varlen_attention(Q, K, V, cq, ck, causal, 0.5, window)
    dQ, dK, dV = oracle.varlen_backward(Q, K, V, O, L, dO, cq, ck, causal, 0.5, window)
    for b in range(3):
        q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
        tr = lambda x, a, c: np.asarray(x[a:c]).transpose(1, 0, 2)[None]
        rq, rk, rv = oracle.dense_backward(tr(Q, q0, q1), tr(K, k0, k1), tr(V, k0, k1),
                                           tr(dO, q0, q1), causal, 0.5, window)
        assert np.max(np.abs(dQ[q0:q1] - rq[0].transpose(1, 0, 2))) <= 1e-12
        assert np.max(np.abs(dK[k0:k1] - rk[0].transpose(1, 0, 2))) <= 1e-12
        assert np.max(np.abs(dV[k0:k1] - rv[0].transpose(1, 0, 2))) <= 1e-12


def test_packed_backward_against_finite_differences():
    # central differences of sum(dO * O) over the whole packed output
    cfg = _cfg(Hq=2, Hkv=1, d=3)
    Q, K, V, cq, ck = inputs.make_packed(cfg, [6, 2, 5], [8, 2, 5])
    Q, K, V = (x.astype(np.float64) for x in (Q, K, V))
    dO = _packed_grad(cfg, cq)
    O, L = oracle.varlen_attention(Q, K, V, cq, ck, True, 0.7)
    dQ, dK, dV = oracle.varlen_backward(Q, K, V, O, L, dO, cq, ck, True, 0.7)
    eps = 1e-5
    for x, g, idx in ((Q, dQ, (3, 1, 2)), (Q, dQ, (7, 0, 0)), (K, dK, (1, 0, 1)),
                      (K, dK, (12, 0, 2)), (V, dV, (0, 0, 0)), (V, dV, (9, 0, 1))):
        keep = x[idx]
        x[idx] = keep + eps
        fp = np.sum(dO * oracle.varlen_attention(Q, K, V, cq, ck, True, 0.7)[0])
        x[idx] = keep - eps
        fm = np.sum(dO * oracle.varlen_attention(Q, K, V, cq, ck, True, 0.7)[0])
        x[idx] = keep
        assert abs((fp - fm) / (2 * eps) - g[idx]) < 1e-7, idx


def test_packed_backward_rows_without_keys():
    cfg = _cfg(Hq=2, Hkv=1, d=4)
    Q, K, V, cq, ck = inputs.make_packed(cfg, [6, 3], [4, 0])
    dO = _packed_grad(cfg, cq)
    O, L = oracle.varlen_attention(Q, K, V, cq, ck, True)
    dQ, dK, dV = oracle.varlen_backward(Q, K, V, O, L, dO, cq, ck, True)
    assert not dQ[0:2].any() and not dQ[6:9].any() and dQ[2:6].any()
    assert np.all(np.isfinite(dK)) and np.all(np.isfinite(dV))
