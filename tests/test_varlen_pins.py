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
