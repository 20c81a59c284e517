"""Pins of the paged-decode oracle (CPU only): gathering through a block table reproduces the
contiguous cache, so paged decode equals the dense definition on the original keys."""

import numpy as np
import pytest

import oracle
from tests import inputs
from tests.inputs import AttnConfig


def _cfg(B=3, Hq=8, Hkv=2, Tk=70, d=16, seed=4):
    return AttnConfig("paged pin", B=B, Hq=Hq, Hkv=Hkv, Tq=1, Tk=Tk, d=d, dtype="f32",
                      causal=False, dist="normal", seed=seed)


@pytest.mark.parametrize("bs", [16, 32, 128])
def test_gather_reproduces_the_contiguous_cache(bs):
    cfg = _cfg()
    _, K, V = inputs.make_inputs(cfg)
    lens = [70, 1, 33]
    Kc, Vc, table, sl = inputs.make_paged(cfg, bs, lens)
    for b, n in enumerate(lens):
        for g in range(cfg.Hkv):
            k, v = oracle.gather_sequence(Kc, Vc, table[b], n, g)
            assert np.array_equal(k, K[b, g, :n]) and np.array_equal(v, V[b, g, :n])


@pytest.mark.parametrize("bs", [16, 64])
def test_paged_decode_equals_dense_on_the_contiguous_cache(bs):
    cfg = _cfg()
    Q, K, V = inputs.make_inputs(cfg)
    lens = [70, 5, 48]
    Kc, Vc, table, sl = inputs.make_paged(cfg, bs, lens)
    O, L = oracle.paged_decode(Q[:, :, 0], Kc, Vc, table, sl, 0.3)
    for b, n in enumerate(lens):
        o, l = oracle.dense_attention(Q[b:b + 1], K[b:b + 1, :, :n], V[b:b + 1, :, :n], False, 0.3)
        assert np.max(np.abs(O[b] - o[0, :, 0])) <= 1e-13
        assert np.max(np.abs(L[b] - l[0, :, 0])) <= 1e-13


def test_one_position_returns_its_value_and_brute_force():
    cfg = _cfg(B=2, Hq=2, Hkv=1, Tk=20, d=2)
    Q, K, V = inputs.make_inputs(cfg)
    Kc, Vc, table, sl = inputs.make_paged(cfg, 16, [1, 20])
    O, L = oracle.paged_decode(Q[:, :, 0], Kc, Vc, table, sl)
    # one visible position: the output is its value, LSE its scaled score
    assert np.allclose(O[0], V[0, 0, 0], atol=0, rtol=0)
    assert np.allclose(L[0], Q[0, :, 0] @ K[0, 0, 0] / np.sqrt(2), atol=1e-12)
    # brute force (scalar loops) on the second sequence
    bq = oracle.brute_attention(Q[1, 0], K[1, 0], V[1, 0], False)
    assert np.max(np.abs(np.asarray(bq[0])[0] - O[1, 0])) <= 1e-12


def test_empty_sequence_convention():
    cfg = _cfg(B=2, Hq=2, Hkv=1, Tk=20, d=4)
    Q, _, _ = inputs.make_inputs(cfg)
    Kc, Vc, table, sl = inputs.make_paged(cfg, 16, [0, 20])
    O, L = oracle.paged_decode(Q[:, :, 0], Kc, Vc, table, sl)
    assert not O[0].any() and np.all(np.isneginf(L[0]))
    assert np.all(np.isfinite(L[1]))
