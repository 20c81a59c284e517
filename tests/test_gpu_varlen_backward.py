"""GPU parity of the packed-batch backward (attn_bwd_varlen) against the fp64 oracle.

Bounds as for the dense backward: max |G - R| <= 2e-2 * max(1, max|R|) and
sum |G - R| <= 1e-2 * sum |R| (+ 1e-6 per element), per gradient tensor. O and LSE come from the
oracle's packed forward, rounded to bf16 and fp32, and go to both sides, except in the end-to-end
case, where the GPU forward feeds the GPU backward and the oracle starts from Q, K, V and dO.
"""

import sys

import numpy as np
import pytest

import oracle
from tests import inputs
from tests.inputs import AttnConfig
from tests.test_gpu_backward import check_grad

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[varlen backward] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def fa():
    import torch

    assert torch.cuda.is_available(), "GPU parity tests need a GPU"
    import io_aware_tiled_amd as fa

    return fa


def _cfg(Hq, Hkv, d, seed=5, causal=True):
    return AttnConfig("varlen bwd", B=1, Hq=Hq, Hkv=Hkv, Tq=1, Tk=1, d=d, dtype="bf16",
                      causal=causal, dist="normal", seed=seed)


def _dev(x):
    return inputs.to_torch(x, "bf16", "cuda")


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _grad(cfg, total):
    rng = np.random.default_rng(cfg.seed + 7)
    return inputs.round_to_bf16(rng.standard_normal((total, cfg.Hq, cfg.d)).astype(np.float32))


def case(fa, cfg, lens_q, lens_k=None, window=None, scale=None):
    import torch

    sc = cfg.scale if scale is None else scale
    Q, K, V, cq, ck = inputs.make_packed(cfg, lens_q, lens_k)
    dO = _grad(cfg, int(cq[-1]))
    O, L = oracle.varlen_attention(Q, K, V, cq, ck, cfg.causal, sc, window)
    Ob, Lf = inputs.round_to_bf16(O), L.astype(np.float32)
    mq = int(max(np.diff(cq).max(initial=0), 1))
    mk = int(max(np.diff(ck).max(initial=0), 1))
    dq, dk, dv = fa.attn_bwd_varlen(_dev(Q), _dev(K), _dev(V), _dev(Ob),
                                    torch.from_numpy(np.ascontiguousarray(Lf)).cuda(), _dev(dO),
                                    torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda(), mq,
                                    mk, causal=cfg.causal, scale=sc, window=window)
    torch.cuda.synchronize()
    ref = oracle.varlen_backward(Q, K, V, Ob, Lf, dO, cq, ck, cfg.causal, sc, window)
    for n, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        check_grad(_np(g), r, f"packed lens={list(lens_q)[:6]} W={window} {n}")


MIX = [1, 2, 33, 64, 65, 257, 300, 700]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_length_mix(fa, d, causal):
    _say(f"d={d} causal={causal}")
    case(fa, _cfg(4, 2, d, seed=d, causal=causal), MIX)


def test_more_keys_than_queries(fa):
    case(fa, _cfg(4, 2, 128), [5, 100, 64, 1], [40, 300, 64, 129])


def test_more_queries_than_keys_and_empty_documents(fa):
    case(fa, _cfg(4, 2, 64), [50, 0, 70, 9, 3], [20, 10, 70, 0, 300])


@pytest.mark.parametrize("G", [1, 4, 16])
def test_gqa_groups(fa, G):
    case(fa, _cfg(2 * G, 2, 128, seed=G), [130, 7, 260])


@pytest.mark.parametrize("W", [1, 17, 200])
def test_sliding_window(fa, W):
    case(fa, _cfg(4, 2, 128, seed=W), MIX, window=W)


def test_scales(fa):
    for sc in (-0.25, 0.0, 0.6):
        case(fa, _cfg(2, 2, 64, seed=9), [100, 31, 257], scale=sc)


def test_equal_lengths_match_the_batched_backward_bitwise(fa):
    import torch

    cfg = _cfg(8, 2, 128, seed=31)
    B, T = 3, 700
    Q, K, V, cq, ck = inputs.make_packed(cfg, [T] * B)
    dO = _grad(cfg, B * T)
    q, k, v, do = _dev(Q), _dev(K), _dev(V), _dev(dO)
    cu = torch.from_numpy(cq).cuda()
    o, lse = fa.attn_fwd_varlen(q, k, v, cu, cu, T, T, causal=True)
    dq, dk, dv = fa.attn_bwd_varlen(q, k, v, o, lse, do, cu, cu, T, T, causal=True)
    bt = lambda x, H: x.view(B, T, H, 128).permute(0, 2, 1, 3).contiguous()
    dqb, dkb, dvb = fa.attn_bwd(bt(q, 8), bt(k, 2), bt(v, 2), bt(o, 8),
                                lse.view(8, B, T).permute(1, 0, 2).contiguous(), bt(do, 8),
                                causal=True)
    torch.cuda.synchronize()
    for a, b_, H in ((dq, dqb, 8), (dk, dkb, 2), (dv, dvb, 2)):
        assert torch.equal(bt(a, H).view(torch.int16), b_.view(torch.int16))


def test_end_to_end_training_batch_sampled(fa):
    # 32768 tokens in documents of U[128, 8192] tokens, H=32, d=128, causal: the GPU forward
    # feeds the GPU backward; sampled rows and keys of four documents against the oracle.
    import torch

    from tests.test_gpu_varlen import _doc_lengths

    cfg = AttnConfig("varlen bwd packed", B=1, Hq=32, Hkv=32, Tq=1, Tk=1, d=128, dtype="bf16",
                     causal=True, dist="normal", seed=77)
    lens = _doc_lengths(32768, 128, 8192, 77)
    _say(f"packed batch of {len(lens)} documents: inputs")
    Q, K, V, cq, ck = inputs.make_packed(cfg, lens)
    dO = _grad(cfg, int(cq[-1]))
    q, k, v, do = _dev(Q), _dev(K), _dev(V), _dev(dO)
    cu = torch.from_numpy(cq).cuda()
    o, lse = fa.attn_fwd_varlen(q, k, v, cu, cu, max(lens), max(lens), causal=True)
    dq, dk, dv = fa.attn_bwd_varlen(q, k, v, o, lse, do, cu, cu, max(lens), max(lens),
                                    causal=True)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t).all())
    rng = np.random.default_rng(3)
    docs = sorted({0, len(lens) - 1, int(np.argmax(lens))})
    for b in docs:
        n, q0 = lens[b], int(cq[b])
        pick = sorted({0, 1, 63, 64, n // 2, n - 1} & set(range(n))
                      | set(rng.choice(n, size=min(n, 12), replace=False).tolist()))
        for h in (0, 31):
            sl = slice(q0, q0 + n)
            _say(f"document {b} ({n} tokens), head {h}: oracle")
            rq = oracle.backward_rows(Q[sl, h], K[sl, h], V[sl, h], dO[sl, h], pick, True,
                                      cfg.scale)
            check_grad(_np(dq[[q0 + r for r in pick], h]), rq, f"doc {b} head {h} dQ")
            rk, rv = oracle.backward_cols(Q[sl, h], K[sl, h], V[sl, h], dO[sl, h], pick, True,
                                          cfg.scale)
            check_grad(_np(dk[[q0 + r for r in pick], h]), rk, f"doc {b} head {h} dK")
            check_grad(_np(dv[[q0 + r for r in pick], h]), rv, f"doc {b} head {h} dV")
