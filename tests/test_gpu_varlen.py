"""GPU parity of packed variable-length attention (attn_fwd_varlen) against the fp64 oracle.

Bounds as for every bf16 case: max abs error <= 2e-2 and mean-relative error <= 1e-2, on O and on
LSE (rows that see no key are compared exactly: O = 0, LSE = -inf).
"""

import sys

import numpy as np
import pytest

import oracle
from tests import inputs
from tests.inputs import AttnConfig
from tests.test_gpu_parity import check

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[varlen] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def fa():
    import torch

    assert torch.cuda.is_available(), "GPU parity tests need a GPU"
    import io_aware_tiled_amd as fa

    return fa


def _cfg(Hq, Hkv, d, seed=5, causal=True):
    return AttnConfig("varlen", B=1, Hq=Hq, Hkv=Hkv, Tq=1, Tk=1, d=d, dtype="bf16",
                      causal=causal, dist="normal", seed=seed)


def _dev(x):
    return inputs.to_torch(x, "bf16", "cuda")


def run_varlen(fa, Q, K, V, cq, ck, causal, scale, window=None):
    import torch

    lq, lk = np.diff(cq), np.diff(ck)
    o, l = fa.attn_fwd_varlen(_dev(Q), _dev(K), _dev(V), torch.from_numpy(cq).cuda(),
                              torch.from_numpy(ck).cuda(), int(max(lq.max(initial=0), 1)),
                              int(max(lk.max(initial=0), 1)), causal=causal, scale=scale,
                              window=window)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), l.cpu().numpy().astype(np.float64)


def varlen_case(fa, cfg, lens_q, lens_k=None, window=None, scale=None):
    sc = cfg.scale if scale is None else scale
    Q, K, V, cq, ck = inputs.make_packed(cfg, lens_q, lens_k)
    o, l = run_varlen(fa, Q, K, V, cq, ck, cfg.causal, sc, window)
    o_ref, l_ref = oracle.varlen_attention(Q, K, V, cq, ck, cfg.causal, sc, window)
    empty = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(l), empty), "rows without keys differ"
    assert not o[np.moveaxis(empty, 0, 1)].any(), "rows without keys must be 0"
    keep = ~empty
    check(np.moveaxis(o, 1, 0)[keep], l[keep], np.moveaxis(o_ref, 1, 0)[keep], l_ref[keep],
          "bf16", f"varlen lens={list(lens_q)[:8]} W={window}")


MIX = [1, 2, 33, 64, 65, 257, 300, 700]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_length_mix(fa, d, causal):
    _say(f"d={d} causal={causal}")
    varlen_case(fa, _cfg(4, 2, d, seed=d, causal=causal), MIX)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("d", [64, 128])
def test_whole_tile_lengths(fa, d, causal):
    # every document a multiple of the key tile: no tile has rows past its document's end, the
    # case where the kernels skip clearing their value stages
    varlen_case(fa, _cfg(4, 2, d, seed=d + 3, causal=causal), [64, 128, 256, 32, 512])


def test_more_keys_than_queries(fa):
    varlen_case(fa, _cfg(4, 2, 128), [5, 100, 64, 1], [40, 300, 64, 129])


def test_more_queries_than_keys_and_empty_documents(fa):
    varlen_case(fa, _cfg(4, 2, 64), [50, 0, 70, 9, 3], [20, 10, 70, 0, 300])
    varlen_case(fa, _cfg(2, 1, 64, causal=False), [50, 0, 7], [20, 5, 0])


@pytest.mark.parametrize("G", [1, 4, 16])
def test_gqa_groups(fa, G):
    varlen_case(fa, _cfg(2 * G, 2, 128, seed=G), [130, 7, 260])


@pytest.mark.parametrize("W", [1, 17, 64, 200])
def test_sliding_window(fa, W):
    varlen_case(fa, _cfg(4, 2, 128, seed=W), MIX, window=W)


@pytest.mark.parametrize("scale", [-0.25, 0.0, 0.6])
def test_scales(fa, scale):
    varlen_case(fa, _cfg(2, 2, 64, seed=9), [100, 31, 257], scale=scale)


def test_equal_lengths_match_the_batched_call_bitwise(fa):
    # B documents of one length packed = the batched [B, H, T, d] call with the same launch
    # configuration, bit for bit.
    import torch

    cfg = _cfg(8, 2, 128, seed=31)
    B, T = 3, 700
    Q, K, V, cq, ck = inputs.make_packed(cfg, [T] * B)
    o, l = fa.attn_fwd_varlen(_dev(Q), _dev(K), _dev(V), torch.from_numpy(cq).cuda(),
                              torch.from_numpy(ck).cuda(), T, T, causal=True)
    qb = _dev(Q).view(B, T, 8, 128).permute(0, 2, 1, 3).contiguous()
    kb = _dev(K).view(B, T, 2, 128).permute(0, 2, 1, 3).contiguous()
    vb = _dev(V).view(B, T, 2, 128).permute(0, 2, 1, 3).contiguous()
    ob, lb = fa.attn_fwd(qb, kb, vb, causal=True,
                         cfg=dict(kernel=1, block_kv=64, waves=8, schedule=2))
    torch.cuda.synchronize()
    assert torch.equal(o.view(B, T, 8, 128).permute(0, 2, 1, 3).contiguous().view(torch.int16),
                       ob.view(torch.int16))
    assert torch.equal(l.view(8, B, T).permute(1, 0, 2), lb)


def _doc_lengths(total, lo, hi, seed):
    rng = np.random.default_rng(seed)
    lens = []
    while sum(lens) < total:
        lens.append(int(rng.integers(lo, hi + 1)))
    lens[-1] -= sum(lens) - total
    return [x for x in lens if x > 0]


def test_workload_packed_training_batch_sampled(fa):
    # 32768 tokens of documents with lengths U[128, 8192], H=32, d=128, causal: the training
    # shape of the varlen interface; rows sampled in four documents, computed one by one.
    import torch

    cfg = AttnConfig("varlen packed", B=1, Hq=32, Hkv=32, Tq=1, Tk=1, d=128, dtype="bf16",
                     causal=True, dist="normal", seed=77)
    lens = _doc_lengths(32768, 128, 8192, 77)
    _say(f"packed batch of {len(lens)} documents: inputs")
    Q, K, V, cq, ck = inputs.make_packed(cfg, lens)
    o, l = fa.attn_fwd_varlen(_dev(Q), _dev(K), _dev(V), torch.from_numpy(cq).cuda(),
                              torch.from_numpy(ck).cuda(), max(lens), max(lens), causal=True)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(l).all())
    rng = np.random.default_rng(5)
    docs = sorted({0, len(lens) - 1, int(np.argmax(lens)), int(rng.integers(len(lens)))})
    og, lg, orf, lrf = [], [], [], []
    for b in docs:
        n = lens[b]
        rows = sorted({0, 1, 63, 64, n // 2, n - 65, n - 1} & set(range(n))
                      | set(rng.choice(n, size=min(n, 16), replace=False).tolist()))
        for h in (0, 17, 31):
            ref_o, ref_l = oracle.dense_head(Q[cq[b]:cq[b + 1], h], K[ck[b]:ck[b + 1], h],
                                             V[ck[b]:ck[b + 1], h], True, cfg.scale, rows=rows)
            idx = [cq[b] + r for r in rows]
            og.append(o[idx, h].float().cpu().numpy())
            lg.append(l[h, idx].cpu().numpy())
            orf.append(ref_o)
            lrf.append(ref_l)
    check(np.concatenate(og).astype(np.float64), np.concatenate(lg).astype(np.float64),
          np.concatenate(orf), np.concatenate(lrf), "bf16", "packed training batch")
