"""GPU parity of sliding-window attention (attn_fwd_window) against the fp64 oracle.

A query at position p = i + Tk - Tq sees keys p - W < j <= p. Same bounds as the other parity
tests: fp32 max abs error <= 1e-5; bf16 max abs error <= 2e-2 and mean-relative error <= 1e-2,
on O and on LSE.
"""

import sys

import numpy as np
import pytest

import oracle
from tests import inputs
from tests.inputs import AttnConfig
from tests.test_gpu_parity import check, _to_dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[window] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def fa():
    import torch

    assert torch.cuda.is_available(), "GPU parity tests need a GPU"
    import io_aware_tiled_amd as fa

    return fa


def _cfg(name, B, Hq, Hkv, Tq, Tk, d, dtype="bf16", seed=31, dist="normal"):
    return AttnConfig(name, B=B, Hq=Hq, Hkv=Hkv, Tq=Tq, Tk=Tk, d=d, dtype=dtype, causal=True,
                      dist=dist, seed=seed)


def run_window(fa, Q, K, V, W, scale, dtype, launch=None):
    import torch

    o, l = fa.attn_fwd(_to_dev(Q, dtype), _to_dev(K, dtype), _to_dev(V, dtype), causal=True,
                       scale=scale, cfg=launch, window=W)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), l.cpu().numpy().astype(np.float64)


def window_case(fa, cfg, W, launch=None):
    Q, K, V = inputs.make_inputs(cfg)
    o, l = run_window(fa, Q, K, V, W, cfg.scale, cfg.dtype, launch)
    o_ref, l_ref = oracle.dense_attention(Q, K, V, True, cfg.scale, window=W)
    check(o, l, o_ref, l_ref, cfg.dtype, f"{cfg.name} W={W} {launch}")


PREFILL_LAUNCHES = [dict(kernel=1, block_kv=bc, waves=nw, schedule=sch)
                    for bc in (32, 64) for nw in (4, 8) for sch in (1, 2, 4) if sch != 4 or nw == 8]


@pytest.mark.parametrize("launch", PREFILL_LAUNCHES,
                         ids=lambda c: "bc{block_kv}_w{waves}_s{schedule}".format(**c))
@pytest.mark.parametrize("d", [32, 64, 128])
def test_window_prefill_every_launch_config(fa, d, launch):
    for (Tq, Tk) in ((300, 300), (129, 200), (64, 64)):
        for W in (1, 5, 64, 100, 257):
            cfg = _cfg(f"swa d{d} Tq{Tq} Tk{Tk}", 2, 4, 2, Tq, Tk, d, seed=d + Tq + W)
            _say(f"{cfg.name} W={W} {launch}")
            window_case(fa, cfg, W, launch)


@pytest.mark.parametrize("T", [1, 2, 33, 65, 257, 513])
def test_window_ragged_lengths(fa, T):
    for W in (1, 31, 32, 33, 256):
        cfg = _cfg(f"swa ragged T{T}", 1, 2, 1, T, T, 128, seed=T + W)
        _say(f"{cfg.name} W={W}")
        window_case(fa, cfg, W)


@pytest.mark.parametrize("G", [1, 4, 16])
def test_window_gqa_groups(fa, G):
    cfg = _cfg(f"swa gqa G{G}", 2, 16, 16 // G, 200, 260, 64, seed=50 + G)
    window_case(fa, cfg, 70)


@pytest.mark.parametrize("d", [32, 64, 128])
def test_window_f32(fa, d):
    for (Tq, Tk) in ((100, 100), (37, 150), (1, 77)):
        for W in (1, 9, 64):
            cfg = _cfg(f"swa f32 d{d} Tq{Tq} Tk{Tk}", 1, 2, 1, Tq, Tk, d, dtype="f32", seed=W)
            window_case(fa, cfg, W)


@pytest.mark.parametrize("Tk", [1, 33, 1000, 4099])
@pytest.mark.parametrize("splits", [0, 1, 3, 16])
def test_window_decode(fa, Tk, splits):
    launch = None if splits == 0 else dict(kernel=3, splits=splits)
    for W in (1, 31, 32, 100, 5000):
        cfg = _cfg(f"swa decode Tk{Tk}", 2, 16, 2, 1, Tk, 128, seed=Tk + W)
        window_case(fa, cfg, W, launch)


def test_window_covering_every_key_equals_causal_bitwise(fa):
    import torch

    cfg = _cfg("swa wide", 1, 4, 2, 200, 300, 64, seed=77)
    Q, K, V = inputs.make_inputs(cfg)
    q, k, v = (_to_dev(x, "bf16") for x in (Q, K, V))
    o1, l1 = fa.attn_fwd(q, k, v, causal=True, window=300)
    o2, l2 = fa.attn_fwd(q, k, v, causal=True, window=10 ** 6)
    o3, l3 = fa.attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o3) and torch.equal(l1, l3)
    assert torch.equal(o2, o3) and torch.equal(l2, l3)


def test_window_deterministic_and_no_out_of_bounds_writes(fa):
    import torch

    cfg = _cfg("swa canary", 2, 4, 2, 200, 200, 128, seed=3)
    Q, K, V = inputs.make_inputs(cfg)
    q, k, v = (_to_dev(x, "bf16") for x in (Q, K, V))
    pad = 4096
    n_o, n_l = q.numel(), cfg.B * cfg.Hq * cfg.Tq
    outs = []
    for _ in range(2):
        obuf = torch.full((n_o + 2 * pad,), 7.0, dtype=torch.bfloat16, device="cuda")
        lbuf = torch.full((n_l + 2 * pad,), 7.0, dtype=torch.float32, device="cuda")
        o = obuf[pad:pad + n_o].view(q.shape)
        l = lbuf[pad:pad + n_l].view(cfg.B, cfg.Hq, cfg.Tq)
        fa.attn_fwd(q, k, v, causal=True, out=o, lse=l, window=48)
        torch.cuda.synchronize()
        for buf, n in ((obuf, n_o), (lbuf, n_l)):
            assert torch.all(buf[:pad] == 7.0) and torch.all(buf[pad + n:] == 7.0)
        outs.append((o.clone(), l.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def _sample_rows(T, W, rng, n=24):
    edge = [0, 1, W - 2, W - 1, W, W + 1, T // 2, T - 2, T - 1]
    rows = set(r for r in edge if 0 <= r < T)
    rows.update(rng.choice(T, size=min(n, T), replace=False).tolist())
    return sorted(rows)


def test_window_prefill_t8192_w4096_sampled(fa):
    import torch

    cfg = inputs.CONFIGS["bf16_causal_b1_h32_t8192_d128"]
    W = 4096
    _say(f"{cfg.name} W={W}: inputs")
    Q, K, V = inputs.make_inputs(cfg)
    q, k, v = (_to_dev(x, cfg.dtype) for x in (Q, K, V))
    o, l = fa.attn_fwd(q, k, v, causal=True, scale=cfg.scale, window=W)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(l).all())
    rng = np.random.default_rng(4096)
    og, lg, orf, lrf = [], [], [], []
    for h in (0, 17, 31):
        rows = _sample_rows(cfg.Tq, W, rng)
        o_ref, l_ref = oracle.dense_head(Q[0, h], K[0, h], V[0, h], True, cfg.scale, rows=rows,
                                         window=W)
        og.append(o[0, h, rows].float().cpu().numpy())
        lg.append(l[0, h, rows].cpu().numpy())
        orf.append(o_ref)
        lrf.append(l_ref)
    check(np.concatenate(og).astype(np.float64), np.concatenate(lg).astype(np.float64),
          np.concatenate(orf), np.concatenate(lrf), cfg.dtype, "t8192 w4096")


def test_window_decode_gqa_tk8192_w4096_full(fa):
    cfg = inputs.CONFIGS["bf16_gqa_decode_b64_hq64_hkv8_tk8192_d128"]
    W = 4096
    _say(f"{cfg.name} W={W}: inputs")
    Q, K, V = inputs.make_inputs(cfg)
    o, l = run_window(fa, Q, K, V, W, cfg.scale, cfg.dtype)
    o_ref = np.empty_like(o)
    l_ref = np.empty_like(l)
    G = cfg.group
    for b in range(cfg.B):
        for g in range(cfg.Hkv):
            qs = Q[b, g * G:(g + 1) * G, 0, :]
            # the window of the single decode row is the last W keys
            ob, lb = oracle.dense_head(qs, K[b, g, cfg.Tk - W:], V[b, g, cfg.Tk - W:], False,
                                       cfg.scale)
            o_ref[b, g * G:(g + 1) * G, 0] = ob
            l_ref[b, g * G:(g + 1) * G, 0] = lb
    check(o, l, o_ref, l_ref, cfg.dtype, "decode w4096")
