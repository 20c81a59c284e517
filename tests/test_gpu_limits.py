"""GPU checks at the size limits of the C ABI (Tq*d and Tk*d just under 2^31, head offsets past
2^31 elements) and at long sequence lengths.

Inputs are drawn on the device from seeded generators; the reference values are the oracle on
sampled rows (copied back) or closed forms that hold at any size (with scale 0 every visible key
has the same weight, so O is the mean of V over the visible keys and LSE = ln(number of keys)).
Bounds as elsewhere for bf16: max abs error <= 2e-2 and mean-relative error <= 1e-2.
"""

import math
import sys

import numpy as np
import pytest

import oracle
from tests.test_gpu_parity import check

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[limits] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def fa():
    import torch

    assert torch.cuda.is_available(), "GPU checks need a GPU"
    import io_aware_tiled_amd as fa

    return fa


def _randn(torch, shape, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn(shape, device="cuda", generator=g).to(torch.bfloat16)


def _host(t):
    return t.float().cpu().numpy().astype(np.float64)


def test_query_tensor_past_2pow31_elements(fa):
    # Two query heads of 2^23 + 5 rows, d = 128: Q and O hold 2.15e9 elements, so the second
    # head starts past 2^31; rows near its end are checked against the oracle.
    import torch

    Tq, Tk, d = (1 << 23) + 5, 100, 128
    _say(f"prefill Tq={Tq} Tk={Tk}: inputs")
    q = _randn(torch, (1, 2, Tq, d), 1)
    k = _randn(torch, (1, 1, Tk, d), 2)
    v = _randn(torch, (1, 1, Tk, d), 3)
    o, lse = fa.attn_fwd(q, k, v, causal=False)
    torch.cuda.synchronize()
    rows = [0, 1, 255, 256, Tq // 2, Tq - 257, Tq - 256, Tq - 2, Tq - 1]
    K, V = _host(k[0, 0]), _host(v[0, 0])
    og, lg, orf, lrf = [], [], [], []
    for h in (0, 1):
        Qr = _host(q[0, h, rows])
        ro, rl = oracle.dense_head(Qr, K, V, False, 1 / math.sqrt(d))
        og.append(_host(o[0, h, rows]))
        lg.append(lse[0, h, rows].cpu().numpy().astype(np.float64))
        orf.append(ro)
        lrf.append(rl)
    check(np.concatenate(og), np.concatenate(lg), np.concatenate(orf), np.concatenate(lrf),
          "bf16", "query tensor past 2^31 elements")


def test_decode_at_the_key_limit(fa):
    # Tk * d = 2^31 - 128: the largest cache one call accepts at d = 128. V ramps from 0 to 1
    # across the keys, so a row read from the wrong place moves the mean.
    import torch

    d = 128
    Tk = (1 << 31) // d - 1
    _say(f"decode Tk={Tk}: inputs")
    ramp = (torch.arange(Tk, device="cuda", dtype=torch.float32) / Tk).to(torch.bfloat16)
    v = ramp[:, None].expand(Tk, d).contiguous().view(1, 1, Tk, d)
    k = torch.zeros(1, 1, Tk, d, dtype=torch.bfloat16, device="cuda")
    q = _randn(torch, (1, 8, 1, d), 4)
    o, lse = fa.attn_fwd(q, k, v, causal=False, scale=0.0)
    torch.cuda.synchronize()
    mean = float(np.mean(_host(ramp)))
    o_ref = np.full((8, d), mean)
    l_ref = np.full(8, math.log(Tk))
    check(_host(o[0, :, 0]), lse[0, :, 0].cpu().numpy().astype(np.float64), o_ref, l_ref, "bf16",
          "decode at the key limit")
    # the same cache behind a causal single row and a window of the last 1000 keys
    o, lse = fa.attn_fwd(q, k, v, causal=True, scale=0.0, window=1000)
    torch.cuda.synchronize()
    tail = float(np.mean(_host(ramp[Tk - 1000:])))
    check(_host(o[0, :, 0]), lse[0, :, 0].cpu().numpy().astype(np.float64),
          np.full((8, d), tail), np.full(8, math.log(1000)), "bf16", "decode window at the limit")


@pytest.mark.parametrize("T", [65536, 131072])
def test_long_causal_sequence_sampled(fa, T):
    import torch

    d = 128
    _say(f"causal T={T}")
    q = _randn(torch, (1, 1, T, d), 10 + T)
    k = _randn(torch, (1, 1, T, d), 20 + T)
    v = _randn(torch, (1, 1, T, d), 30 + T)
    o, lse = fa.attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    rows = sorted({0, 1, 255, 4096, T // 2, T - 257, T - 1}
                  | set(np.random.default_rng(T).choice(T, 8, replace=False).tolist()))
    ro, rl = oracle.dense_head(_host(q[0, 0]), _host(k[0, 0]), _host(v[0, 0]), True,
                               1 / math.sqrt(d), rows=rows)
    check(_host(o[0, 0, rows]), lse[0, 0, rows].cpu().numpy().astype(np.float64), ro, rl, "bf16",
          f"causal T={T}")
