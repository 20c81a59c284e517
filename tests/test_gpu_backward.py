"""GPU parity of the bf16 backward (attn_bwd) against the fp64 oracle.

Bound, per gradient tensor G with oracle value R (derivation: the kernels round P, dS and the
outputs to bf16, unit roundoff 2^-9, and accumulate in fp32; a CPU model of exactly that
rounding gives max errors of at most 0.5% of max|R| and mean-relative errors of about 0.23%):
    max |G - R| <= 2e-2 * max(1, max |R|)    and    sum |G - R| <= 1e-2 * sum |R| (+ 1e-6 each).
This is the forward's bf16 pair of bounds with the absolute one scaled by the tensor's largest
value when that exceeds 1 (gradients of early keys grow with the number of rows that see them).

Inputs: Q, K, V and dO from the seeded generators; O and LSE from the oracle's forward, rounded to
bf16 and fp32, go to both the GPU backward and the oracle's backward (which, like the pages'
backward, takes O and L as inputs). In the end-to-end cases the GPU forward's own outputs feed the
GPU backward and the oracle recomputes everything from Q, K, V and dO alone.
"""

import sys

import numpy as np
import pytest

import oracle
from tests import inputs
from tests.inputs import AttnConfig

pytestmark = pytest.mark.gpu

REL_MAX = 2e-2
MEAN_REL = 1e-2


def _say(msg):
    print(f"[backward] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def fa():
    import torch

    assert torch.cuda.is_available(), "GPU parity tests need a GPU"
    import io_aware_tiled_amd as fa

    return fa


def _dev(x):
    return inputs.to_torch(x, "bf16", "cuda")


def check_grad(got, ref, what):
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), (what, "non-finite")
    bound = REL_MAX * max(1.0, float(np.abs(ref).max()))
    assert err.max() <= bound, (what, "max abs", float(err.max()), bound)
    # 1e-6 per element of slack: a reference that is exactly zero (one visible key: dS = 0)
    # leaves only fp32 rounding of dP - D on the GPU side
    assert err.sum() <= MEAN_REL * float(np.abs(ref).sum()) + 1e-6 * err.size, \
        (what, "mean-rel", float(err.sum() / max(np.abs(ref).sum(), 1e-30)))


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def nan_grads(q, k):
    """dQ, dK, dV buffers filled with NaN: an element the kernels do not write fails the check."""
    import torch

    return (torch.full_like(q, float("nan")), torch.full_like(k, float("nan")),
            torch.full_like(k, float("nan")))


def run_bwd(fa, Q, K, V, O, L, dO, causal, scale, window=None):
    import torch

    lse = torch.from_numpy(np.ascontiguousarray(L, dtype=np.float32)).cuda()
    q, k = _dev(Q), _dev(K)
    dq, dk, dv = nan_grads(q, k)
    fa.attn_bwd(q, k, _dev(V), _dev(inputs.round_to_bf16(O)), lse, _dev(dO), causal=causal,
                scale=scale, window=window, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return _np(dq), _np(dk), _np(dv)


def bwd_case(fa, cfg: AttnConfig, window=None, scale=None):
    """The GPU backward and the oracle's backward on the same inputs: O rounded to bf16 and LSE
    to fp32 are what both receive (the pages' backward takes O and L as inputs)."""
    sc = cfg.scale if scale is None else scale
    Q, K, V = inputs.make_inputs(cfg)
    dO = inputs.make_grad(cfg)
    O, L = oracle.dense_attention(Q, K, V, cfg.causal, sc, window=window)
    Ob, Lf = inputs.round_to_bf16(O), L.astype(np.float32)
    got = run_bwd(fa, Q, K, V, Ob, Lf, dO, cfg.causal, sc, window)
    ref = oracle.tiled_backward(Q, K, V, Ob, Lf, dO, cfg.causal, sc, window=window)
    for n, g, r in zip(("dQ", "dK", "dV"), got, ref):
        check_grad(g, r, f"{cfg.name} W={window} scale={sc} {n}")


def _cfg(name, B, Hq, Hkv, Tq, Tk, d, causal=True, seed=17, dist="normal"):
    return AttnConfig(name, B=B, Hq=Hq, Hkv=Hkv, Tq=Tq, Tk=Tk, d=d, dtype="bf16", causal=causal,
                      dist=dist, seed=seed)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_shapes(fa, d, causal):
    for (Tq, Tk) in ((64, 64), (300, 300), (129, 200), (1, 77), (200, 129)):
        if causal and Tq > Tk:
            continue
        cfg = _cfg(f"bwd d{d} c{int(causal)} Tq{Tq} Tk{Tk}", 2, 4, 2, Tq, Tk, d, causal,
                   seed=d + Tq + Tk)
        _say(cfg.name)
        bwd_case(fa, cfg)


@pytest.mark.parametrize("T", [1, 2, 31, 33, 65, 257, 513])
def test_ragged_lengths(fa, T):
    cfg = _cfg(f"bwd ragged T{T}", 1, 2, 1, T, T, 128, seed=T)
    _say(cfg.name)
    bwd_case(fa, cfg)


@pytest.mark.parametrize("G", [1, 4, 16])
def test_gqa_groups(fa, G):
    cfg = _cfg(f"bwd gqa G{G}", 1, 2 * G, 2, 200, 200, 64, seed=G)
    _say(cfg.name)
    bwd_case(fa, cfg)


@pytest.mark.parametrize("d", [64, 128])
def test_sliding_window(fa, d):
    for (Tq, Tk) in ((300, 300), (129, 200), (1, 90)):
        for W in (1, 5, 64, 100, 257):
            cfg = _cfg(f"bwd swa d{d} Tq{Tq} Tk{Tk}", 1, 4, 2, Tq, Tk, d, seed=W + Tq)
            _say(f"{cfg.name} W={W}")
            bwd_case(fa, cfg, window=W)


@pytest.mark.parametrize("scale", [-0.3, 0.0, 0.5])
def test_scales(fa, scale):
    cfg = _cfg("bwd scale", 1, 2, 1, 150, 150, 64, seed=3)
    _say(f"{cfg.name} {scale}")
    bwd_case(fa, cfg, scale=scale)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("shape", ["noncausal_T2100", "causal_T4400_W2100", "gqa4_Tq300_Tk2300"])
def test_long_row_workgroups(fa, shape, d):
    # Rows that see over 2048 keys on average select the 8-wave workgroups (at d = 128 the dK/dV
    # kernel then keeps its K block in LDS): a ragged last key block, a window, GQA and Tk > Tq
    # at sizes the oracle runs in full.
    Tq, Tk, Hq, causal, W = {"noncausal_T2100": (2100, 2100, 2, False, None),
                             "causal_T4400_W2100": (4400, 4400, 2, True, 2100),
                             "gqa4_Tq300_Tk2300": (300, 2300, 4, False, None)}[shape]
    # GPU forward then GPU backward, against the oracle's dense backward from Q, K, V and dO (the
    # pages' tiled backward is too slow in fp64 at these lengths; the two are pinned equal).
    import torch

    cfg = _cfg(f"bwd long rows {shape} d{d}", 1, Hq, 1, Tq, Tk, d, causal, seed=Tk + d)
    _say(cfg.name)
    Q, K, V = inputs.make_inputs(cfg)
    dO = inputs.make_grad(cfg)
    q, k, v, do = _dev(Q), _dev(K), _dev(V), _dev(dO)
    o, lse = fa.attn_fwd(q, k, v, causal=causal, window=W)
    dq, dk, dv = fa.attn_bwd(q, k, v, o, lse, do, causal=causal, window=W)
    torch.cuda.synchronize()
    ref = oracle.dense_backward(Q, K, V, dO, causal, cfg.scale, window=W)
    for n, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        check_grad(_np(g), r, f"{cfg.name} {n}")


def test_keys_no_row_sees_have_zero_gradients(fa):
    # Tk > Tq with a narrow window: keys before position Tk - Tq - W + 1 are seen by no row.
    cfg = _cfg("bwd unseen keys", 1, 2, 1, 40, 300, 64, seed=8)
    Q, K, V = inputs.make_inputs(cfg)
    dO = inputs.make_grad(cfg)
    O, L = oracle.dense_attention(Q, K, V, True, cfg.scale, window=16)
    _, dk, dv = run_bwd(fa, Q, K, V, O, L, dO, True, cfg.scale, 16)
    first_seen = 300 - 40 - 16 + 1
    assert not dk[:, :, :first_seen].any() and not dv[:, :, :first_seen].any()
    assert dk[:, :, first_seen:].any()


def test_causal_b4_h16_t1024_d64_full(fa):
    # B=4, H=16, T=1024, d=64, U(-0.8, 0.8), causal: every gradient element against the oracle.
    cfg = inputs.CONFIGS["bf16_causal_b4_h16_t1024_d64"]
    _say(cfg.name)
    bwd_case(fa, cfg)


def test_bitwise_reproducible(fa):
    import torch

    cfg = _cfg("bwd determinism", 1, 8, 2, 700, 700, 128, seed=5)
    Q, K, V = inputs.make_inputs(cfg)
    dO = inputs.make_grad(cfg)
    O, L = oracle.dense_attention(Q, K, V, True, cfg.scale)
    args = (_dev(Q), _dev(K), _dev(V), _dev(inputs.round_to_bf16(O)),
            torch.from_numpy(L.astype(np.float32)).cuda(), _dev(dO))
    a = fa.attn_bwd(*args, causal=True)
    b = fa.attn_bwd(*args, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_end_to_end_small(fa):
    # The GPU forward's O and LSE feed the GPU backward.
    import torch

    cfg = _cfg("bwd end-to-end", 2, 8, 2, 333, 333, 128, seed=12)
    Q, K, V = inputs.make_inputs(cfg)
    dO = inputs.make_grad(cfg)
    q, k, v, do = _dev(Q), _dev(K), _dev(V), _dev(dO)
    o, lse = fa.attn_fwd(q, k, v, causal=True)
    dq, dk, dv = fa.attn_bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    ref = oracle.dense_backward(Q, K, V, dO, True, cfg.scale)
    for n, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        check_grad(_np(g), r, f"{cfg.name} {n}")


def _sample(T, rng, n=24, lo=0):
    """Sorted distinct indices in [lo, T): tile edges and the end, plus n drawn from the seed."""
    fixed = [lo, lo + 1, lo + 31, lo + 32, lo + 127, lo + 128, (lo + T) // 2, T - 129, T - 33,
             T - 32, T - 2, T - 1]
    return sorted({x for x in fixed + (lo + rng.choice(T - lo, size=n, replace=False)).tolist()
                   if lo <= x < T})


def sampled_e2e(fa, cfg: AttnConfig, late_keys=None, full_range_kv=None):
    """Full-size forward then backward on the GPU into NaN-filled gradient buffers; every element
    must be written and finite. Sampled dQ rows of every query head and sampled dK/dV keys of
    every kv head are compared with the oracle.

    The oracle's column form costs a whole forward per query head for keys near the start of the
    sequence (every later row sees them). With ``late_keys`` set, kv heads other than those in
    ``full_range_kv`` sample keys from the last ``late_keys`` positions only, which only the
    rows after them see."""
    import torch

    _say(f"{cfg.name}: inputs")
    Q, K, V = inputs.make_inputs(cfg)
    dO = inputs.make_grad(cfg)
    q, k, v, do = _dev(Q), _dev(K), _dev(V), _dev(dO)
    _say(f"{cfg.name}: forward + backward")
    o, lse = fa.attn_fwd(q, k, v, causal=cfg.causal)
    dq, dk, dv = nan_grads(q, k)
    fa.attn_bwd(q, k, v, o, lse, do, causal=cfg.causal, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t).all())
    del o, lse, q, k, v, do
    rng = np.random.default_rng(cfg.seed + 2000)
    G = cfg.group
    got_q, ref_q = [], []
    _say(f"{cfg.name}: oracle dQ rows of all {cfg.B * cfg.Hq} query heads")
    for b in range(cfg.B):
        for h in range(cfg.Hq):
            rows = _sample(cfg.Tq, rng)
            ref_q.append(oracle.backward_rows(Q[b, h], K[b, h // G], V[b, h // G], dO[b, h], rows,
                                              cfg.causal, cfg.scale))
            got_q.append(_np(dq[b, h, rows]))
    check_grad(np.concatenate(got_q), np.concatenate(ref_q), f"{cfg.name} dQ")
    got_k, ref_k, got_v, ref_v = [], [], [], []
    for b in range(cfg.B):
        for g in range(cfg.Hkv):
            full = late_keys is None or (b, g) in (full_range_kv or [])
            keys = _sample(cfg.Tk, rng, lo=0 if full else cfg.Tk - late_keys)
            _say(f"{cfg.name}: oracle dK/dV of kv head ({b}, {g}), keys {keys[0]}..{keys[-1]}")
            rk = np.zeros((len(keys), cfg.d))
            rv = np.zeros((len(keys), cfg.d))
            for h in range(g * G, (g + 1) * G):
                sk, sv = oracle.backward_cols(Q[b, h], K[b, g], V[b, g], dO[b, h], keys,
                                              cfg.causal, cfg.scale)
                rk += sk
                rv += sv
            got_k.append(_np(dk[b, g, keys]))
            got_v.append(_np(dv[b, g, keys]))
            ref_k.append(rk)
            ref_v.append(rv)
            check_grad(got_k[-1], rk, f"{cfg.name} dK ({b},{g})")
            check_grad(got_v[-1], rv, f"{cfg.name} dV ({b},{g})")
    check_grad(np.concatenate(got_k), np.concatenate(ref_k), f"{cfg.name} dK")
    check_grad(np.concatenate(got_v), np.concatenate(ref_v), f"{cfg.name} dV")


def test_causal_t8192_d128_every_head_sampled(fa):
    # B=1, H=32, T=8192, d=128, causal: the forward's headline shape; sampled rows and keys of
    # every head, keys over the whole sequence
    sampled_e2e(fa, inputs.CONFIGS["bf16_causal_b1_h32_t8192_d128"])


def test_noncausal_t8000_d128_every_head_sampled(fa):
    cfg = inputs.CONFIGS["bf16_causal_b1_h32_t8000_d128"].replace(causal=False, name="noncausal t8000")
    sampled_e2e(fa, cfg)


def test_gqa_causal_t16384_d128_every_head_sampled(fa):
    # B=2, Hq=32, Hkv=8, T=16384, d=128, causal, 1% of K rows x8: a kv head's gradient sums
    # four query heads. dQ rows of all 64 query heads; dK/dV keys of all 16 kv heads, over the
    # whole sequence for two of them and from the last 1024 positions for the rest.
    sampled_e2e(fa, inputs.CONFIGS["bf16_gqa_causal_b2_hq32_hkv8_t16384_d128"], late_keys=1024,
                full_range_kv=[(0, 3), (1, 6)])
