"""GPU parity: libfattn through its C ABI against the fp64 oracle, element by element.

Bounds (on both O and LSE): fp32 inputs, max abs error <= 1e-5; bf16 inputs, max abs error
<= 2e-2 and mean-relative error sum|gpu - ref| / sum|ref| <= 1e-2. The oracle reads the same
rounded input values widened exactly to float64.

Small problems are compared in full (several tiles, ragged tails, every launch configuration).
The five full-size workloads run at their real shape in the default configuration, into
NaN-filled output buffers: the fp32 T=128, bf16 T=1024, the T=8192 causal prefill and its three
variants and the GQA decode are compared on every element; the GQA T=16384 prefill on sampled
rows of every one of its 64 heads, which the oracle computes one by one.
"""

import math
import sys

import numpy as np
import pytest

import oracle
from tests import inputs
from tests.inputs import AttnConfig

pytestmark = pytest.mark.gpu

F32_MAX_ABS = 1e-5
BF16_MAX_ABS = 2e-2
BF16_MEAN_REL = 1e-2


def _say(msg):
    print(f"[parity] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def fa():
    import torch

    assert torch.cuda.is_available(), "GPU parity tests need a GPU"
    import io_aware_tiled_amd as fa

    return fa


def _to_dev(x, dtype):
    return inputs.to_torch(x, dtype, "cuda")


def run_gpu(fa, Q, K, V, causal, scale, dtype, cfg=None):
    """One call through the C ABI into NaN-filled O and LSE buffers (an element the kernels do
    not write stays NaN and fails the comparison)."""
    import torch

    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    B, Hq, Tq, d = Q.shape
    o = torch.full((B, Hq, Tq, d), float("nan"), dtype=tdt, device="cuda")
    lse = torch.full((B, Hq, Tq), float("nan"), dtype=torch.float32, device="cuda")
    fa.attn_fwd(_to_dev(Q, dtype), _to_dev(K, dtype), _to_dev(V, dtype), causal=causal,
                scale=scale, cfg=cfg, out=o, lse=lse)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check(o, l, o_ref, l_ref, dtype, what="", f32_bound=F32_MAX_ABS):
    eo, el = np.abs(o - o_ref), np.abs(l - l_ref)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), what
    if dtype == "f32":
        assert eo.max() <= f32_bound, (what, "O", eo.max())
        assert el.max() <= f32_bound, (what, "LSE", el.max())
    else:
        assert eo.max() <= BF16_MAX_ABS, (what, "O", eo.max())
        assert el.max() <= BF16_MAX_ABS, (what, "LSE", el.max())
        assert eo.sum() <= BF16_MEAN_REL * np.abs(o_ref).sum(), (what, "O mean-rel")
        assert el.sum() <= BF16_MEAN_REL * max(np.abs(l_ref).sum(), 1e-30), (what, "LSE mean-rel")


def f32_bound_for_scale(scale, d):
    """fp32 bound for a literal scale: 1e-5 up to the default 1/sqrt(d), growing in proportion
    beyond it, because a logit's fp32 rounding error is proportional to its magnitude (about
    |scale| * sqrt(d) for unit-variance q and k) and the output error follows it."""
    return F32_MAX_ABS * max(1.0, abs(scale) * math.sqrt(d))


def full_case(fa, cfg: AttnConfig, launch=None, scale=None):
    Q, K, V = inputs.make_inputs(cfg)
    sc = cfg.scale if scale is None else scale
    o, l = run_gpu(fa, Q, K, V, cfg.causal, sc, cfg.dtype, launch)
    o_ref, l_ref = oracle.dense_attention(Q, K, V, cfg.causal, sc)
    check(o, l, o_ref, l_ref, cfg.dtype, f"{cfg.name} {launch}", f32_bound_for_scale(sc, cfg.d))
    return o, l


def _small(name, B, Hq, Hkv, Tq, Tk, d, dtype="bf16", causal=True, dist="normal", seed=11):
    return AttnConfig(name, B=B, Hq=Hq, Hkv=Hkv, Tq=Tq, Tk=Tk, d=d, dtype=dtype, causal=causal,
                      dist=dist, seed=seed)


# ------------------------------------------------------------------ small problems, in full

# schedule 1: row-major grid; 2: XCD-grouped, longest causal blocks first; 4: paired blocks
PREFILL_LAUNCHES = [dict(block_kv=bc, waves=nw, schedule=sch)
                    for bc in (32, 64) for nw in (4, 8) for sch in (1, 2, 4) if sch != 4 or nw == 8]


@pytest.mark.parametrize("launch", PREFILL_LAUNCHES, ids=lambda c: "bc{block_kv}_w{waves}_s{schedule}".format(**c))
@pytest.mark.parametrize("d", [32, 64, 128])
def test_prefill_bf16_every_launch_config(fa, d, launch):
    for causal in (True, False):
        for (Tq, Tk) in ((300, 300), (129, 129), (64, 200), (1, 77)):
            if causal and Tq > Tk:
                continue
            cfg = _small(f"bf16 d{d} Tq{Tq} Tk{Tk} c{int(causal)}", 2, 4, 2, Tq, Tk, d,
                         causal=causal, seed=d + Tq)
            _say(f"{cfg.name} {launch}")
            full_case(fa, cfg, dict(launch, kernel=fa.FATTN_KERNEL_PREFILL_MFMA))


@pytest.mark.parametrize("launch", [dict(block_kv=bc, waves=8) for bc in (32, 64)],
                         ids=lambda c: "bc{block_kv}_w{waves}".format(**c))
@pytest.mark.parametrize("d", [32, 64, 128])
def test_paired_blocks(fa, d, launch):
    # Schedule 4 runs query blocks nqb-1-p and p of a (batch, head) in one workgroup, the second
    # with its Q prefetched into LDS and its first K and V tiles issued early. Block counts here
    # are even and odd (an odd count leaves the middle block alone in its workgroup), the last
    # block is ragged, and GQA groups differ.
    cases = [(True, 2, 16, 4, 4100), (False, 4, 16, 16, 2100), (True, 2, 16, 2, 1500),
             (True, 1, 4, 1, 300), (False, 3, 2, 2, 129)]
    for causal, B, Hq, Hkv, T in cases:
        cfg = _small(f"paired d{d} B{B} Hq{Hq} Hkv{Hkv} T{T} c{int(causal)}", B, Hq, Hkv, T, T, d,
                     causal=causal, seed=d + T)
        _say(f"{cfg.name} {launch}")
        full_case(fa, cfg, dict(launch, kernel=fa.FATTN_KERNEL_PREFILL_MFMA, schedule=4))


@pytest.mark.parametrize("T", [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 257, 513])
def test_prefill_bf16_ragged_lengths(fa, T):
    for causal in (True, False):
        cfg = _small(f"ragged T{T}", 1, 2, 1, T, T, 128, causal=causal, seed=T)
        _say(cfg.name)
        full_case(fa, cfg)


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_prefill_bf16_gqa_groups(fa, G):
    cfg = _small(f"gqa G{G}", 2, 16, 16 // G, 200, 200, 64, seed=100 + G)
    _say(cfg.name)
    full_case(fa, cfg)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("Tq,Tk", [(1, 1), (1, 300), (7, 300), (64, 64), (100, 129), (300, 300)])
def test_prefill_f32(fa, d, Tq, Tk):
    for causal in (True, False):
        cfg = _small(f"f32 d{d} Tq{Tq} Tk{Tk}", 2, 4, 2, Tq, Tk, d, dtype="f32", causal=causal,
                     seed=7 * d + Tq)
        _say(cfg.name)
        full_case(fa, cfg)


@pytest.mark.parametrize("splits", [0, 1, 2, 5, 16])
@pytest.mark.parametrize("Tk", [1, 31, 32, 33, 100, 1000, 4099])
def test_decode_splits(fa, Tk, splits):
    for d, G in ((128, 8), (64, 4), (32, 16), (128, 1), (64, 32)):
        cfg = _small(f"decode d{d} G{G} Tk{Tk} s{splits}", 3, 2 * G, 2, 1, Tk, d, causal=False,
                     seed=Tk + d + G)
        _say(cfg.name)
        full_case(fa, cfg, dict(kernel=fa.FATTN_KERNEL_DECODE_SPLITK, splits=splits))


def test_decode_causal_single_row_equals_full_prefix(fa):
    cfg = _small("decode causal", 2, 8, 2, 1, 1000, 128, causal=True)
    full_case(fa, cfg)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("scale", [-0.3, 0.0, 0.02, 1.7])
def test_literal_scales(fa, dtype, scale):
    cfg = _small(f"scale {scale}", 1, 4, 2, 130, 130, 64, dtype=dtype, seed=5)
    full_case(fa, cfg, scale=scale)
    dec = _small(f"scale {scale} decode", 2, 8, 2, 1, 300, 64, dtype=dtype, causal=False, seed=6)
    full_case(fa, dec, scale=scale)


def test_zero_queries_give_prefix_means(fa):
    import torch

    T, d = 200, 64
    cfg = _small("q0", 1, 2, 2, T, T, d, seed=9)
    Q, K, V = inputs.make_inputs(cfg)
    Q[:] = 0
    o, l = run_gpu(fa, Q, K, V, True, cfg.scale, "bf16")
    cnt = np.arange(1, T + 1)
    expect = np.cumsum(V.astype(np.float64), axis=2) / cnt[:, None]
    check(o, l, expect, np.broadcast_to(np.log(cnt), l.shape), "bf16", "q=0 prefix means")


@pytest.mark.parametrize("d", [32, 64, 128])
def test_large_logit_spikes(fa, d):
    # 1% of the K rows scaled x8 (the spiked-key stress of the GQA T=16384 workload) on a small
    # problem, compared in full
    cfg = AttnConfig(f"spikes d{d}", B=1, Hq=4, Hkv=1, Tq=700, Tk=700, d=d, dtype="bf16",
                     causal=True, dist="normal", seed=21, k_spike=(0.01, 8.0))
    full_case(fa, cfg)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_scores_growing_along_the_keys(fa, d, causal):
    # The keys' scale grows 16-fold along the sequence, so tile after tile exceeds the exponent
    # base the rows have so far: the re-base paths of the steady state run again and again (for
    # d <= 64 that is the fallback behind the weight-sum check).
    cfg = _small(f"growing d{d} c{int(causal)}", 1, 4, 2, 900, 900, d, causal=causal, seed=d + 5)
    Q, K, V = inputs.make_inputs(cfg)
    K = inputs.round_to_bf16(K * np.linspace(0.25, 4.0, cfg.Tk)[None, None, :, None])
    o, l = run_gpu(fa, Q, K, V, causal, cfg.scale, "bf16")
    o_ref, l_ref = oracle.dense_attention(Q, K, V, causal, cfg.scale)
    check(o, l, o_ref, l_ref, "bf16", cfg.name)


def test_deterministic_and_no_out_of_bounds_writes(fa):
    import torch

    cfg = _small("canary", 2, 4, 2, 200, 200, 128, seed=3)
    Q, K, V = inputs.make_inputs(cfg)
    q, k, v = (_to_dev(x, "bf16") for x in (Q, K, V))
    pad = 4096
    n_o, n_l = q.numel(), cfg.B * cfg.Hq * cfg.Tq
    for launch in [None, dict(block_kv=32, waves=8, schedule=1)]:
        outs = []
        for _ in range(2):
            obuf = torch.full((n_o + 2 * pad,), 7.0, dtype=torch.bfloat16, device="cuda")
            lbuf = torch.full((n_l + 2 * pad,), 7.0, dtype=torch.float32, device="cuda")
            o = obuf[pad:pad + n_o].view(q.shape)
            l = lbuf[pad:pad + n_l].view(cfg.B, cfg.Hq, cfg.Tq)
            fa.attn_fwd(q, k, v, causal=True, out=o, lse=l, cfg=launch)
            torch.cuda.synchronize()
            for buf, n in ((obuf, n_o), (lbuf, n_l)):
                assert torch.all(buf[:pad] == 7.0) and torch.all(buf[pad + n:] == 7.0)
            outs.append((o.clone(), l.clone()))
        assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_decode_deterministic_and_no_out_of_bounds_writes(fa):
    import torch

    cfg = _small("decode canary", 4, 16, 2, 1, 3000, 128, causal=False, seed=4)
    Q, K, V = inputs.make_inputs(cfg)
    q, k, v = (_to_dev(x, "bf16") for x in (Q, K, V))
    pad = 4096
    n_o, n_l = q.numel(), cfg.B * cfg.Hq
    outs = []
    for _ in range(2):
        obuf = torch.full((n_o + 2 * pad,), 7.0, dtype=torch.bfloat16, device="cuda")
        lbuf = torch.full((n_l + 2 * pad,), 7.0, dtype=torch.float32, device="cuda")
        o = obuf[pad:pad + n_o].view(q.shape)
        l = lbuf[pad:pad + n_l].view(cfg.B, cfg.Hq, 1)
        fa.attn_fwd(q, k, v, out=o, lse=l)
        torch.cuda.synchronize()
        for buf, n in ((obuf, n_o), (lbuf, n_l)):
            assert torch.all(buf[:pad] == 7.0) and torch.all(buf[pad + n:] == 7.0)
        outs.append((o.clone(), l.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_noop_shapes(fa):
    import torch

    z = torch.zeros(0, 4, 16, 64, dtype=torch.bfloat16, device="cuda")
    o, l = fa.attn_fwd(z, z, z, causal=True)
    assert o.shape == z.shape and l.shape == (0, 4, 16)


# ------------------------------------------------------------------ the five workloads

def _sample_rows(T, rng, n=48):
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 129, 255, 256, T // 2, T - 129, T - 128, T - 65,
             T - 64, T - 2, T - 1]
    rnd = rng.choice(T, size=n, replace=False).tolist()
    return sorted({r for r in fixed + rnd if 0 <= r < T})


def nan_outputs(cfg: AttnConfig, dtype):
    """O and LSE buffers filled with NaN, so that any element the kernels leave unwritten fails
    the comparison (and the finiteness check) instead of passing on leftover memory."""
    import torch

    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    o = torch.full((cfg.B, cfg.Hq, cfg.Tq, cfg.d), float("nan"), dtype=tdt, device="cuda")
    lse = torch.full((cfg.B, cfg.Hq, cfg.Tq), float("nan"), dtype=torch.float32, device="cuda")
    return o, lse


def whole_case(fa, cfg: AttnConfig):
    """Run the whole workload on the GPU into NaN-filled buffers and compare every element of O
    and LSE with the oracle; the mean-relative bound is taken over the whole tensor."""
    import torch

    _say(f"{cfg.name}: generating inputs")
    Q, K, V = inputs.make_inputs(cfg)
    q, k, v = (_to_dev(x, cfg.dtype) for x in (Q, K, V))
    o, lse = nan_outputs(cfg, cfg.dtype)
    _say(f"{cfg.name}: launching")
    fa.attn_fwd(q, k, v, causal=cfg.causal, scale=cfg.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    og = o.float().cpu().numpy().astype(np.float64)
    lg = lse.cpu().numpy().astype(np.float64)
    del q, k, v, o, lse
    _say(f"{cfg.name}: oracle on every head")
    o_ref, l_ref = oracle.dense_attention(Q, K, V, cfg.causal, cfg.scale)
    check(og, lg, o_ref, l_ref, cfg.dtype, cfg.name)


def sampled_case(fa, cfg: AttnConfig, heads=None):
    """Run the whole workload on the GPU into NaN-filled buffers; check that every element was
    written and is finite, and compare sampled rows of the given (b, h) heads (default: every
    head, with its own row sample) with the oracle, the mean-relative bound over all of them."""
    import torch

    _say(f"{cfg.name}: generating inputs")
    Q, K, V = inputs.make_inputs(cfg)
    q, k, v = (_to_dev(x, cfg.dtype) for x in (Q, K, V))
    o, l = nan_outputs(cfg, cfg.dtype)
    _say(f"{cfg.name}: launching")
    fa.attn_fwd(q, k, v, causal=cfg.causal, scale=cfg.scale, out=o, lse=l)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(l).all())
    if heads is None:
        heads = [(b, h) for b in range(cfg.B) for h in range(cfg.Hq)]
    rng = np.random.default_rng(cfg.seed + 1000)
    _say(f"{cfg.name}: oracle on sampled rows of {len(heads)} heads")
    og, lg, orf, lrf = [], [], [], []
    for (b, h) in heads:
        g = h // cfg.group
        rows = _sample_rows(cfg.Tq, rng)
        o_ref, l_ref = oracle.dense_head(Q[b, h], K[b, g], V[b, g], cfg.causal, cfg.scale,
                                         rows=rows)
        og.append(o[b, h, rows].float().cpu().numpy())
        lg.append(l[b, h, rows].cpu().numpy())
        orf.append(o_ref)
        lrf.append(l_ref)
    check(np.concatenate(og).astype(np.float64), np.concatenate(lg).astype(np.float64),
          np.concatenate(orf), np.concatenate(lrf), cfg.dtype, cfg.name)


def test_f32_causal_t128_d32_full(fa):
    full_case(fa, inputs.CONFIGS["f32_causal_b1_h4_t128_d32"])


def test_bf16_causal_t1024_d64_full(fa):
    full_case(fa, inputs.CONFIGS["bf16_causal_b4_h16_t1024_d64"])


@pytest.mark.parametrize("name", ["bf16_causal_b1_h32_t8192_d128", "bf16_noncausal_b1_h32_t4096_d128",
                                  "bf16_causal_b1_h32_t8000_d128"])
def test_bf16_t8192_shapes_whole(fa, name):
    # B=1, H=32, d=128: causal T=8192, its non-causal T=4096 variant and the ragged causal
    # T=8000, every element of O and LSE against the oracle
    whole_case(fa, inputs.CONFIGS[name])


def test_bf16_noncausal_t8000_whole(fa):
    cfg = inputs.CONFIGS["bf16_causal_b1_h32_t8000_d128"].replace(causal=False, name="noncausal t8000")
    whole_case(fa, cfg)


def test_gqa_decode_full(fa):
    import torch

    cfg = inputs.CONFIGS["bf16_gqa_decode_b64_hq64_hkv8_tk8192_d128"]
    _say(f"{cfg.name}: generating inputs")
    Q, K, V = inputs.make_inputs(cfg)
    o, l = run_gpu(fa, Q, K, V, cfg.causal, cfg.scale, cfg.dtype)
    _say(f"{cfg.name}: oracle")
    o_ref = np.empty_like(o)
    l_ref = np.empty_like(l)
    G = cfg.group
    for b in range(cfg.B):
        for g in range(cfg.Hkv):
            qs = Q[b, g * G:(g + 1) * G, 0, :]          # the group's queries as rows
            ob, lb = oracle.dense_head(qs, K[b, g], V[b, g], False, cfg.scale)
            o_ref[b, g * G:(g + 1) * G, 0] = ob
            l_ref[b, g * G:(g + 1) * G, 0] = lb
    check(o, l, o_ref, l_ref, cfg.dtype, cfg.name)


def test_gqa_causal_t16384_every_head_sampled(fa):
    # B=2, Hq=32, Hkv=8, T=16384: all 64 heads written (NaN-filled buffers), 66 sampled rows of
    # every head against the oracle
    sampled_case(fa, inputs.CONFIGS["bf16_gqa_causal_b2_hq32_hkv8_t16384_d128"])
