"""Pins of the oracle's accounting to the numbers the pages print (CPU only)."""

import json
import os

import pytest

from oracle import accounting as acc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_logical_access_sweep_reproduces_the_lab():
    g = _golden("lab_recorded_result.json")
    p = g["sweep_model_parameters"]
    for rec in g["hbm_traffic_sweep"]:
        got = acc.logical_access_model(rec["seq_len"], rec["num_heads"], rec["head_dim"],
                                       p["bytes_per_elem"], p["block_q"])
        for key, val in got.items():
            assert val == rec[key], key


def test_access_count_exceeds_compulsory_and_grows_superlinearly():
    g = _golden("lab_checks.json")["access_count"]
    small = acc.logical_access_model(g["small_seq_len"])
    large = acc.logical_access_model(g["large_seq_len"])
    assert small["tiled_logical_access_mb_no_cache_reuse"] > small["qkvo_compulsory_bytes_mb"]
    ratio = (large["tiled_logical_access_mb_no_cache_reuse"]
             / small["tiled_logical_access_mb_no_cache_reuse"])
    assert ratio > g["large_over_small_ratio_above"]


def test_memory_exercise():
    g = _golden("memory_exercise.json")
    a = g["answers_worked_by_hand"]
    s = acc.score_matrix_bytes(g["N"], g["dtype_bytes"])
    o = acc.saved_output_bytes(g["N"], g["d"], g["dtype_bytes"], g["lse_bytes"])
    assert s == a["score_matrix_bytes"]
    assert o == a["o_plus_l_bytes"]
    assert round(s / o, 2) == a["ratio"]
    assert g["M_elements"] // g["d"] ** 2 == a["reduction_factor_M_over_d2"]


def test_notebook_intensity_checks():
    # "Attention from scratch + roofline": AI doubles with T; prefill above the quoted ridges,
    # decode below 20 FLOP/byte
    r = acc.arithmetic_intensity(1, 32, 2048, 128) / acc.arithmetic_intensity(1, 32, 1024, 128)
    assert 1.8 <= r <= 2.2
    assert acc.arithmetic_intensity(1, 32, 1024, 128) > 203
    assert acc.decode_intensity(1, 8, 8, 128, 2048) < 20
    # exercise 1: with a quarter of the kv heads decode intensity rises about fourfold
    mha = acc.decode_intensity(1, 32, 32, 128, 8192)
    gqa = acc.decode_intensity(1, 32, 8, 128, 8192)
    assert gqa / mha == pytest.approx(4.0, rel=1e-3)


def test_causal_halving_convention_against_exact_pair_count():
    exact = acc.attention_flops_exact(1, 32, 8192, 8192, 128, True)
    halved = acc.attention_flops(1, 32, 8192, 8192, 128, True)
    assert exact / halved == pytest.approx(1 + 1 / 8192, rel=1e-12)
    assert acc.visible_pairs(4, 4, True) == 10
    assert acc.visible_pairs(1, 9, True) == 9
    assert acc.visible_pairs(3, 5, True) == 3 + 4 + 5


def test_decode_bytes_of_gqa_step():
    # K and V of 64 x 8 heads x 8192 keys x 128 dims in bf16 dominate: 2.1475 GB
    b = acc.decode_bytes(64, 64, 8, 8192, 128)
    assert b == 2 * 64 * 8 * 8192 * 128 * 2 + 2 * 64 * 64 * 128 * 2 + 4 * 64 * 64
    assert round(b / 1e9, 4) == 2.1496


def test_prefill_compulsory_bytes():
    # B=1, H=32, T=8192, d=128 bf16: Q, K, V read once and O written (4 x 64 MiB) plus the fp32
    # LSE (1 MiB) = 269.48 MB. Under GQA only K and V shrink with the kv head count, and the
    # byte count is linear in the element size except for the fp32 LSE.
    assert acc.prefill_compulsory_bytes(1, 32, 32, 8192, 8192, 128) == 4 * 2**26 + 2**20
    full = acc.prefill_compulsory_bytes(2, 32, 32, 4096, 4096, 128)
    gqa = acc.prefill_compulsory_bytes(2, 32, 8, 4096, 4096, 128)
    kv_mha = 2 * 2 * 32 * 4096 * 128 * 2
    assert full - gqa == kv_mha - kv_mha // 4
    lse = 4 * 2 * 32 * 4096
    assert acc.prefill_compulsory_bytes(2, 32, 8, 4096, 4096, 128, dtype_bytes=4) - lse == \
        2 * (gqa - lse)
    # the attention_bytes model (Q, K, V, O of equal length, MHA) agrees without the LSE
    assert acc.attention_bytes(2, 32, 4096, 128) == full - lse


# ---- the same figures by routes that do not restate the formulas

def _bytes_of(*tensors):
    return sum(t.numel() * t.element_size() for t in tensors)


def _call_tensors(B, Hq, Hkv, Tq, Tk, d, device):
    """Every tensor one forward call reads or writes, as the binding allocates them: bf16 Q, K,
    V and O of the (B, H, T, d) layout and the fp32 LSE."""
    import torch

    bf = torch.bfloat16
    return (torch.empty(B, Hq, Tq, d, dtype=bf, device=device),
            torch.empty(B, Hkv, Tk, d, dtype=bf, device=device),
            torch.empty(B, Hkv, Tk, d, dtype=bf, device=device),
            torch.empty(B, Hq, Tq, d, dtype=bf, device=device),
            torch.empty(B, Hq, Tq, dtype=torch.float32, device=device))


def test_decode_bytes_are_the_bytes_of_the_generated_tensors():
    # a small GQA decode built by the seeded generator, converted to the bf16 tensors the GPU
    # receives, plus the O and LSE the binding allocates
    import torch

    from tests import inputs

    cfg = inputs.CONFIGS["bf16_gqa_decode_b64_hq64_hkv8_tk8192_d128"].replace(B=3, Tk=257)
    q, k, v = (inputs.to_torch(x, "bf16") for x in inputs.make_inputs(cfg))
    o = torch.empty_like(q)
    lse = torch.empty(cfg.B, cfg.Hq, cfg.Tq, dtype=torch.float32)
    assert _bytes_of(q, k, v, o, lse) == acc.decode_bytes(3, 64, 8, 257, 128)
    # the full GQA decode, by the sizes of meta tensors of its shapes (nothing is allocated)
    full = _call_tensors(64, 64, 8, 1, 8192, 128, "meta")
    assert _bytes_of(*full) == acc.decode_bytes(64, 64, 8, 8192, 128) == 2149597184


@pytest.mark.parametrize("shape", [(1, 32, 32, 8192, 8192, 128), (2, 32, 8, 16384, 16384, 128),
                                   (4, 16, 16, 1024, 1024, 64), (3, 8, 2, 5, 77, 32)])
def test_prefill_compulsory_bytes_are_the_bytes_of_the_call_tensors(shape):
    B, Hq, Hkv, Tq, Tk, d = shape
    assert _bytes_of(*_call_tensors(B, Hq, Hkv, Tq, Tk, d, "meta")) == \
        acc.prefill_compulsory_bytes(B, Hq, Hkv, Tq, Tk, d)


def test_prefill_compulsory_bytes_of_generated_inputs():
    import torch

    from tests import inputs

    cfg = inputs.CONFIGS["bf16_gqa_causal_b2_hq32_hkv8_t16384_d128"].replace(Tq=96, Tk=96)
    q, k, v = (inputs.to_torch(x, "bf16") for x in inputs.make_inputs(cfg))
    lse = torch.empty(cfg.B, cfg.Hq, cfg.Tq, dtype=torch.float32)
    assert _bytes_of(q, k, v, torch.empty_like(q), lse) == \
        acc.prefill_compulsory_bytes(2, 32, 8, 96, 96, 128)


@pytest.mark.parametrize("Tq,Tk", [(1, 1), (7, 7), (64, 64), (5, 77), (300, 301)])
def test_visible_pairs_by_brute_force_mask(Tq, Tk):
    # count the entries a bottom-right causal mask keeps, with the mask built element by element
    kept = sum(1 for i in range(Tq) for j in range(Tk) if j <= i + Tk - Tq)
    assert acc.visible_pairs(Tq, Tk, True) == kept
    assert acc.visible_pairs(Tq, Tk, False) == Tq * Tk
    for W in (1, 3, 50):
        kept_w = sum(1 for i in range(Tq) for j in range(Tk)
                     if i + Tk - Tq - W < j <= i + Tk - Tq)
        assert acc.visible_pairs(Tq, Tk, True, W) == kept_w


@pytest.mark.parametrize("shape", [(1, 32, 8192, 128), (2, 32, 16384, 128), (4, 16, 1024, 64),
                                   (1, 2, 5, 8)])
def test_backward_flops_from_visible_pairs(shape):
    # five products (S, dP, dV, dK, dQ), each one multiply-add of d terms per visible pair:
    # 10 d FLOPs per pair. Without a mask every pair is visible; with it the causal-halved
    # convention counts T^2 / 2 pairs against the T (T + 1) / 2 a square causal mask keeps.
    import oracle

    B, H, T, d = shape
    pairs_full = B * H * T * T
    assert oracle.backward_flops(B, H, T, T, d, False) == 10 * d * pairs_full
    pairs_causal = B * H * acc.visible_pairs(T, T, True)
    assert oracle.backward_flops(B, H, T, T, d, True) * (T + 1) == 10 * d * pairs_causal * T
