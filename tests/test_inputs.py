"""Checks of the seeded input generators (CPU only)."""

import numpy as np
import pytest

from tests import inputs


def test_bf16_rounding_matches_torch():
    import torch

    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 7
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 3.0]   # exact ties and an exact value
    ours = inputs.round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours, ref)
    bits = inputs.bf16_bits(ours)
    back = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(back, ours)


def test_slices_are_reproducible_and_distinct():
    cfg = inputs.CONFIGS["bf16_causal_b4_h16_t1024_d64"]
    a = inputs.head_slice(cfg, inputs.Q_ID, 1, 3)
    b = inputs.head_slice(cfg, inputs.Q_ID, 1, 3)
    c = inputs.head_slice(cfg, inputs.K_ID, 1, 3)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert a.shape == (1024, 64) and np.all(np.abs(a) <= 0.8 * (1 + 2.0 ** -8))
    assert np.array_equal(inputs.round_to_bf16(a), a)


def test_k_spikes():
    cfg = inputs.CONFIGS["bf16_gqa_causal_b2_hq32_hkv8_t16384_d128"].replace(Tq=1000, Tk=1000)
    k = inputs.head_slice(cfg, inputs.K_ID, 0, 1)
    plain = inputs.head_slice(cfg.replace(k_spike=None), inputs.K_ID, 0, 1)
    changed = np.nonzero(np.any(k != plain, axis=1))[0]
    assert len(changed) == 10
    assert np.array_equal(k[changed], plain[changed] * 8)


def test_lab_generator_order():
    q, k, v = inputs.lab_qkv(2, 3, seed=42)
    import random

    rng = random.Random(42)
    flat = [rng.uniform(-0.8, 0.8) for _ in range(18)]
    assert np.array_equal(np.concatenate([q.ravel(), k.ravel(), v.ravel()]), flat)


@pytest.mark.parametrize("name", list(inputs.CONFIGS))
def test_configs_are_consistent(name):
    cfg = inputs.CONFIGS[name]
    assert cfg.Hq % cfg.Hkv == 0
    assert (not cfg.causal) or cfg.Tq <= cfg.Tk
