"""GPU parity of paged-KV decode (attn_fwd_paged) against the fp64 oracle.

Bounds as for every bf16 case: max abs error <= 2e-2 and mean-relative error <= 1e-2 on O and
on LSE. Caches come from ``tests.inputs.make_paged``: physical blocks in a seeded random order,
filler in unreferenced blocks and block tails, table entries past each sequence naming valid
blocks that must not be read.
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
    print(f"[paged] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def fa():
    import torch

    assert torch.cuda.is_available(), "GPU parity tests need a GPU"
    import io_aware_tiled_amd as fa

    return fa


def _cfg(B, Hq, Hkv, Tk, d, seed=7):
    return AttnConfig("paged", B=B, Hq=Hq, Hkv=Hkv, Tq=1, Tk=Tk, d=d, dtype="bf16",
                      causal=False, dist="normal", seed=seed)


def _dev(x):
    return inputs.to_torch(x, "bf16", "cuda")


def run_paged(fa, Q, Kc, Vc, table, lens, scale):
    import torch

    o, l = fa.attn_fwd_paged(_dev(Q[:, :, 0]), _dev(Kc), _dev(Vc),
                             torch.from_numpy(np.ascontiguousarray(table)).cuda(),
                             torch.from_numpy(np.ascontiguousarray(lens)).cuda(), scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), l.cpu().numpy().astype(np.float64)


def paged_case(fa, cfg, bs, lens, scale=None):
    sc = cfg.scale if scale is None else scale
    Q, _, _ = inputs.make_inputs(cfg)
    Kc, Vc, table, sl = inputs.make_paged(cfg, bs, lens)
    o, l = run_paged(fa, Q, Kc, Vc, table, sl, sc)
    o_ref, l_ref = oracle.paged_decode(Q[:, :, 0], Kc, Vc, table, sl, sc)
    check(o, l, o_ref, l_ref, "bf16", f"paged bs={bs} lens={list(lens)[:6]}")


@pytest.mark.parametrize("bs", [16, 32, 64, 256])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_block_sizes_and_ragged_lengths(fa, d, bs):
    cfg = _cfg(5, 8, 2, 700, d, seed=d + bs)
    lens = [700, 1, 17, 333, 256]
    _say(f"d={d} bs={bs}")
    paged_case(fa, cfg, bs, lens)


@pytest.mark.parametrize("G", [1, 4, 16, 32])
def test_gqa_groups(fa, G):
    cfg = _cfg(3, 2 * G, 2, 400, 128, seed=G)
    _say(f"G={G}")
    paged_case(fa, cfg, 16, [400, 31, 129])


@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.7])
def test_scales(fa, scale):
    paged_case(fa, _cfg(2, 4, 1, 300, 64, seed=3), 32, [300, 77], scale=scale)


def test_empty_sequence(fa):
    cfg = _cfg(3, 4, 2, 100, 64, seed=11)
    Q, _, _ = inputs.make_inputs(cfg)
    Kc, Vc, table, sl = inputs.make_paged(cfg, 16, [100, 0, 5])
    o, l = run_paged(fa, Q, Kc, Vc, table, sl, cfg.scale)
    assert not o[1].any() and np.all(np.isneginf(l[1]))
    o_ref, l_ref = oracle.paged_decode(Q[:, :, 0], Kc, Vc, table, sl, cfg.scale)
    keep = [0, 2]
    check(o[keep], l[keep], o_ref[keep], l_ref[keep], "bf16", "paged with an empty sequence")


def test_out_of_range_table_entries_read_as_zero_rows(fa):
    # The library never dereferences a table entry outside [0, num_blocks): those positions act
    # as zero keys and values. The reference is the oracle on the cache with those rows zeroed.
    cfg = _cfg(2, 4, 2, 96, 64, seed=13)
    Q, K, V = inputs.make_inputs(cfg)
    Kc, Vc, table, sl = inputs.make_paged(cfg, 16, [96, 96])
    table = table.copy()
    table[0, 2] = -7
    table[1, 4] = Kc.shape[0] + 100
    o, l = run_paged(fa, Q, Kc, Vc, table, sl, cfg.scale)
    K0, V0 = K.copy(), V.copy()
    K0[0, :, 32:48] = 0
    V0[0, :, 32:48] = 0
    K0[1, :, 64:80] = 0
    V0[1, :, 64:80] = 0
    o_ref, l_ref = oracle.dense_attention(Q, K0, V0, False, cfg.scale)
    check(o, l, o_ref[:, :, 0], l_ref[:, :, 0], "bf16", "invalid table entries")


def test_bitwise_equal_to_the_contiguous_decode(fa):
    # Same kernel, same split plan: a paged cache of full sequences gives the contiguous result
    # bit for bit.
    import torch

    cfg = _cfg(4, 16, 2, 1024, 128, seed=21)
    Q, K, V = inputs.make_inputs(cfg)
    Kc, Vc, table, sl = inputs.make_paged(cfg, 64, [1024] * 4)
    o_p, l_p = fa.attn_fwd_paged(_dev(Q[:, :, 0]), _dev(Kc), _dev(Vc),
                                 torch.from_numpy(table).cuda(), torch.from_numpy(sl).cuda())
    o_c, l_c = fa.attn_fwd(_dev(Q), _dev(K), _dev(V), causal=False)
    torch.cuda.synchronize()
    assert torch.equal(o_p.view(torch.int16), o_c[:, :, 0].view(torch.int16))
    assert torch.equal(l_p, l_c[:, :, 0])


def test_workload_gqa_decode_paged_full(fa):
    # The GQA decode workload (B=64, Hq=64, Hkv=8, 8192 cached positions, d=128) in 16-position
    # pages, every output against the oracle.
    cfg = inputs.CONFIGS["bf16_gqa_decode_b64_hq64_hkv8_tk8192_d128"]
    _say("gqa decode paged: inputs")
    paged_case(fa, cfg, 16, [8192] * cfg.B)


def test_workload_gqa_decode_paged_ragged(fa):
    cfg = inputs.CONFIGS["bf16_gqa_decode_b64_hq64_hkv8_tk8192_d128"].replace(B=16, name="gqa decode ragged lengths")
    lens = np.random.default_rng(99).integers(1, 8193, size=16)
    lens[0], lens[1] = 8192, 1
    _say("gqa decode paged ragged")
    paged_case(fa, cfg, 16, lens)
