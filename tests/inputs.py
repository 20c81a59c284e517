"""Seeded synthetic inputs shared by the oracle checks, the GPU parity tests and the benchmark.

This module only draws random numbers and rounds them to the storage precision; it holds none of
the attention arithmetic, so both sides of a parity comparison can take their inputs from here
without sharing any of the method.

Recipe (every tensor is reproducible slice by slice):
  * one head slice ``[T, d]`` of tensor ``which`` (Q=0, K=1, V=2) at batch ``b``, head ``h`` is drawn
    from ``numpy.random.default_rng([seed, which, b, h])`` in float32;
  * distribution ``normal`` is N(0, 1); ``uniform08`` is U(-0.8, 0.8), the distribution of the lab
    generator on "Explain tiled attention and verify its output" (section "Read lab.py");
  * ``k_spike=(frac, factor)`` multiplies round(frac*T) K rows per (b, kv-head), chosen without
    replacement by ``default_rng([seed, 3, b, h])``, by ``factor`` before rounding (factor 8 is exact
    in both fp32 and bf16);
  * the upstream gradient dO of a backward case: slice [Tq, d] at (b, h) from
    ``default_rng([seed, 4, b, h])``, N(0, 1) whatever ``dist`` is, rounded like Q;
  * a paged cache (``make_paged``) holds the K and V above for sequences of given lengths: the
    logical blocks of all sequences are dealt to physical blocks in the order of a permutation
    from ``default_rng([seed, 5])``, a few spare blocks and the tails of partly filled blocks hold
    N(0, 1) filler that no visible position reads, and table entries past a sequence's last
    block name arbitrary valid blocks;
  * a packed batch (``make_packed``) of documents with lengths (Lq_b, Lk_b): the rows of document b,
    head h are ``head_slice`` of the config with Tq = Lq_b (Q) or Tk = Lk_b (K, V), laid out as
    [total, H, d] with cumulative offsets;
  * bf16 tensors are the float32 draws rounded to nearest-even; the oracle reads those same rounded
    values, widened exactly to float64.
"""

from __future__ import annotations

import dataclasses
import math
import random
from typing import Optional, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class AttnConfig:
    """One attention workload: shapes, dtype, mask, value distribution and seed."""

    name: str
    B: int
    Hq: int
    Hkv: int
    Tq: int
    Tk: int
    d: int
    dtype: str  # "f32" or "bf16"
    causal: bool
    dist: str  # "normal" or "uniform08"
    seed: int
    k_spike: Optional[Tuple[float, float]] = None

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    def replace(self, **kw) -> "AttnConfig":
        return dataclasses.replace(self, **kw)


# The five workloads the method is measured on, plus the two prefill variants of the T=8192 case.
CONFIGS = {
    "f32_causal_b1_h4_t128_d32": AttnConfig(
        "f32_causal_b1_h4_t128_d32", B=1, Hq=4, Hkv=4, Tq=128, Tk=128, d=32,
        dtype="f32", causal=True, dist="normal", seed=0),
    "bf16_causal_b4_h16_t1024_d64": AttnConfig(
        "bf16_causal_b4_h16_t1024_d64", B=4, Hq=16, Hkv=16, Tq=1024, Tk=1024, d=64,
        dtype="bf16", causal=True, dist="uniform08", seed=42),
    "bf16_causal_b1_h32_t8192_d128": AttnConfig(
        "bf16_causal_b1_h32_t8192_d128", B=1, Hq=32, Hkv=32, Tq=8192, Tk=8192, d=128,
        dtype="bf16", causal=True, dist="normal", seed=1),
    "bf16_noncausal_b1_h32_t4096_d128": AttnConfig(
        "bf16_noncausal_b1_h32_t4096_d128", B=1, Hq=32, Hkv=32, Tq=4096, Tk=4096, d=128,
        dtype="bf16", causal=False, dist="normal", seed=2),
    "bf16_causal_b1_h32_t8000_d128": AttnConfig(
        "bf16_causal_b1_h32_t8000_d128", B=1, Hq=32, Hkv=32, Tq=8000, Tk=8000, d=128,
        dtype="bf16", causal=True, dist="normal", seed=3),
    "bf16_gqa_decode_b64_hq64_hkv8_tk8192_d128": AttnConfig(
        "bf16_gqa_decode_b64_hq64_hkv8_tk8192_d128", B=64, Hq=64, Hkv=8, Tq=1, Tk=8192, d=128,
        dtype="bf16", causal=False, dist="normal", seed=4),
    "bf16_gqa_causal_b2_hq32_hkv8_t16384_d128": AttnConfig(
        "bf16_gqa_causal_b2_hq32_hkv8_t16384_d128", B=2, Hq=32, Hkv=8, Tq=16384, Tk=16384, d=128,
        dtype="bf16", causal=True, dist="normal", seed=5, k_spike=(0.01, 8.0)),
}

Q_ID, K_ID, V_ID = 0, 1, 2
SPIKE_ID, DO_ID, PAGE_ID = 3, 4, 5


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32 holding them."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = ((u + bias) & np.uint32(0xFFFF0000)).astype(np.uint32)
    return r.view(np.float32)


def bf16_bits(x_rounded: np.ndarray) -> np.ndarray:
    """The uint16 bit patterns of float32 values that are already exact bfloat16 values."""
    u = np.ascontiguousarray(x_rounded, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def _draw(rng: np.random.Generator, dist: str, shape) -> np.ndarray:
    if dist == "normal":
        return rng.standard_normal(shape, dtype=np.float32)
    if dist == "uniform08":
        return rng.uniform(-0.8, 0.8, size=shape).astype(np.float32)
    raise ValueError(f"unknown distribution {dist!r}")


def head_slice(cfg: AttnConfig, which: int, b: int, h: int) -> np.ndarray:
    """One [T, d] float32 slice (already rounded when the config is bf16)."""
    T = cfg.Tq if which == Q_ID else cfg.Tk
    rng = np.random.default_rng([cfg.seed, which, b, h])
    x = _draw(rng, cfg.dist, (T, cfg.d))
    if which == K_ID and cfg.k_spike is not None:
        frac, factor = cfg.k_spike
        n = int(round(frac * T))
        if n > 0:
            pick = np.random.default_rng([cfg.seed, SPIKE_ID, b, h]).choice(T, size=n, replace=False)
            x[pick] *= np.float32(factor)
    if cfg.dtype == "bf16":
        x = round_to_bf16(x)
    return x


def make_inputs(cfg: AttnConfig):
    """Full Q [B,Hq,Tq,d], K and V [B,Hkv,Tk,d] as float32 arrays (bf16-exact when bf16)."""
    Q = np.empty((cfg.B, cfg.Hq, cfg.Tq, cfg.d), np.float32)
    K = np.empty((cfg.B, cfg.Hkv, cfg.Tk, cfg.d), np.float32)
    V = np.empty((cfg.B, cfg.Hkv, cfg.Tk, cfg.d), np.float32)
    for b in range(cfg.B):
        for h in range(cfg.Hq):
            Q[b, h] = head_slice(cfg, Q_ID, b, h)
        for h in range(cfg.Hkv):
            K[b, h] = head_slice(cfg, K_ID, b, h)
            V[b, h] = head_slice(cfg, V_ID, b, h)
    return Q, K, V


def grad_slice(cfg: AttnConfig, b: int, h: int) -> np.ndarray:
    """One [Tq, d] float32 slice of the upstream gradient dO (rounded when the config is bf16)."""
    x = np.random.default_rng([cfg.seed, DO_ID, b, h]).standard_normal((cfg.Tq, cfg.d),
                                                                      dtype=np.float32)
    return round_to_bf16(x) if cfg.dtype == "bf16" else x


def make_grad(cfg: AttnConfig) -> np.ndarray:
    """The upstream gradient dO [B, Hq, Tq, d] of a backward case."""
    dO = np.empty((cfg.B, cfg.Hq, cfg.Tq, cfg.d), np.float32)
    for b in range(cfg.B):
        for h in range(cfg.Hq):
            dO[b, h] = grad_slice(cfg, b, h)
    return dO


def make_paged(cfg: AttnConfig, block_size: int, seq_lens, spare: int = 3):
    """A paged cache holding the K, V of ``cfg`` (Tk = the longest sequence) for sequences of the
    given lengths. Returns (K_cache, V_cache [num_blocks, Hkv, block_size, d] float32,
    block_table [B, max_blocks] int32, seq_lens [B] int32)."""
    _, K, V = make_inputs(cfg)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    bs = int(block_size)
    max_blocks = max(1, -(-cfg.Tk // bs))
    need = [-(-int(n) // bs) for n in seq_lens]
    num_blocks = sum(need) + spare
    rng = np.random.default_rng([cfg.seed, PAGE_ID])
    perm = rng.permutation(num_blocks)
    shape = (num_blocks, cfg.Hkv, bs, cfg.d)
    Kc = rng.standard_normal(shape, dtype=np.float32)
    Vc = rng.standard_normal(shape, dtype=np.float32)
    if cfg.dtype == "bf16":
        Kc, Vc = round_to_bf16(Kc), round_to_bf16(Vc)
    table = rng.integers(0, num_blocks, size=(cfg.B, max_blocks)).astype(np.int32)
    n = 0
    for b in range(cfg.B):
        for i in range(need[b]):
            blk = int(perm[n])
            n += 1
            table[b, i] = blk
            rows = min(bs, int(seq_lens[b]) - i * bs)
            Kc[blk, :, :rows] = K[b, :, i * bs:i * bs + rows]
            Vc[blk, :, :rows] = V[b, :, i * bs:i * bs + rows]
    return Kc, Vc, table, seq_lens


def make_packed(cfg: AttnConfig, lens_q, lens_k=None):
    """Packed Q [total_q, Hq, d], K, V [total_k, Hkv, d] (float32) and int32 cumulative offsets
    cu_q, cu_k [n + 1] for documents of the given lengths (lens_k defaults to lens_q)."""
    lens_q = [int(x) for x in lens_q]
    lens_k = lens_q if lens_k is None else [int(x) for x in lens_k]
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    Q = np.empty((int(cu_q[-1]), cfg.Hq, cfg.d), np.float32)
    K = np.empty((int(cu_k[-1]), cfg.Hkv, cfg.d), np.float32)
    V = np.empty((int(cu_k[-1]), cfg.Hkv, cfg.d), np.float32)
    for b, (lq, lk) in enumerate(zip(lens_q, lens_k)):
        c = cfg.replace(Tq=max(lq, 1), Tk=max(lk, 1))
        for h in range(cfg.Hq):
            Q[cu_q[b]:cu_q[b + 1], h] = head_slice(c, Q_ID, b, h)[:lq]
        for h in range(cfg.Hkv):
            K[cu_k[b]:cu_k[b + 1], h] = head_slice(c, K_ID, b, h)[:lk]
            V[cu_k[b]:cu_k[b + 1], h] = head_slice(c, V_ID, b, h)[:lk]
    return Q, K, V, cu_q, cu_k


def to_torch(x: np.ndarray, dtype: str, device=None):
    """Wrap a float32 array as a torch tensor of the config dtype (bit-exact for bf16)."""
    import torch

    if dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    elif dtype == "bf16":
        t = torch.from_numpy(bf16_bits(x).view(np.int16)).view(torch.bfloat16)
    else:
        raise ValueError(dtype)
    return t if device is None else t.to(device)


def lab_qkv(seq_len: int, head_dim: int, seed: int = 42):
    """The lab generator on "Explain tiled attention and verify its output" (section "Read lab.py").

    A ``random.Random(seed)`` stream draws q, then k, then v, row by row, each element from
    U(-0.8, 0.8). Returns three float64 arrays of shape [seq_len, head_dim].
    """
    rng = random.Random(seed)
    out = []
    for _ in range(3):
        out.append(np.array([[rng.uniform(-0.8, 0.8) for _ in range(head_dim)]
                             for _ in range(seq_len)], dtype=np.float64))
    return out[0], out[1], out[2]
