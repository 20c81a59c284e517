"""Launch-configuration sweep for libfattn (the source of the table in csrc/tune_table.h).

    python -m io_aware_tiled_amd.tune [--reps N] [--shapes prefill,decode]

Times every prefill configuration (block_kv x waves x schedule) on causal and non-causal bf16
prefill shapes for d = 64 and d = 128, and every decode split count on the GQA decode shape,
with HIP events on the launch stream; prints one JSON line per (shape, configuration) and a
summary of the fastest configuration per shape. Inputs are seeded N(0, 1) draws in bf16.
Correctness of every configuration is covered by the parity tests; this tool only times.
"""

from __future__ import annotations

import argparse
import json
import math
import sys

import torch

import io_aware_tiled_amd as fa

PREFILL_SHAPES = [
    # B, Hq, Hkv, T, d, causal
    (1, 32, 32, 8192, 128, True),
    (1, 32, 32, 8192, 128, False),
    (1, 32, 32, 4096, 128, True),
    (1, 32, 32, 4096, 128, False),
    (4, 32, 32, 2048, 128, True),
    (16, 32, 32, 1024, 128, True),
    (16, 32, 32, 1024, 128, False),
    (2, 32, 8, 16384, 128, True),
    (4, 16, 16, 1024, 64, True),
    (4, 16, 16, 1024, 64, False),
    (16, 32, 32, 1024, 64, True),
    (2, 32, 32, 8192, 64, True),
    (2, 32, 32, 8192, 64, False),
]
DECODE_SHAPES = [
    # B, Hq, Hkv, Tk, d
    (64, 64, 8, 8192, 128),
    (16, 32, 8, 32768, 128),
    (64, 32, 8, 4096, 64),
]


def _time(fn, reps):
    fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(reps):
        fn()
    ev[1].record()
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[1]) / reps


def sweep_prefill(reps):
    best = {}
    g = torch.Generator(device="cuda").manual_seed(0)
    for (B, Hq, Hkv, T, d, causal) in PREFILL_SHAPES:
        q = torch.randn(B, Hq, T, d, device="cuda", generator=g).to(torch.bfloat16)
        k = torch.randn(B, Hkv, T, d, device="cuda", generator=g).to(torch.bfloat16)
        v = torch.randn(B, Hkv, T, d, device="cuda", generator=g).to(torch.bfloat16)
        o, lse = torch.empty_like(q), torch.empty(B, Hq, T, device="cuda")
        flops = 4.0 * B * Hq * T * T * d / (2 if causal else 1)
        for bc in (32, 64):
            for nw in (4, 8):
                for sch in (1, 2):
                    cfg = dict(kernel=fa.FATTN_KERNEL_PREFILL_MFMA, block_kv=bc, waves=nw,
                               schedule=sch)
                    ms = _time(lambda: fa.attn_fwd(q, k, v, causal=causal, out=o, lse=lse,
                                                   cfg=cfg), reps)
                    rec = {"shape": [B, Hq, Hkv, T, d, int(causal)], "cfg": cfg, "ms": round(ms, 4),
                           "tflops": round(flops / ms / 1e9, 1)}
                    print(json.dumps(rec), flush=True)
                    key = tuple(rec["shape"])
                    if key not in best or ms < best[key]["ms"]:
                        best[key] = rec
        del q, k, v, o, lse
    return best


def sweep_decode(reps):
    best = {}
    g = torch.Generator(device="cuda").manual_seed(1)
    for (B, Hq, Hkv, Tk, d) in DECODE_SHAPES:
        q = torch.randn(B, Hq, 1, d, device="cuda", generator=g).to(torch.bfloat16)
        k = torch.randn(B, Hkv, Tk, d, device="cuda", generator=g).to(torch.bfloat16)
        v = torch.randn(B, Hkv, Tk, d, device="cuda", generator=g).to(torch.bfloat16)
        o, lse = torch.empty_like(q), torch.empty(B, Hq, 1, device="cuda")
        nbytes = (2 * B * Hkv * Tk * d + 2 * B * Hq * d) * 2 + 4 * B * Hq
        for splits in (1, 2, 4, 8, 16, 32):
            cfg = dict(kernel=fa.FATTN_KERNEL_DECODE_SPLITK, splits=splits)
            ms = _time(lambda: fa.attn_fwd(q, k, v, out=o, lse=lse, cfg=cfg), reps)
            rec = {"shape": [B, Hq, Hkv, Tk, d], "cfg": cfg, "ms": round(ms, 4),
                   "gbs": round(nbytes / ms / 1e6, 1)}
            print(json.dumps(rec), flush=True)
            key = tuple(rec["shape"])
            if key not in best or ms < best[key]["ms"]:
                best[key] = rec
        del q, k, v, o, lse
    return best


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--shapes", default="prefill,decode")
    args = ap.parse_args()
    torch.cuda.set_device(0)
    best = {}
    if "prefill" in args.shapes:
        best.update(sweep_prefill(args.reps))
    if "decode" in args.shapes:
        best.update(sweep_decode(args.reps))
    print("best per shape:", file=sys.stderr)
    for key, rec in best.items():
        print(json.dumps({"best": rec}), flush=True)


if __name__ == "__main__":
    main()
