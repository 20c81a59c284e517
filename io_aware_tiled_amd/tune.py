"""Launch-configuration sweep for libfattn and the generator of its table (csrc/tune_table.h).

    python -m io_aware_tiled_amd.tune sweep [--rounds N] [--out PATH]   # GPU: time, write JSON
    python -m io_aware_tiled_amd.tune emit [--sweep PATH] [--out PATH]  # CPU: JSON -> header
    python -m io_aware_tiled_amd.tune check [--sweep PATH]              # CPU: header up to date?
    python -m io_aware_tiled_amd.tune rates [--out PATH]                # GPU: rates across shapes

The block size is a performance choice, not a numerical one: every configuration computes the
same function (the parity tests run each one), so the table only records which one is fastest.

`sweep` times every prefill configuration (keys per tile x waves per workgroup x grid order) on
the shapes of PREFILL_SHAPES and every split count on DECODE_SHAPES, with HIP events on the launch
stream. Each shape's configurations are timed round-robin, `rounds` times over, and the median
of the rounds is kept, so a drift of the clock during the sweep does not favour whichever
configuration ran first. Inputs are seeded N(0, 1) draws in bf16. The record (every timing, the
device, the library's source hashes) goes to tune_sweep.json beside this file.

`emit` turns that record into csrc/tune_table.h without a GPU. For each head dim and mask, the
swept shapes are ordered by key length, and at one key length by batch x heads, largest first;
every shape contributes the row "Tk <= its key length (and B*Hq >= its batch x heads, unless it is
the smallest at that length) -> its fastest configuration", the largest key length's rows
covering every longer one. Consecutive rows that pick the same configuration without a batch
bound are merged. d = 32 (no sweep: one configuration serves it) and the decode targets are fixed
and written as they are. `check` regenerates the header and compares it with the file.

`rates` times attn_fwd and attn_bwd with the table's configurations on the shapes of RATE_SHAPES
(B*T = 16384 tokens, 32 heads) and writes a markdown table.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SWEEP_PATH = os.path.join(HERE, "tune_sweep.json")
HEADER_PATH = os.path.join(HERE, "csrc", "tune_table.h")

PREFILL_SHAPES = [
    # B, Hq, Hkv, T, d, causal
    (16, 32, 32, 1024, 128, True),
    (4, 32, 32, 2048, 128, True),
    (1, 32, 32, 4096, 128, True),
    (1, 32, 32, 8192, 128, True),
    (2, 32, 8, 16384, 128, True),
    (16, 32, 32, 1024, 128, False),
    (1, 32, 32, 4096, 128, False),
    (1, 32, 32, 8192, 128, False),
    (16, 32, 32, 1024, 64, True),
    (4, 16, 16, 1024, 64, True),
    (2, 32, 32, 8192, 64, True),
    (4, 16, 16, 1024, 64, False),
    (2, 32, 32, 8192, 64, False),
]
DECODE_SHAPES = [
    # B, Hq, Hkv, Tk, d
    (64, 64, 8, 8192, 128),
    (16, 32, 8, 32768, 128),
    (64, 32, 8, 4096, 64),
]
RATE_SHAPES = [(16384 // T, 32, 32, T, d, c) for d in (64, 128) for T in (1024, 2048, 4096, 8192, 16384)
               for c in (True, False)]
SOURCES = ["prefill_bf16.hip", "decode_bf16.hip", "backward_bf16.hip", "api.cpp"]

# every prefill configuration the kernels implement (paired blocks need 8 waves)
PREFILL_CFGS = [(bc, nw, sch) for bc in (64, 32) for nw in (8, 4) for sch in (2, 4, 1)
                if sch != 4 or nw == 8]
DECODE_SPLITS = (1, 2, 4, 8, 16, 32)

# fixed rows of the generated header
D32_ROW = (32, -1, 0, 0, 64, 4, 2)
DECODE_ROWS = [(128, 2048, 256), (64, 2048, 256), (32, 2048, 256)]


def _source_hashes():
    out = {}
    for name in SOURCES:
        with open(os.path.join(HERE, "csrc", name), "rb") as f:
            out[name] = hashlib.sha256(f.read()).hexdigest()[:16]
    return out


# ------------------------------------------------------------------------------ GPU: timing

def _time(torch, fn, reps):
    fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(reps):
        fn()
    ev[1].record()
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[1]) / reps


def _warm(torch, fn, ms=300.0):
    """Back-to-back calls until `ms` of GPU time has run (the clock leaves its idle state)."""
    spent = 0.0
    while spent < ms:
        spent += _time(torch, fn, 10) * 10


def sweep(rounds, reps, out_path):
    import torch

    import io_aware_tiled_amd as fa

    torch.cuda.set_device(0)
    records = []
    g = torch.Generator(device="cuda").manual_seed(0)
    for (B, Hq, Hkv, T, d, causal) in PREFILL_SHAPES:
        q = torch.randn(B, Hq, T, d, device="cuda", generator=g).to(torch.bfloat16)
        k = torch.randn(B, Hkv, T, d, device="cuda", generator=g).to(torch.bfloat16)
        v = torch.randn(B, Hkv, T, d, device="cuda", generator=g).to(torch.bfloat16)
        o, lse = torch.empty_like(q), torch.empty(B, Hq, T, device="cuda")
        flops = 4.0 * B * Hq * T * T * d / (2 if causal else 1)
        calls = {}
        for (bc, nw, sch) in PREFILL_CFGS:
            cfg = dict(kernel=fa.FATTN_KERNEL_PREFILL_MFMA, block_kv=bc, waves=nw, schedule=sch)
            calls[(bc, nw, sch)] = (lambda cfg=cfg: fa.attn_fwd(q, k, v, causal=causal, out=o,
                                                                lse=lse, cfg=cfg))
        _warm(torch, next(iter(calls.values())))
        times = {key: [] for key in calls}
        for _ in range(rounds):
            for key, fn in calls.items():
                times[key].append(_time(torch, fn, reps))
        for (bc, nw, sch), ts in times.items():
            ms = statistics.median(ts)
            rec = {"kind": "prefill", "shape": [B, Hq, Hkv, T, d, int(causal)],
                   "cfg": [bc, nw, sch], "ms": round(ms, 5), "ms_rounds": [round(t, 5) for t in ts],
                   "tflops": round(flops / ms / 1e9, 1)}
            records.append(rec)
            print(json.dumps(rec), flush=True)
        del q, k, v, o, lse
    g = torch.Generator(device="cuda").manual_seed(1)
    for (B, Hq, Hkv, Tk, d) in DECODE_SHAPES:
        q = torch.randn(B, Hq, 1, d, device="cuda", generator=g).to(torch.bfloat16)
        k = torch.randn(B, Hkv, Tk, d, device="cuda", generator=g).to(torch.bfloat16)
        v = torch.randn(B, Hkv, Tk, d, device="cuda", generator=g).to(torch.bfloat16)
        o, lse = torch.empty_like(q), torch.empty(B, Hq, 1, device="cuda")
        nbytes = (2 * B * Hkv * Tk * d + 2 * B * Hq * d) * 2 + 4 * B * Hq
        calls = {s: (lambda s=s: fa.attn_fwd(q, k, v, out=o, lse=lse,
                                             cfg=dict(kernel=fa.FATTN_KERNEL_DECODE_SPLITK,
                                                      splits=s)))
                 for s in DECODE_SPLITS}
        _warm(torch, calls[DECODE_SPLITS[0]])
        times = {s: [] for s in calls}
        for _ in range(rounds):
            for s, fn in calls.items():
                times[s].append(_time(torch, fn, reps))
        default = fa.attn_fwd_plan(B, Hq, Hkv, 1, Tk, d, False, fa.FATTN_BF16)["splits"]
        for s, ts in times.items():
            ms = statistics.median(ts)
            rec = {"kind": "decode", "shape": [B, Hq, Hkv, Tk, d], "splits": s,
                   "table_splits": default, "ms": round(ms, 5),
                   "ms_rounds": [round(t, 5) for t in ts], "gbs": round(nbytes / ms / 1e6, 1)}
            records.append(rec)
            print(json.dumps(rec), flush=True)
        del q, k, v, o, lse
    props = torch.cuda.get_device_properties(0)
    doc = {"device": getattr(props, "gcnArchName", props.name).split(":")[0], "rounds": rounds,
           "reps": reps,
           "sources_sha256_16": _source_hashes(), "records": records}
    with open(out_path, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    print(f"wrote {out_path}", file=sys.stderr)


def rates(out_path):
    import torch

    import io_aware_tiled_amd as fa

    torch.cuda.set_device(0)
    g = torch.Generator(device="cuda").manual_seed(2)
    lines = ["| d | T | B x H | causal | forward ms | forward TFLOP/s | backward ms | "
             "backward TFLOP/s |", "|---|---|---|---|---|---|---|---|"]
    for (B, H, _, T, d, causal) in RATE_SHAPES:
        q = torch.randn(B, H, T, d, device="cuda", generator=g).to(torch.bfloat16)
        k = torch.randn(B, H, T, d, device="cuda", generator=g).to(torch.bfloat16)
        v = torch.randn(B, H, T, d, device="cuda", generator=g).to(torch.bfloat16)
        do = torch.randn(B, H, T, d, device="cuda", generator=g).to(torch.bfloat16)
        o, lse = fa.attn_fwd(q, k, v, causal=causal)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        fwd = lambda: fa.attn_fwd(q, k, v, causal=causal, out=o, lse=lse)
        bwd = lambda: fa.attn_bwd(q, k, v, o, lse, do, causal=causal, dq=dq, dk=dk, dv=dv)
        _warm(torch, fwd)
        tf = statistics.median(_time(torch, fwd, 5) for _ in range(5))
        tb = statistics.median(_time(torch, bwd, 3) for _ in range(5))
        flops = 4.0 * B * H * T * T * d / (2 if causal else 1)
        line = (f"| {d} | {T} | {B}x{H} | {'yes' if causal else 'no'} | {tf:.3f} | "
                f"{flops / tf / 1e9:.0f} | {tb:.3f} | {2.5 * flops / tb / 1e9:.0f} |")
        lines.append(line)
        print(line, flush=True)
        del q, k, v, do, o, lse, dq, dk, dv
    text = ("Forward (attn_fwd) and backward (attn_bwd) with the default table on "
            f"{torch.cuda.get_device_name(0)}: bf16, B*T = 16384 tokens, 32 heads, N(0, 1) inputs; "
            "median of 5 rounds; FLOPs 4*B*H*T^2*d (halved when causal), 2.5 times that for the "
            "backward.\n\n" + "\n".join(lines) + "\n")
    with open(out_path, "w") as f:
        f.write(text)
    print(f"wrote {out_path}", file=sys.stderr)


# ------------------------------------------------------------------------------ CPU: the table

def _fastest(recs):
    """The fastest record; ties (equal median) go to the earlier configuration of PREFILL_CFGS."""
    order = {c: i for i, c in enumerate(PREFILL_CFGS)}
    return min(recs, key=lambda r: (r["ms"], order[tuple(r["cfg"])]))


def prefill_rows(doc):
    """(d, causal, tk_max, min_bh, block_kv, waves, schedule, note) rows from a sweep record."""
    by_shape = {}
    for r in doc["records"]:
        if r["kind"] == "prefill":
            by_shape.setdefault(tuple(r["shape"]), []).append(r)
    rows = []
    for d in (128, 64):
        for causal in (1, 0):
            shapes = [s for s in by_shape if s[4] == d and s[5] == causal]
            lengths = sorted({s[3] for s in shapes})
            cand = []
            for i, T in enumerate(lengths):
                at = sorted((s for s in shapes if s[3] == T), key=lambda s: -(s[0] * s[1]))
                for j, s in enumerate(at):
                    recs = by_shape[s]
                    best = _fastest(recs)
                    rest = [r for r in recs if r is not best]
                    second = _fastest(rest) if rest else None
                    note = (f"B={s[0]} Hq={s[1]} Hkv={s[2]} T={T}: {best['tflops']:.0f} TFLOP/s"
                            + (f" (next {tuple(second['cfg'])} {second['tflops']:.0f})"
                               if second else ""))
                    cand.append((d, causal, 0 if i == len(lengths) - 1 else T,
                                 0 if j == len(at) - 1 else s[0] * s[1], *best["cfg"], note))
            merged = []
            for row in cand:
                if merged and merged[-1][3] == 0 and row[3] == 0 and merged[-1][4:7] == row[4:7]:
                    notes = merged[-1][7] + "; " + row[7]
                    merged[-1] = row[:7] + (notes,)
                else:
                    merged.append(row)
            rows.extend(merged)
    return rows


def render(doc, sweep_name):
    rows = prefill_rows(doc)
    out = []
    w = out.append
    w("// Launch-configuration table of libfattn. GENERATED by `python -m io_aware_tiled_amd.tune emit`")
    w(f"// from the sweep record {sweep_name} (device: {doc['device']}, {doc['rounds']} rounds")
    w("// per configuration); do not edit by hand.")
    w("//")
    w("// The block size is a performance choice, not a numerical one (\"SDPA and FlashAttention's")
    w("// tiling\", section \"A softmax you can compute one block at a time\"; \"Explain tiled attention")
    w("// and verify its output\", section \"Separate storage savings from runtime\": tile size,")
    w("// register pressure and cache reuse decide the speed). Every entry computes the same function;")
    w("// the parity tests run each one.")
    w("//")
    w("// Prefill rows are matched in order: the first row whose d matches, whose causal flag matches")
    w("// (-1 = either), whose Tk is at most tk_max (0 = no bound) and whose batch x query heads is at")
    w("// least min_bh wins. Each swept shape gave the row of its fastest configuration (block_kv,")
    w("// waves, schedule), noted below with its rate and the next best.")
    w("#pragma once")
    w("")
    w("namespace fattn {")
    w("")
    w("struct PrefillEntry {")
    w("  int d;")
    w("  int causal;   // -1 = any")
    w("  int tk_max;   // 0 = unbounded")
    w("  int min_bh;   // B * Hq at least this (0 = any)")
    w("  int block_kv;")
    w("  int waves;")
    w("  int schedule;")
    w("};")
    w("")
    w("static const PrefillEntry kPrefillTable[] = {")
    w("    // d, causal, tk_max, min_bh, block_kv, waves, schedule")
    for r in rows:
        for note in r[7].split("; "):
            w(f"    // {note}")
        w(f"    {{{r[0]}, {r[1]}, {r[2]}, {r[3]}, {r[4]}, {r[5]}, {r[6]}}},")
    w("    // d = 32: not swept, one configuration")
    w("    {%d, %d, %d, %d, %d, %d, %d}," % D32_ROW)
    w("};")
    w("")
    w("// Decode: number of workgroups to aim for across the whole grid and the smallest key chunk a")
    w("// split may have (keys, multiple of 32). Split counts of the sweep (GB/s, table's choice *):")
    for r in doc["records"]:
        if r["kind"] == "decode" and r["splits"] == r["table_splits"]:
            B, Hq, Hkv, Tk, d = r["shape"]
            alts = sorted((x for x in doc["records"] if x["kind"] == "decode"
                           and x["shape"] == r["shape"]), key=lambda x: x["splits"])
            w(f"//   B={B} Hq={Hq} Hkv={Hkv} Tk={Tk} d={d}: " + ", ".join(
                f"{x['splits']}{'*' if x['splits'] == r['splits'] else ''} {x['gbs']:.0f}"
                for x in alts))
    w("struct DecodeEntry {")
    w("  int d;")
    w("  int target_workgroups;")
    w("  int min_chunk;")
    w("};")
    w("")
    w("static const DecodeEntry kDecodeTable[] = {")
    for r in DECODE_ROWS:
        w("    {%d, %d, %d}," % r)
    w("};")
    w("")
    w("}  // namespace fattn")
    return "\n".join(out) + "\n"


def emit(sweep_path, out_path):
    with open(sweep_path) as f:
        doc = json.load(f)
    text = render(doc, os.path.basename(sweep_path))
    with open(out_path, "w") as f:
        f.write(text)
    print(f"wrote {out_path}", file=sys.stderr)


def check(sweep_path):
    with open(sweep_path) as f:
        doc = json.load(f)
    with open(HEADER_PATH) as f:
        have = f.read()
    return have == render(doc, os.path.basename(sweep_path))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("sweep")
    s.add_argument("--rounds", type=int, default=3)
    s.add_argument("--reps", type=int, default=5)
    s.add_argument("--out", default=SWEEP_PATH)
    e = sub.add_parser("emit")
    e.add_argument("--sweep", default=SWEEP_PATH)
    e.add_argument("--out", default=HEADER_PATH)
    c = sub.add_parser("check")
    c.add_argument("--sweep", default=SWEEP_PATH)
    r = sub.add_parser("rates")
    r.add_argument("--out", required=True)
    args = ap.parse_args()
    if args.cmd == "sweep":
        sweep(args.rounds, args.reps, args.out)
    elif args.cmd == "emit":
        emit(args.sweep, args.out)
    elif args.cmd == "check":
        ok = check(args.sweep)
        print("tune_table.h matches the sweep record" if ok else "tune_table.h is stale")
        sys.exit(0 if ok else 1)
    else:
        rates(args.out)


if __name__ == "__main__":
    main()
