"""Benchmark of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--cpu-baseline auto|off]

One step is one pass of the whole hot path on synthetic, seeded inputs already resident in HBM:
  * causal prefill, bf16, B=1, H=32, T=8192, d=128 (one attn_fwd call: the MFMA prefill kernel);
  * GQA decode, bf16, B=64, Hq=64, Hkv=8, Tq=1, Tk=8192, d=128 (one attn_fwd call: split-K
    partial kernel + combine kernel).
Each call is bracketed by HIP events recorded on the stream the kernels are launched on. The
headline value is the prefill rate in TFLOP/s from the median call time, counting 4*B*H*T^2*d
halved for the causal mask; the decode rate is reported as algorithmic HBM bytes per second
(K and V read once, Q read, O and LSE written). Every step's call times are in the line
(`ms_steps`), with their median, mean, p10 and p90.

Warm-up: the W steps asked for, then, if those took less than CLOCK_WARMUP_MS of GPU time, more
of the same steps until that much has run (the clock climbs from its idle state over the first
tens of milliseconds of back-to-back work). The extra steps are untimed and reported in the line
(`warmup_extra`).

After the timed steps, and outside them: the probes (matrix-core rate on register operands,
nontemporal HBM read rate; a separate library, libfattn_probe.so) give the achievable rates the
two kernels are also quoted against; then the sliding-window variants of both calls (window
4096, work of the visible (query, key) pairs only), a packed batch of variable-length documents
(attn_fwd_varlen and attn_bwd_varlen, 32768 tokens), the decode call over a paged copy of its
cache (attn_fwd_paged, 16-position pages in a random order, checked bitwise equal to the
contiguous result) and the backward of the prefill call (attn_bwd, seeded upstream gradient,
10*B*H*T^2*d/2 FLOPs) are timed.

With the CPU baseline on (the default), the fp64 oracle is timed first, before this process
touches the GPU, one child process per measurement: each of the five workloads on all host cores
(the large ones on a stated subset of heads or sequences, scaled by their count, which is exact
because they cost the same), and the small ones and the decode on one core too. One JSON line is
printed.

    python bench.py --calibrate-copy BYTES

runs a device-to-device copy of BYTES bytes a few times (for scaling hardware byte counters) and
prints one JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "causal prefill TFLOP/s (% MFMA peak) at T=8192,d=128; decode HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak (published)
PREFILL = "bf16_causal_b1_h32_t8192_d128"
DECODE = "bf16_gqa_decode_b64_hq64_hkv8_tk8192_d128"
PROFILES = os.path.join(ROOT, "profiles")
PROBE_LIB = os.path.join(ROOT, "io_aware_tiled_amd", "libfattn_probe.so")
CLOCK_WARMUP_MS = 300.0


def prefill_flops(B, H, Tq, Tk, d, causal):
    """4*B*H*Tq*Tk*d, halved under a causal mask."""
    f = 4.0 * B * H * Tq * Tk * d
    return f / 2 if causal else f


def decode_bytes(B, Hq, Hkv, Tk, d, eb=2):
    """K and V read once, Q read, O written (element size eb), LSE written in fp32."""
    return (2 * B * Hkv * Tk * d + 2 * B * Hq * d) * eb + 4 * B * Hq


def window_pairs(T, W):
    """Visible (query, key) pairs of a square causal window: row i sees min(i + 1, W) keys."""
    if W >= T:
        return T * (T + 1) // 2
    return W * (W + 1) // 2 + (T - W) * W


def window_decode_bytes(B, Hq, Hkv, W, d, eb=2):
    """A decode step under a window reads only the last W keys and values."""
    return decode_bytes(B, Hq, Hkv, W, d, eb)


def backward_flops(B, H, Tq, Tk, d, causal):
    """The backward's five products (S, dP, dV, dK, dQ): 10*B*H*Tq*Tk*d, halved under a causal
    mask, the forward's convention for its two."""
    f = 10.0 * B * H * Tq * Tk * d
    return f / 2 if causal else f


VARLEN_TOKENS = 32768
VARLEN_SEED = 77


def varlen_doc_lengths(total, lo, hi, seed):
    """Document lengths drawn U[lo, hi] from the seed until they cover `total` tokens; the last
    one is cut to fit."""
    import numpy as np

    rng = np.random.default_rng(seed)
    lens = []
    while sum(lens) < total:
        lens.append(int(rng.integers(lo, hi + 1)))
    lens[-1] -= sum(lens) - total
    return [x for x in lens if x > 0]


def stats_ms(times):
    """median, mean, p10, p90 of a list of call times in ms."""
    import numpy as np

    a = np.asarray(times, dtype=np.float64)
    return {"median": float(np.median(a)), "mean": float(a.mean()),
            "p10": float(np.percentile(a, 10)), "p90": float(np.percentile(a, 90))}


def time_calls(torch, fn, warmup, reps):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    for e in ev:
        e[0].record()
        fn()
        e[1].record()
    torch.cuda.synchronize()
    return [e[0].elapsed_time(e[1]) for e in ev]


def probes(torch):
    """Matrix-core TFLOP/s and HBM read GB/s of the probes (best of a few launches)."""
    import ctypes

    plib = ctypes.CDLL(PROBE_LIB)
    plib.probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_void_p]
    plib.probe_mfma_bf16.restype = ctypes.c_int
    plib.probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                    ctypes.c_int, ctypes.c_void_p]
    plib.probe_hbm_read.restype = ctypes.c_int
    wgs, iters = 2048, 100
    out = torch.empty(wgs * 512, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def mfma_rate(random):
        def call():
            rc = plib.probe_mfma_bf16(out.data_ptr(), wgs, iters, random, stream)
            assert rc == 0, rc

        t = time_calls(torch, call, 3, 5)
        return wgs * 8 * 32 * iters * 32768.0 / (min(t) * 1e-3) / 1e12

    mfma_tflops = mfma_rate(0)
    mfma_random_tflops = mfma_rate(1)
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    rwgs = 16384
    words = torch.empty(rwgs * 4, dtype=torch.int32, device="cuda")

    def read():
        rc = plib.probe_hbm_read(buf.data_ptr(), nbytes, words.data_ptr(), rwgs, stream)
        assert rc == 0, rc

    t = time_calls(torch, read, 20, 10)
    read_gbs = nbytes / (min(t) * 1e-3) / 1e9
    del buf, words, out
    return {"mfma_bf16_tflops": round(mfma_tflops, 1),
            "mfma_bf16_random_tflops": round(mfma_random_tflops, 1),
            "hbm_read_gbs": round(read_gbs, 1),
            "what": "best of 5 (matrix) and 10 (read) launches: 4 chains of "
                    "v_mfma_f32_32x32x16_bf16 per wavefront on register operands (2048 x 8 "
                    "wavefronts), small slowly varying operands, then hashed uniform(-1, 1) "
                    "operands (the clock under matrix load drops with the operand bits that "
                    "toggle); 16-byte nontemporal loads over a 4 GiB buffer, one contiguous "
                    "256 KiB chunk per workgroup (16384 x 256 threads)"}


def source_hash(name):
    with open(os.path.join(ROOT, "io_aware_tiled_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def device_inputs(cfg, torch):
    """Seeded inputs, generated head by head on the host and copied to the GPU."""
    from tests import inputs

    def build(which, H, T):
        t = torch.empty((cfg.B, H, T, cfg.d), dtype=torch.bfloat16, device="cuda")
        for b in range(cfg.B):
            for h in range(H):
                t[b, h].copy_(inputs.to_torch(inputs.head_slice(cfg, which, b, h), "bf16"))
        return t

    return (build(inputs.Q_ID, cfg.Hq, cfg.Tq), build(inputs.K_ID, cfg.Hkv, cfg.Tk),
            build(inputs.V_ID, cfg.Hkv, cfg.Tk))


def device_grad(cfg, torch):
    """The seeded upstream gradient dO of a backward case, on the GPU."""
    from tests import inputs

    t = torch.empty((cfg.B, cfg.Hq, cfg.Tq, cfg.d), dtype=torch.bfloat16, device="cuda")
    for b in range(cfg.B):
        for h in range(cfg.Hq):
            t[b, h].copy_(inputs.to_torch(inputs.grad_slice(cfg, b, h), "bf16"))
    return t


def traffic_for(kernel_source, key):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE/WRITE_SIZE counters, read from the
    `traffic-record:` line of the committed profile summaries; None when no summary has it or
    the kernel source changed since the counters were taken."""
    import glob

    want = source_hash(kernel_source)
    for path in sorted(glob.glob(os.path.join(PROFILES, "*.md"))):
        with open(path) as f:
            for line in f:
                if line.startswith("traffic-record:"):
                    try:
                        rec = json.loads(line.split(":", 1)[1])
                    except ValueError:
                        continue
                    if (rec.get("key") == key and rec.get("source") == kernel_source
                            and rec.get("source_sha256_16") == want):
                        return rec.get("hbm_bytes_per_launch")
    return None


def counters_for(kernel_source, key):
    """Utilisation counters of the dominant kernel of a call (matrix-core busy share, LDS bank
    conflict cycles per LDS-active cycle, HBM bytes per launch), read from the `counter-record:`
    line of the committed profile summaries; None when no summary has it or the kernel source
    changed since the counters were taken."""
    import glob

    want = source_hash(kernel_source)
    for path in sorted(glob.glob(os.path.join(PROFILES, "*.md"))):
        with open(path) as f:
            for line in f:
                if line.startswith("counter-record:"):
                    try:
                        rec = json.loads(line.split(":", 1)[1])
                    except ValueError:
                        continue
                    if (rec.get("key") == key and rec.get("source") == kernel_source
                            and rec.get("source_sha256_16") == want):
                        return {k: v for k, v in rec.items() if k not in ("key", "source")}
    return None


# ---- the CPU oracle, timed in child processes (one per measurement) before the GPU is touched

SMALL_F32 = "f32_causal_b1_h4_t128_d32"
SMALL_BF16 = "bf16_causal_b4_h16_t1024_d64"
GQA_LONG = "bf16_gqa_causal_b2_hq32_hkv8_t16384_d128"
# workload -> (what is timed, units timed, units in the workload, unit name)
ORACLE_CASES = {
    SMALL_F32: ("all 4 heads", None, None, "heads"),
    SMALL_BF16: ("all 64 heads", None, None, "heads"),
    PREFILL: ("all 32 heads", None, None, "heads"),
    DECODE: ("sequences 0-7 of 64 (all 64 query heads each)", 8, 64, "sequences"),
    GQA_LONG: ("query heads 0 and 1 of sequence 0 (kv head 0) of 64 heads", 2, 64, "heads"),
}
# the workloads also timed on one core
ONE_CORE = (SMALL_F32, SMALL_BF16, DECODE)
# the calls timed after the steps, each on a bounded sample: name -> sample description
BESIDE_CASES = {
    "sliding_window_prefill": "heads 0-3 of 32 of the W=4096 causal T=8192 d=128 prefill, fp64 "
                              "dense",
    "backward": "heads 0-2 of 32 of the causal T=8192 d=128 backward, fp64 chain rule with P "
                "materialised",
    "varlen": "head 0 of the first two documents of the packed batch, fp64 dense per document",
    "paged_decode": "sequences 0-1 of 64 of the paged GQA decode (16-position pages), gather then "
                    "fp64 dense",
}


def _slices(cfg, which, bs, hs):
    import numpy as np

    from tests import inputs

    T = cfg.Tq if which == inputs.Q_ID else cfg.Tk
    out = np.empty((len(bs), len(hs), T, cfg.d), np.float32)
    for i, b in enumerate(bs):
        for j, h in enumerate(hs):
            out[i, j] = inputs.head_slice(cfg, which, b, h)
    return out


def oracle_case(name):
    """In a child process: generate the inputs of one measurement (untimed), time the oracle on
    them and return {"seconds", "threads", "timed", "total", "work", "unit"}: `work` is the
    algorithmic FLOPs (or bytes, for a decode) of the timed part."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    from tests import inputs

    res = {}
    if name in ORACLE_CASES:
        _, timed, total, _ = ORACLE_CASES[name]
        cfg = inputs.CONFIGS[name]
        bs, hq, hk = range(cfg.B), range(cfg.Hq), range(cfg.Hkv)
        if name == DECODE:
            bs = range(timed)
        elif name == GQA_LONG:
            bs, hq, hk = [0], [0, 1], [0]
        Q = _slices(cfg, inputs.Q_ID, bs, hq)
        K = _slices(cfg, inputs.K_ID, bs, hk)
        V = _slices(cfg, inputs.V_ID, bs, hk)
        t0 = time.perf_counter()
        oracle.dense_attention(Q, K, V, cfg.causal, cfg.scale)
        el = time.perf_counter() - t0
        if name == DECODE:
            work, unit = decode_bytes(len(bs), cfg.Hq, cfg.Hkv, cfg.Tk, cfg.d), "bytes"
        else:
            work = prefill_flops(len(bs), len(hq), cfg.Tq, cfg.Tk, cfg.d, cfg.causal)
            unit = "FLOPs"
        n = len(bs) if name == DECODE else len(bs) * len(hq)
        res = {"timed": n, "total": cfg.B if name == DECODE else cfg.B * cfg.Hq}
    else:
        cfg = inputs.CONFIGS[PREFILL]
        if name == "sliding_window_prefill":
            W, hs = 4096, range(4)
            Q, K, V = (_slices(cfg, w, [0], hs) for w in (inputs.Q_ID, inputs.K_ID, inputs.V_ID))
            t0 = time.perf_counter()
            oracle.dense_attention(Q, K, V, True, cfg.scale, window=W)
            el = time.perf_counter() - t0
            work, unit = 4.0 * cfg.d * len(hs) * window_pairs(cfg.Tq, W), "FLOPs"
        elif name == "backward":
            hs = range(3)
            Q, K, V = (_slices(cfg, w, [0], hs) for w in (inputs.Q_ID, inputs.K_ID, inputs.V_ID))
            dO = np.stack([inputs.grad_slice(cfg, 0, h) for h in hs])[None]
            t0 = time.perf_counter()
            oracle.dense_backward(Q, K, V, dO, True, cfg.scale)
            el = time.perf_counter() - t0
            work, unit = backward_flops(1, len(hs), cfg.Tq, cfg.Tk, cfg.d, True), "FLOPs"
        elif name == "varlen":
            lens = varlen_doc_lengths(VARLEN_TOKENS, 128, 8192, VARLEN_SEED)[:2]
            vc = inputs.AttnConfig("varlen oracle sample", B=1, Hq=1, Hkv=1, Tq=1, Tk=1, d=cfg.d,
                                   dtype="bf16", causal=True, dist="normal", seed=VARLEN_SEED)
            Q, K, V, cq, ck = inputs.make_packed(vc, lens)
            t0 = time.perf_counter()
            oracle.varlen_attention(Q, K, V, cq, ck, True, cfg.scale)
            el = time.perf_counter() - t0
            work, unit = sum(prefill_flops(1, 1, m, m, cfg.d, True) for m in lens), "FLOPs"
        elif name == "paged_decode":
            dc = inputs.CONFIGS[DECODE].replace(B=2, name="paged oracle sample")
            Qd, _, _ = inputs.make_inputs(dc)
            Kc, Vc, table, sl = inputs.make_paged(dc, 16, [dc.Tk] * dc.B)
            t0 = time.perf_counter()
            oracle.paged_decode(Qd[:, :, 0], Kc, Vc, table, sl, dc.scale)
            el = time.perf_counter() - t0
            work, unit = decode_bytes(dc.B, dc.Hq, dc.Hkv, dc.Tk, dc.d), "bytes"
        else:
            raise ValueError(name)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    res.update({"seconds": el, "threads": threads, "work": work, "unit": unit,
                "cpus": len(os.sched_getaffinity(0))})
    return res


def _oracle_child(name, one_core):
    """Runs `bench.py --oracle-case name` as a child process (all host cores, or one)."""
    import subprocess

    env = dict(os.environ)
    cmd = [sys.executable, os.path.abspath(__file__), "--oracle-case", name]
    if one_core:
        for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
            env[v] = "1"
        cmd.append("--one-core")
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=300)
    if r.returncode != 0:
        raise RuntimeError(f"oracle child {name} failed ({r.returncode}): {r.stderr[-2000:]}")
    return json.loads(r.stdout.strip().splitlines()[-1])


def cpu_oracle_leg():
    """The oracle timed per workload (all cores; one core for the three small ones), then on
    samples of the calls timed after the steps. Returns (cpu_baseline, per_config, beside)."""
    per = {}
    for name, (what, timed, total, unit) in ORACLE_CASES.items():
        print(f"[bench] CPU oracle {name}", file=sys.stderr, flush=True)
        r = _oracle_child(name, False)
        scale = r["total"] / r["timed"]
        rate = r["work"] / r["seconds"]
        e = {"timed": what, "threads": r["threads"], "host_cpus": r["cpus"],
             "seconds": round(r["seconds"], 4),
             "seconds_whole_workload": round(r["seconds"] * scale, 4),
             "extrapolated": scale != 1,
             ("gbs" if r["unit"] == "bytes" else "tflops"):
                 rate / 1e9 if r["unit"] == "bytes" else rate / 1e12}
        if name in ONE_CORE:
            r1 = _oracle_child(name, True)
            e["seconds_one_core"] = round(r1["seconds"], 4)
            e["seconds_one_core_whole_workload"] = round(r1["seconds"] * scale, 4)
        per[name] = e
    beside = {}
    for name, what in BESIDE_CASES.items():
        print(f"[bench] CPU oracle beside: {name}", file=sys.stderr, flush=True)
        r = _oracle_child(name, False)
        rate = r["work"] / r["seconds"]
        beside[name] = {"value": rate / 1e9 if r["unit"] == "bytes" else rate / 1e12,
                        "unit": "GB/s" if r["unit"] == "bytes" else "TFLOP/s",
                        "cores": r["threads"], "kind": "oracle",
                        "sample": f"{what}, {r['seconds']:.2f} s"}
    pre = per[PREFILL]
    head = {"value": pre["tflops"], "unit": "TFLOP/s", "cores": pre["threads"], "kind": "oracle",
            "sample": f"the whole causal T=8192 d=128 prefill (32 heads, all 8192 rows each), fp64 "
                      f"dense with S and P materialised, {pre['seconds']:.2f} s in its own process; "
                      f"the matrix products use {pre['threads']} BLAS threads, the exponentials and "
                      f"other elementwise steps one; TFLOP/s with the causal-halved FLOP count of "
                      f"the GPU figure",
            "seconds": pre["seconds"], "host_cpus": pre["host_cpus"]}
    return head, per, beside


def _r(d):
    return {k: round(v, 4) for k, v in d.items()}


def calibrate_copy(nbytes, reps=3):
    import torch

    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n * 4, "reps": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the clock ramps up over the first ~20 ms of back-to-back work; warm up past that
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--cpu-baseline", choices=["auto", "off"], default="auto")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES")
    # internal: one oracle measurement in a child process (see cpu_oracle_leg)
    ap.add_argument("--oracle-case", default=None, help=argparse.SUPPRESS)
    ap.add_argument("--one-core", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()

    if args.oracle_case:
        if args.one_core:
            os.sched_setaffinity(0, {min(os.sched_getaffinity(0))})
        print(json.dumps(oracle_case(args.oracle_case)), flush=True)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "libfattn has no multi-GPU path; shard (batch, kv-head) groups across GPUs "
              "with one process each instead.", file=sys.stderr)
        sys.exit(2)

    # the CPU oracle first: its child processes start before this process touches the GPU
    cpu = per_config = beside = None
    if args.cpu_baseline == "auto" and not args.calibrate_copy:
        cpu, per_config, beside = cpu_oracle_leg()

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    import numpy as np

    import io_aware_tiled_amd as fa
    from tests import inputs

    pc, dc = inputs.CONFIGS[PREFILL], inputs.CONFIGS[DECODE]
    print(f"[bench] generating inputs: {pc.name}, {dc.name}", file=sys.stderr, flush=True)
    q3, k3, v3 = device_inputs(pc, torch)
    q4, k4, v4 = device_inputs(dc, torch)
    o3, l3 = torch.empty_like(q3), torch.empty(pc.B, pc.Hq, pc.Tq, device="cuda")
    o4, l4 = torch.empty_like(q4), torch.empty(dc.B, dc.Hq, dc.Tq, device="cuda")
    plan3 = fa.attn_fwd_plan(pc.B, pc.Hq, pc.Hkv, pc.Tq, pc.Tk, pc.d, pc.causal, fa.FATTN_BF16)
    plan4 = fa.attn_fwd_plan(dc.B, dc.Hq, dc.Hkv, dc.Tq, dc.Tk, dc.d, dc.causal, fa.FATTN_BF16)

    def step():
        fa.attn_fwd(q3, k3, v3, causal=pc.causal, scale=pc.scale, out=o3, lse=l3)
        fa.attn_fwd(q4, k4, v4, causal=dc.causal, scale=dc.scale, out=o4, lse=l4)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    w0 = torch.cuda.Event(enable_timing=True)
    w1 = torch.cuda.Event(enable_timing=True)
    w0.record()
    for _ in range(args.warmup):
        step()
    w1.record()
    torch.cuda.synchronize()
    warm_ms = w0.elapsed_time(w1) if args.warmup else 0.0
    # more untimed steps until CLOCK_WARMUP_MS of back-to-back work has run (reported)
    extra, extra_ms = 0, 0.0
    while warm_ms + extra_ms < CLOCK_WARMUP_MS:
        w0.record()
        for _ in range(10):
            step()
        w1.record()
        torch.cuda.synchronize()
        extra += 10
        extra_ms += w0.elapsed_time(w1)
    if extra:
        print(f"[bench] {extra} more warm-up steps ({extra_ms:.0f} ms)", file=sys.stderr,
              flush=True)

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    print(f"[bench] timing {K} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record()
        fa.attn_fwd(q3, k3, v3, causal=pc.causal, scale=pc.scale, out=o3, lse=l3)
        ev[i][1].record()
        fa.attn_fwd(q4, k4, v4, causal=dc.causal, scale=dc.scale, out=o4, lse=l4)
        ev[i][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    p_steps = [e[0].elapsed_time(e[1]) for e in ev]
    d_steps = [e[1].elapsed_time(e[2]) for e in ev]
    pst, dst = stats_ms(p_steps), stats_ms(d_steps)
    prefill_ms, decode_ms = pst["median"], dst["median"]
    if not (bool(torch.isfinite(o3).all()) and bool(torch.isfinite(o4).all())):
        print("non-finite output", file=sys.stderr)
        sys.exit(1)

    flops = prefill_flops(pc.B, pc.Hq, pc.Tq, pc.Tk, pc.d, pc.causal)
    tflops = flops / (prefill_ms * 1e-3) / 1e12
    dbytes = decode_bytes(dc.B, dc.Hq, dc.Hkv, dc.Tk, dc.d)
    gbs = dbytes / (decode_ms * 1e-3) / 1e9

    # ---- outside the timed steps: achievable rates, then the sliding-window variants
    print("[bench] probes and sliding-window calls", file=sys.stderr, flush=True)
    pr = probes(torch)
    W = 4096
    sw_p = stats_ms(time_calls(torch, lambda: fa.attn_fwd(q3, k3, v3, causal=True, scale=pc.scale,
                                                         out=o3, lse=l3, window=W), 10, 20))
    sw_d = stats_ms(time_calls(torch, lambda: fa.attn_fwd(q4, k4, v4, causal=True, scale=dc.scale,
                                                         out=o4, lse=l4, window=W), 10, 20))
    sw_flops = 4.0 * pc.d * pc.B * pc.Hq * window_pairs(pc.Tq, W)
    sw_tflops = sw_flops / (sw_p["median"] * 1e-3) / 1e12
    sw_bytes = window_decode_bytes(dc.B, dc.Hq, dc.Hkv, W, dc.d)
    sw_gbs = sw_bytes / (sw_d["median"] * 1e-3) / 1e9

    # ---- the decode call over a paged cache: the same keys and values in 16-position pages,
    # dealt to physical blocks in a seeded random order
    print("[bench] paged decode", file=sys.stderr, flush=True)
    BS = 16
    mb = dc.Tk // BS
    gen = torch.Generator(device="cpu")
    gen.manual_seed(dc.seed)
    perm = torch.randperm(dc.B * mb, generator=gen).to("cuda")
    def paged(x):
        blocks = x.view(dc.B, dc.Hkv, mb, BS, dc.d).permute(0, 2, 1, 3, 4)
        c = torch.empty((dc.B * mb, dc.Hkv, BS, dc.d), dtype=x.dtype, device="cuda")
        c[perm] = blocks.reshape(dc.B * mb, dc.Hkv, BS, dc.d)
        return c
    kc4, vc4 = paged(k4), paged(v4)
    table4 = perm.view(dc.B, mb).to(torch.int32).contiguous()
    lens4 = torch.full((dc.B,), dc.Tk, dtype=torch.int32, device="cuda")
    q4p, o4p = q4[:, :, 0].contiguous(), torch.empty(dc.B, dc.Hq, dc.d, dtype=torch.bfloat16,
                                                     device="cuda")
    l4p = torch.empty(dc.B, dc.Hq, device="cuda")
    pg = stats_ms(time_calls(torch, lambda: fa.attn_fwd_paged(q4p, kc4, vc4, table4, lens4,
                                                             scale=dc.scale, out=o4p, lse=l4p),
                             10, 20))
    fa.attn_fwd(q4, k4, v4, causal=dc.causal, scale=dc.scale, out=o4, lse=l4)
    torch.cuda.synchronize()
    if not torch.equal(o4p.view(torch.int16), o4[:, :, 0].view(torch.int16)):
        print("paged decode differs from the contiguous decode", file=sys.stderr)
        sys.exit(1)
    pg_bytes = dbytes + 4 * dc.B * mb + 4 * dc.B  # plus the block table and lengths
    pg_gbs = pg_bytes / (pg["median"] * 1e-3) / 1e9
    del kc4, vc4

    # ---- a packed training batch: 32768 tokens of documents with lengths U[128, 8192]
    print("[bench] packed variable-length prefill", file=sys.stderr, flush=True)
    lens = varlen_doc_lengths(VARLEN_TOKENS, 128, 8192, VARLEN_SEED)
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32, device="cuda")
    gv = torch.Generator(device="cuda")
    gv.manual_seed(VARLEN_SEED)
    qv = torch.randn(VARLEN_TOKENS, pc.Hq, pc.d, device="cuda", generator=gv).to(torch.bfloat16)
    kv = torch.randn(VARLEN_TOKENS, pc.Hkv, pc.d, device="cuda", generator=gv).to(torch.bfloat16)
    vv = torch.randn(VARLEN_TOKENS, pc.Hkv, pc.d, device="cuda", generator=gv).to(torch.bfloat16)
    ov = torch.empty_like(qv)
    lv = torch.empty(pc.Hq, VARLEN_TOKENS, device="cuda")
    vl = stats_ms(time_calls(torch, lambda: fa.attn_fwd_varlen(qv, kv, vv, cu, cu, max(lens),
                                                              max(lens), causal=True,
                                                              scale=pc.scale, out=ov, lse=lv),
                             10, 20))
    if not bool(torch.isfinite(ov).all()):
        print("non-finite packed output", file=sys.stderr)
        sys.exit(1)
    vl_flops = sum(prefill_flops(1, pc.Hq, n, n, pc.d, True) for n in lens)
    vl_tflops = vl_flops / (vl["median"] * 1e-3) / 1e12
    # and its backward (attn_bwd_varlen) with a seeded upstream gradient
    dov = torch.randn(VARLEN_TOKENS, pc.Hq, pc.d, device="cuda", generator=gv).to(torch.bfloat16)
    gq, gk, gvv = torch.empty_like(qv), torch.empty_like(kv), torch.empty_like(vv)
    vb = stats_ms(time_calls(torch, lambda: fa.attn_bwd_varlen(
        qv, kv, vv, ov, lv, dov, cu, cu, max(lens), max(lens), causal=True, scale=pc.scale,
        dq=gq, dk=gk, dv=gvv), 5, 10))
    if not all(bool(torch.isfinite(t).all()) for t in (gq, gk, gvv)):
        print("non-finite packed gradient", file=sys.stderr)
        sys.exit(1)
    vb_flops = 2.5 * vl_flops
    vb_tflops = vb_flops / (vb["median"] * 1e-3) / 1e12
    del qv, kv, vv, ov, lv, dov, gq, gk, gvv

    # ---- the backward of the prefill call (O and LSE of the last forward call above)
    print("[bench] backward", file=sys.stderr, flush=True)
    fa.attn_fwd(q3, k3, v3, causal=pc.causal, scale=pc.scale, out=o3, lse=l3)
    do3 = device_grad(pc, torch)
    dq3, dk3, dv3 = torch.empty_like(q3), torch.empty_like(k3), torch.empty_like(v3)
    bw = stats_ms(time_calls(torch, lambda: fa.attn_bwd(q3, k3, v3, o3, l3, do3, causal=pc.causal,
                                                       scale=pc.scale, dq=dq3, dk=dk3, dv=dv3),
                             10, 20))
    if not all(bool(torch.isfinite(t).all()) for t in (dq3, dk3, dv3)):
        print("non-finite gradient", file=sys.stderr)
        sys.exit(1)
    bw_flops = backward_flops(pc.B, pc.Hq, pc.Tq, pc.Tk, pc.d, pc.causal)
    bw_tflops = bw_flops / (bw["median"] * 1e-3) / 1e12
    del do3, dq3, dk3, dv3

    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "warmup_extra": {"steps": extra, "ms": round(extra_ms, 1),
                         "why": f"untimed steps after the {args.warmup} asked for, until "
                                f"{CLOCK_WARMUP_MS:.0f} ms of back-to-back work had run (the "
                                f"{args.warmup} took {warm_ms:.1f} ms): the clock climbs "
                                f"from its idle state over the first tens of ms"},
        "ms_per_step": round(wall * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "causal prefill bf16 B=1 H=32 T=8192 d=128 + GQA decode bf16 B=64 "
                        "Hq=64 Hkv=8 Tq=1 Tk=8192 d=128",
            "prefill_launch": plan3,
            "decode_launch": plan4,
            "inputs": "N(0,1) per-head seeded draws rounded to bf16, resident in HBM",
        },
        "prefill": {"ms": round(prefill_ms, 4), "tflops": round(tflops, 2),
                    "pct_mfma_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
                    "pct_of_probe": round(100 * tflops / pr["mfma_bf16_tflops"], 2),
                    "pct_of_random_operand_probe":
                        round(100 * tflops / pr["mfma_bf16_random_tflops"], 2),
                    "flops_per_call": flops, "ms_stats": _r(pst),
                    "ms_steps": [round(x, 4) for x in p_steps]},
        "decode": {"ms": round(decode_ms, 4), "gbs": round(gbs, 1),
                   "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
                   "pct_of_probe": round(100 * gbs / pr["hbm_read_gbs"], 2),
                   "bytes_per_call": dbytes, "ms_stats": _r(dst),
                   "ms_steps": [round(x, 4) for x in d_steps],
                   "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": round(gbs / PEAK_HBM_GBS, 4),
                                "traffic": traffic_for("decode_bf16.hip", "decode"),
                                "counters": counters_for("decode_bf16.hip", "decode")}},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_for("prefill_bf16.hip", "prefill"),
                     "counters": counters_for("prefill_bf16.hip", "prefill")},
        "probes": pr,
        "sliding_window": {
            "window": W,
            "prefill": {"ms": round(sw_p["median"], 4), "tflops": round(sw_tflops, 2),
                        "pct_mfma_peak": round(100 * sw_tflops / PEAK_BF16_TFLOPS, 2),
                        "flops_per_call": sw_flops, "ms_stats": _r(sw_p),
                        "work": "4*d FLOPs per visible (query, key) pair, window 4096",
                        "traffic": traffic_for("prefill_bf16.hip", "prefill_window")},
            "decode": {"ms": round(sw_d["median"], 4), "gbs": round(sw_gbs, 1),
                       "pct_hbm_peak": round(100 * sw_gbs / PEAK_HBM_GBS, 2),
                       "bytes_per_call": sw_bytes, "ms_stats": _r(sw_d),
                       "work": "K and V of the last 4096 keys read once, Q read, O and LSE "
                               "written",
                       "traffic": traffic_for("decode_bf16.hip", "decode_window")},
        },
        "varlen": {
            "workload": f"causal packed batch bf16: {VARLEN_TOKENS} tokens in {len(lens)} "
                        f"documents with lengths U[128, 8192] (seed {VARLEN_SEED}), H=32, d=128",
            "ms": round(vl["median"], 4), "tflops": round(vl_tflops, 2),
            "pct_mfma_peak": round(100 * vl_tflops / PEAK_BF16_TFLOPS, 2),
            "flops_per_call": vl_flops, "ms_stats": _r(vl),
            "work": "sum over documents of 4*H*L^2*d/2 (the causal count of each document)",
            "traffic": traffic_for("prefill_bf16.hip", "prefill_varlen"),
            "backward": {"ms": round(vb["median"], 4), "tflops": round(vb_tflops, 2),
                         "pct_mfma_peak": round(100 * vb_tflops / PEAK_BF16_TFLOPS, 2),
                         "flops_per_call": vb_flops, "ms_stats": _r(vb),
                         "work": "2.5 times the forward count: the five backward products",
                         "traffic": traffic_for("backward_bf16.hip", "backward_varlen")},
        },
        "paged_decode": {
            "workload": "GQA decode bf16 B=64 Hq=64 Hkv=8 Tk=8192 d=128 over a paged cache, "
                        "16 positions per page, pages in a seeded random order",
            "ms": round(pg["median"], 4), "gbs": round(pg_gbs, 1),
            "pct_hbm_peak": round(100 * pg_gbs / PEAK_HBM_GBS, 2),
            "bytes_per_call": pg_bytes, "ms_stats": _r(pg),
            "work": "the contiguous decode's bytes plus the block table and lengths",
            "bitwise_equal_to_contiguous": True,
            "traffic": traffic_for("decode_bf16.hip", "decode_paged"),
        },
        "backward": {
            "workload": "backward of the causal prefill bf16 B=1 H=32 T=8192 d=128",
            "ms": round(bw["median"], 4), "tflops": round(bw_tflops, 2),
            "pct_mfma_peak": round(100 * bw_tflops / PEAK_BF16_TFLOPS, 2),
            "flops_per_call": bw_flops, "ms_stats": _r(bw),
            "work": "10*B*H*T^2*d/2: the five products S, dP, dV, dK, dQ; the kernels run seven "
                    "(S and dP once in the dQ kernel and once in the dK/dV kernel)",
            "traffic": traffic_for("backward_bf16.hip", "backward"),
            "counters": counters_for("backward_bf16.hip", "backward"),
        },
        "cpu_baseline": cpu,
        "cpu_oracle_per_config": per_config,
        "cpu_oracle_beside": beside,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
