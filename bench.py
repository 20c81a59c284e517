"""Benchmark of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--cpu-baseline auto|off]

One step is one pass of the whole hot path on synthetic, seeded inputs already resident in HBM:
  * causal prefill, bf16, B=1, H=32, T=8192, d=128 (one attn_fwd call: the MFMA prefill kernel);
  * GQA decode, bf16, B=64, Hq=64, Hkv=8, Tq=1, Tk=8192, d=128 (one attn_fwd call: split-K
    partial kernel + combine kernel).
Each call is bracketed by HIP events recorded on the stream the kernels are launched on. The
headline value is the prefill rate in TFLOP/s from the median call time, counting 4*B*H*T^2*d
halved for the causal mask; the decode rate is reported as algorithmic HBM bytes per second
(K and V read once, Q read, O and LSE written). Mean, p10 and p90 call times are reported too.

After the timed steps, and outside them: the library's two probes (matrix-core rate on
register operands, nontemporal HBM read rate) give the achievable rates the two kernels are also
quoted against; then the sliding-window variants of both calls (window 4096, work of the visible
(query, key) pairs only), a packed batch of variable-length documents (attn_fwd_varlen and
attn_bwd_varlen, 32768 tokens), the decode call over a paged copy of its cache (attn_fwd_paged,
16-position pages in a random order, checked bitwise equal to the contiguous result) and the
backward of the prefill call (attn_bwd, seeded upstream gradient, 10*B*H*T^2*d/2 FLOPs) are timed.
With the CPU baseline on, the fp64 oracle is also timed on bounded samples of those calls
(`cpu_oracle_beside`). One JSON line is printed.

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


def probes(fa, torch):
    """Matrix-core TFLOP/s and HBM read GB/s of the library's probes (best of a few launches)."""
    wgs, iters = 2048, 100
    out = torch.empty(wgs * 512, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def mfma():
        rc = fa.lib.fattn_probe_mfma(out.data_ptr(), wgs, iters, stream)
        assert rc == fa.FATTN_OK, rc

    t = time_calls(torch, mfma, 3, 5)
    mfma_tflops = wgs * 8 * 32 * iters * 32768.0 / (min(t) * 1e-3) / 1e12
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    rwgs = 16384
    words = torch.empty(rwgs * 4, dtype=torch.int32, device="cuda")

    def read():
        rc = fa.lib.fattn_probe_hbm_read(buf.data_ptr(), nbytes, words.data_ptr(), rwgs, stream)
        assert rc == fa.FATTN_OK, rc

    t = time_calls(torch, read, 20, 10)
    read_gbs = nbytes / (min(t) * 1e-3) / 1e9
    del buf, words, out
    return {"mfma_bf16_tflops": round(mfma_tflops, 1), "hbm_read_gbs": round(read_gbs, 1),
            "what": "best of 5 (matrix) and 10 (read) launches: 4 chains of v_mfma_f32_32x32x16_bf16 per wavefront on "
                    "register operands (2048 x 8 wavefronts); 16-byte nontemporal loads over a "
                    "4 GiB buffer, one contiguous 256 KiB chunk per workgroup (16384 x 256 "
                    "threads)"}


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


def cpu_baseline(budget_s=12.0, max_heads=32):
    """The fp64 oracle timed on the host cores on a bounded sample of the prefill workload."""
    import numpy as np  # noqa: F401
    from threadpoolctl import threadpool_info

    import oracle
    from tests import inputs

    cfg = inputs.CONFIGS[PREFILL]
    heads, elapsed = 0, 0.0
    while heads < max_heads and (heads == 0 or elapsed < budget_s):
        q = inputs.head_slice(cfg, inputs.Q_ID, 0, heads)
        k = inputs.head_slice(cfg, inputs.K_ID, 0, heads)
        v = inputs.head_slice(cfg, inputs.V_ID, 0, heads)
        t0 = time.perf_counter()
        oracle.dense_head(q, k, v, cfg.causal, cfg.scale)
        elapsed += time.perf_counter() - t0
        heads += 1
    flops = prefill_flops(1, heads, cfg.Tq, cfg.Tk, cfg.d, cfg.causal)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{heads} of 32 heads of the causal T=8192 d=128 prefill, all 8192 rows "
                      f"each, fp64 dense (S and P materialised), {elapsed:.2f} s; TFLOP/s with "
                      f"the same causal-halved FLOP count as the GPU figure",
            "seconds": elapsed, "host_cpus": len(os.sched_getaffinity(0))}


def oracle_beside(budget_s=3.0):
    """The fp64 oracle timed on bounded samples of the other measured calls (sliding window,
    packed prefill, paged decode, backward), each in the unit of its GPU figure: heads (or
    sequences) are added until `budget_s` seconds of oracle time have run."""
    import numpy as np

    import oracle
    from tests import inputs

    from threadpoolctl import threadpool_info

    cfg = inputs.CONFIGS[PREFILL]
    out = {"kind": "oracle",
           "cores": max([i.get("num_threads", 1) for i in threadpool_info()] or [1])}

    def heads_until(fn):
        n, el = 0, 0.0
        while n < cfg.Hq and (n == 0 or el < budget_s):
            args = fn(n)
            t0 = time.perf_counter()
            args[0](*args[1:])
            el += time.perf_counter() - t0
            n += 1
        return n, el

    def head(h):
        return (inputs.head_slice(cfg, inputs.Q_ID, 0, h), inputs.head_slice(cfg, inputs.K_ID, 0, h),
                inputs.head_slice(cfg, inputs.V_ID, 0, h))

    W = 4096
    n, el = heads_until(lambda h: (lambda q, k, v: oracle.dense_head(q, k, v, True, cfg.scale,
                                                                      window=W), *head(h)))
    out["sliding_window_prefill"] = {
        "value": 4.0 * cfg.d * n * window_pairs(cfg.Tq, W) / el / 1e12, "unit": "TFLOP/s",
        "sample": f"{n} heads of the W=4096 T=8192 d=128 prefill, fp64 dense, {el:.2f} s"}

    n, el = heads_until(lambda h: (lambda q, k, v, do: oracle.dense_backward_head(
        q, k, v, do, True, cfg.scale), *head(h), inputs.grad_slice(cfg, 0, h)))
    out["backward"] = {
        "value": backward_flops(1, n, cfg.Tq, cfg.Tk, cfg.d, True) / el / 1e12, "unit": "TFLOP/s",
        "sample": f"{n} heads of the causal T=8192 d=128 backward, fp64 chain rule with P "
                  f"materialised, {el:.2f} s"}

    lens = varlen_doc_lengths(VARLEN_TOKENS, 128, 8192, VARLEN_SEED)
    vc = inputs.AttnConfig("varlen oracle sample", B=1, Hq=1, Hkv=1, Tq=1, Tk=1, d=cfg.d,
                           dtype="bf16", causal=True, dist="normal", seed=VARLEN_SEED)
    Q, K, V, cq, ck = inputs.make_packed(vc, lens[:2])
    t0 = time.perf_counter()
    oracle.varlen_attention(Q, K, V, cq, ck, True, cfg.scale)
    el = time.perf_counter() - t0
    out["varlen"] = {
        "value": sum(prefill_flops(1, 1, m, m, cfg.d, True) for m in lens[:2]) / el / 1e12,
        "unit": "TFLOP/s",
        "sample": f"one head of the first two documents ({lens[0]} and {lens[1]} tokens) of the "
                  f"packed batch, fp64 dense per document, {el:.2f} s"}

    dc = inputs.CONFIGS[DECODE].replace(B=2, name="paged oracle sample")
    Qd, _, _ = inputs.make_inputs(dc)
    Kc, Vc, table, sl = inputs.make_paged(dc, 16, [dc.Tk] * dc.B)
    t0 = time.perf_counter()
    oracle.paged_decode(Qd[:, :, 0], Kc, Vc, table, sl, dc.scale)
    el = time.perf_counter() - t0
    out["paged_decode"] = {
        "value": decode_bytes(dc.B, dc.Hq, dc.Hkv, dc.Tk, dc.d) / el / 1e9, "unit": "GB/s",
        "sample": f"2 of the 64 sequences of the paged GQA decode (16-position pages), gather then "
                  f"fp64 dense, {el:.2f} s"}
    del np
    return out


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
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "libfattn has no multi-GPU path; shard (batch, kv-head) groups across GPUs "
              "with one process each instead.", file=sys.stderr)
        sys.exit(2)

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
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

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
    pst = stats_ms([e[0].elapsed_time(e[1]) for e in ev])
    dst = stats_ms([e[1].elapsed_time(e[2]) for e in ev])
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
    pr = probes(fa, torch)
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

    cpu = None
    beside = None
    if args.cpu_baseline == "auto":
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline()
        print("[bench] timing the CPU oracle beside the other calls", file=sys.stderr, flush=True)
        beside = oracle_beside()

    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
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
                    "flops_per_call": flops, "ms_stats": _r(pst)},
        "decode": {"ms": round(decode_ms, 4), "gbs": round(gbs, 1),
                   "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
                   "pct_of_probe": round(100 * gbs / pr["hbm_read_gbs"], 2),
                   "bytes_per_call": dbytes, "ms_stats": _r(dst),
                   "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": round(gbs / PEAK_HBM_GBS, 4),
                                "traffic": traffic_for("decode_bf16.hip", "decode")}},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_for("prefill_bf16.hip", "prefill")},
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
        },
        "cpu_baseline": cpu,
        "cpu_oracle_beside": beside,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
