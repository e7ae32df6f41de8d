#!/usr/bin/env python3
"""Throughput of the exact-attention forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config causal_32k|f32_causal_256|causal_4k_b4|swa4096_32k|causal_131k|band256_globals_16k]
    python bench.py --sweep       (causal d=128 H=8 B=1, N = 512 ... 131072)
    python bench.py --config band256_globals_16k --cold   (a 1 GiB scratch write before every
                                           timed call, so no input is in MALL)

One step = one attn_fwd call (every pass the mask needs) over one batch of
seeded synthetic inputs already resident in HBM. The untimed warm-up steps
(20 by default) let the clocks leave their idle state first. The default workload is
causal attention at B=1, H=32, N=32768, d=128 in bf16, the shape the
throughput target is quoted on. Useful FLOPs count visible pairs only:
4*d per visible (query, key) pair (QK^T and PV, two flops per multiply-add).

Prints one JSON line with the metric, a roofline object for the forward
kernel (HIP events on the launch stream) and the CPU oracle timed on a bounded
sample of the same workload. --sweep prints one JSON line per sequence length
instead (time, useful TFLOP/s, free device memory before and after the call).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X dense bf16 MFMA peak: 256 CUs x 2.4 GHz x 4096 flop/clk/CU = 2516.6
# TFLOP/s (AMD's published 2.5 PFLOP/s); dense fp32 MFMA: 157.3 TFLOP/s.
PEAK_BF16 = 2516.6
PEAK_HBM_GBS = 8000.0   # MI355X HBM3E, published
PEAK_F32 = 157.3
METRIC = "fwd attention TFLOP/s (unmasked FLOPs only) + % of bf16 MFMA peak"
KERNEL_SRC = os.path.join(ROOT, "efficient_exact_attention_amd", "csrc", "attn_fwd.hip")


def mask_name(w):
    if w.global_idx:
        return f"band -{w.win_left}/+{w.win_right} + {len(w.global_idx)} global tokens"
    if w.causal and w.win_left >= 0:
        return f"causal sliding window {w.win_left + 1}"
    return "causal" if w.causal else "full"


DECODE_SRC = os.path.join(ROOT, "efficient_exact_attention_amd", "csrc", "attn_decode.hip")


def source_hash(path=KERNEL_SRC):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_for(config, src=KERNEL_SRC):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if the
    kernel source has not changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{config}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256") != source_hash(src):
        return None
    return t.get("hbm_bytes_per_launch")


def calibration_copy(nbytes):
    """One plain device copy of nbytes (the dispatch the HBM byte counters are
    scaled by)."""
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[bench] calibration copy of {nbytes} bytes done", file=sys.stderr, flush=True)


def blas_build():
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                return f"{i.get('internal_api')} {i.get('version')} ({i.get('threading_layer', '')})"
    except Exception:
        pass
    return "unknown"


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline(w, budget_s, gpu_out=None, gpu_lse=None):
    """Time the oracle on a bounded, seeded sample of query rows of the same
    workload (same input values as the GPU run)."""
    import numpy as np
    import oracle
    from efficient_exact_attention_amd import workloads as W

    rng = np.random.default_rng(w.seed + 1000)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    order = [heads[i] for i in rng.permutation(len(heads))]
    t_used = 0.0
    flops = 0
    nrows = 0
    nheads = 0
    max_err = 0.0
    rows_per_head = 64
    for (b, h) in order:
        q, k, v = (W.head_values(w, t, b, h).astype(np.float64) for t in range(3))
        rows = np.sort(rng.choice(w.N, size=min(rows_per_head, w.N), replace=False))
        t0 = time.perf_counter()
        O, L = oracle.attention(q[None, None], k[None, None], v[None, None], causal=w.causal,
                                win_left=w.win_left, win_right=w.win_right,
                                global_idx=w.global_idx, rows=rows)
        dt = time.perf_counter() - t0
        t_used += dt
        vis = oracle.mask_rows(rows, w.N, w.causal, w.win_left, w.win_right, w.global_idx)
        flops += 4 * w.d * int(vis.sum())
        nrows += len(rows)
        nheads += 1
        if gpu_out is not None:
            go = gpu_out[b, h, rows].float().cpu().numpy().astype(np.float64)
            max_err = max(max_err, float(np.max(np.abs(go - O[0, 0]))))
        if t_used >= budget_s:
            break
        # scale the next heads' row count towards the budget
        per_row = t_used / nrows
        rows_per_head = int(min(w.N, max(16, (budget_s - t_used) / per_row / 2)))
    return dict(value=flops / t_used / 1e12, unit="TFLOP/s", cores=blas_threads(), kind="oracle",
                sample=f"{nrows} seeded query rows over {nheads} head(s) of the same workload, "
                       f"numpy fp64 full masked score rows, {t_used:.1f} s",
                seconds=round(t_used, 2), rows=nrows, blas=blas_build(),
                full_call_seconds_extrapolated=round(t_used * w.B * w.H * w.N / nrows, 1)), max_err


def gemm_reference(args):
    """The vendor library's dense bf16 GEMM (torch.matmul, hipBLASLt on ROCm)
    on large shapes: the matrix-core rate the GPU sustains under its power
    limit, beside which the attention kernels' TFLOP/s can be read. One JSON
    line per shape; not part of the attention path."""
    import torch
    for m, n, k in ((8192, 8192, 8192), (16384, 16384, 8192)):
        g = torch.Generator(device="cuda").manual_seed(11)
        a = torch.randn(m, k, device="cuda", dtype=torch.bfloat16, generator=g)
        b = torch.randn(k, n, device="cuda", dtype=torch.bfloat16, generator=g)
        for _ in range(max(args.warmup, 5)):
            c = a @ b
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            c = a @ b
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        tf = 2.0 * m * n * k / ms / 1e9
        print(json.dumps({"metric": "library bf16 GEMM throughput", "value": round(tf, 1), "unit": "TFLOP/s",
                          "shape": [m, n, k], "ms_per_call": round(ms, 4), "steps": args.steps,
                          "frac_of_published_peak": round(tf / PEAK_BF16, 4)}), flush=True)
        del a, b, c
    return 0


def main():
    from efficient_exact_attention_amd import workloads as W
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="causal_32k", choices=sorted(W.WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="causal d=128 H=8 B=1 sequence-length sweep, one JSON line per N")
    ap.add_argument("--bwd", action="store_true",
                    help="time the backward pass (attn_bwd) of the workload instead; useful FLOP = "
                         "10*d per visible pair (five matrix products)")
    ap.add_argument("--decode", default=None, choices=sorted(W.DECODE_WORKLOADS),
                    help="time one decoding step (attn_decode) of this cache workload instead; "
                         "HBM-bound, reported in GB/s of K/V cache read")
    ap.add_argument("--pattern", default=None, choices=sorted(W.PATTERN_WORKLOADS),
                    help="time the forward of a strided or random-block (BigBird-style) workload instead")
    ap.add_argument("--cold", action="store_true",
                    help="write a 1 GiB scratch buffer before every timed call (cold MALL)")
    ap.add_argument("--gemm-reference", action="store_true",
                    help="time the library bf16 GEMM (torch.matmul: hipBLASLt) on large square shapes instead: "
                         "the dense matrix-core rate this GPU sustains at its power limit, for comparison")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after timing, run one plain device copy of this many bytes "
                         "(calibration dispatch for HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures a single GPU: the attention forward of one GPU's share "
              "(heads are independent) is what this library runs; --gpus must be 1.",
              file=sys.stderr)
        return 2

    import torch
    import efficient_exact_attention_amd as ea
    ea.lib()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1

    if args.gemm_reference:
        return gemm_reference(args)
    if args.sweep:
        return sweep(args)
    if args.bwd:
        return bench_bwd(args)
    if args.decode:
        return bench_decode(args)
    if args.pattern:
        return bench_pattern(args)

    w = W.WORKLOADS[args.config]
    print(f"[bench] generating {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype}", file=sys.stderr,
          flush=True)
    qkv = W.make_qkv(w)

    def dev(x):
        if w.dtype == "bf16":
            return torch.from_numpy(x.view("int16")).view(torch.bfloat16).cuda()
        return torch.from_numpy(x).cuda()
    q, k, v = (dev(x) for x in qkv)
    del qkv
    out = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, w.N, dtype=torch.float32, device="cuda")
    pairs = ea.attn_plan_stats(w.N, w.causal, w.win_left, w.win_right, w.global_idx, 128, 64)[0]
    flops = 4 * w.d * pairs * w.B * w.H
    esize = 2 if w.dtype == "bf16" else 4
    alg_bytes = 4 * w.B * w.H * w.N * w.d * esize + w.B * w.H * w.N * 4
    ws = None
    if w.global_idx:
        ws = torch.empty(ea.attn_workspace_bytes(w.B, w.H, w.N, w.d, len(w.global_idx)),
                         dtype=torch.uint8, device="cuda")

    stream = torch.cuda.current_stream()

    def step():
        ea.fwd(q, k, v, causal=w.causal, win_left=w.win_left, win_right=w.win_right,
               global_idx=w.global_idx or None, out=out, lse=lse, workspace=ws, stream=stream)

    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda") if args.cold else None

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup}), timing {args.steps} steps"
          + (" (cold MALL: 1 GiB scratch write before each call)" if args.cold else ""),
          file=sys.stderr, flush=True)

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for s, e in ev:
        if scratch is not None:
            scratch.fill_(1)
        s.record(stream)
        step()
        e.record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    launch_ms = sorted(s.elapsed_time(e) for s, e in ev)
    avg_launch_ms = sum(launch_ms) / len(launch_ms)
    # with --cold the step is the call alone (the scratch writes are not attention work)
    ms_step = avg_launch_ms if args.cold else t_start.elapsed_time(t_end) / args.steps
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (avg_launch_ms * 1e-3) / 1e12
    peak = PEAK_F32 if w.dtype == "f32" else PEAK_BF16
    print(f"[bench] {ms_step:.3f} ms/step, {value:.1f} TFLOP/s, launch avg {avg_launch_ms:.3f} ms "
          f"(min {launch_ms[0]:.3f}, max {launch_ms[-1]:.3f}), wall {wall:.2f} s", file=sys.stderr,
          flush=True)

    if args.copy_bytes > 0:
        calibration_copy(args.copy_bytes)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{mask_name(w)} attention forward B={w.B} H={w.H} N={w.N} d={w.d}",
                   "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "win_left": w.win_left, "win_right": w.win_right,
                   "n_global": len(w.global_idx), "seed": w.seed,
                   "inputs": f"{w.dtype} ~N(0,{w.sigma}^2)", "useful_flop_per_step": flops},
        "pct_bf16_peak": round(100.0 * value / PEAK_BF16, 2),
        "median_launch_ms": round(launch_ms[len(launch_ms) // 2], 4),
        # Q, K, V read once and out, LSE written once, over the call: the rate
        # that matters where the band is short and d small
        "hbm_algorithmic_bytes": alg_bytes,
        "hbm_algorithmic_gbs": round(alg_bytes / (avg_launch_ms * 1e-3) / 1e9, 1),
        "mall": "cold" if args.cold else "warm",
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic_for(args.config),
                     "kernel": "attn_fwd (band pass)" if not w.global_idx
                     else "attn_fwd call (band pass + global rows + merge)"},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print(f"[bench] timing the CPU oracle for ~{args.cpu_seconds:.0f} s", file=sys.stderr, flush=True)
        cb, err = cpu_baseline(w, args.cpu_seconds, out, lse)
        cb["gpu_over_oracle"] = round(value / cb["value"], 1)
        result["cpu_baseline"] = cb
        result["sample_max_abs_err_vs_oracle"] = err
    print(json.dumps(result), flush=True)
    return 0


def bench_bwd(args):
    """Backward pass of the workload: one step = one attn_bwd call (row
    terms, dK/dV pass, dQ pass) with the forward's output and LSE and a
    seeded upstream gradient resident in HBM. Prints one JSON line."""
    import torch
    import efficient_exact_attention_amd as ea
    from efficient_exact_attention_amd import workloads as W
    w = W.WORKLOADS[args.config]
    if w.dtype != "bf16":
        print("the backward pass covers bf16 inputs only", file=sys.stderr)
        return 2
    q, k, v, g = (torch.from_numpy(x.view("int16")).view(torch.bfloat16).cuda()
                  for x in (*W.make_qkv(w), W.make_tensor(w.with_(seed=w.seed + 7), 0)))
    kw = dict(causal=w.causal, win_left=w.win_left, win_right=w.win_right, global_idx=w.global_idx or None)
    out, lse = ea.fwd(q, k, v, **kw)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    stream = torch.cuda.current_stream()
    pairs = ea.attn_plan_stats(w.N, w.causal, w.win_left, w.win_right, w.global_idx or None, 128, 64)[0]
    flops = 10 * w.d * pairs * w.B * w.H

    def step():
        ea.bwd(q, k, v, out, g, lse, dq=dq, dk=dk, dv=dv, stream=stream, **kw)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for s_, e_ in ev:
        s_.record(stream)
        step()
        e_.record(stream)
    torch.cuda.synchronize()
    ms = sorted(s_.elapsed_time(e_) for s_, e_ in ev)
    avg = sum(ms) / len(ms)
    value = flops / (avg * 1e-3) / 1e12
    print(json.dumps({"metric": "bwd attention TFLOP/s (unmasked FLOPs only: 10*d per visible pair)",
                      "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
                      "warmup": args.warmup, "ms_per_step": round(avg, 4), "median_launch_ms": round(ms[len(ms) // 2], 4),
                      "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
                      "config": {"workload": f"{mask_name(w)} attention backward B={w.B} H={w.H} N={w.N} d={w.d}",
                                 "useful_flop_per_step": flops},
                      "pct_bf16_peak": round(100 * value / PEAK_BF16, 2),
                      "scaling": "weak", "vs_baseline": None,
                      "roofline": {"bound": "mfma", "achieved": round(value, 2), "peak": PEAK_BF16,
                                   "unit": "TFLOP/s", "frac": round(value / PEAK_BF16, 4), "traffic": None,
                                   "kernel": "attn_bwd call (row terms, dK/dV, dQ; split passes and merges "
                                             "with global tokens)"}}), flush=True)
    return 0


def bench_pattern(args):
    """Forward of a strided or random-block workload: one attn_fwd_masked call
    per step; useful FLOP = 4*d per visible pair (from the planner, which
    reads the random lists back from the device)."""
    import torch
    import efficient_exact_attention_amd as ea
    from efficient_exact_attention_amd import workloads as W
    pw = W.PATTERN_WORKLOADS[args.pattern]
    w = pw["workload"]
    print(f"[bench] generating {w.name}: {w.desc}", file=sys.stderr, flush=True)
    q, k, v = (torch.from_numpy(x.view("int16")).view(torch.bfloat16).cuda() for x in W.make_qkv(w))
    kw = dict(causal=w.causal, win_left=w.win_left, win_right=w.win_right, global_idx=w.global_idx or None,
              stride=pw["stride"], rand_block=pw["rand_block"])
    lists = None
    if pw["rand_block"]:
        lists = torch.from_numpy(W.random_block_lists(w.N, pw["rand_block"], pw["n_rand"], w.seed + 9)).cuda()
        kw["rand_idx"] = lists
    pairs = ea.attn_plan_stats_masked(w.N, 128, 64, causal=w.causal, win_left=w.win_left, win_right=w.win_right,
                                      global_idx=list(w.global_idx), stride=pw["stride"],
                                      rand_block=pw["rand_block"], n_rand=pw["n_rand"],
                                      rand_idx=lists.data_ptr() if lists is not None else None)[0]
    flops = 4 * w.d * pairs * w.B * w.H
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        ea.fwd(q, k, v, out=out, lse=lse, stream=stream, **kw)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for s_, e_ in ev:
        s_.record(stream)
        step()
        e_.record(stream)
    torch.cuda.synchronize()
    ms = sorted(s_.elapsed_time(e_) for s_, e_ in ev)
    avg = sum(ms) / len(ms)
    value = flops / (avg * 1e-3) / 1e12
    print(json.dumps({"metric": "fwd attention TFLOP/s (unmasked FLOPs only)", "value": round(value, 2),
                      "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                      "ms_per_step": round(avg, 4), "median_launch_ms": round(ms[len(ms) // 2], 4),
                      "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
                      "config": {"workload": f"{w.desc}: B={w.B} H={w.H} N={w.N} d={w.d}",
                                 "visible_pairs_per_head": pairs, "useful_flop_per_step": flops},
                      "roofline": {"bound": "mfma", "achieved": round(value, 2), "peak": PEAK_BF16, "unit": "TFLOP/s",
                                   "frac": round(value / PEAK_BF16, 4), "traffic": None}}), flush=True)
    return 0


def decode_bytes(w):
    """Algorithmic HBM bytes of one decoding step: the K and V rows of every
    position some new query sees (each read once), the queries, the bf16
    outputs and the fp32 LSE."""
    seen = 0
    for L in w.seq_len:
        span = L if w.win_left < 0 else min(L, w.Nq + w.win_left)
        seen += min(span, w.S)
    return 2 * seen * w.H_kv * w.d * 2 + w.B * w.H * w.Nq * (2 * w.d * 2 + 4)


def bench_decode(args):
    """One decoding step over a K/V cache resident in HBM: the split-KV pass
    and the merge (one attn_decode call). Prints one JSON line whose
    roofline is HBM bandwidth over the algorithmic bytes."""
    import torch
    import efficient_exact_attention_amd as ea
    from efficient_exact_attention_amd import workloads as W
    w = W.DECODE_WORKLOADS[args.decode]
    print(f"[bench] generating {w.name}: {w.desc}", file=sys.stderr, flush=True)
    q, kc, vc, seq = W.make_decode(w)
    dq, dk, dv = (torch.from_numpy(x.view("int16")).view(torch.bfloat16).cuda() for x in (q, kc, vc))
    ds = torch.from_numpy(seq).cuda()
    out = torch.empty_like(dq)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    nbytes = decode_bytes(w)

    def step():
        ea.decode(dq, dk, dv, ds, win_left=w.win_left, rolling=bool(w.rolling), out=out, lse=lse, stream=stream)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for s_, e_ in ev:
        s_.record(stream)
        step()
        e_.record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = sorted(s_.elapsed_time(e_) for s_, e_ in ev)
    avg = sum(ms) / len(ms)
    gbs = nbytes / (avg * 1e-3) / 1e9
    steps_s = 1e3 / avg
    if args.copy_bytes > 0:
        calibration_copy(args.copy_bytes)
    print(json.dumps({"metric": "decode steps/s (one new token per sequence, all heads)",
                      "value": round(steps_s, 2), "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
                      "warmup": args.warmup, "ms_per_step": round(t0.elapsed_time(t1) / args.steps, 4),
                      "median_launch_ms": round(ms[len(ms) // 2], 4), "higher_is_better": True,
                      "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
                      "config": {"workload": f"decode {w.desc}: B={w.B} H={w.H} H_kv={w.H_kv} Nq={w.Nq} "
                                             f"S={w.S} d={w.d}", "algorithmic_bytes_per_step": nbytes},
                      "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                   "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                                   "traffic": traffic_for(w.name, DECODE_SRC)}}),
          flush=True)
    return 0


def sweep(args):
    """Causal d=128, H=8, B=1 over N = 512 ... 131072: median launch time of
    the attn_fwd call (at least 20 calls or 1 s), useful TFLOP/s, and the free
    device memory just before and just after the call."""
    import torch
    import efficient_exact_attention_amd as ea
    from efficient_exact_attention_amd import workloads as W
    N = 512
    while N <= 131072:
        w = W.random_workload(f"sweep{N}", 1, 8, N, 128, causal=1, seed=200 + N.bit_length())
        q, k, v = (torch.from_numpy(x.view("int16")).view(torch.bfloat16).cuda() for x in W.make_qkv(w))
        out = torch.empty_like(q)
        lse = torch.empty(1, 8, N, dtype=torch.float32, device="cuda")
        pairs = ea.attn_plan_stats(N, 1, -1, -1, None, 128, 64)[0]
        flops = 4 * 128 * pairs * 8
        stream = torch.cuda.current_stream()

        def call():
            ea.fwd(q, k, v, causal=1, out=out, lse=lse, stream=stream)
        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()
        free0, total = torch.cuda.mem_get_info()
        call()
        torch.cuda.synchronize()
        free1, _ = torch.cuda.mem_get_info()
        times = []
        t_end = time.perf_counter() + 1.0
        while len(times) < max(20, args.steps) or time.perf_counter() < t_end:
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record(stream)
            call()
            e.record(stream)
            e.synchronize()
            times.append(s.elapsed_time(e))
            if len(times) >= 2000:
                break
        times.sort()
        ms = times[len(times) // 2]
        print(json.dumps({"N": N, "B": 1, "H": 8, "d": 128, "causal": 1, "calls": len(times),
                          "median_ms": round(ms, 4), "useful_tflops": round(flops / ms / 1e9, 1),
                          "pct_bf16_peak": round(100 * flops / ms / 1e9 / PEAK_BF16, 2),
                          "free_gib_before": round(free0 / 2**30, 3), "free_gib_after": round(free1 / 2**30, 3),
                          "inputs_outputs_mib": round((4 * q.numel() * 2 + lse.numel() * 4) / 2**20, 1)}),
              flush=True)
        del q, k, v, out, lse
        torch.cuda.empty_cache()
        N *= 2
    return 0


if __name__ == "__main__":
    sys.exit(main())
