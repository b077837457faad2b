#!/usr/bin/env python3
"""Benchmark of the AWQ hot path on one MI355X.

One step = one pass of the whole path over the 4096x4096 layer with 8192 calibration tokens
(INT4 asymmetric, g = 128, 21-point alpha grid), inputs resident in HBM:
    act_stats -> search (scale table, fused loss kernel, loss reduction, argmin) -> pack
    -> W4A16 product at M = 1, 16 and 256 tokens.
``value`` is search TFLOP/s over the whole step: 21 * 2*T*K*N flops of X.E products divided
by the step time (stats, pack and the products included), so it never exceeds the search
kernels' own rate.

Also reported on the same JSON line:
  roofline      the search (dominant kernels) against the bf16 matrix-core peak; its duration
                is measured with HIP events on the stream the library launches on;
  cpu_baseline  the fp64 oracle timed on this host on a bounded sample of the same workload;
  clip_search   the clip-ratio search on the same layer at the chosen s* (21 ratios 1 .. 0.5,
                the same number of X.E products) against the bf16 matrix-core peak;
  multi_search  the joint search of the q, k and v projections of a 70B-shaped block, which read
                one X [4096, 8192] (W [8192, 8192 | 1024 | 1024]), against the three searches
                run one by one and against the bf16 matrix-core peak;
  greedy        the power-of-two per-group greedy (20 candidates, 3 passes) on the same layer,
                a VALU-bound workload: element evaluations per second against the vector-ALU
                peak divided by the 7 operations one exact evaluation needs;
  gemv          the M = 1 W4A16 product over the seven linears of a 70B-shaped block
                (462 MB of packed weights, rotated so the 256 MB Infinity Cache cannot hold
                them) against HBM peak;
  gemv_fused    the same block with the projections that share an input searched jointly
                (awq_search_multi), so q|k|v and gate|up share s and run as one product each
                (4 launches instead of 7);
  block_quantization  the quantization of that whole block at full size on the way there
                (statistic, joint or single search and packing of each input group, one timed
                pass each) against the bf16 matrix-core peak;
  other_configs the statistic and search at full size on the 11008 -> 4096 layer (8192 tokens)
                and the symmetric g = 64 5120 -> 13824 layer (16384 tokens).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-gemv] [--no-clip]
                    [--no-multi] [--no-greedy] [--no-configs]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

METRIC = "AWQ search TFLOP/s (% bf16 MFMA peak), 4096x4096 layer, 8192 calib tokens"
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 matrix-core peak (256 CU x 2.4 GHz x 4096 flop/clk)
SPEC_MHZ = 2400                # the clock those peaks assume
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_VALU_TOPS = 39.32         # 256 CU x 4 SIMD x 16 lanes x 2.4 GHz: vector ops/s (fp32 unpacked = fp64 rate)
GREEDY_OPS_PER_EVAL = 7        # multiply, round, clamp (2), fma, multiply, fma: one exact element error


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)   # ~50 ms: the shader clock ramps up over the first ~30 ms
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gemv", action="store_true")
    ap.add_argument("--no-clip", action="store_true")
    ap.add_argument("--clip-iters", type=int, default=5)
    ap.add_argument("--no-multi", action="store_true")
    ap.add_argument("--no-greedy", action="store_true")
    ap.add_argument("--no-configs", action="store_true")
    ap.add_argument("--no-clock", action="store_true")
    ap.add_argument("--greedy-iters", type=int, default=3)
    ap.add_argument("--multi-iters", type=int, default=3)
    ap.add_argument("--gemv-iters", type=int, default=50)
    ap.add_argument("--cpu-cols", type=int, default=4096,
                    help="output columns of the oracle's bounded sample (of 4096)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one device copy of known size (for HBM counter calibration)")
    return ap.parse_args()


def search_source_digest():
    """SHA-256 of the search kernel's code (its source file and the device helpers it includes),
    with `//` comments and blank lines dropped, so that only a change to the code itself makes the
    recorded counters stale."""
    import hashlib
    h = hashlib.sha256()
    for f in ("awq_search.hip", "awq_device.h"):
        with open(os.path.join(HERE, "weight_only_int4_act_amd", "csrc", f), encoding="utf-8") as fh:
            for line in fh:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()


def search_traffic():
    """HBM-side bytes per search launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE runs
    (scaled by the copy-kernel calibration), or None once the kernel code changed since then."""
    prof = os.path.join(HERE, "profiles", "search_c2_hbm_traffic.md")
    try:
        text = open(prof, encoding="utf-8").read()
        rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
        if search_source_digest() != rec["source_sha256"]:
            return None
        # bytes the L2s fetched from and wrote to the fabric per launch, each counter scaled by
        # what it reads for a copy of known size
        return float(rec["fetch_kib"]) * 1024 * float(rec["fetch_factor"]) + \
            float(rec["write_kib"]) * 1024 * float(rec["write_factor"])
    except (OSError, IndexError, KeyError, ValueError):
        return None


def cpu_baseline(layer, n_cols):
    """The fp64 oracle as it stands, on the first n_cols output columns of the same layer:
    statistic + all 21 losses + argmin.  Returns TFLOP/s of X.E products (same count as value)."""
    from oracle import awq_oracle as O
    from weight_only_int4_act_amd import inputs as I
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [os.cpu_count()])
    except Exception:
        threads = os.cpu_count()
    X = I.bf16_to_f64(layer.X)
    W = I.bf16_to_f64(layer.W)[:, :n_cols].copy()
    T, K = X.shape
    t0 = time.perf_counter()
    _, m = O.act_stats(X)
    res = O.search(X, W, m, layer.group_size, layer.zero_point, 21)
    dt = time.perf_counter() - t0
    # the rest of the step, timed beside it: packing at the chosen scales and the W4A16 reference
    # product at M = 1, 16 and 256
    t1 = time.perf_counter()
    s_best = O.scale_table(m, 21)[int(res["best"])]
    w, d, z = O.pack(W, s_best, layer.group_size, layer.zero_point)
    t2 = time.perf_counter()
    for M in (1, 16, 256):
        O.w4a16_ref(X[:M], s_best, w, d, z, layer.group_size)
    t3 = time.perf_counter()
    flops = 21 * 2.0 * T * K * n_cols
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "seconds": round(dt, 3), "pack_seconds": round(t2 - t1, 3), "w4a16_ref_seconds": round(t3 - t2, 3),
            "best_alpha_index": int(res["best"]),
            "sample": f"oracle (numpy float64) statistic + 21-alpha search of the 4096x4096 layer restricted to "
                      f"its first {n_cols} of 4096 output columns, all 8192 tokens ({flops / 1e12:.3f} TFLOP)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the AWQ path here runs on one GPU; run with --gpus 1",
                          "n_gpus_requested": args.gpus}), flush=True)
        sys.exit(2)

    import torch
    from weight_only_int4_act_amd import awq as A
    from weight_only_int4_act_amd import inputs as I

    dev = torch.device("cuda:0")
    log("[bench] generating the 4096x4096x8192 layer (seed 0)")
    layer = I.make_config("c2", seed=0).layers[0]
    X = layer.X.to(dev)
    W = layer.W.to(dev)
    T, K = X.shape
    N = W.shape[1]
    g = layer.group_size
    cfg = A.qconfig(g, layer.zero_point, 21)

    # device buffers (allocated once, outside the timed region)
    sum_abs = torch.empty(K, dtype=torch.float64, device=dev)
    mean_abs = torch.empty(K, dtype=torch.float32, device=dev)
    ws_stats = A.workspace(A.awq_act_stats_workspace_size(T, K), dev)
    ws_search = A.workspace(A.awq_search_workspace_size(T, K, N, cfg), dev)
    losses = torch.empty(21, dtype=torch.float64, device=dev)
    best = torch.empty(1, dtype=torch.int32, device=dev)
    s_best = torch.empty(K, dtype=torch.float32, device=dev)
    codes = torch.empty((K // 8, N), dtype=torch.int32, device=dev)
    scales = torch.empty((K // g, N), dtype=torch.float32, device=dev)
    zeros = torch.empty((K // g, N), dtype=torch.uint8, device=dev)
    Ms = (1, 16, 256)
    Xm = {M: X[:M].contiguous() for M in Ms}
    Ys = {M: torch.empty((M, N), dtype=torch.bfloat16, device=dev) for M in Ms}
    ws_gemm = {M: A.workspace(A.awq_w4a16_gemm_workspace_size(M, K, N, g), dev) for M in Ms}
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]

    def step(i=None):
        A.awq_act_stats(X, sum_abs, False, T, mean_abs, ws_stats, stream)
        if i is not None:
            ev[i][0].record(stream)
        A.awq_search(X, W, mean_abs, cfg, ws_search, losses, best, s_best, stream)
        if i is not None:
            ev[i][1].record(stream)
        A.awq_pack(W, s_best, cfg, codes, scales, zeros, stream)
        for M in Ms:
            A.awq_w4a16_gemm(Xm[M], s_best, codes, scales, zeros, g, Ys[M], ws_gemm[M], stream)

    if args.calib_copy:
        src = torch.empty(1 << 28, dtype=torch.uint8, device=dev)   # 256 MiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    search_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    flops = 21 * 2.0 * T * K * N
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (search_ms * 1e-3) / 1e12
    log(f"[bench] step {ms_step:.3f} ms, search {search_ms:.3f} ms -> {achieved:.1f} TFLOP/s, best alpha "
        f"index {int(best.item())}")

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "c2: Llama-7B-shaped 4096x4096 linear, 8192 calibration tokens, INT4 asymmetric "
                               "g=128, 21-point alpha grid; step = stats + search + pack + W4A16 at M=1,16,256",
                   "T": T, "K": K, "N": N, "group_size": g, "zero_point": True, "n_grid": 21},
        "pct_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": search_traffic(),
                     "kernel": "awq_search call: k_search (the fused loss kernel, ~98% of the call) plus the "
                               "scale table, W and X tiling, loss reduction and argmin kernels",
                     "duration": "mean over the timed steps of HIP events recorded around each awq_search call "
                                 "on the stream the library launches on",
                     "algorithmic_flops_per_launch": flops, "avg_launch_ms": round(search_ms, 4)},
        "best_alpha_index": int(best.item()),
    }
    if not args.no_clock:
        out["clock"] = observed_clock(lambda: A.awq_search(X, W, mean_abs, cfg, ws_search, losses, best, s_best,
                                                           stream), torch, achieved)

    if not args.no_clip:
        out["clip_search"] = bench_clip(A, torch, dev, X, W, s_best, g, layer.zero_point, ws_search, stream,
                                        args.clip_iters)

    if not args.no_greedy:
        out["greedy"] = bench_greedy(A, torch, dev, W, mean_abs, g, stream, args.greedy_iters)

    if not args.no_multi:
        out["multi_search"] = bench_multi(A, I, torch, dev, args.multi_iters)

    if not args.no_configs:
        out["other_configs"] = bench_configs(A, I, torch, dev, 3)

    if not args.no_gemv:
        out["gemv"] = bench_gemv(A, I, torch, dev, args.gemv_iters)
        out["gemv_fused"], out["block_quantization"] = bench_gemv_fused(A, I, torch, dev, args.gemv_iters)

    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle on {args.cpu_cols} columns")
        out["cpu_baseline"] = cpu_baseline(layer, args.cpu_cols)

    print(json.dumps(out), flush=True)


def bench_clip(A, torch, dev, X, W, s_best, g, zp, ws, stream, iters):
    """The clip-ratio search on the same layer at the alpha search's s*: 21 ratios 1 .. 0.5, so the
    X.E work equals the alpha search's (same fused kernel, clipped quantizer, 512-row tiles)."""
    T, K = X.shape
    N = W.shape[1]
    cfg = A.qconfig(g, zp, 21)
    losses = torch.empty(21, dtype=torch.float64, device=dev)
    best = torch.empty(1, dtype=torch.int32, device=dev)
    cbest = torch.empty(1, dtype=torch.float32, device=dev)
    A.awq_clip_search(X, W, s_best, cfg, 0.5, ws, losses, best, cbest, stream)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(iters):
        A.awq_clip_search(X, W, s_best, cfg, 0.5, ws, losses, best, cbest, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    flops = 21 * 2.0 * T * K * N
    tf = flops / (ms * 1e-3) / 1e12
    log(f"[bench] clip search {ms:.3f} ms -> {tf:.1f} TFLOP/s, best ratio {float(cbest.item())}")
    return {"workload": "c2 layer at s*: 21 clip ratios 1 .. 0.5", "ms": round(ms, 4), "achieved": round(tf, 3),
            "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4), "best_index": int(best.item()),
            "best_ratio": float(cbest.item())}


def bench_greedy(A, torch, dev, W, mean_abs, g, stream, iters):
    """The power-of-two greedy over the same layer's scales: 20 candidates, 3 passes, asymmetric."""
    K, N = W.shape
    cfg = A.qconfig(g, True, 21)
    ws = A.workspace(A.awq_greedy_workspace_size(K, N, cfg, 20), dev)
    s = torch.empty(K, dtype=torch.float32, device=dev)
    er = torch.empty(K // g, dtype=torch.float64, device=dev)
    e = torch.empty_like(er)
    A.awq_greedy_search(W, mean_abs, cfg, 20, 3, ws, s, er, e, stream)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(iters):
        A.awq_greedy_search(W, mean_abs, cfg, 20, 3, ws, s, er, e, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    evals = 3.0 * K * 20 * N * g            # passes x K x candidates x N x g element evaluations
    rate = evals / (ms * 1e-3) / 1e12
    peak = PEAK_VALU_TOPS / GREEDY_OPS_PER_EVAL
    ratio = float(er.sum().item() / e.sum().item())
    log(f"[bench] greedy {ms:.2f} ms ({ms * 1e3 / (3 * g):.1f} us per step) -> {rate:.2f} T evals/s, "
        f"rounding error / greedy error = {ratio:.3f}")
    return {"workload": "c2 layer: power-of-two greedy, 20 candidates 2^-10..2^9, 3 passes, g=128 asymmetric",
            "ms": round(ms, 3), "launches": 3 * g + 2,
            "roofline": {"bound": "alu", "achieved": round(rate, 3), "peak": round(peak, 3),
                         "unit": "T element-evaluations/s", "frac": round(rate / peak, 4), "traffic": None},
            "algorithmic_evals_per_call": evals, "err_rtn_over_err": round(ratio, 4),
            "scales_above_1": int((s > 1).sum().item()), "scales_below_1": int((s < 1).sum().item())}


def bench_configs(A, I, torch, dev, iters):
    """The search (statistic + 21-point search + argmin) at the full size of the other single-layer
    configurations: the 11008 -> 4096 down projection with silu-like activations and 8192 tokens,
    and the 5120 -> 13824 symmetric g=64 projection with 16384 tokens."""
    res = {}
    for name in ("c3", "c4"):
        log(f"[bench] {name}: generating the full-size layer")
        L = I.make_config(name, seed=0).layers[0]
        X, W = L.X.to(dev), L.W.to(dev)
        T, K = X.shape
        N = W.shape[1]
        cfg = A.qconfig(L.group_size, L.zero_point, 21)
        stream = torch.cuda.current_stream()
        sum_abs = torch.empty(K, dtype=torch.float64, device=dev)
        m = torch.empty(K, dtype=torch.float32, device=dev)
        ws_stats = A.workspace(A.awq_act_stats_workspace_size(T, K), dev)
        ws = A.workspace(A.awq_search_workspace_size(T, K, N, cfg), dev)
        losses = torch.empty(21, dtype=torch.float64, device=dev)
        best = torch.empty(1, dtype=torch.int32, device=dev)
        s_best = torch.empty(K, dtype=torch.float32, device=dev)

        def search():
            A.awq_act_stats(X, sum_abs, False, T, m, ws_stats, stream)
            A.awq_search(X, W, m, cfg, ws, losses, best, s_best, stream)

        search()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(iters):
            search()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        flops = 21 * 2.0 * T * K * N
        tf = flops / (ms * 1e-3) / 1e12
        log(f"[bench] {name} ({T}x{K} -> {N}, g={L.group_size}, {'asym' if L.zero_point else 'sym'}): statistic + "
            f"search {ms:.3f} ms -> {tf:.1f} TFLOP/s, alpha* {int(best.item())}")
        res[name] = {"workload": f"{name}: T={T}, K={K}, N={N}, g={L.group_size}, "
                                 f"{'asymmetric' if L.zero_point else 'symmetric'}, 21-point alpha grid",
                     "ms": round(ms, 4), "algorithmic_flops": flops, "achieved": round(tf, 3), "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_BF16_TFLOPS, 4), "best_index": int(best.item())}
        del X, W, ws, L
    return res


def bench_multi(A, I, torch, dev, iters):
    """Joint search of q, k and v (one X) against the three single searches, same inputs."""
    log("[bench] multi: building X_attn [4096, 8192] and q, k, v")
    X = I.c5_input(0, 0).to(dev)
    Ws = [I.c5_weight(0, l).to(dev) for l in range(3)]
    T, K = X.shape
    Ns = [W.shape[1] for W in Ws]
    cfg = A.qconfig(128, True, 21)
    stream = torch.cuda.current_stream()
    sum_abs = torch.empty(K, dtype=torch.float64, device=dev)
    m = torch.empty(K, dtype=torch.float32, device=dev)
    A.awq_act_stats(X, sum_abs, False, T, m, A.workspace(A.awq_act_stats_workspace_size(T, K), dev), stream)
    ws = A.workspace(max([A.awq_search_multi_workspace_size(T, K, Ns, cfg)] +
                         [A.awq_search_workspace_size(T, K, n, cfg) for n in Ns]), dev)
    losses = torch.empty(21, dtype=torch.float64, device=dev)
    each = torch.empty((3, 21), dtype=torch.float64, device=dev)
    best = torch.empty(1, dtype=torch.int32, device=dev)
    s_best = torch.empty(K, dtype=torch.float32, device=dev)

    def joint():
        A.awq_search_multi(X, Ws, m, cfg, ws, losses, each, best, s_best, stream)

    def singles():
        for W in Ws:
            A.awq_search(X, W, m, cfg, ws, losses, best, s_best, stream)

    res = {}
    for name, fn in (("singles", singles), ("joint", joint)):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(iters):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / iters
    flops = 21 * 2.0 * T * K * sum(Ns)
    tf = flops / (res["joint"] * 1e-3) / 1e12
    log(f"[bench] multi search q,k,v: joint {res['joint']:.3f} ms ({tf:.1f} TFLOP/s), one by one "
        f"{res['singles']:.3f} ms, alpha* {int(best.item())}")
    return {"workload": "c5 attention: X [4096, 8192] shared by q, k, v; W [8192, 8192 | 1024 | 1024]; "
                        "INT4 asym g=128, 21-point alpha grid",
            "joint_ms": round(res["joint"], 4), "one_by_one_ms": round(res["singles"], 4),
            "speedup": round(res["singles"] / res["joint"], 3), "achieved": round(tf, 3), "unit": "TFLOP/s",
            "frac": round(tf / PEAK_BF16_TFLOPS, 4), "algorithmic_flops_per_call": flops,
            "best_index": int(best.item())}


def _gemv_bytes(K, N, g=128):
    return K * N // 2 + 4 * (K // g) * N + (K // g) * N + 4 * K + 2 * K + 2 * N


def observed_clock(run_once, torch, achieved):
    """The shader clock the chip holds under the search: the search runs back to back for ~3 s
    while `amd-smi metric -c` is read five times from 1 s in (per-XCD gfx clocks, MHz; the SMU reports a short
    average, so single readings scatter).  The matrix-core peak scales with the clock, so the
    fraction of the peak at the median observed clock is given beside the spec one.  Null fields if
    the tool is missing or fails."""
    import subprocess
    import threading
    samples = []

    def sample():
        time.sleep(1.0)         # past the ramp from idle: earlier readings still average in the idle clock
        for _ in range(5):
            try:
                r = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "--json"], capture_output=True,
                                   text=True, timeout=10)
                clk = json.loads(r.stdout)["gpu_data"][0]["clock"] if r.returncode == 0 else {}
                per_xcd = [float(v["clk"]["value"]) for k, v in sorted(clk.items()) if k.startswith("gfx_")]
                if per_xcd:
                    samples.append(per_xcd)
            except Exception:   # tool missing, hung or unexpected output: no sample
                pass
            time.sleep(0.3)

    th = threading.Thread(target=sample)
    th.start()
    t0 = time.perf_counter()
    while th.is_alive():
        for _ in range(10):
            run_once()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 > 30.0:
            break
    th.join()
    means = sorted(sum(x) / len(x) for x in samples)
    med = means[len(means) // 2] if means else None
    out = {"observed_gfx_mhz": round(med, 1) if med else None,
           "samples_mhz": [round(m, 1) for m in means], "spec_mhz": SPEC_MHZ,
           "method": "amd-smi metric -c, read five times from 1 s into ~3 s of back-to-back searches of "
                     "the same layer; the median of the per-reading means over the 8 XCDs"}
    if med:
        out["frac_of_peak_at_observed_clock"] = round(achieved / (PEAK_BF16_TFLOPS * med / SPEC_MHZ), 4)
        log(f"[bench] observed shader clock during the search {med:.0f} MHz (readings "
            f"{', '.join(f'{m:.0f}' for m in means)}; spec {SPEC_MHZ}): "
            f"{100 * achieved / (PEAK_BF16_TFLOPS * med / SPEC_MHZ):.1f}% of the peak at that clock")
    return out


def bench_gemv_fused(A, I, torch, dev, iters):
    """M = 1 block with q|k|v and gate|up each searched jointly and packed side by side.  The
    quantization of each group (statistic, joint search, packing) is timed on the way: the whole
    70B-shaped block at full size."""
    log("[bench] gemv_fused: joint searches of q,k,v and gate,up; o and down alone (timed)")
    cfg = A.qconfig(128, True, 21)
    stream = torch.cuda.current_stream()
    groups = (("qkv", 0, (0, 1, 2)), ("o", 1, (3,)), ("gate_up", 2, (4, 5)), ("down", 3, (6,)))
    layers = []
    quant = {}
    xm = {}
    for name, j, ls in groups:
        X = I.c5_input(0, j).to(dev)
        Ws = [I.c5_weight(0, l).to(dev) for l in ls]
        T, K = X.shape
        Ns = [W.shape[1] for W in Ws]
        sum_abs = torch.empty(K, dtype=torch.float64, device=dev)
        m = torch.empty(K, dtype=torch.float32, device=dev)
        ws_stats = A.workspace(A.awq_act_stats_workspace_size(T, K), dev)
        ws = A.workspace(A.awq_search_multi_workspace_size(T, K, Ns, cfg), dev)
        losses = torch.empty(21, dtype=torch.float64, device=dev)
        each = torch.empty((len(Ws), 21), dtype=torch.float64, device=dev)
        best = torch.empty(1, dtype=torch.int32, device=dev)
        s_best = torch.empty(K, dtype=torch.float32, device=dev)
        outs = [(torch.empty((K // 8, n), dtype=torch.int32, device=dev),
                 torch.empty((K // 128, n), dtype=torch.float32, device=dev),
                 torch.empty((K // 128, n), dtype=torch.uint8, device=dev)) for n in Ns]

        def quantize():
            A.awq_act_stats(X, sum_abs, False, T, m, ws_stats, stream)
            A.awq_search_multi(X, Ws, m, cfg, ws, losses, each, best, s_best, stream)
            for W, (c, sc, z) in zip(Ws, outs):
                A.awq_pack(W, s_best, cfg, c, sc, z, stream)

        quantize()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        quantize()
        e1.record(stream)
        torch.cuda.synchronize()
        quant[name] = {"ms": e0.elapsed_time(e1), "flops": 21 * 2.0 * T * K * sum(Ns),
                       "best_index": int(best.item())}
        q = A.Quantized(torch.cat([o[0] for o in outs], 1).contiguous(), torch.cat([o[1] for o in outs], 1).contiguous(),
                        torch.cat([o[2] for o in outs], 1).contiguous(), s_best, 128)
        N = q.codes.shape[1]
        x1 = X[:1].contiguous()
        xm[name] = {M: X[:M].contiguous() for M in (16, 256)}
        del X, Ws, ws, outs
        y = torch.empty((1, N), dtype=torch.bfloat16, device=dev)
        wsg = A.workspace(A.awq_w4a16_gemm_workspace_size(1, K, N, 128), dev)
        layers.append((name, K, N, x1, q, y, wsg, _gemv_bytes(K, N)))
    qms = sum(v["ms"] for v in quant.values())
    qfl = sum(v["flops"] for v in quant.values())
    qtf = qfl / (qms * 1e-3) / 1e12
    log(f"[bench] 70B block quantization (stats + joint searches + pack): {qms:.2f} ms, search flops "
        f"{qfl / 1e12:.1f} TFLOP -> {qtf:.1f} TFLOP/s")
    block_quant = {"workload": "c5 block, all 7 linears at full size, 4096 tokens: q,k,v searched jointly on X_attn, "
                               "o alone, gate,up jointly on X_mlp, down alone (K=28672); each group = statistic + "
                               "search + pack",
                   "ms": round(qms, 3), "algorithmic_flops": qfl, "achieved": round(qtf, 3), "unit": "TFLOP/s",
                   "frac": round(qtf / PEAK_BF16_TFLOPS, 4),
                   "groups": {k: {"ms": round(v["ms"], 3), "best_index": v["best_index"]} for k, v in quant.items()}}
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def block():
        for (name, K, N, x1, q, y, ws, byts) in layers:
            A.awq_w4a16_gemm(x1, q.s, q.codes, q.scales, q.zeros, 128, y, ws, stream)

    for _ in range(3):
        block()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(iters):
        block()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    total = sum(l[-1] for l in layers)
    gbs = total / (ms * 1e-3) / 1e9
    log(f"[bench] gemv_fused block {ms * 1e3:.2f} us -> {gbs:.1f} GB/s ({100 * gbs / PEAK_HBM_GBS:.1f}% of HBM)")
    res = {"workload": "c5 block M=1 with shared-input projections fused: q|k|v [8192x10240], o [8192x8192], "
                       "gate|up [8192x57344], down [28672x8192] (462 MB rotated per iteration)",
           "iters": iters, "block_us": round(ms * 1e3, 2), "block_bytes": total, "achieved_GBs": round(gbs, 1),
           "peak_GBs": PEAK_HBM_GBS, "frac": round(gbs / PEAK_HBM_GBS, 4)}
    # the fused block at M = 16 and M = 256: four launches instead of seven
    res["M16_M256"] = _block_at_m(A, torch, dev, layers, xm, iters, total, "gemv_fused block")
    return res, block_quant


def _block_at_m(A, torch, dev, layers, xm, iters, m1_bytes, label):
    """The block of products at M = 16 (weight bytes still dominate) and M = 256 (matrix cores):
    back-to-back launches, each layer with its own output and workspace."""
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    out = {}
    for M in (16, 256):
        ys = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for (name, K, N, *_r) in layers]
        wss = [A.workspace(A.awq_w4a16_gemm_workspace_size(M, K, N, 128), dev) for (name, K, N, *_r) in layers]

        def blockm():
            for (name, K, N, x1, q, y, ws, byts), yy, ww in zip(layers, ys, wss):
                A.awq_w4a16_gemm(xm[name][M], q.s, q.codes, q.scales, q.zeros, 128, yy, ww, stream)

        blockm()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(iters):
            blockm()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        flops = sum(2.0 * M * K * N for (name, K, N, *_r) in layers)
        byts = m1_bytes + sum(2 * M * (K + N) for (name, K, N, *_r) in layers)
        out[f"M{M}"] = {"block_us": round(ms * 1e3, 2), "GBs": round(byts / (ms * 1e-3) / 1e9, 1),
                        "frac_hbm": round(byts / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                        "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 2),
                        "frac_bf16": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        log(f"[bench] {label} at M={M}: {ms * 1e3:.1f} us -> {byts / (ms * 1e-3) / 1e9:.0f} GB/s, "
            f"{flops / (ms * 1e-3) / 1e12:.1f} TFLOP/s")
        del ys, wss
    return out


def bench_gemv(A, I, torch, dev, iters):
    """M = 1 W4A16 product over the seven linears of the 70B-shaped block.  Each layer is run
    through stats -> search -> pack once (untimed) to produce its packed weights."""
    layers = []
    xs = {}
    xm = {}
    log("[bench] gemv: building the 70B-shaped block (7 linears, T=4096)")
    for l, (name, K, N, j) in enumerate(I.C5_LAYERS):
        if j not in xs:
            xs[j] = I.c5_input(0, j).to(dev)
        Wl = I.c5_weight(0, l).to(dev)
        r = A.run_layer(xs[j], Wl, A.qconfig(128, True, 21))
        del Wl
        q = r["q"]
        x1 = xs[j][:1].contiguous()
        xm[name] = {M: xs[j][:M].contiguous() for M in (16, 256)}
        y = torch.empty((1, N), dtype=torch.bfloat16, device=dev)
        ws = A.workspace(A.awq_w4a16_gemm_workspace_size(1, K, N, 128), dev)
        byts = _gemv_bytes(K, N)
        layers.append((name, K, N, x1, q, y, ws, byts))
    xs.clear()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def block():
        for (name, K, N, x1, q, y, ws, byts) in layers:
            A.awq_w4a16_gemm(x1, q.s, q.codes, q.scales, q.zeros, 128, y, ws, stream)

    for _ in range(3):
        block()
    torch.cuda.synchronize()
    per = {name: [] for (name, *_r) in layers}
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in layers]
           for _ in range(iters)]
    # block time: back-to-back launches only
    e0.record(stream)
    for it in range(iters):
        block()
    e1.record(stream)
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1) / iters
    # per-layer times: events around each launch
    for it in range(iters):
        for li, (name, K, N, x1, q, y, ws, byts) in enumerate(layers):
            evs[it][li][0].record(stream)
            A.awq_w4a16_gemm(x1, q.s, q.codes, q.scales, q.zeros, 128, y, ws, stream)
            evs[it][li][1].record(stream)
    torch.cuda.synchronize()
    total_bytes = sum(l[-1] for l in layers)
    res = {"workload": "c5 block M=1: q,k,v,o [8192x8192|1024], gate,up [8192x28672], down [28672x8192], "
                       "INT4 asym g=128, weights rotated through 7 layers (462 MB) per iteration",
           "iters": iters, "block_us": round(total_ms * 1e3, 2), "block_bytes": total_bytes,
           "achieved_GBs": round(total_bytes / (total_ms * 1e-3) / 1e9, 1), "peak_GBs": PEAK_HBM_GBS,
           "layers": {}}
    res["frac"] = round(res["achieved_GBs"] / PEAK_HBM_GBS, 4)
    for li, (name, K, N, x1, q, y, ws, byts) in enumerate(layers):
        us = float(np.median([evs[it][li][0].elapsed_time(evs[it][li][1]) for it in range(iters)])) * 1e3
        res["layers"][name] = {"us": round(us, 2), "GBs": round(byts / (us * 1e-6) / 1e9, 1)}
    log(f"[bench] gemv block {res['block_us']} us -> {res['achieved_GBs']} GB/s ({100 * res['frac']:.1f}% of HBM)")
    # the same block at M = 16 (weight bytes still dominate) and M = 256 (matrix cores)
    res["M16_M256"] = _block_at_m(A, torch, dev, layers, xm, iters, total_bytes, "block")
    return res


if __name__ == "__main__":
    main()
