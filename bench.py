#!/usr/bin/env python3
"""Benchmark: batch-1 decode through a 27B-class stack of low-bit layers.

One step = one token through 64 layers; each layer runs the batch-1 products
of its projections in the order a decoder layer uses them: q/k/v (one fused
15360 x 5120 matrix), o (5120 x 5120), gate/up (one fused 34816 x 5120
matrix) and down (5120 x 17408), with group-128 fp16 scales and bf16
activations.  All weights (3.35 GB binary, 6.33 GB ternary 2-bit) are
resident in HBM; the step is captured once as a HIP graph and replayed.

Prints one JSON line (see --help for options).  The CPU-baseline leg times
the fp64 oracle on one layer of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
LAYERS = 64
HIDDEN, FFN = 5120, 17408
# (name, N, K) of the per-layer products, fused where the inputs are shared
MATS = [("qkv", 3 * HIDDEN, HIDDEN), ("o", HIDDEN, HIDDEN), ("gateup", 2 * FFN, HIDDEN),
        ("down", HIDDEN, FFN)]
FMT_NAMES = {1: "binary", 2: "ternary-2bit", 3: "ternary-base3"}
SEED = 1002  # 1000 + config index of the decode-step workload


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_model(lb, synth, torch, fmt, layers):
    tern = fmt != 1
    W = []
    t0 = time.time()
    for l in range(layers):
        mats = []
        for j, (name, N, K) in enumerate(MATS):
            tid = 16 * l + 2 * j
            codes = synth.device_codes(tern, SEED, tid, N, K, "cuda", chunk_rows=2048)
            scales = synth.device_scales(SEED, tid + 1, N, K // 128, "cuda")
            pc, ps = lb.pack(fmt, codes, scales)
            del codes, scales
            mats.append((pc, ps))
        W.append(mats)
        if l % 16 == 15:
            torch.cuda.synchronize()
            log(f"  built {l + 1}/{layers} layers ({time.time() - t0:.1f}s)")
    torch.cuda.synchronize()
    return W


def packed_step_bytes(lb, fmt, layers):
    tot = 0
    for _, N, K in MATS:
        cb, sb = lb.packed_bytes(fmt, N, K)
        tot += cb + sb
    return tot * layers


def run_step(lb, torch, fmt, W, xs, ys, layers):
    for l in range(layers):
        for j, (name, N, K) in enumerate(MATS):
            pc, ps = W[l][j]
            lb.gemv(fmt, N, K, pc, ps, xs[j], y=ys[j], y_dtype=lb.F32)


def cpu_baseline(fmt, budget_s):
    """The oracle, as it stands, on a bounded sample: 64-row slices of the four
    layer matrices (regenerated bit-exactly on the host), timed over as many
    calls as fit the budget and scaled to tokens per second."""
    import numpy as np
    import synth
    from oracle import oracle as O
    gen = synth.ternary_codes if fmt != 1 else synth.binary_codes
    rows = np.arange(64)
    sample = []
    for j, (name, N, K) in enumerate(MATS):
        sample.append((gen(SEED, 2 * j, N, K, rows=rows),
                       synth.group_scales(SEED, 2 * j + 1, N, K // 128, rows=rows),
                       synth.normal_bf16(SEED, 900 + j, 1, K), K))
    macs_done, t_used, calls = 0, 0.0, 0
    while t_used < budget_s:
        codes, scales, x, K = sample[calls % len(sample)]
        t0 = time.perf_counter()
        O.matmul(codes, scales, O.X_BF16, x, with_abs=False)
        t_used += time.perf_counter() - t0
        macs_done += len(rows) * K
        calls += 1
    layer_macs = sum(N * K for _, N, K in MATS)
    sec_per_token = t_used / macs_done * layer_macs * LAYERS
    return {"value": 1.0 / sec_per_token, "unit": "tok/s", "cores": 1, "kind": "oracle",
            "sample": f"{calls} oracle calls on 64-row slices of the four layer-0 matrices "
                      f"({macs_done / 1e6:.0f}M weight MACs, {t_used:.1f}s, 1 thread), scaled to "
                      f"{layer_macs * LAYERS / 1e9:.2f}G MACs per token"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--fmt", type=int, default=2, choices=[1, 2])
    ap.add_argument("--layers", type=int, default=LAYERS)
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported in this build "
              "(every box has one MI355X)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from ultra_bit_dit_amd import lowbit as lb

    fmt, layers = args.fmt, args.layers
    log(f"building {layers} layers, {FMT_NAMES[fmt]}")
    W = build_model(lb, synth, torch, fmt, layers)
    xs = [torch.from_numpy(synth.normal_bf16(SEED, 900 + j, 1, K).view(np.int16)).cuda()
          .view(torch.bfloat16)[0] for j, (_, _, K) in enumerate(MATS)]
    ys = [torch.empty(N, dtype=torch.float32, device="cuda") for _, N, _ in MATS]
    step_bytes = packed_step_bytes(lb, fmt, layers)

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        run_step(lb, torch, fmt, W, xs, ys, layers)  # eager warm-up (allocates the workspace)
    torch.cuda.synchronize()
    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            run_step(lb, torch, fmt, W, xs, ys, layers)
        torch.cuda.synchronize()

    def step():
        if graph is not None:
            graph.replay()
        else:
            run_step(lb, torch, fmt, W, xs, ys, layers)

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(args.steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / args.steps
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    log(f"step {ms_step:.3f} ms, {gbs:.0f} GB/s, {1000 / ms_step:.1f} tok/s (wall {wall:.2f}s)")

    out = {
        "metric": "decode GEMV HBM GB/s (% peak) & tok/s; pp512 GEMM TFLOP/s (% MFMA peak)",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"27B-class decode step, {FMT_NAMES[fmt]}: {layers} layers x "
                               "(qkv 15360x5120, o 5120x5120, gate/up 34816x5120, down 5120x17408), "
                               "group-128 fp16 scales, bf16 activations, batch 1",
                   "tok_s": round(1000.0 / ms_step, 2),
                   "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1),
                   "bytes_per_step": step_bytes,
                   "graph": graph is not None},
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(fmt, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
