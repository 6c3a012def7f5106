#!/usr/bin/env python3
"""Benchmark of the group-scaled binary / ternary matmul on one MI355X.

Headline (``value``): batch-1 decode through a 27B-class stack of low-bit
layers.  One step = one token through 64 layers; each layer runs the batch-1
products of its projections in the order a decoder layer uses them: q/k/v
(one fused 15360 x 5120 matrix), o (5120 x 5120), gate/up (one fused
34816 x 5120 matrix) and down (5120 x 17408), with group-128 fp16 scales and
bf16 activations (a fixed synthetic x per shape, outputs not fed back).  All
weights (3.35 GB binary, 6.33 GB ternary 2-bit) are resident in HBM.  By
default the step is one persistent launch (lowbit_chain_run) that streams
the weights of all 256 products; the same step with sequential dependencies
between products, and as 256 separate launches in a HIP graph, is reported
beside it.  ``value`` is packed-weight GB/s (weights + scales read per step /
step time).

Also reported: the pp512 prefill pass (M = 512 tokens through the same four
ternary layer products, bf16 activations and int8 activations) and the
diffusion-transformer block GEMMs (binary, M = 4608 and 18432) in TFLOP/s;
the roofline of the decode kernel (HBM) with its measured HBM traffic; and
the fp64 oracle timed on the host as a CPU baseline.

Prints one JSON line (see --help for options).
"""
import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_PEAK_F16_TFLOPS = 2516.6  # dense fp16 / bf16 MFMA
MFMA_PEAK_I8_TOPS = 5033.2     # dense int8 MFMA
MFMA_PEAK_F4_TOPS = 10100.0    # dense fp4 MFMA
LAYERS = 64
HIDDEN, FFN = 5120, 17408
# (name, N, K) of the per-layer products, fused where the inputs are shared
MATS = [("qkv", 3 * HIDDEN, HIDDEN), ("o", HIDDEN, HIDDEN), ("gateup", 2 * FFN, HIDDEN),
        ("down", HIDDEN, FFN)]
# diffusion-transformer block: q, k, v, out (3072^2), FFN up 3072 -> 9216, down 9216 -> 3072
DIT = [("q", 3072, 3072), ("k", 3072, 3072), ("v", 3072, 3072), ("out", 3072, 3072),
       ("up", 9216, 3072), ("down", 3072, 9216)]
FMT_NAMES = {1: "binary", 2: "ternary-2bit", 3: "ternary-base3"}
SEED = 1002  # decode-step workload
PP_SEED, DIT_SEED = 1003, 1004
PMC_SUMMARY = os.path.join(ROOT, "profiles", "{kernel}_decode_step_pmc.txt")
# sources the decode kernels are built from (their hash ties a counter summary to them)
GEMV_SOURCES = [os.path.join(ROOT, "ultra_bit_dit_amd", "csrc", f)
                for f in ("gemv.hip", "fp4.hpp", "common.hpp")]


def gemv_source_hash():
    """sha256 of the decode kernel's sources with comments and blank space
    removed: an edit of a comment leaves the kernel, and its counters, valid."""
    h = hashlib.sha256()
    for path in GEMV_SOURCES:
        with open(path, encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_mats(lb, synth, fmt, seed, tid0, shapes, chunk_rows=2048):
    out = []
    for j, (name, N, K) in enumerate(shapes):
        tid = tid0 + 2 * j
        codes = synth.device_codes(fmt != 1, seed, tid, N, K, "cuda", chunk_rows=chunk_rows)
        scales = synth.device_scales(seed, tid + 1, N, K // 128, "cuda")
        out.append(lb.pack(fmt, codes, scales))
        del codes, scales
    return out


def build_model(lb, synth, torch, fmt, layers):
    W = []
    t0 = time.time()
    for l in range(layers):
        W.append(build_mats(lb, synth, fmt, SEED, 16 * l, MATS))
        if l % 16 == 15:
            torch.cuda.synchronize()
            log(f"  built {l + 1}/{layers} layers ({time.time() - t0:.1f}s)")
    torch.cuda.synchronize()
    return W


def packed_bytes(lb, fmt, shapes):
    tot = 0
    for _, N, K in shapes:
        cb, sb = lb.packed_bytes(fmt, N, K)
        tot += cb + sb
    return tot


def run_step(lb, fmt, W, xs, ys, layers):
    for l in range(layers):
        for j, (name, N, K) in enumerate(MATS):
            pc, ps = W[l][j]
            lb.gemv(fmt, N, K, pc, ps, xs[j], y=ys[j], y_dtype=lb.F32)


def time_region(torch, stream, fn, steps, warmup):
    """Warm-up, then `steps` calls bracketed by synchronisations; HIP events
    on `stream` (the stream every launch goes to).  Returns ms per call."""
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def pmc_traffic(launch_bytes, kernel):
    """HBM bytes per launch of the decode kernel from the committed rocprofv3
    counter summary, scaled by the same counters read on a plain copy of
    known size; None when the summary is missing or the kernel source changed
    since the counters were taken."""
    try:
        kv = {}
        with open(PMC_SUMMARY.format(kernel=kernel)) as f:
            for line in f:
                if "=" in line and not line.startswith("#"):
                    k, v = line.split("=", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("gemv_source_sha256_16") != gemv_source_hash() or kv.get("kernel") != kernel:
            return None, "kernel changed since the counters were taken"
        copy_bytes = float(kv["copy_bytes_each_way"])
        f_scale = copy_bytes / (float(kv["copy_FETCH_SIZE_KiB"]) * 1024.0)
        w_scale = copy_bytes / (float(kv["copy_WRITE_SIZE_KiB"]) * 1024.0)
        fetch = float(kv["gemv_FETCH_SIZE_KiB_per_dispatch"]) * 1024.0 * f_scale
        write = float(kv["gemv_WRITE_SIZE_KiB_per_dispatch"]) * 1024.0 * w_scale
        # the counters were taken on a launch of the same kernel over fewer
        # layers (the profiler cannot count the full build); traffic per
        # algorithmic byte carries over to this launch
        ratio = (fetch + write) / float(kv["profiled_algorithmic_bytes_per_dispatch"])
        return ratio * launch_bytes, (
            f"rocprofv3 FETCH_SIZE + WRITE_SIZE per dispatch, scaled by a "
            f"{copy_bytes / 2**20:.0f} MiB copy (x{f_scale:.3f} / x{w_scale:.3f}), measured on a "
            f"launch of {float(kv['profiled_algorithmic_bytes_per_dispatch']) / 1e6:.0f} MB and "
            f"carried over per byte: {ratio:.3f} x the algorithmic bytes")
    except (OSError, KeyError, ValueError):
        return None, "no counter summary"


def copy_calibration(torch):
    """A plain elementwise copy of known size (read 256 MiB, write 256 MiB):
    the reference the HBM byte counters are scaled by."""
    src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def hbm_read_rate(lb, torch, steps=10, warmup=2, nbytes=4 << 30):
    """Sustained HBM read rate of this device: a plain streaming read of a
    4 GiB buffer (lowbit_hbm_read_probe), timed like the decode step."""
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    ms = time_region(torch, stream, lambda: lb.hbm_read_probe(buf, out, stream), steps, warmup)
    del buf, out
    torch.cuda.synchronize()
    return nbytes / (ms * 1e-3) / 1e9


def chain_for(lb, fmt, W, xs, ys, layers, wait, torch=None):
    """One persistent chain over every product of the step.  With waits the
    chain is a sequential decode layer: the gate/up product runs the SiLU-mul
    epilogue and the down projection reads its output z (bf16 activations
    throughout); q/k/v and o read fixed activations (attention is not part of
    the path)."""
    if not wait:
        stages = []
        for l in range(layers):
            for j, (name, N, K) in enumerate(MATS):
                stages.append((fmt, N, K, W[l][j][0], W[l][j][1], xs[j], ys[j], 0))
        return lb.Chain(stages, x_dtype=lb.BF16, y_dtype=lb.F32)
    names = [m[0] for m in MATS]
    gu, dn = names.index("gateup"), names.index("down")
    outs = [torch.empty(N // 2 if j == gu else N, dtype=torch.bfloat16, device="cuda")
            for j, (_, N, _) in enumerate(MATS)]
    stages = []
    for l in range(layers):
        for j, (name, N, K) in enumerate(MATS):
            x = outs[gu] if j == dn else xs[j]
            epi = lb.EPI_SILU_MUL if j == gu else lb.EPI_NONE
            stages.append((fmt, N, K, W[l][j][0], W[l][j][1], x, outs[j], 1, epi))
    ch = lb.Chain(stages, x_dtype=lb.BF16, y_dtype=lb.BF16)
    ch._outs = outs
    return ch


def bench_decode(args, lb, synth, torch, np):
    """Times the decode step three ways (see --modes):
    chain      one persistent launch per step streams all 4 x layers products
               (the products of this workload are independent: fixed x per shape);
    chain_dep  the same launch with every product waiting for the previous one
               to complete before reading its activations (sequential decode),
               gate/up with the SiLU-mul epilogue feeding the down projection;
    separate   one lowbit_gemv launch per product, the step captured as a HIP graph.
    The first mode listed is the headline."""
    fmt, layers = args.fmt, args.layers
    modes = [m for m in args.modes.split(",") if m]
    log(f"building {layers} layers, {FMT_NAMES[fmt]}")
    W = build_model(lb, synth, torch, fmt, layers)
    xs = [torch.from_numpy(synth.normal_bf16(SEED, 900 + j, 1, K).view(np.int16)).cuda()
          .view(torch.bfloat16)[0] for j, (_, _, K) in enumerate(MATS)]
    ys = [torch.empty(N, dtype=torch.float32, device="cuda") for _, N, _ in MATS]
    step_bytes = packed_bytes(lb, fmt, MATS) * layers
    stream = torch.cuda.Stream()
    res = {}
    for mode in modes:
        if mode in ("chain", "chain_dep"):
            ch = chain_for(lb, fmt, W, xs, ys, layers, 1 if mode == "chain_dep" else 0, torch)
            ms = time_region(torch, stream, lambda: ch.run(stream), args.steps, args.warmup)
            if ch.failed_waits():
                raise RuntimeError("chain wait gave up")
            ch.close()
            res[mode] = (ms, 1)
        elif mode == "separate":
            with torch.cuda.stream(stream):
                run_step(lb, fmt, W, xs, ys, layers)  # eager warm-up (allocates the workspace)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                run_step(lb, fmt, W, xs, ys, layers)
            torch.cuda.synchronize()
            ms = time_region(torch, stream, graph.replay, args.steps, args.warmup)
            del graph
            res[mode] = (ms, len(MATS) * layers)
        else:
            raise SystemExit(f"unknown mode {mode}")
        log(f"decode [{mode}] {ms:.3f} ms/step, {step_bytes / ms / 1e6:.0f} GB/s, "
            f"{1000 / ms:.1f} tok/s")
    head = modes[0]
    ms, launches = res[head]
    gbs = step_bytes / (ms * 1e-3) / 1e9
    launch_bytes = step_bytes / launches
    launch_us = ms * 1e3 / launches
    kbase = {"chain": "gemv_stream", "chain_dep": "gemv_chain", "separate": "gemv_mfma"}[head]
    traffic, tnote = pmc_traffic(launch_bytes, kbase)
    kname = kbase + (" (ternary 2-bit" if fmt == 2 else " (binary") + ", bf16 x, fp32 y)"
    roof = {"bound": "hbm", "kernel": kname,
            "achieved": round(launch_bytes / (launch_us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(launch_bytes / (launch_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": None if traffic is None else round(traffic),
            "algorithmic_bytes_per_launch": round(launch_bytes),
            "avg_launch_us": round(launch_us, 3),
            "note": f"{launches} launch(es) per step, durations from HIP events over the timed "
                    f"region; traffic: {tnote}"}
    modes_out = {m: {"ms_per_step": round(v[0], 4), "gb_s": round(step_bytes / v[0] / 1e6, 1),
                     "tok_s": round(1000.0 / v[0], 2), "launches_per_step": v[1]}
                 for m, v in res.items()}
    if args.verify_rows > 1:
        # one pass of `verify_rows` activation rows through every product of
        # the step (checking verify_rows - 1 drafted tokens and the next one)
        M = args.verify_rows
        xv = [torch.from_numpy(synth.normal_bf16(SEED, 950 + j, M, K).view(np.int16)).cuda()
              .view(torch.bfloat16) for j, (_, _, K) in enumerate(MATS)]
        yv = [torch.empty((M, N), dtype=torch.float32, device="cuda") for _, N, _ in MATS]
        stages = [(fmt, N, K, W[l][j][0], W[l][j][1], xv[j], yv[j], 0)
                  for l in range(layers) for j, (name, N, K) in enumerate(MATS)]
        ch = lb.Chain(stages, x_dtype=lb.BF16, y_dtype=lb.F32, rows=M)
        vms = time_region(torch, stream, lambda: ch.run(stream), args.steps, args.warmup)
        ch.close()
        log(f"verify pass, {M} rows: {vms:.3f} ms, {step_bytes / vms / 1e6:.0f} GB/s, "
            f"{M * 1000 / vms:.1f} tokens checked/s")
        modes_out["verify_pass"] = {"rows": M, "ms_per_pass": round(vms, 4),
                                    "gb_s": round(step_bytes / vms / 1e6, 1),
                                    "tokens_per_s": round(M * 1000.0 / vms, 1)}
    del W
    torch.cuda.synchronize()
    return ms, gbs, step_bytes, roof, head, modes_out


def bench_gemm_pass(lb, synth, torch, np, fmt, M, shapes, seed, xkind, reps):
    """One pass = every GEMM of `shapes` at M rows (activation staging and,
    for int8, per-token quantization included).  Returns (ms, TFLOP/s)."""
    mats = build_mats(lb, synth, fmt, seed, 0, shapes)
    Xs = [torch.from_numpy(synth.normal_bf16(seed, 700 + j, M, K).view(np.int16)).cuda()
          .view(torch.bfloat16) for j, (_, _, K) in enumerate(shapes)]
    Ys = [torch.empty((M, N), dtype=torch.float32, device="cuda") for _, N, _ in shapes]
    Qs = [torch.empty((M, K), dtype=torch.int8, device="cuda") for _, _, K in shapes]
    Ss = [torch.empty(M, dtype=torch.float32, device="cuda") for _ in shapes]
    if xkind == "sign":
        Bs = [torch.from_numpy(synth.sign_bits(seed, 800 + j, M, K)).cuda()
              for j, (_, _, K) in enumerate(shapes)]
        alpha = torch.ones(M, dtype=torch.float32, device="cuda")

    def one():
        for j, (name, N, K) in enumerate(shapes):
            pc, ps = mats[j]
            if xkind == "i8":
                lb.quantize_act_i8(Xs[j], Q=Qs[j], s_x=Ss[j])
                lb.gemm(fmt, M, N, K, pc, ps, Qs[j], x_scales=Ss[j], Y=Ys[j])
            elif xkind == "sign":
                lb.gemm(fmt, M, N, K, pc, ps, Bs[j], x_scales=alpha, Y=Ys[j], x_dtype=lb.SIGN1)
            else:
                lb.gemm(fmt, M, N, K, pc, ps, Xs[j], Y=Ys[j])

    stream = torch.cuda.Stream()
    ms = time_region(torch, stream, one, reps, 2)
    flops = sum(2.0 * M * N * K for _, N, K in shapes)
    del mats, Xs, Ys, Qs, Ss
    torch.cuda.synchronize()
    return ms, flops / (ms * 1e-3) / 1e12


def bench_gemv_product(lb, synth, torch, np, fmt, N, K, copies, mode, reps):
    """One product per launch over `copies` distinct weight matrices (more
    packed bytes than the 256 MB last-level cache, so every launch streams
    from HBM), the launches replayed as one HIP graph.  mode "sign": batch-1
    binary weights x sign activations (XOR + popcount, lowbit_gemv SIGN1);
    "m<M>": M bf16 activation rows (M = 5: the small-M verification pass).
    Returns (us per product, GB/s of packed weight bytes)."""
    mats = build_mats(lb, synth, fmt, SEED + 10, 0, [("w", N, K)] * copies)
    if mode == "sign":
        xb = torch.from_numpy(synth.sign_bits(SEED + 10, 850, 1, K)).cuda()[0]
        y = torch.empty(N, dtype=torch.float32, device="cuda")

        def one():
            for pc, ps in mats:
                lb.gemv(1, N, K, pc, ps, xb, x_scale=1.0, y=y, x_dtype=lb.SIGN1)
    else:
        M = int(mode[1:])  # "m<rows>"
        X = torch.from_numpy(synth.normal_bf16(SEED + 10, 851, M, K).view(np.int16)).cuda() \
            .view(torch.bfloat16)
        Y = torch.empty((M, N), dtype=torch.float32, device="cuda")

        def one():
            for pc, ps in mats:
                if M == 1:
                    lb.gemv(fmt, N, K, pc, ps, X[0], y=Y[0])
                else:
                    lb.gemm(fmt, M, N, K, pc, ps, X, Y=Y)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        one()  # eager warm-up (allocates the workspace)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        one()
    torch.cuda.synchronize()
    ms = time_region(torch, stream, graph.replay, reps, 2)
    nbytes = packed_bytes(lb, fmt, [("w", N, K)]) * copies
    del graph, mats
    torch.cuda.synchronize()
    return ms * 1e3 / copies, nbytes / (ms * 1e-3) / 1e9


def bench_quantizer(lb, synth, torch, np, N, K, reps):
    """lowbit_quantize_weights with rotation on an N x K bf16 matrix; returns
    (ms, GB/s of bf16 read + codes and scales written)."""
    W = torch.randn(N, K, device="cuda").mul_(0.02).to(torch.bfloat16).view(torch.int16)
    d = torch.from_numpy(np.where(np.random.default_rng(5).random(K) < 0.5, -1, 1)
                         .astype(np.int8)).cuda()
    codes = torch.empty((N, K), dtype=torch.int8, device="cuda")
    scales = torch.empty((N, K // 128), dtype=torch.int16, device="cuda")
    stream = torch.cuda.Stream()

    def one():
        lb._check("lowbit_quantize_weights",
                  lb.lib().lowbit_quantize_weights(2, N, K, lb._ptr(W), lb._ptr(d), lb._ptr(codes),
                                                   lb._ptr(scales), lb._stream(stream)))

    ms = time_region(torch, stream, one, reps, 2)
    nbytes = N * K * 2 + N * K + N * (K // 128) * 2
    del W, codes, scales
    torch.cuda.synchronize()
    return ms, nbytes / (ms * 1e-3) / 1e9


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
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--fmt", type=int, default=2, choices=[1, 2])
    ap.add_argument("--layers", type=int, default=LAYERS)
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--gemm-reps", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--modes", default="chain,chain_dep,separate",
                    help="decode-step modes to time, headline first (chain, chain_dep, separate)")
    ap.add_argument("--no-gemm", action="store_true")
    ap.add_argument("--no-other-format", action="store_true",
                    help="skip the decode step in the other weight format")
    ap.add_argument("--verify-rows", type=int, default=5,
                    help="rows of the small-M verification pass through the whole step (0: skip)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures a single GPU; --gpus {args.gpus} is not supported (the "
              "kernels run on one device's share; multi-GPU sharding is not implemented)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from ultra_bit_dit_amd import lowbit as lb

    copy_calibration(torch)
    read_gbs = hbm_read_rate(lb, torch)
    log(f"streaming read of 4 GiB: {read_gbs:.0f} GB/s")
    ms, gbs, step_bytes, roof, head, modes_out = bench_decode(args, lb, synth, torch, np)
    roof["measured_read_gb_s"] = round(read_gbs, 1)
    roof["frac_of_measured_read"] = round(roof["achieved"] / read_gbs, 4)
    # the same step with the other weight format (the workload has binary and
    # ternary variants): streaming and sequential chains
    other = None
    if not args.no_other_format:
        a2 = argparse.Namespace(**vars(args))
        a2.fmt = 1 if args.fmt == 2 else 2
        a2.modes = "chain,chain_dep"
        a2.verify_rows = 0
        oms, ogbs, obytes, oroof, _, omodes = bench_decode(a2, lb, synth, torch, np)
        other = {"format": FMT_NAMES[a2.fmt], "mode": "chain", "ms_per_step": round(oms, 4),
                 "gb_s": round(ogbs, 1), "pct_hbm_peak": round(100 * ogbs / HBM_PEAK_GBS, 1),
                 "tok_s": round(1000.0 / oms, 2), "bytes_per_step": obytes,
                 "kernel": oroof["kernel"], "decode_modes": omodes}

    out = {
        "metric": "decode GEMV HBM GB/s (% peak) & tok/s; pp512 GEMM TFLOP/s (% MFMA peak)",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"27B-class decode step, {FMT_NAMES[args.fmt]}: {args.layers} layers x "
                               "(qkv 15360x5120, o 5120x5120, gate/up 34816x5120, down 5120x17408), "
                               "group-128 fp16 scales, bf16 activations, batch 1",
                   "tok_s": round(1000.0 / ms, 2),
                   "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1),
                   "bytes_per_step": step_bytes,
                   "mode": head,
                   "decode_modes": modes_out},
        "roofline": roof,
    }
    if other is not None:
        out["config"]["decode_" + other["format"].split("-")[0]] = other
    if not args.no_gemm:
        pp = {}
        for xk, peak in (("bf16", MFMA_PEAK_F16_TFLOPS), ("i8", MFMA_PEAK_I8_TOPS)):
            pms, tf = bench_gemm_pass(lb, synth, torch, np, 2, 512, MATS, PP_SEED, xk, args.gemm_reps)
            log(f"pp512 {xk}: {pms:.3f} ms per layer, {tf:.1f} TFLOP/s")
            pp[xk] = {"ms_per_layer": round(pms, 4), "tflops": round(tf, 1),
                      "pct_mfma_peak": round(100 * tf / peak, 1),
                      "tok_s_64_layers": round(512 / (pms * LAYERS * 1e-3), 1)}
        out["config"]["pp512_ternary"] = pp
        dit = {}
        for M in (4608, 18432):
            dms, tf = bench_gemm_pass(lb, synth, torch, np, 1, M, DIT, DIT_SEED, "bf16",
                                      max(2, args.gemm_reps // (M // 4608)))
            log(f"DiT block M={M}: {dms:.3f} ms, {tf:.1f} TFLOP/s")
            dit[str(M)] = {"ms_per_block": round(dms, 4), "tflops": round(tf, 1),
                           "pct_mfma_peak": round(100 * tf / MFMA_PEAK_F16_TFLOPS, 1)}
        out["config"]["dit_block_binary_bf16"] = dit
        # the same blocks with sign activations (binary x binary on the fp4 MFMA)
        sg = {}
        for M in (4608, 18432):
            dms, tf = bench_gemm_pass(lb, synth, torch, np, 1, M, DIT, DIT_SEED, "sign",
                                      max(2, args.gemm_reps // (M // 4608)))
            log(f"DiT block sign M={M}: {dms:.3f} ms, {tf:.1f} TOP/s")
            sg[str(M)] = {"ms_per_block": round(dms, 4), "tops": round(tf, 1),
                          "pct_mfma_peak_fp4": round(100 * tf / MFMA_PEAK_F4_TOPS, 1)}
        out["config"]["dit_block_binary_sign"] = sg
        # batch-1 XOR + popcount and the five-row verification pass, gate/up shape
        gv = {}
        us, gb = bench_gemv_product(lb, synth, torch, np, 1, 34816, 5120, 16, "sign", args.gemm_reps)
        log(f"XOR+popcount GEMV 34816x5120 binary: {us:.1f} us per product, {gb:.0f} GB/s")
        gv["xor_popcount_binary_34816x5120"] = {"us_per_product": round(us, 2), "gb_s": round(gb, 1),
                                                "pct_hbm_peak": round(100 * gb / HBM_PEAK_GBS, 1)}
        us, gb = bench_gemv_product(lb, synth, torch, np, 2, 34816, 5120, 8, "m5", args.gemm_reps)
        log(f"M=5 ternary 34816x5120: {us:.1f} us per product, {gb:.0f} GB/s")
        gv["m5_ternary_34816x5120"] = {"us_per_product": round(us, 2), "gb_s": round(gb, 1),
                                       "pct_hbm_peak": round(100 * gb / HBM_PEAK_GBS, 1)}
        out["config"]["gemv_products"] = gv
        # data-free quantizer front end on the gate/up matrix (rotated, ternary)
        qms, qgbs = bench_quantizer(lb, synth, torch, np, 34816, 5120, args.gemm_reps)
        log(f"quantizer 34816x5120: {qms:.3f} ms, {qgbs:.0f} GB/s")
        out["config"]["quantizer_gate_up"] = {"ms": round(qms, 4), "gb_s": round(qgbs, 1),
                                              "pct_hbm_peak": round(100 * qgbs / HBM_PEAK_GBS, 1),
                                              "bytes": "bf16 in + int8 codes + fp16 scales out"}
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(args.fmt, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
