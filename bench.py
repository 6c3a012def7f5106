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
C0_SEED, C1_SEED, PP_SEED, DIT_SEED = 1000, 1001, 1003, 1004
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


def time_region(torch, stream, fn, steps, warmup, per_step=None):
    """Warm-up, then `steps` calls bracketed by synchronisations; HIP events
    on `stream` (the stream every launch goes to).  Returns ms per call (the
    mean over the bracketed region).  With `per_step` (a list) an event is
    also recorded between consecutive calls and the per-call durations are
    appended to it."""
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True)
              for _ in range(steps + 1 if per_step is not None else 2)]
        ev[0].record(stream)
        for i in range(steps):
            fn()
            if per_step is not None:
                ev[i + 1].record(stream)
        ev[-1].record(stream)
        torch.cuda.synchronize()
    if per_step is not None:
        per_step.extend(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return ev[0].elapsed_time(ev[-1]) / steps


def median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def pmc_traffic(launch_bytes, kernel, fmt=2):
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
        if kv.get("format", FMT_NAMES[2]) != FMT_NAMES[fmt]:
            return None, f"counters taken for {kv.get('format')}, not {FMT_NAMES[fmt]}"
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


GEMM_LEGS = ("pp512_bf16", "pp512_i8", "dit_bf16", "dit_sign", "gemv_products", "quantizer")

MODE_WHAT = {
    "chain": "the step as specified (fixed x per shape, products independent): one persistent "
             "launch streams every product's weights; the streaming bound",
    "chain_dep": "sequential decode: every product waits for the previous one, gate/up's "
                 "SiLU-mul output feeds down (bf16 activations); one persistent launch",
    "separate": "one launch per product, the step captured as one HIP graph",
}


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
        per = []
        if mode in ("chain", "chain_dep"):
            ch = chain_for(lb, fmt, W, xs, ys, layers, 1 if mode == "chain_dep" else 0, torch)
            ms = time_region(torch, stream, lambda: ch.run(stream), args.steps, args.warmup, per)
            if ch.failed_waits():
                raise RuntimeError("chain wait gave up")
            ch.close()
            res[mode] = (ms, 1, median(per))
        elif mode == "separate":
            with torch.cuda.stream(stream):
                run_step(lb, fmt, W, xs, ys, layers)  # eager warm-up (allocates the workspace)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                run_step(lb, fmt, W, xs, ys, layers)
            torch.cuda.synchronize()
            ms = time_region(torch, stream, graph.replay, args.steps, args.warmup, per)
            del graph
            res[mode] = (ms, len(MATS) * layers, median(per))
        else:
            raise SystemExit(f"unknown mode {mode}")
        log(f"decode [{mode}] {ms:.3f} ms/step, {step_bytes / ms / 1e6:.0f} GB/s, "
            f"{1000 / ms:.1f} tok/s")
    head = modes[0]
    ms, launches, _ = res[head]
    gbs = step_bytes / (ms * 1e-3) / 1e9
    launch_bytes = step_bytes / launches
    launch_us = ms * 1e3 / launches
    kbase = {"chain": "gemv_stream", "chain_dep": "gemv_chain", "separate": "gemv_mfma"}[head]
    traffic, tnote = pmc_traffic(launch_bytes, kbase, fmt)
    kname = kbase + f" ({FMT_NAMES[fmt]}, bf16 x, fp32 y)"
    roof = {"bound": "hbm", "kernel": kname,
            "achieved": round(launch_bytes / (launch_us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(launch_bytes / (launch_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": None if traffic is None else round(traffic),
            "algorithmic_bytes_per_launch": round(launch_bytes),
            "avg_launch_us": round(launch_us, 3),
            "note": f"{launches} launch(es) per step, durations from HIP events over the timed "
                    f"region; traffic: {tnote}"}
    modes_out = {m: {"ms_per_step": round(v[0], 4), "median_ms_per_step": round(v[2], 4),
                     "gb_s": round(step_bytes / v[0] / 1e6, 1),
                     "tok_s": round(1000.0 / v[0], 2), "launches_per_step": v[1],
                     "what": MODE_WHAT[m]}
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


def bench_gemv_product(lb, synth, torch, np, fmt, N, K, copies, mode, reps, launches=None,
                       seed=SEED + 10):
    """One product per launch, the launches cycling over `copies` distinct
    weight matrices (more packed bytes than the 256 MB last-level cache: every
    launch streams from HBM; one copy: the weights stay cache-resident),
    `launches` of them (default one per copy) replayed as one HIP graph.
    mode "sign": batch-1 binary weights x sign activations (XOR + popcount,
    lowbit_gemv SIGN1); "m<M>": M bf16 activation rows (M = 1: lowbit_gemv,
    M = 5: the small-M verification pass).  Returns (us per product, GB/s of
    packed weight bytes)."""
    launches = launches or copies
    mats = build_mats(lb, synth, fmt, seed, 0, [("w", N, K)] * copies)
    order = [mats[i % copies] for i in range(launches)]
    if mode == "sign":
        xb = torch.from_numpy(synth.sign_bits(SEED + 10, 850, 1, K)).cuda()[0]
        y = torch.empty(N, dtype=torch.float32, device="cuda")

        def one():
            for pc, ps in order:
                lb.gemv(1, N, K, pc, ps, xb, x_scale=1.0, y=y, x_dtype=lb.SIGN1)
    else:
        M = int(mode[1:])  # "m<rows>"
        X = torch.from_numpy(synth.normal_bf16(SEED + 10, 851, M, K).view(np.int16)).cuda() \
            .view(torch.bfloat16)
        Y = torch.empty((M, N), dtype=torch.float32, device="cuda")

        def one():
            for pc, ps in order:
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
    nbytes = packed_bytes(lb, fmt, [("w", N, K)]) * launches
    del graph, mats, order
    torch.cuda.synchronize()
    return ms * 1e3 / launches, nbytes / (ms * 1e-3) / 1e9


def bench_c0_latency(lb, synth, torch, np, reps=200):
    """The binary GEMV correctness configuration (N = 256, K = 1024, fp32 x and
    y): 36,864 packed bytes, far below the cache, so the figure is latency.
    Reports the median of `reps` single calls, each bracketed by its own
    events on an idle stream, and the per-call time of 100 calls replayed as
    one HIP graph."""
    N, K = 256, 1024
    codes = synth.device_codes(False, C0_SEED, 0, N, K, "cuda")
    scales = synth.device_scales(C0_SEED, 1, N, K // 128, "cuda")
    pc, ps = lb.pack(1, codes, scales)
    x = torch.from_numpy(synth.normal_f32(C0_SEED, 2, 1, K)).cuda()[0]
    y = torch.empty(N, dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()
    one = lambda: lb.gemv(1, N, K, pc, ps, x, y=y)  # noqa: E731
    single = []
    with torch.cuda.stream(stream):
        for _ in range(10):
            one()
        torch.cuda.synchronize()
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            one()
            e1.record(stream)
            e1.synchronize()
            single.append(e0.elapsed_time(e1) * 1e3)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for _ in range(100):
            one()
    torch.cuda.synchronize()
    gms = time_region(torch, stream, graph.replay, 20, 2)
    del graph
    torch.cuda.synchronize()
    return {"us_single_call_median": round(median(single), 2),
            "us_single_call_min": round(min(single), 2),
            "us_per_call_in_graph": round(gms * 1e3 / 100, 3),
            "packed_bytes": packed_bytes(lb, 1, [("w", N, K)]),
            "what": "binary GEMV N=256 K=1024, fp32 x, fp32 y (C0); latency-bound"}


def bench_c1(lb, synth, torch, np, reps):
    """The ternary 5120 x 5120 GEMV (bf16 x, fp32 y) in both packings: cold,
    the launches rotating over enough distinct copies (>= 512 MB) that every
    launch streams from HBM, and hot, 100 launches on one cache-resident
    matrix.  Each labelled."""
    out = {}
    N = K = 5120
    for fmt in (2, 3):
        nb = packed_bytes(lb, fmt, [("w", N, K)])
        copies = max(80, -(-(512 << 20) // nb))
        us, gb = bench_gemv_product(lb, synth, torch, np, fmt, N, K, copies, "m1", reps,
                                    seed=C1_SEED)
        uh, gh = bench_gemv_product(lb, synth, torch, np, fmt, N, K, 1, "m1", reps, launches=100,
                                    seed=C1_SEED)
        name = FMT_NAMES[fmt]
        log(f"C1 {name}: cold {us:.2f} us ({gb:.0f} GB/s), hot {uh:.2f} us ({gh:.0f} GB/s)")
        out[name] = {
            "packed_bytes": nb,
            "cold": {"us_per_product": round(us, 3), "gb_s": round(gb, 1),
                     "pct_hbm_peak": round(100 * gb / HBM_PEAK_GBS, 1),
                     "what": f"rotated over {copies} copies ({copies * nb / 1e6:.0f} MB), "
                             "each launch streams from HBM"},
            "hot": {"us_per_product": round(uh, 3), "gb_s": round(gh, 1),
                    "what": "one matrix, 100 launches: cache-resident (not an HBM figure)"}}
    return out


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


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_threads():
    """Threads for the multi-threaded oracle runs: the CPUs this process may
    run on, at most 16 (one GPU's share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def oracle_time(O, calls, threads):
    """Wall seconds for the oracle products `calls` (tuples codes, scales,
    xkind, X), each split by weight rows over `threads` threads (the
    oracle's C library runs without the interpreter lock)."""
    from concurrent.futures import ThreadPoolExecutor
    jobs = []
    for codes, scales, xk, X in calls:
        N = codes.shape[0]
        step = -(-N // threads)
        for r in range(0, N, step):
            jobs.append((codes[r:r + step], scales[r:r + step], xk, X))
    t0 = time.perf_counter()
    if threads == 1:
        for c, sc, xk, X in jobs:
            O.matmul(c, sc, xk, X, with_abs=False)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(lambda a: O.matmul(a[0], a[1], a[2], a[3], with_abs=False), jobs))
    return time.perf_counter() - t0


def cpu_baseline(fmt, step_bytes, budget_s, device_gen=None):
    """The oracle, as it stands, timed on the host: fp64 dequantize-then-
    multiply (plain C, -O2), once on 1 thread and once on T threads.  Inputs
    are the same seeded synthetic tensors, regenerated bit-exactly on the host.
      C0   binary GEMV N=256 K=1024 (fp32 x), timed in full;
      C1   ternary GEMV 5120 x 5120 (bf16 x), timed in full (dequantize-
           multiply only; the oracle's unpacker is timed on its own);
      C2   decode step: a row sample of the four layer matrices (64 rows on
           1 thread; the full layer on T threads when it fits the budget),
           extrapolated per weight to 64 layers;
      C3   pp512: 512 rows x 8 weight rows of each layer matrix, extrapolated
           to one layer and to 64 layers;
      C4   DiT block M=4608: 256 activation rows x 4 weight rows of each block
           matrix, extrapolated to the block.
    `value` is the T-thread decode rate in the headline's unit (packed-weight
    bytes of one step / seconds per step); tok/s beside it.  device_gen (not
    None: a GPU is present) lets whole inputs be generated on the device."""
    import numpy as np
    import synth
    from oracle import oracle as O
    T = cpu_threads()
    gen = synth.ternary_codes if fmt != 1 else synth.binary_codes
    out = {"kind": "oracle", "cores": T, "cpu_model": cpu_model(), "threads_available": T}
    layer_macs = sum(N * K for _, N, K in MATS)

    # C0 and C1 in full
    c0 = (synth.binary_codes(C0_SEED, 0, 256, 1024), synth.group_scales(C0_SEED, 1, 256, 8),
          O.X_F32, synth.normal_f32(C0_SEED, 2, 1, 1024))
    t_c0 = min(oracle_time(O, [c0], 1) for _ in range(5))
    c1 = (synth.ternary_codes(C1_SEED, 0, 5120, 5120), synth.group_scales(C1_SEED, 1, 5120, 40),
          O.X_BF16, synth.normal_bf16(C1_SEED, 2, 1, 5120))
    t_c1_1 = oracle_time(O, [c1], 1)
    t_c1_T = oracle_time(O, [c1], T)
    pc, ps, _ = O.pack(2, c1[0], c1[1])
    t0 = time.perf_counter()
    O.unpack(2, 5120, 5120, pc, ps)
    t_unpack = time.perf_counter() - t0
    out["c0_binary_gemv"] = {"us_1_thread": round(t_c0 * 1e6, 1), "measured": "in full"}
    out["c1_ternary_gemv"] = {"ms_1_thread": round(t_c1_1 * 1e3, 2), f"ms_{T}_threads":
                              round(t_c1_T * 1e3, 2), "unpack_2bit_ms_1_thread":
                              round(t_unpack * 1e3, 2), "measured": "in full"}

    # C2: 1-thread row sample, T-thread full layer (or the largest sample that fits)
    full_layer = None
    if device_gen is not None:
        # whole matrices generated on the device (the same values as the host
        # generators, much faster) and copied to the host once
        full_layer = []
        for j, (name, N, K) in enumerate(MATS):
            full_layer.append(
                (synth.device_codes(fmt != 1, SEED, 2 * j, N, K, "cuda").cpu().numpy(),
                 synth.device_scales(SEED, 2 * j + 1, N, K // 128, "cuda").cpu().numpy()
                 .view(np.uint16)))

    def layer_calls(rows):
        calls = []
        for j, (name, N, K) in enumerate(MATS):
            if full_layer is not None:
                codes, scales = full_layer[j][0][:rows], full_layer[j][1][:rows]
            else:
                r = np.arange(min(rows, N))
                codes = gen(SEED, 2 * j, N, K, rows=r)
                scales = synth.group_scales(SEED, 2 * j + 1, N, K // 128, rows=r)
            calls.append((codes, scales, O.X_BF16, synth.normal_bf16(SEED, 900 + j, 1, K)))
        return calls

    # rows of each matrix: 64 to probe the rate, then as many as a quarter of
    # the budget allows on 1 thread and half of it on T threads (up to the
    # whole layer); host-generated inputs stay small
    probe = layer_calls(64)
    rate_1 = sum(c[0].size for c in probe) / oracle_time(O, probe, 1)
    cap = max(N for _, N, _ in MATS) if full_layer is not None else 256
    rows_1 = int(min(cap, max(64, budget_s * 0.25 * rate_1 / 32768)))
    s1 = layer_calls(rows_1)
    t1 = oracle_time(O, s1, 1)
    macs1 = sum(c[0].size for c in s1)
    sec_tok_1 = t1 / macs1 * layer_macs * LAYERS
    rows_T = int(min(cap, max(64, budget_s * 0.5 * rate_1 * T / 32768)))
    sT = layer_calls(rows_T)
    tT = oracle_time(O, sT, T)
    macsT = sum(c[0].size for c in sT)
    full = macsT == layer_macs
    sec_tok_T = tT / macsT * layer_macs * LAYERS
    del sT, s1, full_layer
    out["value"] = round(step_bytes / sec_tok_T / 1e9, 4)
    out["unit"] = "GB/s"
    out["tok_s"] = round(1.0 / sec_tok_T, 6)
    out["sample"] = (f"decode step ({FMT_NAMES[fmt]}): {'one full layer' if full else f'{rows_T} rows of each layer matrix'} "
                     f"({macsT / 1e6:.0f}M weight MACs) in {tT:.2f}s on {T} threads, "
                     f"extrapolated per weight to {LAYERS} layers ({layer_macs * LAYERS / 1e9:.2f}G MACs); "
                     f"value = packed bytes of one step / seconds per step")
    out["single_thread"] = {"tok_s": round(1.0 / sec_tok_1, 6),
                            "gb_s": round(step_bytes / sec_tok_1 / 1e9, 4),
                            "sample": f"{rows_1} rows of each layer matrix ({macs1 / 1e6:.0f}M MACs) "
                                      f"in {t1:.2f}s, extrapolated to {LAYERS} layers"}

    # C3: pp512 layer sample (T threads)
    c3 = []
    for j, (name, N, K) in enumerate(MATS):
        r = np.arange(8)
        c3.append((synth.ternary_codes(PP_SEED, 2 * j, N, K, rows=r),
                   synth.group_scales(PP_SEED, 2 * j + 1, N, K // 128, rows=r),
                   O.X_BF16, synth.normal_bf16(PP_SEED, 700 + j, 512, K)))
    t3 = oracle_time(O, c3, min(T, 8))
    m3 = sum(512 * c[0].size for c in c3)
    s_layer = t3 / m3 * 512 * layer_macs
    out["c3_pp512"] = {"s_per_layer": round(s_layer, 2), "s_per_pass_64_layers": round(s_layer * LAYERS, 1),
                       "gflop_s": round(2 * m3 / t3 / 1e9, 3), "threads": min(T, 8),
                       "measured": f"512 rows x 8 weight rows of each layer matrix ({m3 / 1e6:.0f}M MACs, "
                                   f"{t3:.2f}s); extrapolated"}
    # C4: DiT block sample (T threads)
    c4 = []
    for j, (name, N, K) in enumerate(DIT):
        r = np.arange(4)
        c4.append((synth.binary_codes(DIT_SEED, 2 * j, N, K, rows=r),
                   synth.group_scales(DIT_SEED, 2 * j + 1, N, K // 128, rows=r),
                   O.X_BF16, synth.normal_bf16(DIT_SEED, 700 + j, 256, K)))
    t4 = oracle_time(O, c4, min(T, 4))
    m4 = sum(256 * c[0].size for c in c4)
    block_macs = 4608 * sum(N * K for _, N, K in DIT)
    out["c4_dit_block_4608"] = {"s_per_block": round(t4 / m4 * block_macs, 1),
                                "gflop_s": round(2 * m4 / t4 / 1e9, 3), "threads": min(T, 4),
                                "measured": f"256 activation rows x 4 weight rows of each block "
                                            f"matrix ({m4 / 1e6:.0f}M MACs, {t4:.2f}s); extrapolated"}
    return out


# ------------------------------------------------------------------ profiles
# Summaries of rocprofv3 output for profiles/: `python bench.py --summarize
# KIND --prof-dir DIR [--prof-dir2 DIR2] --out FILE --cmd "..."`.

def _csv_rows(d, suffix):
    """Rows of every `*<suffix>` CSV rocprofv3 wrote under directory d."""
    import csv
    import glob
    rows = []
    for path in sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def _col(row, *names):
    for n in names:
        if n in row:
            return row[n]
    raise KeyError(f"none of {names} in {sorted(row)}")


def _demangle(names):
    import subprocess
    try:
        out = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True,
                             timeout=60).stdout.split("\n")
    except (OSError, subprocess.SubprocessError):
        out = list(names)
    out = [o.replace("lowbit::(anonymous namespace)::", "") for o in out[:len(names)]]
    return [o[5:] if o.startswith("void ") else o for o in out]


def _dispatches(d):
    """Per dispatch of a --pmc run: {"id", "kernel", "grid", "counters": {...}} in
    dispatch order (counter values of one dispatch summed over their rows)."""
    acc = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        did = int(_col(r, "Dispatch_Id", "Dispatch_ID"))
        e = acc.setdefault(did, {"id": did, "kernel": _col(r, "Kernel_Name"),
                                 "grid": _col(r, "Grid_Size", "Grid_Size_X"), "counters": {},
                                 "ns": int(_col(r, "End_Timestamp")) - int(_col(r, "Start_Timestamp"))})
        c = _col(r, "Counter_Name")
        e["counters"][c] = e["counters"].get(c, 0.0) + float(_col(r, "Counter_Value"))
    out = [acc[k] for k in sorted(acc)]
    dm = _demangle([e["kernel"] for e in out])
    for e, n in zip(out, dm):
        e["kernel"] = n
    return out


def _trace(d):
    """Per dispatch of a --kernel-trace run: (kernel, duration ns) in order."""
    rows = _csv_rows(d, "kernel_trace.csv")
    rows.sort(key=lambda r: int(_col(r, "Dispatch_Id", "Dispatch_ID")))
    names = _demangle([_col(r, "Kernel_Name") for r in rows])
    return [(n, int(_col(r, "End_Timestamp")) - int(_col(r, "Start_Timestamp")))
            for n, r in zip(names, rows)]


def _kbase(name):
    return name.split("<", 1)[0].split("(", 1)[0].strip()


def summarize_stats(d, out, cmd):
    """Kernel-trace statistics (rocprofv3 --stats): every kernel's calls and
    average / min / max duration."""
    rows = _csv_rows(d, "kernel_stats.csv")
    names = _demangle([_col(r, "Name", "Kernel_Name") for r in rows])
    lines = ["# rocprofv3 kernel statistics (--kernel-trace --stats) of the library's kernels "
             "(torch's input-generation kernels omitted)", f"# command: {cmd}",
             "# kernel | calls | total ms | average us | min us | max us"]
    for n, r in sorted(zip(names, rows), key=lambda t: -float(_col(t[1], "TotalDurationNs"))):
        if n.startswith(("at::", "(anonymous namespace)::", "__amd_rocclr")):
            continue
        lines.append(f"{n[:150]} | {_col(r, 'Calls')} | {float(_col(r, 'TotalDurationNs')) / 1e6:.3f} | "
                     f"{float(_col(r, 'AverageNs')) / 1e3:.3f} | {float(_col(r, 'MinNs')) / 1e3:.3f} | "
                     f"{float(_col(r, 'MaxNs')) / 1e3:.3f}")
    _write(out, lines)


def summarize_hbm(dfetch, dwrite, out, cmds, fmt, layers):
    """FETCH_SIZE / WRITE_SIZE per dispatch of the streaming decode kernel and
    of the copy it is scaled by, in the key = value form pmc_traffic reads.
    cmds: the two rocprofv3 commands, or one with @PMC@ for the counter."""
    fcmd = cmds[0].replace("@PMC@", "FETCH_SIZE")
    wcmd = cmds[1] if len(cmds) > 1 else cmds[0].replace("@PMC@", "WRITE_SIZE")
    from ultra_bit_dit_amd import lowbit as lb
    name = f"gemv_stream<{fmt},"

    def pick(d, counter):
        ds = _dispatches(d)
        g = [e["counters"][counter] for e in ds if e["kernel"].startswith(name)]
        c = [e["counters"][counter] for e in ds if "neg" in e["kernel"]]
        if not g or not c:
            raise SystemExit(f"no {name} or copy dispatch with {counter} under {d}")
        return sum(g) / len(g), max(c), len(g)

    gf, cf, nf = pick(dfetch, "FETCH_SIZE")
    gw, cw, nw = pick(dwrite, "WRITE_SIZE")
    lines = [
        "# rocprofv3 HBM byte counters of the decode GEMV kernel (gemv_stream)",
        f"# FETCH_SIZE command: {fcmd}",
        f"# WRITE_SIZE command: {wcmd}",
        "# copy reference: torch.neg over 64 Mi fp32 (256 MiB read, 256 MiB written)",
        f"# gemv dispatches counted: {nf} (FETCH), {nw} (WRITE); per-dispatch KiB averaged",
        "kernel = gemv_stream",
        f"format = {FMT_NAMES[fmt]}",
        "# hash of the code of gemv.hip + fp4.hpp + common.hpp (the sources the kernel is built "
        "from; comments and blank space removed)",
        f"gemv_source_sha256_16 = {gemv_source_hash()}",
        f"profiled_algorithmic_bytes_per_dispatch = {packed_bytes(lb, fmt, MATS) * layers}",
        f"gemv_FETCH_SIZE_KiB_per_dispatch = {gf:.1f}",
        f"gemv_WRITE_SIZE_KiB_per_dispatch = {gw:.1f}",
        f"copy_bytes_each_way = {256 << 20}",
        f"copy_FETCH_SIZE_KiB = {cf:.1f}",
        f"copy_WRITE_SIZE_KiB = {cw:.1f}",
    ]
    _write(out, lines)


def gemm_dispatch_labels(legs, reps):
    """The (leg, M, product, timed) label of every gemm_f8 dispatch of a bench
    run over `legs` with --gemm-reps `reps`, in launch order (two warm-up
    passes, then the timed ones, per bench_gemm_pass call)."""
    out = []
    for leg in [l for l in GEMM_LEGS if l in legs]:
        if leg.startswith("pp512"):
            runs = [(512, MATS, reps)]
        elif leg.startswith("dit"):
            runs = [(M, DIT, max(2, reps // (M // 4608))) for M in (4608, 18432)]
        else:
            continue
        for M, shapes, r in runs:
            for p in range(2 + r):
                for name, N, K in shapes:
                    out.append((leg, M, name, N, K, p >= 2))
    return out


def summarize_mfma(dpmc, dtrace, out, cmd_pmc, cmd_trace, legs, reps):
    """MFMA counters and durations per GEMM product (pp512 and DiT legs).
    Dispatches are matched to products by launch order."""
    labels = gemm_dispatch_labels(legs, reps)
    pm = [e for e in _dispatches(dpmc) if _kbase(e["kernel"]) == "gemm_f8"]
    tr = [t for t in _trace(dtrace) if _kbase(t[0]) == "gemm_f8"]
    if len(pm) != len(labels) or len(tr) != len(labels):
        raise SystemExit(f"{len(pm)} counted / {len(tr)} traced gemm_f8 dispatches, "
                         f"{len(labels)} expected")
    groups = {}
    for lab, e, t in zip(labels, pm, tr):
        g = groups.setdefault(lab[:5], {"n": 0, "c": {}, "dur": [], "kernel": e["kernel"], "pns": 0})
        g["n"] += 1
        g["pns"] += e["ns"]
        for k, v in e["counters"].items():
            g["c"][k] = g["c"].get(k, 0.0) + v
        if lab[5]:
            g["dur"].append(t[1])
    lines = ["# rocprofv3 MFMA counters of the GEMM kernel (gemm_f8), per product",
             f"# counters: {cmd_pmc}", f"# durations: {cmd_trace}",
             "# dispatches matched to products by launch order; durations: median over the "
             "timed passes of the trace run; counters: mean per dispatch",
             "# flop = 2 M N K; mfma_ops = SQ_INSTS_VALU_MFMA_MOPS_* x 512 (operations the "
             "MFMA pipe executed, split terms and padding included)",
             "# mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8 XCDs): "
             "the fraction of SIMD cycles the MFMA pipe was busy while the kernel ran; "
             "clock = GRBM_GUI_ACTIVE / 8 / dispatch time of the counter run; "
             "cycles_per_mfma = SQ_VALU_MFMA_BUSY_CYCLES / SQ_INSTS_MFMA (32: the 16x16x128 "
             "fp8 x fp4 MFMA at the fp8 rate; 16: fp4 x fp4)",
             "# product: time | TFLOP/s (2MNK) | % of the dtype's dense peak | MFMA ops executed / "
             "2MNK | mfma_busy | clock GHz | cycles_per_mfma | VALU instructions per MFMA"]
    for (leg, M, name, N, K), g in groups.items():
        c = {k: v / g["n"] for k, v in g["c"].items()}
        pns = g["pns"] / g["n"]
        dur = median(g["dur"]) if g["dur"] else float("nan")
        flop = 2.0 * M * N * K
        mops = sum(v for k, v in c.items() if k.startswith("SQ_INSTS_VALU_MFMA_MOPS")) * 512
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan"))
        gui = c.get("GRBM_GUI_ACTIVE", float("nan")) / 8
        nm = c.get("SQ_INSTS_MFMA", float("nan"))
        peak = (MFMA_PEAK_F16_TFLOPS if leg.endswith("bf16") else MFMA_PEAK_I8_TOPS
                if leg.endswith("i8") else MFMA_PEAK_F4_TOPS)
        pname = "bf16" if leg.endswith("bf16") else "int8" if leg.endswith("i8") else "fp4"
        lines.append(
            f"{leg} M={M} {name} {N}x{K}: {dur / 1e3:.2f} us | {flop / dur / 1e3:.1f} | "
            f"{100 * flop / dur / 1e3 / peak:.1f}% {pname} | {mops / flop:.2f} | "
            f"{busy / (1024 * gui):.3f} | {gui / pns:.2f} | {busy / nm:.1f} | "
            f"{c.get('SQ_INSTS_VALU', float('nan')) / nm:.1f}")
        lines.append("    raw: " + "; ".join(f"{k} {v:.6g}" for k, v in sorted(c.items())))
    lines.append(f"# kernel instances: {sorted(set(g['kernel'][:120] for g in groups.values()))}")
    _write(out, lines)


def summarize_valu(d, out, cmd, fmt, layers):
    """Instruction counters of the streaming decode kernel per weight."""
    ds = [e for e in _dispatches(d) if e["kernel"].startswith(f"gemv_stream<{fmt},")]
    if not ds:
        raise SystemExit(f"no gemv_stream<{fmt}, dispatch under {d}")
    c = {}
    for e in ds:
        for k, v in e["counters"].items():
            c[k] = c.get(k, 0.0) + v / len(ds)
    weights = sum(N * K for _, N, K in MATS) * layers
    lines = [f"# rocprofv3 instruction counters of the decode GEMV kernel (gemv_stream, "
             f"{FMT_NAMES[fmt]}), mean per dispatch", f"# command: {cmd}",
             f"# one dispatch = {layers} layers = {weights} weights; SQ_INSTS_* count wave "
             "instructions (64 lanes each)"]
    for k, v in sorted(c.items()):
        lines.append(f"{k} = {v:.6g}")
    for k in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD", "SQ_INSTS_LDS"):
        if k in c:
            lines.append(f"{k}_per_1k_weights = {1000 * c[k] / weights:.4f}")
    if "SQ_WAIT_INST_ANY" in c and "SQ_WAVE_CYCLES" in c:
        lines.append(f"wait_inst_any_frac_of_wave_cycles = {c['SQ_WAIT_INST_ANY'] / c['SQ_WAVE_CYCLES']:.4f}")
    if "GRBM_GUI_ACTIVE" in c:
        ns = sum(e["ns"] for e in ds) / len(ds)
        lines.append(f"dispatch_us = {ns / 1e3:.1f}")
        # GRBM_GUI_ACTIVE sums the 8 XCDs' busy cycles
        lines.append(f"sustained_clock_ghz = {c['GRBM_GUI_ACTIVE'] / 8 / ns:.3f}")
    _write(out, lines)


def _write(path, lines):
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--fmt", type=int, default=2, choices=[1, 2, 3],
                    help="headline weight format: 1 binary, 2 ternary 2-bit, 3 ternary base-3")
    ap.add_argument("--layers", type=int, default=LAYERS)
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--gemm-reps", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--modes", default="chain,chain_dep,separate",
                    help="decode-step modes to time, headline first (chain, chain_dep, separate)")
    ap.add_argument("--no-gemm", action="store_true")
    ap.add_argument("--gemm-legs", default=",".join(GEMM_LEGS),
                    help="legs after the decode step (comma list of " + ", ".join(GEMM_LEGS) + ")")
    ap.add_argument("--no-other-format", action="store_true",
                    help="skip the decode step in the other weight formats")
    ap.add_argument("--no-c01", action="store_true",
                    help="skip the C0 latency and C1 single-product legs")
    ap.add_argument("--verify-rows", type=int, default=5,
                    help="rows of the small-M verification pass through the whole step (0: skip)")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode step (and the streaming-read probe)")
    ap.add_argument("--summarize", choices=["stats", "hbm", "mfma", "valu"],
                    help="write a profiles/ summary of rocprofv3 output instead of benchmarking")
    ap.add_argument("--prof-dir", action="append", default=[])
    ap.add_argument("--out")
    ap.add_argument("--cmd", action="append", default=[],
                    help="the rocprofv3 command(s) the summary states")
    args = ap.parse_args()
    if args.summarize:
        legs = [l for l in args.gemm_legs.split(",") if l]
        if args.summarize == "stats":
            summarize_stats(args.prof_dir[0], args.out, args.cmd[0])
        elif args.summarize == "hbm":
            summarize_hbm(args.prof_dir[0], args.prof_dir[1], args.out, args.cmd, args.fmt,
                          args.layers)
        elif args.summarize == "mfma":
            summarize_mfma(args.prof_dir[0], args.prof_dir[1], args.out, args.cmd[0], args.cmd[1],
                           legs, args.gemm_reps)
        else:
            summarize_valu(args.prof_dir[0], args.out, args.cmd[0], args.fmt, args.layers)
        return
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
    out = {
        "metric": "decode GEMV HBM GB/s (% peak) & tok/s; pp512 GEMM TFLOP/s (% MFMA peak)",
        "value": None,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"27B-class decode step, {FMT_NAMES[args.fmt]}: {args.layers} layers x "
                               "(qkv 15360x5120, o 5120x5120, gate/up 34816x5120, down 5120x17408), "
                               "group-128 fp16 scales, bf16 activations, batch 1"},
    }
    others = []
    step_bytes = packed_bytes(lb, args.fmt, MATS) * args.layers
    if not args.no_decode:
        read_gbs = hbm_read_rate(lb, torch)
        log(f"streaming read of 4 GiB: {read_gbs:.0f} GB/s")
        ms, gbs, step_bytes, roof, head, modes_out = bench_decode(args, lb, synth, torch, np)
        roof["measured_read_gb_s"] = round(read_gbs, 1)
        roof["frac_of_measured_read"] = round(roof["achieved"] / read_gbs, 4)
        out["value"] = round(gbs, 1)
        out["ms_per_step"] = round(ms, 4)
        out["config"].update({"tok_s": round(1000.0 / ms, 2),
                              "tok_s_sequential": modes_out.get("chain_dep", {}).get("tok_s"),
                              "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1),
                              "bytes_per_step": step_bytes,
                              "mode": head,
                              "decode_modes": modes_out})
        out["roofline"] = roof
        # the same step in the other weight formats (binary, and both ternary
        # packings): streaming and sequential chains
        if not args.no_other_format:
            for ofmt in (1, 2, 3):
                if ofmt == args.fmt:
                    continue
                a2 = argparse.Namespace(**vars(args))
                a2.fmt = ofmt
                a2.modes = "chain,chain_dep"
                a2.verify_rows = 0
                oms, ogbs, obytes, oroof, _, omodes = bench_decode(a2, lb, synth, torch, np)
                others.append({"format": FMT_NAMES[ofmt], "mode": "chain",
                               "ms_per_step": round(oms, 4), "gb_s": round(ogbs, 1),
                               "pct_hbm_peak": round(100 * ogbs / HBM_PEAK_GBS, 1),
                               "tok_s": round(1000.0 / oms, 2), "bytes_per_step": obytes,
                               "kernel": oroof["kernel"], "decode_modes": omodes})
    for o in others:
        out["config"]["decode_" + o["format"].replace("-", "_")] = o
    if not args.no_c01:
        out["config"]["c0_binary_gemv_latency"] = bench_c0_latency(lb, synth, torch, np)
        log(f"C0: {out['config']['c0_binary_gemv_latency']}")
        out["config"]["c1_ternary_gemv_5120"] = bench_c1(lb, synth, torch, np, args.gemm_reps)
    legs = set() if args.no_gemm else set(l for l in args.gemm_legs.split(",") if l)
    if legs - set(GEMM_LEGS):
        raise SystemExit(f"unknown legs {sorted(legs - set(GEMM_LEGS))}")
    pp = {}
    for xk, peak in (("bf16", MFMA_PEAK_F16_TFLOPS), ("i8", MFMA_PEAK_I8_TOPS)):
        if "pp512_" + xk not in legs:
            continue
        pms, tf = bench_gemm_pass(lb, synth, torch, np, 2, 512, MATS, PP_SEED, xk, args.gemm_reps)
        log(f"pp512 {xk}: {pms:.3f} ms per layer, {tf:.1f} TFLOP/s")
        pp[xk] = {"ms_per_layer": round(pms, 4), "tflops": round(tf, 1),
                  "pct_mfma_peak": round(100 * tf / peak, 1),
                  "tok_s_64_layers": round(512 / (pms * LAYERS * 1e-3), 1)}
    if pp:
        out["config"]["pp512_ternary"] = pp
    if "dit_bf16" in legs:
        dit = {}
        for M in (4608, 18432):
            dms, tf = bench_gemm_pass(lb, synth, torch, np, 1, M, DIT, DIT_SEED, "bf16",
                                      max(2, args.gemm_reps // (M // 4608)))
            log(f"DiT block M={M}: {dms:.3f} ms, {tf:.1f} TFLOP/s")
            dit[str(M)] = {"ms_per_block": round(dms, 4), "tflops": round(tf, 1),
                           "pct_mfma_peak": round(100 * tf / MFMA_PEAK_F16_TFLOPS, 1)}
        out["config"]["dit_block_binary_bf16"] = dit
    if "dit_sign" in legs:
        # the same blocks with sign activations (binary x binary on the fp4 MFMA)
        sg = {}
        for M in (4608, 18432):
            dms, tf = bench_gemm_pass(lb, synth, torch, np, 1, M, DIT, DIT_SEED, "sign",
                                      max(2, args.gemm_reps // (M // 4608)))
            log(f"DiT block sign M={M}: {dms:.3f} ms, {tf:.1f} TOP/s")
            sg[str(M)] = {"ms_per_block": round(dms, 4), "tops": round(tf, 1),
                          "pct_mfma_peak_fp4": round(100 * tf / MFMA_PEAK_F4_TOPS, 1)}
        out["config"]["dit_block_binary_sign"] = sg
    if "gemv_products" in legs:
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
    if "quantizer" in legs:
        # data-free quantizer front end on the gate/up matrix (rotated, ternary)
        qms, qgbs = bench_quantizer(lb, synth, torch, np, 34816, 5120, args.gemm_reps)
        log(f"quantizer 34816x5120: {qms:.3f} ms, {qgbs:.0f} GB/s")
        out["config"]["quantizer_gate_up"] = {"ms": round(qms, 4), "gb_s": round(qgbs, 1),
                                              "pct_hbm_peak": round(100 * qgbs / HBM_PEAK_GBS, 1),
                                              "bytes": "bf16 in + int8 codes + fp16 scales out"}
    # nothing of the library's may outlive the process's GPU work: every
    # chain and graph is closed above; free the per-stream workspaces
    torch.cuda.synchronize()
    lb.release_workspaces()
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(args.fmt, step_bytes, args.cpu_budget, device_gen=True)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
