"""The 27B-class decode step at full size, in the launch configuration that
bench.py times: the same 64-layer weight set (bench.build_model), the same
activations and one chain of all 256 products.

Independent products (the headline streaming launch): every stage gets an
output of its own so that each can be checked; sampled rows of several
layers are regenerated on the host from their tensor ids and must meet the
oracle tolerance.  Sequential decode (waits, gate/up with the SiLU-mul
epilogue feeding the down projection, bf16 outputs; bench.chain_for): the
last layer's outputs are final and are checked, down against the oracle
applied to the GPU's own z.  Also the five-row verification pass and the
256 one-product launches replayed as a HIP graph."""
import numpy as np
import pytest
import torch

import bench
import synth
from oracle import oracle as O
from ultra_bit_dit_amd import lowbit as lb

from helpers import assert_within, codes_for, silu_mul_tolerance, to_np

pytestmark = pytest.mark.gpu

NAMES = [m[0] for m in bench.MATS]
GU, DN = NAMES.index("gateup"), NAMES.index("down")


def step_inputs():
    """bench.py's activations: one bf16 vector per product shape."""
    xh = [synth.normal_bf16(bench.SEED, 900 + j, 1, K) for j, (_, _, K) in enumerate(bench.MATS)]
    xs = [torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)[0] for x in xh]
    return xh, xs


def weights_rows(fmt, layer, j, rows):
    """Codes and scales of rows `rows` of product j of `layer`, regenerated
    from the tensor ids bench.build_model uses."""
    _, N, K = bench.MATS[j]
    tid = 16 * layer + 2 * j
    codes = codes_for(fmt, bench.SEED, tid, N, K, rows=rows)
    scales = synth.group_scales(bench.SEED, tid + 1, N, K // 128, rows=rows)
    return codes, scales


def sample_rows(N, seed, n=6):
    r = np.random.RandomState(seed).choice(np.arange(1, N - 1), size=n, replace=False)
    return np.sort(np.concatenate([[0, N - 1], r]))


@pytest.mark.parametrize("fmt", [1, 2])
def test_decode_step_stream_sampled(fmt):
    print(f"decode step fmt={fmt}: independent products", flush=True)
    W = bench.build_model(lb, synth, torch, fmt, bench.LAYERS)
    xh, xs = step_inputs()
    ys = [[torch.full((N,), float("nan"), device="cuda") for _, N, _ in bench.MATS]
          for _ in range(bench.LAYERS)]
    stages = [(fmt, N, K, W[l][j][0], W[l][j][1], xs[j], ys[l][j], 0)
              for l in range(bench.LAYERS) for j, (_, N, K) in enumerate(bench.MATS)]
    chain = lb.Chain(stages, x_dtype=lb.BF16, y_dtype=lb.F32)
    chain.run()
    torch.cuda.synchronize()
    assert chain.failed_waits() == 0
    chain.close()
    for l in range(bench.LAYERS):
        for j in range(len(bench.MATS)):
            assert not torch.isnan(ys[l][j]).any(), f"layer {l} product {j}: outputs not written"
    for l in (0, 1, 31, bench.LAYERS - 1):
        for j, (name, N, K) in enumerate(bench.MATS):
            rows = sample_rows(N, 97 * l + j)
            codes, scales = weights_rows(fmt, l, j, rows)
            yref, absY = O.matmul(codes, scales, O.X_BF16, xh[j])
            y = ys[l][j].cpu().numpy()[rows]
            assert_within(y[None], yref, absY, what=f"layer {l} {name}")


@pytest.mark.parametrize("fmt", [1, 2])
def test_decode_step_dependent_sampled(fmt):
    print(f"decode step fmt={fmt}: sequential decode with the SiLU-mul epilogue", flush=True)
    W = bench.build_model(lb, synth, torch, fmt, bench.LAYERS)
    xh, xs = step_inputs()
    chain = bench.chain_for(lb, fmt, W, xs, None, bench.LAYERS, 1, torch)
    chain.run()
    torch.cuda.synchronize()
    assert chain.failed_waits() == 0
    outs = chain._outs  # shared by the layers: the last layer's values remain
    chain.close()
    last = bench.LAYERS - 1
    # q/k/v and o read the fixed activations
    for j in (NAMES.index("qkv"), NAMES.index("o")):
        name, N, K = bench.MATS[j]
        rows = sample_rows(N, 31 + j)
        codes, scales = weights_rows(fmt, last, j, rows)
        yref, absY = O.matmul(codes, scales, O.X_BF16, xh[j])
        assert_within(to_np(outs[j])[rows][None], yref, absY, bf16_out=True, what=name)
    # z = silu(g) u: output i pairs fused rows 16 (i // 8) + i % 8 (gate) and + 8 (up)
    F = bench.MATS[GU][1] // 2
    zi = sample_rows(F, 53, n=10)
    grow = 16 * (zi // 8) + zi % 8
    codes, scales = weights_rows(fmt, last, GU, np.concatenate([grow, grow + 8]))
    gu, absGU = O.matmul(codes, scales, O.X_BF16, xh[GU])
    n = len(zi)
    gref, uref, absG, absU = gu[0, :n], gu[0, n:], absGU[0, :n], absGU[0, n:]
    zref = O.silu_mul(gref, uref)
    z = to_np(outs[GU])
    tol = silu_mul_tolerance(gref, uref, absG, absU, zref, True)
    assert np.all(np.abs(z[zi] - zref) <= tol), "z out of tolerance"
    assert np.all(np.isfinite(z)), "non-finite z"
    # down reads the GPU's own z (bf16)
    name, N, K = bench.MATS[DN]
    zbits = outs[GU].view(torch.int16).cpu().numpy().view(np.uint16)[None]
    rows = sample_rows(N, 71)
    codes, scales = weights_rows(fmt, last, DN, rows)
    yref, absY = O.matmul(codes, scales, O.X_BF16, zbits)
    assert_within(to_np(outs[DN])[rows][None], yref, absY, bf16_out=True, what="down")


def test_verify_pass_sampled():
    """bench.py's verification pass: five bf16 activation rows through all
    256 ternary products of the step in one chain (rows = 5)."""
    print("decode step: verification pass, 5 rows", flush=True)
    M, fmt = 5, 2
    W = bench.build_model(lb, synth, torch, fmt, bench.LAYERS)
    xvh = [synth.normal_bf16(bench.SEED, 950 + j, M, K) for j, (_, _, K) in enumerate(bench.MATS)]
    xv = [torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16) for x in xvh]
    yv = [[torch.full((M, N), float("nan"), device="cuda") for _, N, _ in bench.MATS]
          for _ in range(bench.LAYERS)]
    stages = [(fmt, N, K, W[l][j][0], W[l][j][1], xv[j], yv[l][j], 0)
              for l in range(bench.LAYERS) for j, (_, N, K) in enumerate(bench.MATS)]
    chain = lb.Chain(stages, x_dtype=lb.BF16, y_dtype=lb.F32, rows=M)
    chain.run()
    torch.cuda.synchronize()
    assert chain.failed_waits() == 0
    chain.close()
    for l in (0, bench.LAYERS - 1):
        for j, (name, N, K) in enumerate(bench.MATS):
            assert not torch.isnan(yv[l][j]).any(), f"layer {l} {name}: outputs not written"
            rows = sample_rows(N, 13 * l + j)
            codes, scales = weights_rows(fmt, l, j, rows)
            yref, absY = O.matmul(codes, scales, O.X_BF16, xvh[j])
            assert_within(yv[l][j].cpu().numpy()[:, rows], yref, absY, what=f"layer {l} {name}")


def test_separate_launches_graph_replays():
    """bench.py's `separate` mode: one lowbit_gemv launch per product, the
    step captured as one HIP graph.  Every replay (with eager launches and
    synchronisations between them) equals the eager run bit for bit, and a
    sample of the eager run meets the oracle."""
    print("decode step: 256 launches as one HIP graph", flush=True)
    fmt = 2
    W = bench.build_model(lb, synth, torch, fmt, bench.LAYERS)
    xh, xs = step_inputs()
    ys = [[torch.empty(N, device="cuda") for _, N, _ in bench.MATS] for _ in range(bench.LAYERS)]

    def step():
        for l in range(bench.LAYERS):
            for j, (_, N, K) in enumerate(bench.MATS):
                lb.gemv(fmt, N, K, W[l][j][0], W[l][j][1], xs[j], y=ys[l][j], y_dtype=lb.F32)

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        step()  # eager (allocates the split-K workspace outside the capture)
    torch.cuda.synchronize()
    eager = [[y.clone() for y in layer] for layer in ys]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for layer in ys:
            for y in layer:
                y.fill_(float("nan"))
        with torch.cuda.stream(stream):
            graph.replay()
        torch.cuda.synchronize()
        for l in range(bench.LAYERS):
            for j in range(len(bench.MATS)):
                assert torch.equal(ys[l][j], eager[l][j]), f"replay {rep} layer {l} product {j}"
        with torch.cuda.stream(stream):  # eager work between replays
            lb.gemv(fmt, 5120, 5120, W[0][1][0], W[0][1][1], xs[1], y_dtype=lb.F32)
        torch.cuda.synchronize()
    del graph
    for j, (name, N, K) in enumerate(bench.MATS):
        rows = sample_rows(N, 7 + j)
        codes, scales = weights_rows(fmt, bench.LAYERS - 1, j, rows)
        yref, absY = O.matmul(codes, scales, O.X_BF16, xh[j])
        assert_within(eager[-1][j].cpu().numpy()[rows][None], yref, absY, what=f"last layer {name}")
