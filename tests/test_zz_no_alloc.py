"""lowbit_gemv_noalloc, the allocation-free batch-1 product, called through
the C ABI: its output equals lowbit_gemv's bit for bit (the same kernels, a
static scratch array instead of the per-stream workspace) and meets the
oracle's tolerance, over two calls in a row with the second one smaller, in
every weight format and activation type, and inside a replayed HIP graph."""
import numpy as np
import pytest
import torch

import synth
from oracle import oracle as O
from ultra_bit_dit_amd import lowbit as lb

from helpers import SEED, assert_within, codes_for

pytestmark = pytest.mark.gpu


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def make(fmt, N, K, tid):
    codes = codes_for(fmt, SEED, tid, N, K)
    scales = synth.group_scales(SEED, tid + 1, N, K // 128)
    pc, ps = lb.pack(fmt, dev(codes), dev(scales.view(np.int16)))
    return codes, scales, pc, ps


def activation(xk, K, tid):
    if xk == "bf16":
        x = synth.normal_bf16(SEED, tid, 1, K)
        return x, O.X_BF16, dev(x.view(np.int16)).view(torch.bfloat16)[0]
    x = synth.normal_f32(SEED, tid, 1, K)
    return x, O.X_F32, dev(x)[0]


# first call large (the 27B down projection's shape, split over K), second smaller and ragged
CALLS = [(5120, 17408, "bf16"), (37, 384, "f32")]


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_noalloc_equals_gemv_two_calls(fmt):
    for i, (N, K, xk) in enumerate(CALLS):
        print(f"noalloc fmt={fmt} N={N} K={K} x={xk}", flush=True)
        codes, scales, pc, ps = make(fmt, N, K, 300 + 4 * i)
        x, okind, xt = activation(xk, K, 302 + 4 * i)
        ref = lb.gemv(fmt, N, K, pc, ps, xt)
        y = torch.full((N,), float("nan"), device="cuda")
        lb.gemv_noalloc(fmt, N, K, pc, ps, xt, y)
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"call {i}"
        yref, absY = O.matmul(codes, scales, okind, x)
        assert_within(y.cpu().numpy()[None], yref, absY, what=f"call {i}")


@pytest.mark.parametrize("fmt", [2, 3])
def test_noalloc_int8_exact_and_bf16_out(fmt):
    """int8 activations: the I32 output is the exact integer sum of the oracle;
    bf16 output equals lowbit_gemv's."""
    for i, (N, K) in enumerate([(2048, 5120), (48, 1664)]):
        codes, scales, pc, ps = make(fmt, N, K, 320 + 4 * i)
        q = np.random.default_rng(7 + i).integers(-127, 128, size=(1, K), dtype=np.int8)
        qt = dev(q)[0]
        yi = torch.empty(N, dtype=torch.int32, device="cuda")
        lb.gemv_noalloc(fmt, N, K, pc, None, qt, yi, y_dtype=lb.I32)
        yb = torch.empty(N, dtype=torch.bfloat16, device="cuda")
        _, _, xt = activation("bf16", K, 322 + 4 * i)
        lb.gemv_noalloc(fmt, N, K, pc, ps, xt, yb, y_dtype=lb.BF16)
        rb = lb.gemv(fmt, N, K, pc, ps, xt, y_dtype=lb.BF16)
        torch.cuda.synchronize()
        exact = O.group_int_sums(codes, q).sum(axis=-1)
        assert np.array_equal(yi.cpu().numpy(), exact.reshape(-1).astype(np.int64))
        assert torch.equal(yb, rb)


def test_noalloc_in_a_graph():
    """Captured after an eager call: every replay, with eager calls of other
    shapes on the same stream between replays, equals lowbit_gemv."""
    fmt, N, K = 2, 15360, 5120
    codes, scales, pc, ps = make(fmt, N, K, 340)
    _, _, xt = activation("bf16", K, 342)
    ref = lb.gemv(fmt, N, K, pc, ps, xt)
    y = torch.empty(N, device="cuda")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        lb.gemv_noalloc(fmt, N, K, pc, ps, xt, y)
    torch.cuda.synchronize()
    assert torch.equal(y, ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        lb.gemv_noalloc(fmt, N, K, pc, ps, xt, y)
    torch.cuda.synchronize()
    _, _, pc2, ps2 = make(fmt, 640, 17408, 344)
    _, _, x2 = activation("bf16", 17408, 346)
    y2 = torch.empty(640, device="cuda")
    for rep in range(3):
        y.fill_(float("nan"))
        with torch.cuda.stream(stream):
            g.replay()
            lb.gemv_noalloc(fmt, 640, 17408, pc2, ps2, x2, y2)  # after the replay, same stream
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"replay {rep}"
    del g
