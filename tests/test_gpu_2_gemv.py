"""lowbit_gemv / small-M lowbit_gemm on the GPU against the fp64 oracle.

Float outputs must satisfy |y - y_ref| <= 1e-3 * sum_k |w x| per output
(plus 2^-8 |y_ref| for bf16 outputs); integer outputs must be bit-exact."""
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


def make(fmt, N, K, seed=SEED, tid=1):
    codes = codes_for(fmt, seed, tid, N, K)
    scales = synth.group_scales(seed, tid + 1, N, K // 128)
    pc, ps = lb.pack(fmt, dev(codes), dev(scales.view(np.int16)))
    return codes, scales, pc, ps


SHAPES = [(16, 128), (1, 128), (37, 384), (5, 1152), (33, 2048), (100, 640), (256, 1024), (48, 1664)]


@pytest.mark.parametrize("fmt", [1, 2, 3])
@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("xk", ["bf16", "f32"])
def test_gemv_float_parity(fmt, N, K, xk):
    print(f"gemv fmt={fmt} N={N} K={K} x={xk}", flush=True)
    codes, scales, pc, ps = make(fmt, N, K)
    if xk == "bf16":
        x = synth.normal_bf16(SEED, 9, 1, K)
        xt = dev(x.view(np.int16)).view(torch.bfloat16)[0]
        kind = O.X_BF16
    else:
        x = synth.normal_f32(SEED, 9, 1, K)
        xt = dev(x)[0]
        kind = O.X_F32
    yref, absY = O.matmul(codes, scales, kind, x)
    y = lb.gemv(fmt, N, K, pc, ps, xt, y_dtype=lb.F32)
    yb = lb.gemv(fmt, N, K, pc, ps, xt, y_dtype=lb.BF16)
    torch.cuda.synchronize()
    assert_within(y.cpu().numpy()[None], yref, absY, what="f32 out")
    assert_within(yb.float().cpu().numpy()[None], yref, absY, bf16_out=True, what="bf16 out")


def test_c0_binary_256x1024_f32():
    """Binary GEMV N=256, K=1024, fp32 activations N(0,1), scales U[0.01,0.1]."""
    N, K = 256, 1024
    codes, scales, pc, ps = make(1, N, K, seed=SEED, tid=1)
    x = synth.normal_f32(SEED, 3, 1, K)
    yref, absY = O.matmul(codes, scales, O.X_F32, x)
    y = lb.gemv(1, N, K, pc, ps, dev(x)[0])
    torch.cuda.synchronize()
    worst = assert_within(y.cpu().numpy()[None], yref, absY, what="C0")
    print(f"C0 worst err/tol = {worst:.3e}")


@pytest.mark.parametrize("fmt", [1, 2, 3])
@pytest.mark.parametrize("N,K", [(5120, 5120), (17408, 5120), (5120, 17408)])
def test_full_size_shapes(fmt, N, K):
    """27B-class layer shapes, weights generated on the device, full compare."""
    print(f"gemv full fmt={fmt} N={N} K={K}", flush=True)
    tern = fmt != 1
    codes_t = synth.device_codes(tern, SEED + 1, 21, N, K, "cuda")
    scales_t = synth.device_scales(SEED + 1, 22, N, K // 128, "cuda")
    pc, ps = lb.pack(fmt, codes_t, scales_t)
    del codes_t
    x = synth.normal_bf16(SEED + 1, 23, 1, K)
    y = lb.gemv(fmt, N, K, pc, ps, dev(x.view(np.int16)).view(torch.bfloat16)[0])
    torch.cuda.synchronize()
    codes = codes_for(fmt, SEED + 1, 21, N, K)
    scales = synth.group_scales(SEED + 1, 22, N, K // 128)
    yref, absY = O.matmul(codes, scales, O.X_BF16, x)
    worst = assert_within(y.cpu().numpy()[None], yref, absY, what="full")
    print(f"worst err/tol = {worst:.3e}")


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_dyadic_inputs_are_exact(fmt):
    """Small-integer bf16 activations and power-of-two scales: the product is
    exactly representable and the GPU result equals the oracle exactly."""
    rng = np.random.default_rng(4)
    N, K = 64, 1280
    codes = codes_for(fmt, SEED, 31, N, K)
    scales = np.asarray(2.0 ** rng.integers(-7, -2, size=(N, K // 128)), np.float16).view(np.uint16)
    xv = rng.integers(-8, 9, size=(1, K)).astype(np.float32)
    x = synth.f32_to_bf16_bits(xv)
    pc, ps = lb.pack(fmt, dev(codes), dev(scales.view(np.int16)))
    y = lb.gemv(fmt, N, K, pc, ps, dev(x.view(np.int16)).view(torch.bfloat16)[0])
    yref = O.matmul(codes, scales, O.X_BF16, x, with_abs=False)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().astype(np.float64), yref[0])


@pytest.mark.parametrize("fmt", [1, 2, 3])
@pytest.mark.parametrize("N,K", [(37, 384), (5120, 5120)])
def test_int8_activations(fmt, N, K):
    codes, scales, pc, ps = make(fmt, N, K, tid=41)
    xb = synth.normal_bf16(SEED, 43, 1, K)
    q, sx = O.quantize_act_i8(xb)
    qt = dev(q)[0]
    # exact integer path: unit scales, int32 output
    yi = lb.gemv(fmt, N, K, pc, None, qt, y_dtype=lb.I32, x_dtype=lb.I8)
    A = O.group_int_sums(codes, q).sum(axis=2)[0]
    # float path with the group scales and s_x
    yf = lb.gemv(fmt, N, K, pc, ps, qt, x_scale=float(sx[0]), y_dtype=lb.F32, x_dtype=lb.I8)
    torch.cuda.synchronize()
    assert np.array_equal(yi.cpu().numpy().astype(np.int64), A)
    yref, absY = O.matmul(codes, scales, O.X_I8, q, sx)
    assert_within(yf.cpu().numpy()[None], yref, absY, what="i8 float")


# (20480, 5120): two waves of five quads per row-block (rounds of five loads)
@pytest.mark.parametrize("N,K", [(37, 384), (256, 1024), (5120, 5120), (300, 17408), (16, 128),
                                 (48, 640), (16, 393216), (20480, 5120)])
def test_sign_activations_xor_popcount(N, K):
    codes, scales, pc, ps = make(1, N, K, tid=51)
    xb = synth.sign_bits(SEED, 53, 1, K)
    yi = lb.gemv(1, N, K, pc, None, dev(xb)[0], y_dtype=lb.I32, x_dtype=lb.SIGN1)
    yf = lb.gemv(1, N, K, pc, ps, dev(xb)[0], x_scale=0.75, y_dtype=lb.F32, x_dtype=lb.SIGN1)
    torch.cuda.synchronize()
    Y, D = O.xor_popcount(codes, scales, xb, np.array([0.75], np.float32))
    assert np.array_equal(yi.cpu().numpy().astype(np.int64), D[0])
    _, absY = O.matmul(codes, scales, O.X_SIGN1, xb, np.array([0.75], np.float32))
    assert_within(yf.cpu().numpy()[None], Y, absY, what="sign float")


@pytest.mark.parametrize("fmt", [1, 2])
def test_repeat_runs_bit_identical(fmt):
    N, K = 5120, 5120
    codes_t = synth.device_codes(fmt != 1, SEED, 61, N, K, "cuda")
    pc, ps = lb.pack(fmt, codes_t, synth.device_scales(SEED, 62, N, K // 128, "cuda"))
    x = dev(synth.normal_bf16(SEED, 63, 1, K).view(np.int16)).view(torch.bfloat16)[0]
    y1 = lb.gemv(fmt, N, K, pc, ps, x)
    y2 = lb.gemv(fmt, N, K, pc, ps, x)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("fmt", [1, 2, 3])
@pytest.mark.parametrize("M", [1, 2, 5, 8])
def test_small_m_gemm_bf16(fmt, M):
    """Small-M products (M = k+1 = 5 is a speculative-decoding verify pass)."""
    N, K = 96, 1536
    codes, scales, pc, ps = make(fmt, N, K, tid=71)
    X = synth.normal_bf16(SEED, 73, M, K)
    Xt = dev(X.view(np.int16)).view(torch.bfloat16)
    Y = lb.gemm(fmt, M, N, K, pc, ps, Xt)
    torch.cuda.synchronize()
    yref, absY = O.matmul(codes, scales, O.X_BF16, X)
    assert_within(Y.cpu().numpy(), yref, absY, what=f"M={M}")
    if M == 1:
        y = lb.gemv(fmt, N, K, pc, ps, Xt[0])
        torch.cuda.synchronize()
        assert torch.equal(Y[0], y)


@pytest.mark.parametrize("M", [3, 8])
def test_small_m_gemm_int8(M):
    N, K = 80, 1024
    codes, scales, pc, ps = make(2, N, K, tid=81)
    Xb = synth.normal_bf16(SEED, 83, M, K)
    Q, sx = lb.quantize_act_i8(dev(Xb.view(np.int16)).view(torch.bfloat16))
    q_ref, sx_ref = O.quantize_act_i8(Xb)
    Yi = lb.gemm(2, M, N, K, pc, None, Q, y_dtype=lb.I32)
    Yf = lb.gemm(2, M, N, K, pc, ps, Q, x_scales=sx)
    torch.cuda.synchronize()
    assert np.array_equal(Q.cpu().numpy(), q_ref) and np.array_equal(sx.cpu().numpy(), sx_ref)
    assert np.array_equal(Yi.cpu().numpy().astype(np.int64), O.group_int_sums(codes, q_ref).sum(axis=2))
    yref, absY = O.matmul(codes, scales, O.X_I8, q_ref, sx_ref)
    assert_within(Yf.cpu().numpy(), yref, absY, what="i8 gemm")


@pytest.mark.parametrize("N,K", [(37, 384), (100, 1152), (5120, 5120), (16384, 1536)])
@pytest.mark.parametrize("xk", ["bf16", "f32"])
def test_base3_equals_2bit(N, K, xk):
    """The same ternary codes packed as 2-bit and as base-3 decode to the same
    fp4 operands, so the two GEMVs agree bit for bit where both reduce a row
    in one slice (no split-K partials in either workspace).  Rows split into
    K-slices -- long rows, or small products split to reach every CU -- are
    cut into whole quads for 2-bit and whole octets for base-3, which changes
    the fp32 summation order: both are then checked against the oracle."""
    codes = codes_for(2, SEED, 91, N, K)
    scales = synth.group_scales(SEED, 92, N, K // 128)
    pc2, ps2 = lb.pack(2, dev(codes), dev(scales.view(np.int16)))
    pc3, ps3 = lb.pack(3, dev(codes), dev(scales.view(np.int16)))
    if xk == "bf16":
        x = dev(synth.normal_bf16(SEED, 93, 1, K).view(np.int16)).view(torch.bfloat16)[0]
    else:
        x = dev(synth.normal_f32(SEED, 93, 1, K))[0]
    y2 = lb.gemv(2, N, K, pc2, ps2, x)
    y3 = lb.gemv(3, N, K, pc3, ps3, x)
    torch.cuda.synchronize()
    xdt = lb.BF16 if xk == "bf16" else lb.F32
    one_slice = all(lb.workspace_bytes(f, 1, N, K, xdt) == 256 << 10 for f in (2, 3))
    if one_slice:
        assert torch.equal(y2, y3)
    else:
        xh = x.cpu().view(torch.int16).numpy().view(np.uint16) if xk == "bf16" else x.cpu().numpy()
        yref, absY = O.matmul(codes, scales, O.X_BF16 if xk == "bf16" else O.X_F32, xh[None])
        assert_within(y2.cpu().numpy()[None], yref, absY, what="2-bit")
        assert_within(y3.cpu().numpy()[None], yref, absY, what="base-3")
    assert one_slice or (N, K) != (16384, 1536)


@pytest.mark.parametrize("K,offset", [(1024, 0), (17408, 0), (1000, 0), (1024, 1)])
def test_quantize_act_i8_paths(K, offset):
    """Per-row int8 quantization, bit-exact: the 16-byte path (K % 8 == 0,
    aligned) and the element path (K % 8 != 0, or X at a 2-byte offset), with
    a zero row and a row of exact ties (max 127: x * inv = x, so 2.5 -> 2,
    -3.5 -> -4, 0.5 -> 0)."""
    M = 5
    Xb = synth.normal_bf16(SEED, 91, M, K)
    Xb[2] = 0
    ties = np.array([127.0, 2.5, -3.5, 0.5, 1.5, -0.5, -126.5, 63.5], np.float32)
    row3 = np.resize(ties, K).astype(np.float32)
    Xb[3] = (row3.view(np.uint32) >> 16).astype(np.uint16)
    flat = torch.empty(M * K + offset, dtype=torch.int16, device="cuda")
    flat[offset:] = dev(Xb.view(np.int16).reshape(-1))
    X = flat[offset:].view(M, K).view(torch.bfloat16)
    Q, sx = lb.quantize_act_i8(X)
    torch.cuda.synchronize()
    q_ref, sx_ref = O.quantize_act_i8(Xb)
    assert np.array_equal(Q.cpu().numpy(), q_ref)
    assert np.array_equal(sx.cpu().numpy(), sx_ref)
    assert sx_ref[2] == 0 and not q_ref[2].any()
    assert q_ref[3][:8].tolist() == [127, 2, -4, 0, 2, 0, -126, 64]


@pytest.mark.parametrize("fmt", [1, 2])
def test_small_m_graph_replays(fmt):
    """Small-M products (M = 5: the slice images staged once per call, then
    the product) captured as one HIP graph: every replay, with eager
    launches and synchronisations between replays, equals the eager run bit
    for bit; the eager run meets the oracle.  Two shapes, one with K-slices."""
    M = 5
    shapes = [(2048, 5120), (640, 17408)]
    mats, Xs, Ys, refs = [], [], [], []
    for j, (N, K) in enumerate(shapes):
        codes, scales, pc, ps = make(fmt, N, K, tid=95 + 2 * j)
        X = synth.normal_bf16(SEED, 99 + j, M, K)
        mats.append((pc, ps))
        Xs.append(dev(X.view(np.int16)).view(torch.bfloat16))
        Ys.append(torch.empty((M, N), device="cuda"))
        refs.append((X, codes, scales))
    stream = torch.cuda.Stream()

    def step():
        for j, (N, K) in enumerate(shapes):
            lb.gemm(fmt, M, N, K, mats[j][0], mats[j][1], Xs[j], Y=Ys[j])

    with torch.cuda.stream(stream):
        step()  # eager (sizes the workspace outside the capture)
    torch.cuda.synchronize()
    eager = [y.clone() for y in Ys]
    for j, (X, codes, scales) in enumerate(refs):
        yref, absY = O.matmul(codes, scales, O.X_BF16, X)
        assert_within(eager[j].cpu().numpy(), yref, absY, what=f"shape {j}")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for y in Ys:
            y.fill_(float("nan"))
        with torch.cuda.stream(stream):
            graph.replay()
        torch.cuda.synchronize()
        for j in range(len(shapes)):
            assert torch.equal(Ys[j], eager[j]), f"replay {rep} shape {j}"
        with torch.cuda.stream(stream):  # eager work between replays
            lb.gemm(fmt, M, 2048, 5120, mats[0][0], mats[0][1], Xs[0])
        torch.cuda.synchronize()
    del graph


def test_graph_survives_workspace_growth():
    """A graph captured on a stream keeps its workspace after a larger eager
    call on the same stream grows the stream's workspace: replays before and
    after the growth equal the eager result bit for bit.  Capturing a product
    on a stream whose workspace is too small fails with E_NOMEM."""
    fmt, M, N, K = 2, 5, 640, 5120
    print("graph workspace growth", flush=True)
    codes, scales, pc, ps = make(fmt, N, K, tid=121)
    X = synth.normal_bf16(SEED, 123, M, K)
    Xt = dev(X.view(np.int16)).view(torch.bfloat16)
    Y = torch.empty((M, N), device="cuda")
    ref = lb.gemm(fmt, M, N, K, pc, ps, Xt)  # eager, on the default stream
    torch.cuda.synchronize()
    yref, absY = O.matmul(codes, scales, O.X_BF16, X)
    assert_within(ref.cpu().numpy(), yref, absY, what="eager")

    stream = torch.cuda.Stream()
    need = lb.workspace_bytes(fmt, M, N, K, lb.BF16)
    assert need > 0
    lb.reserve_workspace(need, stream=stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        lb.gemm(fmt, M, N, K, pc, ps, Xt, Y=Y)
    torch.cuda.synchronize()

    # a larger product on the same stream grows its workspace
    Nb, Kb, Mb = 2048, 17408, 300
    _, _, pcb, psb = make(fmt, Nb, Kb, tid=125)
    Xb = torch.randn((Mb, Kb), device="cuda").to(torch.bfloat16)
    assert lb.workspace_bytes(fmt, Mb, Nb, Kb, lb.BF16) > need
    for rep in range(3):
        Y.fill_(float("nan"))
        with torch.cuda.stream(stream):
            graph.replay()
            if rep == 0:
                lb.gemm(fmt, Mb, Nb, Kb, pcb, psb, Xb)  # grows while the replay may run
        torch.cuda.synchronize()
        assert torch.equal(Y, ref), f"replay {rep}"
    del graph

    # no reserve: the capture cannot grow the fresh stream's workspace
    fresh = torch.cuda.Stream()
    g2 = torch.cuda.CUDAGraph()
    err = None
    with torch.cuda.graph(g2, stream=fresh):
        Y.fill_(0.0)
        try:
            lb.gemm(fmt, M, N, K, pc, ps, Xt, Y=Y)
        except lb.LowbitError as e:
            err = e
    torch.cuda.synchronize()
    assert err is not None and err.status == lb.E_NOMEM
    del g2
