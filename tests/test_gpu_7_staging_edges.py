"""Activations the split-term staging cannot carry on the fast path, on the GPU
against the fp64 oracle.

Every float output must satisfy |y - y_ref| <= 1e-3 * sum_k |w x| (plus
2^-8 |y_ref| for bf16 outputs) for any finite input.  The hard cases put a
large activation beside much smaller ones in the same 128-weight group and
give the large one a zero ternary code, so that sum |w x| counts only the
small ones: ranges of 2^14, 2^17, 2^24 and 2^60 within a group, tiny and
subnormal bf16 values, fp32 activations with full 24-bit mantissas, and
negative, zero and subnormal fp16 scales.  They run through every path:
the one-product GEMV, small-M products, chains (streaming and waiting,
one and several rows) and the GEMM (its per-group correction lists and the
exact recomputation when a list overflows)."""
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


def bf16_bits(v):
    return synth.f32_to_bf16_bits(np.asarray(v, np.float32))


def bf16_dev(bits):
    return dev(bits.view(np.int16)).view(torch.bfloat16)


def wide_range(seed, tid, M, K, span, every=8):
    """bf16 activations: every `every`-th element 2^span times larger than
    the rest (N(0,1) magnitudes otherwise), so every 32-element block of the
    hardware order holds both scales."""
    x = synth.normal_f32(seed, tid, M, K).astype(np.float64)
    big = (np.arange(K) % every) == 0
    x[:, big] = np.sign(x[:, big]) * (1.0 + np.abs(x[:, big])) * 2.0 ** span
    return bf16_bits(x), big


def zero_at(codes, mask):
    """ternary codes with 0 wherever mask (a K-vector) is set"""
    c = codes.copy()
    c[:, mask] = 0
    return c


def pack(fmt, codes, scales):
    return lb.pack(fmt, dev(codes), dev(scales.view(np.int16)))


def odd_scales(seed, tid, N, G):
    """fp16 scales mixing U[0.01,0.1], their negatives, zeros, positive
    subnormals (multiples of 2^-24) and a negative subnormal (-2^-20)."""
    s = synth.group_scales(seed, tid, N, G).view(np.float16).astype(np.float64)
    pick = synth.rand_u32(seed, tid + 1, np.arange(N * G)).reshape(N, G) % 6
    s = np.where(pick == 1, -s, s)
    s = np.where(pick == 2, 0.0, s)
    s = np.where(pick == 3, 2.0 ** -24 * (1 + (np.arange(N * G).reshape(N, G) % 1000)), s)
    s = np.where(pick == 4, -2.0 ** -20, s)
    return np.asarray(s, np.float16).view(np.uint16)


SPANS = [14, 17, 24, 60]


@pytest.mark.parametrize("fmt", [1, 2, 3])
@pytest.mark.parametrize("span", SPANS)
def test_gemv_wide_range_zero_code_at_max(fmt, span):
    N, K = 96, 1536
    print(f"gemv wide fmt={fmt} span={span}", flush=True)
    x, big = wide_range(SEED, 501, 1, K, span)
    codes = codes_for(fmt, SEED, 502, N, K)
    if fmt != 1:
        codes = zero_at(codes, big)
    scales = synth.group_scales(SEED, 503, N, K // 128)
    pc, ps = pack(fmt, codes, scales)
    y = lb.gemv(fmt, N, K, pc, ps, bf16_dev(x)[0])
    yb = lb.gemv(fmt, N, K, pc, ps, bf16_dev(x)[0], y_dtype=lb.BF16)
    torch.cuda.synchronize()
    yref, absY = O.matmul(codes, scales, O.X_BF16, x)
    w = assert_within(y.cpu().numpy()[None], yref, absY, what="f32 out")
    assert_within(yb.float().cpu().numpy()[None], yref, absY, bf16_out=True, what="bf16 out")
    print(f"  worst err/tol {w:.3e}")


@pytest.mark.parametrize("fmt", [2, 3])
def test_gemv_single_small_weighted_element(fmt):
    """The row weighs one small element of each group (codes zero elsewhere,
    in particular at the block maxima): y is then s c x_small and the bound
    1e-3 |s x_small| leaves no room for a dropped element."""
    N, K = 64, 1024
    x, big = wide_range(SEED, 511, 1, K, 20, every=4)
    rng = np.random.default_rng(5)
    codes = np.zeros((N, K), np.int8)
    for n in range(N):
        for g in range(K // 128):
            k = 128 * g + int(rng.integers(0, 128))
            while big[k]:
                k = 128 * g + int(rng.integers(0, 128))
            codes[n, k] = 1 if rng.random() < 0.5 else -1
    scales = synth.group_scales(SEED, 513, N, K // 128)
    pc, ps = pack(fmt, codes, scales)
    y = lb.gemv(fmt, N, K, pc, ps, bf16_dev(x)[0])
    torch.cuda.synchronize()
    yref, absY = O.matmul(codes, scales, O.X_BF16, x)
    assert_within(y.cpu().numpy()[None], yref, absY, what="single small")


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_gemv_tiny_and_subnormal_bf16(fmt):
    """bf16 subnormals (2^-133 .. 2^-127) beside normal values of 2^-120 and
    of 1, and blocks made only of subnormals."""
    N, K = 80, 1280
    base = synth.normal_f32(SEED, 521, 1, K).astype(np.float64)
    scale = np.where(np.arange(K) % 3 == 0, 2.0 ** -131, np.where(np.arange(K) % 3 == 1, 2.0 ** -120, 1.0))
    scale[:256] = 2.0 ** -131  # two whole groups of subnormals
    x = bf16_bits(base * scale)
    codes = codes_for(fmt, SEED, 522, N, K)
    if fmt != 1:
        codes = zero_at(codes, (np.arange(K) % 3 == 2))
    scales = synth.group_scales(SEED, 523, N, K // 128)
    pc, ps = pack(fmt, codes, scales)
    y = lb.gemv(fmt, N, K, pc, ps, bf16_dev(x)[0])
    torch.cuda.synchronize()
    yref, absY = O.matmul(codes, scales, O.X_BF16, x)
    assert_within(y.cpu().numpy()[None], yref, absY, what="subnormal")


@pytest.mark.parametrize("fmt", [1, 2, 3])
@pytest.mark.parametrize("span", [0, 20, 40])
def test_gemv_f32_full_mantissa(fmt, span):
    """fp32 activations with all 24 significant bits (more than the four
    terms' 16), with and without a wide range inside each block."""
    N, K = 96, 1024
    x = synth.normal_f32(SEED, 531, 1, K).astype(np.float64)
    x *= 1.0 + np.arange(K) * 2.0 ** -23  # fill the low mantissa bits
    big = (np.arange(K) % 8) == 0
    x[:, big] *= 2.0 ** span
    x = x.astype(np.float32)
    codes = codes_for(fmt, SEED, 532, N, K)
    if fmt != 1 and span:
        codes = zero_at(codes, big)
    scales = synth.group_scales(SEED, 533, N, K // 128)
    pc, ps = pack(fmt, codes, scales)
    y = lb.gemv(fmt, N, K, pc, ps, dev(x)[0])
    torch.cuda.synchronize()
    yref, absY = O.matmul(codes, scales, O.X_F32, x)
    assert_within(y.cpu().numpy()[None], yref, absY, what="f32 acts")


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_odd_scales(fmt):
    """Negative, zero and subnormal fp16 scales, GEMV and GEMM."""
    N, K, M = 144, 1152, 70
    codes = codes_for(fmt, SEED, 541, N, K)
    scales = odd_scales(SEED, 542, N, K // 128)
    pc, ps = pack(fmt, codes, scales)
    X = synth.normal_bf16(SEED, 544, M, K)
    y = lb.gemv(fmt, N, K, pc, ps, bf16_dev(X)[0])
    Y = lb.gemm(fmt, M, N, K, pc, ps, bf16_dev(X))
    torch.cuda.synchronize()
    yref, absY = O.matmul(codes, scales, O.X_BF16, X)
    assert_within(y.cpu().numpy()[None], yref[:1], absY[:1], what="gemv")
    assert_within(Y.cpu().numpy(), yref, absY, what="gemm")


@pytest.mark.parametrize("fmt", [2, 3])
@pytest.mark.parametrize("M", [2, 3, 5])
@pytest.mark.parametrize("span", [17, 60])
def test_small_m_wide_range(fmt, M, span):
    N, K = 80, 2048
    X, big = wide_range(SEED, 551, M, K, span)
    codes = zero_at(codes_for(fmt, SEED, 552, N, K), big)
    scales = synth.group_scales(SEED, 553, N, K // 128)
    pc, ps = pack(fmt, codes, scales)
    Y = lb.gemm(fmt, M, N, K, pc, ps, bf16_dev(X))
    torch.cuda.synchronize()
    yref, absY = O.matmul(codes, scales, O.X_BF16, X)
    assert_within(Y.cpu().numpy(), yref, absY, what=f"M={M}")


@pytest.mark.parametrize("fmt", [2, 3])
@pytest.mark.parametrize("wait", [0, 1])
@pytest.mark.parametrize("rows", [1, 3])
def test_chain_wide_range(fmt, wait, rows):
    """Chains: the streaming kernel (no waits) and the waiting kernel, one
    row and several rows, with normal stages around a wide-range stage."""
    shapes = [(64, 1024), (96, 2048), (48, 5120)]
    spans = [0, 60, 24]
    stages, refs, ys = [], [], []
    for j, ((N, K), span) in enumerate(zip(shapes, spans)):
        if span:
            X, big = wide_range(SEED, 561 + j, rows, K, span)
            codes = zero_at(codes_for(fmt, SEED, 571 + j, N, K), big)
        else:
            X = synth.normal_bf16(SEED, 561 + j, rows, K)
            codes = codes_for(fmt, SEED, 571 + j, N, K)
        scales = synth.group_scales(SEED, 581 + j, N, K // 128)
        pc, ps = pack(fmt, codes, scales)
        xt = bf16_dev(X) if rows > 1 else bf16_dev(X)[0]
        y = torch.full((rows, N) if rows > 1 else (N,), float("nan"), device="cuda")
        ys.append(y)
        stages.append((fmt, N, K, pc, ps, xt, y, wait if j else 0))
        refs.append(O.matmul(codes, scales, O.X_BF16, X))
    chain = lb.Chain(stages, x_dtype=lb.BF16, y_dtype=lb.F32, rows=rows)
    for rep in range(2):
        for y in ys:
            y.fill_(float("nan"))
        chain.run()
        torch.cuda.synchronize()
        for j in range(len(shapes)):
            yref, absY = refs[j]
            assert_within(ys[j].cpu().numpy().reshape(rows, -1), yref, absY, what=f"stage {j} rep {rep}")
    assert chain.failed_waits() == 0
    chain.close()


def sparse_small_weighted(seed, tid, M, N, K):
    """bf16 X of N(0,1) values in which one column per 128-group is scaled
    down by 2^20 in rows m % 16 < 8 (the two fp8 terms miss those elements:
    eight list entries per 16-row tile and group), and ternary codes that
    weigh only those columns, so that in those rows sum |w x| counts only
    the small elements: the GEMM's correction lists, without overflow."""
    rng = np.random.default_rng(tid)
    X = synth.normal_f32(seed, tid, M, K).astype(np.float64)
    cols = np.array([128 * g + int(rng.integers(0, 128)) for g in range(K // 128)])
    rows = (np.arange(M) % 16) < 8
    X[np.ix_(rows, cols)] *= 2.0 ** -20
    codes = np.zeros((N, K), np.int8)
    codes[:, cols] = synth.binary_codes(seed, tid + 1, N, K)[:, cols]
    return bf16_bits(X), codes, rows


@pytest.mark.parametrize("fmt", [2, 3])
@pytest.mark.parametrize("M,N,K", [(64, 512, 1024), (200, 2048, 1280), (130, 4096, 640)])
def test_gemm_correction_lists(fmt, M, N, K):
    print(f"gemm lists fmt={fmt} M={M} N={N} K={K}", flush=True)
    X, codes, _ = sparse_small_weighted(SEED, 591, M, N, K)
    scales = synth.group_scales(SEED, 593, N, K // 128)
    pc, ps = pack(fmt, codes, scales)
    Y = lb.gemm(fmt, M, N, K, pc, ps, bf16_dev(X))
    Yb = lb.gemm(fmt, M, N, K, pc, ps, bf16_dev(X), y_dtype=lb.BF16)
    torch.cuda.synchronize()
    yref, absY = O.matmul(codes, scales, O.X_BF16, X)
    w = assert_within(Y.cpu().numpy(), yref, absY, what="f32 out")
    assert_within(Yb.float().cpu().numpy(), yref, absY, bf16_out=True, what="bf16 out")
    print(f"  worst err/tol {w:.3e}")


@pytest.mark.parametrize("fmt", [1, 2, 3])
@pytest.mark.parametrize("span", SPANS)
def test_gemm_wide_range(fmt, span):
    """Every block wide-ranged: the ternary lists overflow and the workgroups
    recompute exactly; binary rows stay on the MFMA path."""
    M, N, K = 100, 1040, 1024
    print(f"gemm wide fmt={fmt} span={span}", flush=True)
    X, big = wide_range(SEED, 601, M, K, span)
    codes = codes_for(fmt, SEED, 602, N, K)
    if fmt != 1:
        codes = zero_at(codes, big)
    scales = synth.group_scales(SEED, 603, N, K // 128)
    pc, ps = pack(fmt, codes, scales)
    Y = lb.gemm(fmt, M, N, K, pc, ps, bf16_dev(X))
    torch.cuda.synchronize()
    yref, absY = O.matmul(codes, scales, O.X_BF16, X)
    w = assert_within(Y.cpu().numpy(), yref, absY, what="gemm wide")
    print(f"  worst err/tol {w:.3e}")


@pytest.mark.parametrize("fmt", [2, 3])
def test_gemm_split_k_lists(fmt):
    """A grid small enough to be split over K: the corrections of each split
    are added before the ordered reduction."""
    M, N, K = 64, 256, 5120
    X, codes, _ = sparse_small_weighted(SEED, 611, M, N, K)
    scales = synth.group_scales(SEED, 613, N, K // 128)
    pc, ps = pack(fmt, codes, scales)
    Y = lb.gemm(fmt, M, N, K, pc, ps, bf16_dev(X))
    torch.cuda.synchronize()
    yref, absY = O.matmul(codes, scales, O.X_BF16, X)
    assert_within(Y.cpu().numpy(), yref, absY, what="split-K lists")


def few_far_below(seed, tid, K, every=256, span=40):
    """One bf16 row: N(0,1) values with one element per `every` scaled down
    by 2^span, far beyond the range the split terms carry beside its block's
    maximum (a few correction-list entries per slice, no overflow)."""
    x = synth.normal_f32(seed, tid, 1, K).astype(np.float64)
    rng = np.random.default_rng(tid)
    cols = np.array([every * j + int(rng.integers(0, every)) for j in range(K // every)])
    x[0, cols] *= 2.0 ** -span
    return bf16_bits(x), cols


@pytest.mark.parametrize("fmt", [2, 3])
def test_waiting_chain_correction_lists(fmt):
    """Waiting chain, one row: the weights see only the elements far below
    their blocks' maxima (codes zero elsewhere), so sum |w x| counts only
    them and the result is what the correction lists add.  The second stage
    has more row groups than the grid has workgroups, so some workgroups
    run a second item on the same staged slice and its list."""
    print(f"waiting chain correction lists fmt={fmt}", flush=True)
    shapes = [(256, 2048), (33792, 1024), (512, 5120)]
    stages, refs, ys = [], [], []
    for j, (N, K) in enumerate(shapes):
        X, cols = few_far_below(SEED, 601 + j, K)
        full = codes_for(fmt, SEED, 611 + j, N, K)
        codes = np.zeros_like(full)
        codes[:, cols] = np.where(full[:, cols] == 0, 1, full[:, cols])
        scales = synth.group_scales(SEED, 621 + j, N, K // 128)
        pc, ps = pack(fmt, codes, scales)
        y = torch.full((N,), float("nan"), device="cuda")
        ys.append(y)
        stages.append((fmt, N, K, pc, ps, bf16_dev(X)[0], y, 1 if j else 0))
        refs.append(O.matmul(codes, scales, O.X_BF16, X))
    chain = lb.Chain(stages, x_dtype=lb.BF16, y_dtype=lb.F32)
    for rep in range(2):
        for y in ys:
            y.fill_(float("nan"))
        chain.run()
        torch.cuda.synchronize()
        for j in range(len(shapes)):
            yref, absY = refs[j]
            assert np.all(absY > 0)
            assert_within(ys[j].cpu().numpy()[None], yref, absY, what=f"stage {j} rep {rep}")
    assert chain.failed_waits() == 0
    chain.close()
