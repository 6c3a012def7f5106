"""Large-M lowbit_gemm (staged-tile MFMA kernels) on the GPU against the fp64
oracle.

Small and medium shapes are compared in full; the prefill (M=512) and
diffusion-transformer block shapes are compared on sampled outputs: whole
rows plus a random block of (row, column) pairs.  Float outputs must satisfy
|y - y_ref| <= 1e-3 * sum_k |w x| (plus 2^-8 |y_ref| for bf16 outputs); the
int8 activation x ternary/binary product with unit scales is int32 and must
be bit-exact."""
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


def bf16_dev(x):
    return dev(x.view(np.int16)).view(torch.bfloat16)


def make(fmt, N, K, tid):
    codes = codes_for(fmt, SEED, tid, N, K)
    scales = synth.group_scales(SEED, tid + 1, N, K // 128)
    pc, ps = lb.pack(fmt, dev(codes), dev(scales.view(np.int16)))
    return codes, scales, pc, ps


# (M, N, K): ragged M and N, one group, several groups per split, split-K
SHAPES = [(9, 48, 128), (128, 256, 1024), (200, 384, 640), (130, 100, 1152), (300, 520, 2560),
          (64, 1040, 5120)]


@pytest.mark.parametrize("fmt", [1, 2, 3])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_bf16_parity(fmt, M, N, K):
    print(f"gemm bf16 fmt={fmt} M={M} N={N} K={K}", flush=True)
    codes, scales, pc, ps = make(fmt, N, K, tid=101)
    X = synth.normal_bf16(SEED, 103, M, K)
    Xt = bf16_dev(X)
    Y = lb.gemm(fmt, M, N, K, pc, ps, Xt, y_dtype=lb.F32)
    Yb = lb.gemm(fmt, M, N, K, pc, ps, Xt, y_dtype=lb.BF16)
    torch.cuda.synchronize()
    yref, absY = O.matmul(codes, scales, O.X_BF16, X)
    w = assert_within(Y.cpu().numpy(), yref, absY, what="f32 out")
    assert_within(Yb.float().cpu().numpy(), yref, absY, bf16_out=True, what="bf16 out")
    print(f"  worst err/tol {w:.3e}")


@pytest.mark.parametrize("fmt", [1, 2, 3])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_int8_parity(fmt, M, N, K):
    print(f"gemm int8 fmt={fmt} M={M} N={N} K={K}", flush=True)
    codes, scales, pc, ps = make(fmt, N, K, tid=111)
    Xb = synth.normal_bf16(SEED, 113, M, K)
    Q, sx = lb.quantize_act_i8(bf16_dev(Xb))
    Yi = lb.gemm(fmt, M, N, K, pc, None, Q, y_dtype=lb.I32)
    Yf = lb.gemm(fmt, M, N, K, pc, ps, Q, x_scales=sx, y_dtype=lb.F32)
    Yb = lb.gemm(fmt, M, N, K, pc, ps, Q, x_scales=sx, y_dtype=lb.BF16)
    torch.cuda.synchronize()
    q_ref, sx_ref = O.quantize_act_i8(Xb)
    assert np.array_equal(Q.cpu().numpy(), q_ref) and np.array_equal(sx.cpu().numpy(), sx_ref)
    A = O.group_int_sums(codes, q_ref).sum(axis=2)
    assert np.array_equal(Yi.cpu().numpy().astype(np.int64), A)
    yref, absY = O.matmul(codes, scales, O.X_I8, q_ref, sx_ref)
    assert_within(Yf.cpu().numpy(), yref, absY, what="i8 f32 out")
    assert_within(Yb.float().cpu().numpy(), yref, absY, bf16_out=True, what="i8 bf16 out")


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_gemm_dyadic_inputs_are_exact(fmt):
    """Small-integer activations and power-of-two scales: every partial sum is
    representable, so the GEMM equals the oracle exactly."""
    rng = np.random.default_rng(5)
    M, N, K = 160, 300, 1280
    codes = codes_for(fmt, SEED, 121, N, K)
    scales = np.asarray(2.0 ** rng.integers(-7, -2, size=(N, K // 128)), np.float16).view(np.uint16)
    X = synth.f32_to_bf16_bits(rng.integers(-8, 9, size=(M, K)).astype(np.float32))
    pc, ps = lb.pack(fmt, dev(codes), dev(scales.view(np.int16)))
    Y = lb.gemm(fmt, M, N, K, pc, ps, bf16_dev(X))
    torch.cuda.synchronize()
    yref = O.matmul(codes, scales, O.X_BF16, X, with_abs=False)
    assert np.array_equal(Y.cpu().numpy().astype(np.float64), yref)


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_gemm_bf16_wide_exponent_range(fmt):
    """bf16 rows far outside the fp16 range (and a zero row, and one tiny
    element beside large ones) are rescaled per row without loss."""
    M, N, K = 136, 96, 768
    codes, scales, pc, ps = make(fmt, N, K, tid=131)
    Xf = synth.bf16_bits_to_f32(synth.normal_bf16(SEED, 133, M, K)).astype(np.float64)
    expo = np.array([(-120, -60, -30, -15, 0, 15, 30, 60, 120)[m % 9] for m in range(M)], np.float64)
    Xf = Xf * 2.0 ** expo[:, None]
    Xf[7] = 0.0
    Xf[8, 5] = 2.0 ** -100
    X = synth.f32_to_bf16_bits(Xf.astype(np.float32))
    Y = lb.gemm(fmt, M, N, K, pc, ps, bf16_dev(X))
    torch.cuda.synchronize()
    yref, absY = O.matmul(codes, scales, O.X_BF16, X)
    assert_within(Y.cpu().numpy(), yref, absY, what="wide range")
    assert not Y[7].any()


def test_gemm_repeat_runs_bit_identical():
    """Split-K partials are added in a fixed order: repeated calls agree bit for bit."""
    M, N, K = 512, 5120, 5120
    codes_t = synth.device_codes(True, SEED, 141, N, K, "cuda")
    pc, ps = lb.pack(2, codes_t, synth.device_scales(SEED, 142, N, K // 128, "cuda"))
    X = bf16_dev(synth.normal_bf16(SEED, 143, M, K))
    Y1 = lb.gemm(2, M, N, K, pc, ps, X)
    Y2 = lb.gemm(2, M, N, K, pc, ps, X)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)


def sample_check(fmt, M, N, K, tid, int8=False, full_rows=2, blk=32):
    """Weights generated on the device; the oracle runs on `full_rows` whole
    output rows and a random blk x blk block of (row, column) pairs."""
    tern = fmt != 1
    codes_t = synth.device_codes(tern, SEED, tid, N, K, "cuda", chunk_rows=2048)
    scales_t = synth.device_scales(SEED, tid + 1, N, K // 128, "cuda")
    pc, ps = lb.pack(fmt, codes_t, scales_t)
    del codes_t, scales_t
    Xb = synth.normal_bf16(SEED, tid + 2, M, K)
    Xt = bf16_dev(Xb)
    rng = np.random.default_rng(tid)
    rows = np.unique(np.concatenate([[0, M - 1][:full_rows], rng.integers(0, M, size=blk)]))
    cols = np.sort(rng.choice(N, size=blk, replace=False))
    whole = np.array([0, M - 1][:full_rows])
    if int8:
        Q, sx = lb.quantize_act_i8(Xt)
        Yi = lb.gemm(fmt, M, N, K, pc, None, Q, y_dtype=lb.I32)
        Yf = lb.gemm(fmt, M, N, K, pc, ps, Q, x_scales=sx)
    else:
        Yf = lb.gemm(fmt, M, N, K, pc, ps, Xt)
    torch.cuda.synchronize()
    scales_all = synth.group_scales(SEED, tid + 1, N, K // 128)
    codes_all = codes_for(fmt, SEED, tid, N, K)
    if int8:
        q_ref, sx_ref = O.quantize_act_i8(Xb[rows])
        assert np.array_equal(Q.cpu().numpy()[rows], q_ref)
        assert np.array_equal(sx.cpu().numpy()[rows], sx_ref)
        Yi_h = Yi.cpu().numpy().astype(np.int64)
        qw = q_ref[np.searchsorted(rows, whole)]
        assert np.array_equal(Yi_h[whole], O.group_int_sums(codes_all, qw).sum(axis=2))
        assert np.array_equal(Yi_h[np.ix_(rows, cols)],
                              O.group_int_sums(codes_all[cols], q_ref).sum(axis=2))
        xs_whole = sx_ref[np.searchsorted(rows, whole)]
        yref, absY = O.matmul(codes_all, scales_all, O.X_I8, qw, xs_whole)
        yref2, absY2 = O.matmul(codes_all[cols], scales_all[cols], O.X_I8, q_ref, sx_ref)
    else:
        yref, absY = O.matmul(codes_all, scales_all, O.X_BF16, Xb[whole])
        yref2, absY2 = O.matmul(codes_all[cols], scales_all[cols], O.X_BF16, Xb[rows])
    Yh = Yf.cpu().numpy()
    w1 = assert_within(Yh[whole], yref, absY, what="whole rows")
    w2 = assert_within(Yh[np.ix_(rows, cols)], yref2, absY2, what="sampled block")
    print(f"  worst err/tol {max(w1, w2):.3e}")


@pytest.mark.parametrize("N,K", [(5120, 5120), (17408, 5120), (5120, 17408)])
def test_pp512_ternary_bf16_sampled(N, K):
    print(f"pp512 ternary bf16 N={N} K={K}", flush=True)
    sample_check(2, 512, N, K, tid=150 + (N + K) % 7)


@pytest.mark.parametrize("N,K", [(5120, 5120), (5120, 17408), (34816, 5120)])
def test_pp512_ternary_int8_sampled(N, K):
    # 34816 x 5120: 544 tiles of 64 x 512, two whole rounds of the 256 compute
    # units and 32 tiles split eight ways along K (exact int32 either way)
    print(f"pp512 ternary int8 N={N} K={K}", flush=True)
    sample_check(2, 512, N, K, tid=160 + (N + K) % 7, int8=True)


@pytest.mark.parametrize("M,N,K", [(4608, 3072, 3072), (4608, 9216, 3072), (4608, 3072, 9216),
                                   (18432, 3072, 3072)])
def test_dit_binary_bf16_sampled(M, N, K):
    print(f"DiT binary bf16 M={M} N={N} K={K}", flush=True)
    sample_check(1, M, N, K, tid=170 + (M + N + K) % 11, full_rows=1)


@pytest.mark.parametrize("N,K", [(5120, 5120), (17408, 5120)])
def test_pp512_ternary_base3_bf16_sampled(N, K):
    print(f"pp512 ternary base-3 bf16 N={N} K={K}", flush=True)
    sample_check(3, 512, N, K, tid=190 + (N + K) % 7)


@pytest.mark.parametrize("M,N,K", [(200, 384, 640), (512, 5120, 5120)])
def test_gemm_base3_equals_2bit(M, N, K):
    """Same ternary codes packed as 2-bit and base-3 decode to the same fp4
    operands: the two GEMMs agree bit for bit."""
    codes = codes_for(2, SEED, 195, N, K)
    scales = synth.group_scales(SEED, 196, N, K // 128)
    pc2, ps2 = lb.pack(2, dev(codes), dev(scales.view(np.int16)))
    pc3, ps3 = lb.pack(3, dev(codes), dev(scales.view(np.int16)))
    X = bf16_dev(synth.normal_bf16(SEED, 197, M, K))
    Y2 = lb.gemm(2, M, N, K, pc2, ps2, X)
    Y3 = lb.gemm(3, M, N, K, pc3, ps3, X)
    torch.cuda.synchronize()
    assert torch.equal(Y2, Y3)


# ------------------------------------------------ sign activations (batched)
def sign_scales(M, tid):
    rng = np.random.default_rng(tid)
    return rng.uniform(0.25, 2.0, size=M).astype(np.float32)


@pytest.mark.parametrize("fmt", [1, 2, 3])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_sign_parity(fmt, M, N, K):
    """Sign-bit activations x = alpha_m (-1)^bit: the unit-scale product is the
    exact integer sum of code x sign (for binary weights the XOR + popcount
    count, checked against the oracle's popcount routine too); scaled outputs
    meet the float bound."""
    print(f"gemm sign fmt={fmt} M={M} N={N} K={K}", flush=True)
    codes, scales, pc, ps = make(fmt, N, K, tid=211)
    xb = synth.sign_bits(SEED, 213, M, K)
    alpha = sign_scales(M, 215)
    Xd = dev(xb)
    Yi = lb.gemm(fmt, M, N, K, pc, None, Xd, y_dtype=lb.I32, x_dtype=lb.SIGN1)
    Yf = lb.gemm(fmt, M, N, K, pc, ps, Xd, x_scales=dev(alpha), y_dtype=lb.F32, x_dtype=lb.SIGN1)
    Yb = lb.gemm(fmt, M, N, K, pc, ps, Xd, x_scales=dev(alpha), y_dtype=lb.BF16, x_dtype=lb.SIGN1)
    torch.cuda.synchronize()
    D = O.matmul(codes, None, O.X_SIGN1, xb, np.ones(M, np.float32), with_abs=False)
    assert np.array_equal(Yi.cpu().numpy().astype(np.float64), D)
    if fmt == 1:
        _, Dpop = O.xor_popcount(codes, None, xb)
        assert np.array_equal(Yi.cpu().numpy().astype(np.int64), Dpop)
    yref, absY = O.matmul(codes, scales, O.X_SIGN1, xb, alpha)
    assert_within(Yf.cpu().numpy(), yref, absY, what="sign f32 out")
    assert_within(Yb.float().cpu().numpy(), yref, absY, bf16_out=True, what="sign bf16 out")


def test_gemm_sign_dit_block_sampled():
    """A DiT projection with sign activations at full size: exact integer
    outputs on whole rows and a sampled block."""
    M, N, K = 4608, 3072, 3072
    print(f"DiT sign binary M={M} N={N} K={K}", flush=True)
    codes_t = synth.device_codes(False, SEED, 221, N, K, "cuda", chunk_rows=2048)
    scales_t = synth.device_scales(SEED, 222, N, K // 128, "cuda")
    pc, ps = lb.pack(1, codes_t, scales_t)
    del codes_t, scales_t
    xb = synth.sign_bits(SEED, 223, M, K)
    Yi = lb.gemm(1, M, N, K, pc, None, dev(xb), y_dtype=lb.I32, x_dtype=lb.SIGN1)
    torch.cuda.synchronize()
    codes_all = codes_for(1, SEED, 221, N, K)
    rng = np.random.default_rng(224)
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, size=32)]))
    cols = np.sort(rng.choice(N, size=32, replace=False))
    Yh = Yi.cpu().numpy().astype(np.int64)
    _, Dw = O.xor_popcount(codes_all, None, xb[[0, M - 1]])
    assert np.array_equal(Yh[[0, M - 1]], Dw)
    _, Db = O.xor_popcount(codes_all[cols], None, xb[rows])
    assert np.array_equal(Yh[np.ix_(rows, cols)], Db)


def test_gemm_sign_rejects():
    _, _, pc, ps = make(1, 64, 256, tid=230)
    xb = dev(synth.sign_bits(SEED, 231, 40, 256))
    with pytest.raises(lb.LowbitError) as e:  # scaled output needs alpha per row
        lb.gemm(1, 40, 64, 256, pc, ps, xb, y_dtype=lb.F32, x_dtype=lb.SIGN1)
    assert e.value.status == lb.E_NULL
    with pytest.raises(lb.LowbitError) as e:  # the exact integer output takes unit scales
        lb.gemm(1, 40, 64, 256, pc, ps, xb, y_dtype=lb.I32, x_dtype=lb.SIGN1)
    assert e.value.status == lb.E_UNSUPPORTED
