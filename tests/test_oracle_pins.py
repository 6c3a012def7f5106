"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each test ties one oracle function to the pages (bit widths, add/sign-flip,
XOR + popcount), to closed forms, to an independent library routine (numpy's
fp16 decoding, integer matmul) or to brute force, so that a dropped term, a
wrong sign, a wrong index or a transposed operand fails somewhere.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import oracle as O


# ------------------------------------------------------------------ helpers

def f16_np(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_np(bits):
    with np.errstate(invalid="ignore"):
        return synth.bf16_bits_to_f32(bits).astype(np.float64)


def f16_bits(values):
    return np.asarray(values, dtype=np.float16).view(np.uint16)


def bf16_bits_exact(values):
    v = np.asarray(values, dtype=np.float32)
    b = synth.f32_to_bf16_bits(v)
    assert np.array_equal(bf16_np(b), v.astype(np.float64)), "value not exact in bf16"
    return b


# ------------------------------------------------------------- decoders

def test_f16_decoder_matches_numpy_exhaustive():
    ref = f16_np(np.arange(65536, dtype=np.uint16))
    got = np.array([O.f16_to_f64(h) for h in range(65536)])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    # a few values fixed by the IEEE binary16 definition
    assert O.f16_to_f64(0x3C00) == 1.0 and O.f16_to_f64(0xC000) == -2.0
    assert O.f16_to_f64(0x0001) == 2.0 ** -24 and O.f16_to_f64(0x7BFF) == 65504.0


def test_bf16_decoder_matches_float32_view_exhaustive():
    ref = bf16_np(np.arange(65536, dtype=np.uint16))
    got = np.array([O.bf16_to_f64(b) for b in range(65536)])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


# ----------------------------------------------------------- P1 bit widths

def test_bit_widths_match_pages(golden_dir):
    gold = json.load(open(os.path.join(golden_dir, "bit_widths.json")))
    grp, sbits = gold["group_size"], gold["scale_bits"]
    # the pages' figures decompose as payload bits + scale bits / group
    assert 1 + sbits / grp == gold["binary_bits_per_weight"]
    assert round(math.log2(3), 2) == gold["ternary_information_bits"]
    assert round(math.log2(3) + sbits / grp, 2) == gold["ternary_bits_per_weight"]
    for N, K in [(16, 1024), (5120, 5120), (17408, 5120), (3072, 9216)]:
        bits = {}
        for fmt in (O.BINARY, O.TERNARY_2BIT, O.TERNARY_BASE3):
            cb, sb = O.packed_bytes(fmt, N, K)
            bits[fmt] = Fraction(8 * (cb + sb), N * K)
        assert bits[O.BINARY] == Fraction(9, 8)  # exactly 1 + 16/128
        assert bits[O.TERNARY_2BIT] == Fraction(17, 8)
        assert bits[O.TERNARY_BASE3] == Fraction(7, 4)
        bound = math.log2(3) + sbits / grp
        assert float(bits[O.TERNARY_2BIT]) >= bound
        assert float(bits[O.TERNARY_BASE3]) >= bound


def test_packed_sizes_of_the_5120_matrix():
    # 5120 x 5120: 2-bit codes 5120*5120/4 bytes, base-3 26 bytes per 128-group
    assert O.packed_bytes(O.TERNARY_2BIT, 5120, 5120) == (6553600, 409600)
    assert O.packed_bytes(O.TERNARY_BASE3, 5120, 5120) == (5324800, 409600)
    assert O.packed_bytes(O.BINARY, 5120, 5120) == (3276800, 409600)
    with pytest.raises(ValueError):
        O.packed_bytes(O.BINARY, 16, 100)


# ------------------------------------------- dequantize-then-multiply (A1)

@pytest.mark.parametrize("M,N,K", [(1, 37, 256), (3, 16, 384), (2, 5, 1024)])
@pytest.mark.parametrize("ternary", [False, True])
def test_matmul_matches_numpy_dequant(M, N, K, ternary):
    G = K // 128
    codes = (synth.ternary_codes if ternary else synth.binary_codes)(11, 1, N, K)
    scales = synth.group_scales(11, 2, N, G)
    x = synth.normal_bf16(11, 3, M, K)
    W = f16_np(scales).repeat(128, axis=1) * codes.astype(np.float64)  # [N][K]
    X = bf16_np(x)
    ref = X @ W.T
    Y, A = O.matmul(codes, scales, O.X_BF16, x)
    assert Y.shape == (M, N)
    assert np.all(np.abs(Y - ref) <= 1e-12 * np.maximum(A, 1e-300))
    assert np.allclose(A, np.abs(X) @ np.abs(W).T, rtol=1e-12, atol=0)


def test_matmul_f32_and_scaled_i8_kinds():
    N, K = 9, 256
    codes = synth.ternary_codes(5, 1, N, K)
    scales = synth.group_scales(5, 2, N, 2)
    W = f16_np(scales).repeat(128, axis=1) * codes
    xf = synth.normal_f32(5, 3, 2, K)
    Y, _ = O.matmul(codes, scales, O.X_F32, xf)
    assert np.allclose(Y, xf.astype(np.float64) @ W.T, rtol=1e-12, atol=1e-12)
    q = np.random.default_rng(0).integers(-127, 128, size=(2, K)).astype(np.int8)
    sx = np.array([0.5, 0.03125], dtype=np.float32)
    Y, _ = O.matmul(codes, scales, O.X_I8, q, sx)
    ref = (q.astype(np.float64) * sx[:, None].astype(np.float64)) @ W.T
    assert np.allclose(Y, ref, rtol=1e-12, atol=1e-12)


def test_unit_scales_reduce_to_integer_matmul():
    N, K, M = 21, 512, 4
    codes = synth.ternary_codes(9, 1, N, K)
    q = np.random.default_rng(1).integers(-127, 128, size=(M, K)).astype(np.int8)
    Y, _ = O.matmul(codes, None, O.X_I8, q)
    ref = q.astype(np.int64) @ codes.astype(np.int64).T
    assert np.array_equal(Y, ref.astype(np.float64))


def test_rows_and_columns_not_transposed():
    # non-square, distinct shapes: W row n only meets x row m at Y[m][n]
    N, K = 3, 128
    codes = np.ones((N, K), dtype=np.int8)
    codes[1, :] = -1
    scales = f16_bits([[1.0], [2.0], [4.0]])
    x = bf16_bits_exact(np.tile(np.arange(1, 129, dtype=np.float32), (2, 1)) * np.array([[1.0], [0.5]], dtype=np.float32))
    Y, _ = O.matmul(codes, scales, O.X_BF16, x)
    s = sum(range(1, 129))
    assert np.array_equal(Y, np.array([[s, -2 * s, 4 * s], [s / 2, -s, 2 * s]], dtype=np.float64))


# ------------------------------------------------- P2 add / sign flip

def _dyadic_case(rng, M, N, K, ternary):
    G = K // 128
    codes = (rng.integers(-1, 2, size=(N, K)) if ternary else 1 - 2 * rng.integers(0, 2, size=(N, K))).astype(np.int8)
    scales = f16_bits(2.0 ** rng.integers(-7, -2, size=(N, G)))
    x = bf16_bits_exact(rng.integers(-8, 9, size=(M, K)).astype(np.float32))
    return codes, scales, x


@pytest.mark.parametrize("ternary", [False, True])
def test_addflip_equals_multiply_exactly_on_dyadic_inputs(ternary):
    rng = np.random.default_rng(7)
    M, N, K = 2, 13, 640
    codes, scales, x = _dyadic_case(rng, M, N, K, ternary)
    Y = O.matmul(codes, scales, O.X_BF16, x, with_abs=False)
    Y2 = O.matmul_addflip(codes, scales, O.X_BF16, x)
    assert np.array_equal(Y, Y2)
    # exact integer arithmetic: scales are 2^e with e in [-7,-3]
    s_int = (f16_np(scales) * 128).astype(np.int64)  # exact
    xv = bf16_np(x).astype(np.int64)
    ref = np.zeros((M, N), dtype=np.int64)
    for g in range(K // 128):
        sl = slice(128 * g, 128 * g + 128)
        ref += (xv[:, sl] @ codes[:, sl].astype(np.int64).T) * s_int[:, g][None, :]
    assert np.array_equal(Y * 128, ref.astype(np.float64))


# ------------------------------------------------- P3 XOR + popcount

def test_xor_popcount_identity_bruteforce():
    for L in range(1, 11):
        for a in range(1 << L):
            for b in range(1 << L):
                dot = sum((-1) ** ((a >> i) & 1) * (-1) ** ((b >> i) & 1) for i in range(L))
                assert dot == L - 2 * bin(a ^ b).count("1")


def test_xor_popcount_identity_random_128bit():
    rng = np.random.default_rng(3)
    a = rng.integers(0, 2, size=(100000, 128), dtype=np.int64)
    b = rng.integers(0, 2, size=(100000, 128), dtype=np.int64)
    dot = ((1 - 2 * a) * (1 - 2 * b)).sum(axis=1)
    assert np.array_equal(dot, 128 - 2 * (a ^ b).sum(axis=1))


def test_oracle_xor_popcount_matches_dense_sign_product():
    M, N, K = 3, 17, 384
    codes = synth.binary_codes(21, 1, N, K)
    scales = synth.group_scales(21, 2, N, 3)
    xb = synth.sign_bits(21, 3, M, K)
    alpha = np.array([1.0, 0.5, 3.0], dtype=np.float32)
    Y, D = O.xor_popcount(codes, scales, xb, alpha)
    # independent: unpack bits with numpy, integer dot products
    bits = np.unpackbits(xb, axis=1, bitorder="little").astype(np.int64)
    xs = 1 - 2 * bits
    assert np.array_equal(D, xs @ codes.astype(np.int64).T)
    Yd = O.matmul(codes, scales, O.X_SIGN1, xb, alpha, with_abs=False)
    assert np.allclose(Y, Yd, rtol=1e-14, atol=0)
    Yu, Du = O.xor_popcount(codes, None, xb)
    assert np.array_equal(Yu, D.astype(np.float64))


# ------------------------------------------------- P4 all-+1 groups

def test_all_plus_and_all_minus_groups_closed_form():
    K = 512
    x = bf16_bits_exact(((np.arange(2 * K) % 61 + 1) * 0.25).astype(np.float32).reshape(2, K))
    xv = bf16_np(x)
    codes = np.ones((4, K), dtype=np.int8)
    codes[1, 128:256] = -1      # group 1 flipped
    codes[2, :] = -1            # every group flipped
    codes[3, 384:] = 0          # ternary row with a zero group
    scales = f16_bits(np.array([[0.5, 0.25, 0.125, 2.0]] * 4))
    Y, A = O.matmul(codes, scales, O.X_BF16, x)
    s = f16_np(scales)[0]
    gsum = np.stack([xv[:, 128 * g:128 * g + 128].sum(axis=1) for g in range(4)], axis=1)
    r0 = gsum @ s
    r1 = r0 - 2 * s[1] * gsum[:, 1]
    assert np.array_equal(Y[:, 0], r0) and np.array_equal(Y[:, 1], r1)
    assert np.array_equal(Y[:, 2], -r0)
    assert np.array_equal(Y[:, 3], r0 - s[3] * gsum[:, 3])
    # positive x: sum |w x| equals |y| on the all-+1 row
    assert np.array_equal(A[:, 0], Y[:, 0])


# ------------------------------------------------- P6 invariants

def test_invariants_linearity_negation_permutation_zero():
    rng = np.random.default_rng(5)
    M, N, K = 2, 11, 384
    codes, scales, x = _dyadic_case(rng, M, N, K, True)
    _, _, z = _dyadic_case(rng, M, N, K, True)
    y = lambda c, s, xx: O.matmul(c, s, O.X_BF16, xx, with_abs=False)
    xv, zv = bf16_np(x), bf16_np(z)
    comb = bf16_bits_exact((2 * xv - zv).astype(np.float32))
    assert np.array_equal(y(codes, scales, comb), 2 * y(codes, scales, x) - y(codes, scales, z))
    assert np.array_equal(y((-codes).astype(np.int8), scales, x), -y(codes, scales, x))
    perm = np.concatenate([128 * g + rng.permutation(128) for g in range(K // 128)])
    assert np.array_equal(y(codes[:, perm], scales, x[:, perm]), y(codes, scales, x))
    assert np.all(y(codes, np.zeros_like(scales), x) == 0)
    assert np.all(y(codes, scales, np.zeros_like(x)) == 0)


# ------------------------------------------------- P7 int8 path

def test_group_int_sums_match_numpy_and_bounds():
    rng = np.random.default_rng(8)
    M, N, K = 3, 10, 640
    codes = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    Q = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    A = O.group_int_sums(codes, Q)
    ref = np.einsum("mgk,ngk->mng", Q.astype(np.int64).reshape(M, -1, 128),
                    codes.astype(np.int64).reshape(N, -1, 128))
    assert np.array_equal(A, ref)
    # extremes: all +1 codes against all 127 activations
    A2 = O.group_int_sums(np.ones((1, 128), np.int8), np.full((1, 128), 127, np.int8))
    assert A2[0, 0, 0] == 16256 and 17408 * 127 == 2210816 < 2 ** 31


def test_quantizer_golden_ties(golden_dir):
    gold = json.load(open(os.path.join(golden_dir, "quantize_ties.json")))
    for row in gold["rows"]:
        x = bf16_bits_exact(np.array([row["x"]], dtype=np.float32))
        q, sx = O.quantize_act_i8(x)
        assert q[0].tolist() == row["q"]
        assert float(sx[0]) == row["s_x"]


def test_quantizer_matches_independent_numpy_fp32():
    x = synth.normal_bf16(17, 1, 8, 1000)
    x[3] = 0  # an all-zero row
    q, sx = O.quantize_act_i8(x)
    v = synth.bf16_bits_to_f32(x)
    a = np.abs(v).max(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        inv = np.float32(127.0) / a
        ref = np.clip(np.rint(v * inv[:, None]), -127, 127)
    ref[a == 0] = 0
    assert np.array_equal(q, ref.astype(np.int8))
    assert np.array_equal(sx, np.where(a == 0, np.float32(0), a / np.float32(127.0)).astype(np.float32))


# ------------------------------------------------- P5 formats agree

def test_same_sign_codes_in_three_formats_give_same_result():
    N, K = 19, 1024
    codes = synth.binary_codes(31, 1, N, K)
    scales = synth.group_scales(31, 2, N, 8)
    x = synth.normal_bf16(31, 3, 1, K)
    ys = []
    for fmt in (O.BINARY, O.TERNARY_2BIT, O.TERNARY_BASE3):
        pc, ps, bad = O.pack(fmt, codes, scales)
        assert bad == 0
        c2, s2, bad2 = O.unpack(fmt, N, K, pc, ps)
        assert bad2 == 0
        ys.append(O.matmul(c2, s2, O.X_BF16, x, with_abs=False))
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[2])
