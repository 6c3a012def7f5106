"""Pins for the oracle's data-free weight quantizer (signed Hadamard rotation
per 128-group, absmean fp16 scale, rounding to binary / ternary codes; the
rotation and the per-128 FP16 scale come from the method list of the
paragraph "工作原理" of the page "我开源了 OpenBonsai：把你自己的 BF16 模型与微调
压缩成约 2 GB 的三值 GGUF").  None of these compares the oracle with itself: the
fp16 encoder against numpy's correctly rounded float16, the rotation against
scipy's Sylvester Hadamard matrix, the scale against a numerical L2
minimisation, and hand-worked groups from tests/golden."""
import json
import os

import numpy as np
import pytest
import scipy.linalg
import scipy.optimize

import synth
from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "weight_quantizer_handworked.json")


def expand(runs):
    return np.concatenate([np.full(c, v) for c, v in runs])


def test_f64_to_f16_matches_numpy():
    rng = np.random.default_rng(1)
    xs = np.concatenate([
        rng.normal(0, 1, 4000), rng.normal(0, 1e-5, 2000), rng.normal(0, 3e4, 1000),
        [0.0, -0.0, 65504.0, 65519.99, 65520.0, 70000.0, -65520.0, 2.0 ** -24, 2.0 ** -25,
         3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1.0 + 2.0 ** -11,
         1.0 + 3 * 2.0 ** -11, 0.1, 1.0 / 3.0]])
    for x in xs:
        with np.errstate(over="ignore"):
            want = np.array([x], np.float64).astype(np.float16).view(np.uint16)[0]
        assert O.f64_to_f16(x) == want, x


def test_handworked_groups_without_rotation():
    g = json.load(open(GOLDEN))["groups"]
    W = np.stack([expand(e["runs"]) for e in g]).astype(np.float32)
    Wb = synth.f32_to_bf16_bits(W)
    assert np.array_equal(synth.bf16_bits_to_f32(Wb), W)  # exact in bf16
    for fmt, key in ((2, "ternary"), (3, "ternary"), (1, "binary")):
        codes, scales = O.quantize_weights(fmt, Wb, None)
        for r, e in enumerate(g):
            assert np.array_equal(codes[r], expand(e[key]).astype(np.int8)), (fmt, r)
            assert scales[r, 0] == np.float16(e["scale"]).view(np.uint16), (fmt, r)


def test_binary_scale_is_the_l2_optimum():
    """Without rotation the binary scale is argmin_s sum (w - s sign(w))^2
    (= mean |w|), found here by numerical minimisation, rounded to fp16."""
    Wb = synth.normal_bf16(7, 1, 6, 256)
    W = synth.bf16_bits_to_f32(Wb).astype(np.float64)
    codes, scales = O.quantize_weights(1, Wb, None)
    assert np.array_equal(codes, np.where(W < 0, -1, 1).astype(np.int8))
    for n in range(6):
        for g in range(2):
            w = W[n, 128 * g:128 * (g + 1)]
            sg = np.where(w < 0, -1.0, 1.0)
            best = scipy.optimize.minimize_scalar(lambda s: np.sum((w - s * sg) ** 2),
                                                  bounds=(0, 10), method="bounded",
                                                  options={"xatol": 1e-12}).x
            s16 = np.float16(best)
            got = scales[n, g].view(np.float16)
            assert abs(float(got) - float(s16)) <= float(np.spacing(s16)), (n, g)


def hadamard_rotate(W, signs):
    """Textbook reference: per 128-block, W diag(d) H / sqrt(128) with scipy's
    Sylvester Hadamard matrix."""
    H = scipy.linalg.hadamard(128).astype(np.float64)
    N, K = W.shape
    out = np.empty_like(W)
    for g in range(K // 128):
        blk = W[:, 128 * g:128 * (g + 1)] * signs[128 * g:128 * (g + 1)]
        out[:, 128 * g:128 * (g + 1)] = blk @ H / np.sqrt(128.0)
    return out


def signs_for(K, seed=3):
    return np.where(np.random.default_rng(seed).random(K) < 0.5, -1, 1).astype(np.int8)


def test_rotation_is_the_signed_hadamard_transform():
    Wb = synth.normal_bf16(7, 2, 5, 384)
    W = synth.bf16_bits_to_f32(Wb).astype(np.float64)
    d = signs_for(384)
    T = O.rotate_rows(Wb, d)
    ref = hadamard_rotate(W, d.astype(np.float64))
    assert np.allclose(T, ref, rtol=0, atol=1e-12 * np.abs(W).max())
    # orthonormal: energy per group preserved
    for g in range(3):
        e0 = np.sum(W[:, 128 * g:128 * (g + 1)] ** 2, axis=1)
        e1 = np.sum(T[:, 128 * g:128 * (g + 1)] ** 2, axis=1)
        assert np.allclose(e0, e1, rtol=1e-12)


def test_rotated_basis_vector_gives_walsh_codes():
    """A group holding one nonzero weight rotates to a constant-magnitude
    Walsh row: every rotated value is +-1/sqrt(128), the scale is fp16 of
    1/sqrt(128) and the ternary and binary codes are the row's signs."""
    H = scipy.linalg.hadamard(128)
    for j in (0, 1, 77, 127):
        w = np.zeros((1, 128), np.float32)
        w[0, j] = 1.0
        Wb = synth.f32_to_bf16_bits(w)
        d = np.ones(128, np.int8)
        for fmt in (1, 2):
            codes, scales = O.quantize_weights(fmt, Wb, d)
            assert np.array_equal(codes[0], H[:, j].astype(np.int8)), (fmt, j)
            assert scales[0, 0] == np.float16(1 / np.sqrt(128.0)).view(np.uint16)


def test_quantizer_invariants():
    Wb = synth.normal_bf16(7, 3, 8, 512)
    d = signs_for(512, 4)
    for fmt in (1, 2):
        c, s = O.quantize_weights(fmt, Wb, d)
        # negating the weights negates ternary codes (binary: except exact zeros)
        neg = Wb ^ np.uint16(0x8000)
        c2, s2 = O.quantize_weights(fmt, neg, d)
        assert np.array_equal(s, s2)
        if fmt == 2:
            assert np.array_equal(c2, -c)
        # flipping the sign vector on a group is the same as negating that group
        d2 = d.copy()
        d2[128:256] = -d2[128:256]
        c3, s3 = O.quantize_weights(fmt, Wb, d2)
        assert np.array_equal(s3, s)
        if fmt == 2:
            assert np.array_equal(c3[:, 128:256], -c[:, 128:256])
            assert np.array_equal(c3[:, :128], c[:, :128])
        # powers of two scale the fp16 scale exactly and leave the codes
        W4 = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(Wb) * 4.0)
        c4, s4 = O.quantize_weights(fmt, W4, d)
        assert np.array_equal(c4, c)
        assert np.array_equal(s4.view(np.float16).astype(np.float64),
                              s.view(np.float16).astype(np.float64) * 4.0)


def test_rotation_spreads_an_outlier():
    """The method's purpose: one large weight in a group dominates the
    unrotated absmean scale (most ternary codes become 0); after rotation the
    group's values all have similar magnitude and most codes are nonzero."""
    rng = np.random.default_rng(9)
    w = rng.normal(0, 0.02, (1, 128)).astype(np.float32)
    w[0, 5] = 40.0
    Wb = synth.f32_to_bf16_bits(w)
    c0, _ = O.quantize_weights(2, Wb, None)
    c1, _ = O.quantize_weights(2, Wb, signs_for(128, 5))
    assert np.count_nonzero(c0) <= 2
    assert np.count_nonzero(c1) >= 100
