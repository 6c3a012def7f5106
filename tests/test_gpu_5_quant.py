"""Data-free weight quantizer (lowbit_quantize_weights) and the matching
activation rotation (lowbit_rotate_act) on the GPU against the oracle: codes
and fp16 scales bit-exact (both sides decide in fp64), rotated activations
within the fp32 transform's rounding bound, and a rotated end-to-end
product."""
import numpy as np
import pytest
import torch

import synth
from oracle import oracle as O
from ultra_bit_dit_amd import lowbit as lb

from helpers import SEED, assert_within

pytestmark = pytest.mark.gpu


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def weights(N, K, tid, scale=0.02):
    W = synth.bf16_bits_to_f32(synth.normal_bf16(SEED, tid, N, K)) * scale
    if N > 3:
        W[1, 7] = 3.0          # an outlier
        W[2, 128:256] = 0.0    # a zero group
    return synth.f32_to_bf16_bits(W.astype(np.float32))


def signs_for(K, tid):
    return np.where(np.random.default_rng(tid).random(K) < 0.5, -1, 1).astype(np.int8)


@pytest.mark.parametrize("fmt", [1, 2, 3])
@pytest.mark.parametrize("rotate", [False, True])
@pytest.mark.parametrize("N,K", [(1, 128), (37, 384), (200, 1024), (64, 5120)])
def test_quantizer_matches_oracle(fmt, rotate, N, K):
    print(f"quantize fmt={fmt} rotate={rotate} N={N} K={K}", flush=True)
    Wb = weights(N, K, 301)
    d = signs_for(K, 302) if rotate else None
    codes, scales = lb.quantize_weights(fmt, dev(Wb.view(np.int16)), None if d is None else dev(d))
    torch.cuda.synchronize()
    c_ref, s_ref = O.quantize_weights(fmt, Wb, d)
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    assert np.array_equal(scales.cpu().numpy().view(np.uint16), s_ref)


def test_quantizer_full_matrix_sampled_rows():
    N, K = 5120, 5120
    print(f"quantize ternary N={N} K={K}", flush=True)
    Wb = weights(N, K, 311)
    d = signs_for(K, 312)
    codes, scales = lb.quantize_weights(2, dev(Wb.view(np.int16)), dev(d))
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(313).choice(N, size=24, replace=False))
    c_ref, s_ref = O.quantize_weights(2, Wb[rows], d)
    assert np.array_equal(codes.cpu().numpy()[rows], c_ref)
    assert np.array_equal(scales.cpu().numpy().view(np.uint16)[rows], s_ref)
    # the codes feed the packer unchanged
    pc, ps = lb.pack(2, codes, scales)
    torch.cuda.synchronize()


@pytest.mark.parametrize("M,K", [(1, 128), (3, 1024), (16, 5120)])
def test_rotate_act_within_fp32_bound(M, K):
    print(f"rotate act M={M} K={K}", flush=True)
    Xb = synth.normal_bf16(SEED, 321, M, K)
    d = signs_for(K, 322)
    Xr = lb.rotate_act(dev(Xb.view(np.int16)), dev(d))
    torch.cuda.synchronize()
    ref = O.rotate_rows(Xb, d)
    X = synth.bf16_bits_to_f32(Xb).astype(np.float64)
    # 7 butterfly levels and one scaling, each rounding once in fp32
    bound = np.repeat(np.abs(X).reshape(M, K // 128, 128).sum(axis=2), 128, axis=1) * 8 * 2.0 ** -24
    err = np.abs(Xr.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= bound)


def test_rotated_weights_and_activations_in_the_product():
    """Quantize with rotation, pack, multiply the rotated activations: the
    product equals the oracle's on the same codes, scales and activations."""
    N, K = 640, 1024
    Wb = weights(N, K, 331)
    d = signs_for(K, 332)
    codes, scales = lb.quantize_weights(2, dev(Wb.view(np.int16)), dev(d))
    pc, ps = lb.pack(2, codes, scales)
    xb = synth.normal_bf16(SEED, 333, 1, K)
    xr = lb.rotate_act(dev(xb.view(np.int16)), dev(d))
    y = lb.gemv(2, N, K, pc, ps, xr[0])
    torch.cuda.synchronize()
    yref, absY = O.matmul(codes.cpu().numpy(), scales.cpu().numpy().view(np.uint16), O.X_F32,
                          xr.cpu().numpy())
    assert_within(y.cpu().numpy()[None], yref, absY, what="rotated product")


def test_quantizer_rejects():
    W = torch.zeros((4, 200), dtype=torch.int16, device="cuda")
    with pytest.raises(lb.LowbitError) as e:
        lb.quantize_weights(2, W)
    assert e.value.status == lb.E_SHAPE
