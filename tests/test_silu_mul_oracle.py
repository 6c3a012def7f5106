"""Pins for the oracle's gated FFN activation z = silu(g) * u (the input of
the down projection; the pages keep the base model's architecture, see the
oracle's header) and for the fused gate/up row order of the SiLU-mul
epilogue.  Each pin is a closed form or an identity of the sigmoid, not a
retyping of the oracle's formula: a dropped term, a wrong sign or a swapped
operand fails one of them."""
import math

import numpy as np

from oracle import oracle as O


def silu(v):
    return O.silu_mul(np.array([v]), np.array([1.0]))[0]


def test_closed_forms():
    # sigma(ln 3) = 3/4, sigma(-ln 3) = 1/4, sigma(0) = 1/2
    assert abs(silu(math.log(3.0)) - 0.75 * math.log(3.0)) < 1e-15
    assert abs(silu(-math.log(3.0)) + 0.25 * math.log(3.0)) < 1e-15
    assert silu(0.0) == 0.0
    # sigma(ln 7) = 7/8
    assert abs(silu(math.log(7.0)) - 0.875 * math.log(7.0)) < 1e-15


def test_odd_part_identity():
    # silu(v) - silu(-v) = v sigma(v) + v (1 - sigma(v)) = v for every v
    rng = np.random.default_rng(5)
    v = rng.normal(0, 4, 2000)
    one = np.ones_like(v)
    d = O.silu_mul(v, one) - O.silu_mul(-v, one)
    assert np.max(np.abs(d - v)) < 1e-12 * (1 + np.max(np.abs(v)))


def test_limits_and_product():
    # silu(v) -> v for large v, -> 0 (from below) for very negative v
    assert abs(silu(40.0) - 40.0) < 1e-12
    assert -1e-15 < silu(-40.0) < 0.0
    # the product is linear in u and symmetric in nothing else: silu(g) * u
    rng = np.random.default_rng(6)
    g, u = rng.normal(0, 2, 500), rng.normal(0, 2, 500)
    z = O.silu_mul(g, u)
    zu1 = O.silu_mul(g, np.ones_like(g))
    assert np.max(np.abs(z - zu1 * u)) < 1e-13
    # swapping the operands changes the result (catches a transposed call)
    assert np.max(np.abs(O.silu_mul(u, g) - z)) > 0.1


def test_fused_row_order_handworked():
    # F = 16 gate rows and 16 up rows, rows tagged by value
    gate = np.arange(16)[:, None] * np.ones((1, 3), int)
    up = 100 + np.arange(16)[:, None] * np.ones((1, 3), int)
    fused = O.fuse_gate_up(gate, up)
    want = [0, 1, 2, 3, 4, 5, 6, 7, 100, 101, 102, 103, 104, 105, 106, 107,
            8, 9, 10, 11, 12, 13, 14, 15, 108, 109, 110, 111, 112, 113, 114, 115]
    assert fused[:, 0].tolist() == want
    g2, u2 = O.split_fused(fused[:, 0])
    assert g2.tolist() == list(range(16)) and u2.tolist() == list(range(100, 116))


def test_fused_product_splits_into_gate_and_up():
    # the fused matrix's product, split back, is the two separate products
    rng = np.random.default_rng(7)
    F, K = 32, 256
    cg = rng.integers(-1, 2, (F, K)).astype(np.int8)
    cu = rng.integers(-1, 2, (F, K)).astype(np.int8)
    sg = np.full((F, K // 128), 0x3C00, np.uint16)  # fp16 1.0
    su = np.full((F, K // 128), 0x4000, np.uint16)  # fp16 2.0
    x = rng.normal(0, 1, (1, K)).astype(np.float32)
    yf = O.matmul(O.fuse_gate_up(cg, cu), O.fuse_gate_up(sg, su), O.X_F32, x, with_abs=False)
    g, u = O.split_fused(yf.reshape(-1))
    yg = O.matmul(cg, sg, O.X_F32, x, with_abs=False).reshape(-1)
    yu = O.matmul(cu, su, O.X_F32, x, with_abs=False).reshape(-1)
    assert np.array_equal(g, yg) and np.array_equal(u, yu)
    assert np.allclose(yu, 2 * (cu.astype(np.float64) @ x[0].astype(np.float64)))
