"""Shared helpers for the GPU parity tests (host side only)."""
import numpy as np

import synth
from oracle import oracle as O

SEED = 1000


def codes_for(fmt, seed, tid, N, K, rows=None):
    gen = synth.binary_codes if fmt == O.BINARY else synth.ternary_codes
    return gen(seed, tid, N, K, rows=rows)


def tolerance(absY, yref, bf16_out):
    """1e-3 * sum|w x| per output (fp32 out); plus 2^-8 |y| for bf16 out."""
    t = 1e-3 * absY
    if bf16_out:
        t = t + 2.0 ** -8 * np.abs(yref)
    return t


def assert_within(y, yref, absY, bf16_out=False, what=""):
    y = np.asarray(y, dtype=np.float64)
    tol = tolerance(absY, yref, bf16_out)
    err = np.abs(y - yref)
    bad = err > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} outputs out of tolerance; first at {tuple(i)}: "
                             f"got {y[tuple(i)]!r} want {yref[tuple(i)]!r} tol {tol[tuple(i)]!r}")
    return float((err / np.maximum(tol, 1e-300)).max())


def silu_mul_tolerance(gref, uref, absG, absU, zref, bf16_out):
    """Bound on |z_gpu - z_ref| for z = silu(g) u when g and u each carry the
    product tolerance t = 1e-3 sum|w x|: |silu'| <= 1.1 and |silu''| <= 0.5,
    so |dz| <= 1.1 |u| tg + |silu(g)| tu + tg tu + 0.5 tg^2 (|u| + tu), plus
    fp32 evaluation (1e-6 |z|) and, for bf16 outputs, one rounding (2^-8 |z|)."""
    tg, tu = 1e-3 * absG, 1e-3 * absU
    sg = np.abs(O.silu_mul(gref, np.ones_like(gref)))
    tol = 1.1 * np.abs(uref) * tg + sg * tu + tg * tu + 0.5 * tg * tg * (np.abs(uref) + tu)
    tol += 1e-6 * np.abs(zref) + 1e-30
    if bf16_out:
        tol += 2.0 ** -8 * np.abs(zref)
    return tol


def to_np(t):
    """fp64 values of a float32 or bfloat16 device vector."""
    import torch

    if t.dtype == torch.bfloat16:
        bits = t.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)
