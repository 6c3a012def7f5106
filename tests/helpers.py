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
