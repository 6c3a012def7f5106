"""ctypes binding of the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's
CPU-baseline leg import this module.  The HIP library never does.
"""
import ctypes
import os

import numpy as np

from . import build as _build

BINARY, TERNARY_2BIT, TERNARY_BASE3 = 1, 2, 3
X_F32, X_BF16, X_I8, X_SIGN1 = 1, 2, 3, 4

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        i64, vp, u16 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_uint16
        L.orc_f16_to_f64.argtypes = [u16]
        L.orc_f16_to_f64.restype = ctypes.c_double
        L.orc_bf16_to_f64.argtypes = [u16]
        L.orc_bf16_to_f64.restype = ctypes.c_double
        L.orc_packed_bytes.argtypes = [ctypes.c_int, i64, i64, ctypes.POINTER(ctypes.c_size_t),
                                       ctypes.POINTER(ctypes.c_size_t)]
        L.orc_pack.argtypes = [ctypes.c_int, i64, i64, vp, vp, vp, vp]
        L.orc_pack.restype = i64
        L.orc_unpack.argtypes = [ctypes.c_int, i64, i64, vp, vp, vp, vp]
        L.orc_unpack.restype = i64
        L.orc_matmul.argtypes = [i64, i64, i64, vp, vp, ctypes.c_int, vp, vp, vp, vp]
        L.orc_matmul_addflip.argtypes = [i64, i64, i64, vp, vp, ctypes.c_int, vp, vp, vp]
        L.orc_group_int_sums.argtypes = [i64, i64, i64, vp, vp, vp]
        L.orc_xor_popcount.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, vp]
        L.orc_quantize_act_i8.argtypes = [i64, i64, vp, vp, vp]
        L.orc_f64_to_f16.argtypes = [ctypes.c_double]
        L.orc_f64_to_f16.restype = ctypes.c_uint16
        L.orc_quantize_weights.argtypes = [ctypes.c_int, i64, i64, vp, vp, vp, vp]
        L.orc_rotate_rows.argtypes = [i64, i64, vp, vp, vp]
        L.orc_silu_mul.argtypes = [i64, vp, vp, vp]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def f16_to_f64(h):
    return lib().orc_f16_to_f64(int(h))


def bf16_to_f64(b):
    return lib().orc_bf16_to_f64(int(b))


def packed_bytes(fmt, N, K):
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    rc = lib().orc_packed_bytes(fmt, N, K, ctypes.byref(cb), ctypes.byref(sb))
    if rc:
        raise ValueError(f"orc_packed_bytes failed: {rc}")
    return cb.value, sb.value


def pack(fmt, codes, scales):
    """Dense codes int8 [N][K] + fp16-bit scales uint16 [N][G] -> (pcodes uint8,
    pscales uint16, bad_count)."""
    codes = _c(codes, np.int8)
    scales = _c(scales, np.uint16)
    N, K = codes.shape
    cb, sb = packed_bytes(fmt, N, K)
    pc = np.empty(cb, dtype=np.uint8)
    ps = np.empty(sb // 2, dtype=np.uint16)
    bad = lib().orc_pack(fmt, N, K, _p(codes), _p(scales), _p(pc), _p(ps))
    if bad < 0:
        raise ValueError(f"orc_pack failed: {bad}")
    return pc, ps, int(bad)


def unpack(fmt, N, K, pcodes, pscales):
    pcodes = _c(pcodes, np.uint8)
    pscales = _c(pscales, np.uint16)
    codes = np.empty((N, K), dtype=np.int8)
    scales = np.empty((N, K // 128), dtype=np.uint16)
    bad = lib().orc_unpack(fmt, N, K, _p(pcodes), _p(pscales), _p(codes), _p(scales))
    if bad < 0:
        raise ValueError(f"orc_unpack failed: {bad}")
    return codes, scales, int(bad)


_XDT = {X_F32: np.float32, X_BF16: np.uint16, X_I8: np.int8, X_SIGN1: np.uint8}


def matmul(codes, scales, xkind, X, xs=None, with_abs=True):
    """fp64 Y [M][N] (and sum |w x| [M][N]) of X [M][K] against W [N][K]."""
    codes = _c(codes, np.int8)
    N, K = codes.shape
    X = _c(X, _XDT[xkind])
    M = X.shape[0]
    Y = np.empty((M, N), dtype=np.float64)
    A = np.empty((M, N), dtype=np.float64) if with_abs else None
    rc = lib().orc_matmul(M, N, K, _p(codes), _p(_c(scales, np.uint16)), xkind, _p(X),
                          _p(_c(xs, np.float32)), _p(Y), _p(A))
    if rc:
        raise ValueError(f"orc_matmul failed: {rc}")
    return (Y, A) if with_abs else Y


def matmul_addflip(codes, scales, xkind, X, xs=None):
    codes = _c(codes, np.int8)
    N, K = codes.shape
    X = _c(X, _XDT[xkind])
    M = X.shape[0]
    Y = np.empty((M, N), dtype=np.float64)
    rc = lib().orc_matmul_addflip(M, N, K, _p(codes), _p(_c(scales, np.uint16)), xkind, _p(X),
                                  _p(_c(xs, np.float32)), _p(Y))
    if rc:
        raise ValueError(f"orc_matmul_addflip failed: {rc}")
    return Y


def group_int_sums(codes, Q):
    codes = _c(codes, np.int8)
    Q = _c(Q, np.int8)
    N, K = codes.shape
    M = Q.shape[0]
    A = np.empty((M, N, K // 128), dtype=np.int64)
    rc = lib().orc_group_int_sums(M, N, K, _p(codes), _p(Q), _p(A))
    if rc:
        raise ValueError(f"orc_group_int_sums failed: {rc}")
    return A


def xor_popcount(codes, scales, xbits, alpha=None):
    codes = _c(codes, np.int8)
    xbits = _c(xbits, np.uint8)
    N, K = codes.shape
    M = xbits.shape[0]
    Y = np.empty((M, N), dtype=np.float64)
    D = np.empty((M, N), dtype=np.int64)
    rc = lib().orc_xor_popcount(M, N, K, _p(codes), _p(_c(scales, np.uint16)), _p(xbits),
                                _p(_c(alpha, np.float32)), _p(Y), _p(D))
    if rc:
        raise ValueError(f"orc_xor_popcount failed: {rc}")
    return Y, D


def quantize_act_i8(X_bf16):
    X = _c(X_bf16, np.uint16)
    M, K = X.shape
    Q = np.empty((M, K), dtype=np.int8)
    sx = np.empty(M, dtype=np.float32)
    rc = lib().orc_quantize_act_i8(M, K, _p(X), _p(Q), _p(sx))
    if rc:
        raise ValueError(f"orc_quantize_act_i8 failed: {rc}")
    return Q, sx


def f64_to_f16(x):
    return lib().orc_f64_to_f16(float(x))


def quantize_weights(fmt, W_bf16, signs=None):
    """Data-free quantizer: (codes int8 [N][K], scales fp16 bits [N][K/128])
    from bf16 bits W [N][K]; signs int8 [K] in {-1, +1} or None (no rotation)."""
    W = _c(W_bf16, np.uint16)
    N, K = W.shape
    codes = np.empty((N, K), dtype=np.int8)
    scales = np.empty((N, K // 128), dtype=np.uint16)
    rc = lib().orc_quantize_weights(fmt, N, K, _p(W), _p(_c(signs, np.int8)), _p(codes), _p(scales))
    if rc:
        raise ValueError(f"orc_quantize_weights failed: {rc}")
    return codes, scales


def rotate_rows(W_bf16, signs):
    """fp64 T [N][K]: the quantizer's per-group signed Hadamard rotation."""
    W = _c(W_bf16, np.uint16)
    N, K = W.shape
    T = np.empty((N, K), dtype=np.float64)
    rc = lib().orc_rotate_rows(N, K, _p(W), _p(_c(signs, np.int8)), _p(T))
    if rc:
        raise ValueError(f"orc_rotate_rows failed: {rc}")
    return T


def silu_mul(g, u):
    """fp64 z = silu(g) * u elementwise (orc_silu_mul)."""
    g = _c(g, np.float64).ravel()
    u = _c(u, np.float64).ravel()
    if g.shape != u.shape:
        raise ValueError("silu_mul: shapes differ")
    z = np.empty_like(g)
    rc = lib().orc_silu_mul(g.size, _p(g), _p(u), _p(z))
    if rc:
        raise ValueError(f"orc_silu_mul failed: {rc}")
    return z


def fuse_gate_up(gate_rows, up_rows):
    """Row order of a fused gate/up matrix for the SiLU-mul epilogue: within
    every 16-row block b, rows 0..7 are gate rows 8b..8b+7 and rows 8..15 the
    up rows 8b..8b+7.  Takes two [F][...] arrays (F % 8 == 0), returns the
    [2F][...] fused array."""
    g = np.asarray(gate_rows)
    u = np.asarray(up_rows)
    F = g.shape[0]
    if u.shape != g.shape or F % 8:
        raise ValueError("fuse_gate_up: gate and up must have the same shape, rows % 8 == 0")
    out = np.empty((2 * F,) + g.shape[1:], dtype=g.dtype)
    for b in range(F // 8):
        out[16 * b:16 * b + 8] = g[8 * b:8 * b + 8]
        out[16 * b + 8:16 * b + 16] = u[8 * b:8 * b + 8]
    return out


def split_fused(y):
    """Inverse of fuse_gate_up on a fused output vector: (gate [F], up [F])."""
    y = np.asarray(y)
    blocks = y.reshape(-1, 2, 8)
    return blocks[:, 0, :].reshape(-1), blocks[:, 1, :].reshape(-1)
