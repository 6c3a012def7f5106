"""The C-ABI library loads on a machine without a GPU, exports every symbol
that include/lowbit.h declares, and rejects bad arguments synchronously
(with no HIP call) with the documented status codes."""
import ctypes
import os
import re

import pytest

from oracle import oracle as O
from ultra_bit_dit_amd import lowbit as lb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_symbols():
    text = open(os.path.join(ROOT, "include", "lowbit.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lowbit_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    syms = header_symbols()
    assert len(syms) >= 8
    L = ctypes.CDLL(lb.LIB_PATH)
    for s in syms:
        assert hasattr(L, s), s
    assert set(syms) == set(lb.EXPORTS)


def test_version_and_status_strings():
    assert lb.lib().lowbit_abi_version() == 3
    for st in range(-9, 1):
        assert isinstance(lb.status_str(st), str) and lb.status_str(st)


@pytest.mark.parametrize("fmt", [1, 2, 3])
@pytest.mark.parametrize("N,K", [(1, 128), (37, 384), (5120, 5120), (17408, 5120), (5120, 17408),
                                 (3072, 9216), (9216, 3072), (256, 1024)])
def test_packed_bytes_agree_with_oracle(fmt, N, K):
    assert lb.packed_bytes(fmt, N, K) == O.packed_bytes(fmt, N, K)


def test_packed_bytes_errors():
    L = lb.lib()
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.lowbit_packed_bytes(1, 16, 100, ctypes.byref(cb), ctypes.byref(sb)) == lb.E_SHAPE
    assert L.lowbit_packed_bytes(1, 0, 128, ctypes.byref(cb), ctypes.byref(sb)) == lb.E_SHAPE
    assert L.lowbit_packed_bytes(9, 16, 128, ctypes.byref(cb), ctypes.byref(sb)) == lb.E_UNSUPPORTED
    assert L.lowbit_packed_bytes(1, 16, 128, None, ctypes.byref(sb)) == lb.E_NULL
    assert L.lowbit_packed_bytes(1, 1 << 40, 1 << 30, ctypes.byref(cb), ctypes.byref(sb)) == lb.E_SHAPE


# fake, never dereferenced device addresses: validation fails before any HIP call
A16 = ctypes.c_void_p(0x10000)
A4 = ctypes.c_void_p(0x10004)
A1 = ctypes.c_void_p(0x10001)


def test_gemv_validation_without_gpu():
    L = lb.lib()
    f = L.lowbit_gemv
    assert f(1, 16, 128, None, A16, lb.BF16, A16, 1.0, lb.F32, A16, None) == lb.E_NULL
    assert f(1, 16, 100, A16, A16, lb.BF16, A16, 1.0, lb.F32, A16, None) == lb.E_SHAPE
    assert f(7, 16, 128, A16, A16, lb.BF16, A16, 1.0, lb.F32, A16, None) == lb.E_UNSUPPORTED
    assert f(1, 16, 128, A16, A16, 9, A16, 1.0, lb.F32, A16, None) == lb.E_UNSUPPORTED
    # I32 output needs an integer activation and unit scales
    assert f(1, 16, 128, A16, A16, lb.I8, A16, 1.0, lb.I32, A16, None) == lb.E_UNSUPPORTED
    assert f(1, 16, 128, A16, None, lb.BF16, A16, 1.0, lb.I32, A16, None) == lb.E_UNSUPPORTED
    # float output needs scales
    assert f(1, 16, 128, A16, None, lb.BF16, A16, 1.0, lb.F32, A16, None) == lb.E_NULL
    # sign activations only with binary weights
    assert f(2, 16, 128, A16, A16, lb.SIGN1, A16, 1.0, lb.F32, A16, None) == lb.E_UNSUPPORTED
    # the sign words of a row must fit the kernel's 48 KiB of LDS
    assert f(1, 16, 393216 + 128, A16, A16, lb.SIGN1, A16, 1.0, lb.F32, A16, None) == lb.E_SHAPE
    assert f(1, 16, 128, A4, A16, lb.BF16, A16, 1.0, lb.F32, A16, None) == lb.E_ALIGN
    assert f(1, 16, 128, A16, A16, lb.BF16, A4, 1.0, lb.F32, A16, None) == lb.E_ALIGN
    assert f(1, 16, 128, A16, A16, lb.BF16, A16, 1.0, lb.F32, A1, None) == lb.E_ALIGN


def test_gemm_pack_quant_validation_without_gpu():
    L = lb.lib()
    g = L.lowbit_gemm
    assert g(1, 0, 16, 128, A16, A16, lb.BF16, A16, None, lb.F32, A16, None) == lb.E_SHAPE
    assert g(1, 4, 16, 128, A16, A16, lb.F32, A16, None, lb.F32, A16, None) == lb.E_UNSUPPORTED
    assert g(1, 4, 16, 128, A16, A16, lb.I8, A16, None, lb.F32, A16, None) == lb.E_NULL
    assert g(1, 4, 16, 128, A16, A16, lb.BF16, A16, None, lb.F32, A4, None) == lb.E_ALIGN
    p = L.lowbit_pack
    assert p(1, 16, 128, None, A16, A16, A16, None, None) == lb.E_NULL
    assert p(1, 16, 256 + 64, A16, A16, A16, A16, None, None) == lb.E_SHAPE
    assert p(4, 16, 128, A16, A16, A16, A16, None, None) == lb.E_UNSUPPORTED
    assert p(1, 16, 128, A16, A16, A4, A16, None, None) == lb.E_ALIGN
    u = L.lowbit_unpack
    assert u(1, 16, 128, A16, A16, None, A16, None, None) == lb.E_NULL
    q = L.lowbit_quantize_act_i8
    assert q(0, 128, A16, A16, A16, None) == lb.E_SHAPE
    assert q(1, 128, None, A16, A16, None) == lb.E_NULL
    assert q(1, 128, A16, A16, A1, None) == lb.E_ALIGN


def test_quantizer_validation_without_gpu():
    f = lb.lib().lowbit_quantize_weights
    assert f(2, 4, 128, None, None, A16, A16, None) == lb.E_NULL
    assert f(7, 4, 128, A16, None, A16, A16, None) == lb.E_UNSUPPORTED
    assert f(2, 4, 200, A16, None, A16, A16, None) == lb.E_SHAPE
    # 16-byte loads of weights and signs, 16-byte stores of codes
    assert f(2, 4, 128, A4, None, A16, A16, None) == lb.E_ALIGN
    assert f(2, 4, 128, A16, A4, A16, A16, None) == lb.E_ALIGN
    assert f(2, 4, 128, A16, None, A4, A16, None) == lb.E_ALIGN
    assert f(2, 4, 128, A16, None, A16, A1, None) == lb.E_ALIGN


def test_workspace_bytes_contract():
    """lowbit_workspace_bytes is host-only: argument errors, the F32 rule of
    lowbit_gemm, and sizes that grow with the product (no GPU needed)."""
    L = lb.lib()
    b = ctypes.c_size_t(7)
    assert L.lowbit_workspace_bytes(1, 1, 16, 128, lb.BF16, None) == lb.E_NULL
    assert L.lowbit_workspace_bytes(9, 1, 16, 128, lb.BF16, ctypes.byref(b)) == lb.E_UNSUPPORTED
    assert b.value == 0
    assert L.lowbit_workspace_bytes(1, 1, 16, 128, 9, ctypes.byref(b)) == lb.E_UNSUPPORTED
    assert L.lowbit_workspace_bytes(1, 1, 16, 100, lb.BF16, ctypes.byref(b)) == lb.E_SHAPE
    assert L.lowbit_workspace_bytes(1, 0, 16, 128, lb.BF16, ctypes.byref(b)) == lb.E_SHAPE
    # lowbit_gemm takes no fp32 activations for M > 1
    assert L.lowbit_workspace_bytes(2, 2, 16, 128, lb.F32, ctypes.byref(b)) == lb.E_UNSUPPORTED
    for fmt in (1, 2, 3):
        for xd in (lb.BF16, lb.I8, lb.SIGN1):
            for M in (1, 4, 64, 512):
                v = lb.workspace_bytes(fmt, M, 5120, 5120, xd)
                assert v >= 0
                assert lb.workspace_bytes(fmt, M, 5120, 5120 * 4, xd) >= v
        assert lb.workspace_bytes(fmt, 1, 5120, 5120, lb.F32) > 0


def test_chain_del_at_finalization_does_nothing():
    """Chain.__del__ leaves the chain alone while the interpreter shuts down
    (the HIP runtime may be gone then)."""
    import sys
    c = lb.Chain.__new__(lb.Chain)
    c._h = ctypes.c_void_p(0x1234)  # never passed to the library here
    c._keep = []
    real = sys.is_finalizing
    try:
        sys.is_finalizing = lambda: True
        c.__del__()
    finally:
        sys.is_finalizing = real
    assert c._h.value == 0x1234
    c._h = None


def test_gemv_noalloc_validation_without_gpu():
    """The allocation-free GEMV checks its arguments as lowbit_gemv does and
    rejects products that need more than its static scratch before any HIP
    call."""
    L = lb.lib()
    f = L.lowbit_gemv_noalloc
    assert f(1, 16, 128, None, A16, lb.BF16, A16, 1.0, lb.F32, A16, None) == lb.E_NULL
    assert f(1, 16, 100, A16, A16, lb.BF16, A16, 1.0, lb.F32, A16, None) == lb.E_SHAPE
    assert f(7, 16, 128, A16, A16, lb.BF16, A16, 1.0, lb.F32, A16, None) == lb.E_UNSUPPORTED
    assert f(2, 16, 128, A16, A16, lb.SIGN1, A16, 1.0, lb.F32, A16, None) == lb.E_UNSUPPORTED
    assert f(1, 16, 128, A16, A16, lb.BF16, A16, 1.0, lb.F32, A1, None) == lb.E_ALIGN
    for fmt in (1, 2, 3):
        N, K = 1 << 17, 1 << 16
        assert lb.workspace_bytes(fmt, 1, N, K, lb.BF16) > 4 << 20
        assert f(fmt, N, K, A16, A16, lb.BF16, A16, 1.0, lb.F32, A16, None) == lb.E_TOO_LARGE
    assert "scratch" in lb.status_str(lb.E_TOO_LARGE)
