"""Thin ctypes binding of liblowbit (include/lowbit.h).

Argument marshalling only: torch tensors are passed as device pointers with
the current HIP stream; every step runs in the library's HIP kernels.  The
library must be built first (``python -m ultra_bit_dit_amd.build``); there is
no fallback.
"""
import ctypes
import os
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "liblowbit.so")

OK, E_NULL, E_SHAPE, E_ALIGN, E_UNSUPPORTED, E_BADCODE, E_HIP, E_NOMEM = 0, -1, -2, -3, -4, -5, -6, -7
E_TOO_LARGE = -8
BINARY, TERNARY_2BIT, TERNARY_BASE3 = 1, 2, 3
F32, BF16, I8, SIGN1, I32 = 1, 2, 3, 4, 5
EPI_NONE, EPI_SILU_MUL = 0, 1

# every symbol the public header declares
EXPORTS = ("lowbit_abi_version", "lowbit_status_str", "lowbit_packed_bytes", "lowbit_pack",
           "lowbit_unpack", "lowbit_quantize_act_i8", "lowbit_gemv", "lowbit_gemm",
           "lowbit_gemv_noalloc", "lowbit_workspace_bytes", "lowbit_reserve_workspace", "lowbit_release_workspaces",
           "lowbit_chain_create", "lowbit_chain_create_rows", "lowbit_chain_run", "lowbit_chain_status",
           "lowbit_chain_destroy",
           "lowbit_hbm_read_probe", "lowbit_quantize_weights", "lowbit_rotate_act")


class GemvStage(ctypes.Structure):
    """lowbit_gemv_stage"""
    _fields_ = [("fmt", ctypes.c_int), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("pcodes", ctypes.c_void_p), ("pscales", ctypes.c_void_p),
                ("x", ctypes.c_void_p), ("y", ctypes.c_void_p), ("wait_prev", ctypes.c_int),
                ("epilogue", ctypes.c_int)]


class LowbitError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn}: {status_str(status)} ({status})")
        self.status = status


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"liblowbit is not built ({LIB_PATH} missing); "
                               "run `python -m ultra_bit_dit_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.lowbit_abi_version.restype = i32
        L.lowbit_status_str.argtypes = [i32]
        L.lowbit_status_str.restype = ctypes.c_char_p
        L.lowbit_packed_bytes.argtypes = [i32, i64, i64, ctypes.POINTER(ctypes.c_size_t),
                                          ctypes.POINTER(ctypes.c_size_t)]
        L.lowbit_pack.argtypes = [i32, i64, i64, vp, vp, vp, vp, vp, vp]
        L.lowbit_unpack.argtypes = [i32, i64, i64, vp, vp, vp, vp, vp, vp]
        L.lowbit_quantize_act_i8.argtypes = [i64, i64, vp, vp, vp, vp]
        L.lowbit_gemv.argtypes = [i32, i64, i64, vp, vp, i32, vp, ctypes.c_float, i32, vp, vp]
        L.lowbit_gemv_noalloc.argtypes = [i32, i64, i64, vp, vp, i32, vp, ctypes.c_float, i32, vp, vp]
        L.lowbit_gemm.argtypes = [i32, i64, i64, i64, vp, vp, i32, vp, vp, i32, vp, vp]
        L.lowbit_workspace_bytes.argtypes = [i32, i64, i64, i64, i32, ctypes.POINTER(ctypes.c_size_t)]
        L.lowbit_reserve_workspace.argtypes = [ctypes.c_size_t, vp]
        L.lowbit_release_workspaces.argtypes = []
        L.lowbit_chain_create.argtypes = [i32, ctypes.POINTER(GemvStage), i32, i32,
                                          ctypes.POINTER(vp)]
        L.lowbit_chain_create_rows.argtypes = [i32, ctypes.POINTER(GemvStage), i64, i32, i32,
                                               ctypes.POINTER(vp)]
        L.lowbit_chain_run.argtypes = [vp, vp]
        L.lowbit_chain_status.argtypes = [vp, ctypes.POINTER(i32)]
        L.lowbit_chain_destroy.argtypes = [vp]
        L.lowbit_hbm_read_probe.argtypes = [vp, i64, vp, vp]
        L.lowbit_quantize_weights.argtypes = [i32, i64, i64, vp, vp, vp, vp, vp]
        L.lowbit_rotate_act.argtypes = [i64, i64, vp, vp, vp, vp]
        for name in EXPORTS[2:]:
            getattr(L, name).restype = i32
        _lib = L
    return _lib


def status_str(status):
    return lib().lowbit_status_str(int(status)).decode()


def _check(fn, status):
    if status != OK:
        raise LowbitError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def packed_bytes(fmt, N, K):
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    _check("lowbit_packed_bytes", lib().lowbit_packed_bytes(fmt, N, K, ctypes.byref(cb), ctypes.byref(sb)))
    return cb.value, sb.value


def empty_packed(fmt, N, K, device="cuda"):
    import torch
    cb, sb = packed_bytes(fmt, N, K)
    return (torch.empty(cb, dtype=torch.uint8, device=device),
            torch.empty(sb // 2, dtype=torch.int16, device=device))


def pack(fmt, codes, scales, pcodes=None, pscales=None, bad=None, stream=None):
    """codes int8 [N][K], scales fp16 (or int16 bits) [N][K/128] -> packed tensors."""
    N, K = codes.shape
    if pcodes is None:
        pcodes, pscales = empty_packed(fmt, N, K, codes.device)
    _check("lowbit_pack", lib().lowbit_pack(fmt, N, K, _ptr(codes), _ptr(scales), _ptr(pcodes),
                                            _ptr(pscales), _ptr(bad), _stream(stream)))
    return pcodes, pscales


def unpack(fmt, N, K, pcodes, pscales, bad=None, stream=None):
    import torch
    codes = torch.empty((N, K), dtype=torch.int8, device=pcodes.device)
    scales = torch.empty((N, K // 128), dtype=torch.int16, device=pcodes.device)
    _check("lowbit_unpack", lib().lowbit_unpack(fmt, N, K, _ptr(pcodes), _ptr(pscales), _ptr(codes),
                                                _ptr(scales), _ptr(bad), _stream(stream)))
    return codes, scales


def quantize_act_i8(X, Q=None, s_x=None, stream=None):
    """bf16 X [M][K] -> (int8 Q [M][K], fp32 s_x [M]); Q and s_x may be given."""
    import torch
    M, K = X.shape
    if Q is None:
        Q = torch.empty((M, K), dtype=torch.int8, device=X.device)
    if s_x is None:
        s_x = torch.empty(M, dtype=torch.float32, device=X.device)
    sx = s_x
    _check("lowbit_quantize_act_i8", lib().lowbit_quantize_act_i8(M, K, _ptr(X), _ptr(Q), _ptr(sx),
                                                                  _stream(stream)))
    return Q, sx


def _xdt(x, x_dtype):
    import torch
    if x_dtype is not None:
        return x_dtype
    return {torch.float32: F32, torch.bfloat16: BF16, torch.int8: I8, torch.uint8: SIGN1}[x.dtype]


def _ytorch(y_dtype):
    import torch
    return {F32: torch.float32, BF16: torch.bfloat16, I32: torch.int32}[y_dtype]


def gemv(fmt, N, K, pcodes, pscales, x, x_scale=1.0, y_dtype=F32, y=None, x_dtype=None,
         stream=None):
    """y[n] = sum_k W[n][k] x[k] (see lowbit_gemv)."""
    import torch
    if y is None:
        y = torch.empty(N, dtype=_ytorch(y_dtype), device=pcodes.device)
    _check("lowbit_gemv", lib().lowbit_gemv(fmt, N, K, _ptr(pcodes), _ptr(pscales), _xdt(x, x_dtype),
                                            _ptr(x), float(x_scale), y_dtype, _ptr(y), _stream(stream)))
    return y


def gemv_noalloc(fmt, N, K, pcodes, pscales, x, y, x_scale=1.0, y_dtype=F32, x_dtype=None,
                 stream=None):
    """lowbit_gemv through the allocation-free entry point (lowbit_gemv_noalloc):
    the caller passes the output y; nothing is allocated."""
    _check("lowbit_gemv_noalloc",
           lib().lowbit_gemv_noalloc(fmt, N, K, _ptr(pcodes), _ptr(pscales), _xdt(x, x_dtype),
                                     _ptr(x), float(x_scale), y_dtype, _ptr(y), _stream(stream)))
    return y


def gemm(fmt, M, N, K, pcodes, pscales, X, x_scales=None, y_dtype=F32, Y=None, x_dtype=None,
         stream=None):
    """Y[m][n] = sum_k W[n][k] X[m][k] (see lowbit_gemm)."""
    import torch
    if Y is None:
        Y = torch.empty((M, N), dtype=_ytorch(y_dtype), device=pcodes.device)
    _check("lowbit_gemm", lib().lowbit_gemm(fmt, M, N, K, _ptr(pcodes), _ptr(pscales), _xdt(X, x_dtype),
                                            _ptr(X), _ptr(x_scales), y_dtype, _ptr(Y), _stream(stream)))
    return Y


def workspace_bytes(fmt, M, N, K, x_dtype):
    """Workspace bytes lowbit_gemm (or lowbit_gemv, M = 1) needs for these arguments."""
    b = ctypes.c_size_t()
    _check("lowbit_workspace_bytes",
           lib().lowbit_workspace_bytes(fmt, M, N, K, x_dtype, ctypes.byref(b)))
    return b.value


def reserve_workspace(nbytes, stream=None):
    """Grow the stream's workspace to at least nbytes (do it before capturing a graph)."""
    _check("lowbit_reserve_workspace", lib().lowbit_reserve_workspace(int(nbytes), _stream(stream)))


def release_workspaces():
    """Wait for the devices, then free every workspace (no graph using one may be replayed after)."""
    _check("lowbit_release_workspaces", lib().lowbit_release_workspaces())


def quantize_weights(fmt, W, signs=None, stream=None):
    """Dense (codes int8 [N][K], scales int16 fp16 bits [N][K/128]) from bf16
    weights W [N][K] (see lowbit_quantize_weights); signs int8 [K] or None."""
    import torch
    N, K = W.shape
    codes = torch.empty((N, K), dtype=torch.int8, device=W.device)
    scales = torch.empty((N, K // 128), dtype=torch.int16, device=W.device)
    _check("lowbit_quantize_weights",
           lib().lowbit_quantize_weights(fmt, N, K, _ptr(W), _ptr(signs), _ptr(codes),
                                         _ptr(scales), _stream(stream)))
    return codes, scales


def rotate_act(X, signs, stream=None):
    """fp32 X_rot [M][K] from bf16 X [M][K] (see lowbit_rotate_act)."""
    import torch
    M, K = X.shape
    Xr = torch.empty((M, K), dtype=torch.float32, device=X.device)
    _check("lowbit_rotate_act",
           lib().lowbit_rotate_act(M, K, _ptr(X), _ptr(signs), _ptr(Xr), _stream(stream)))
    return Xr


def hbm_read_probe(src, out, stream=None):
    """Stream-read every byte of device tensor `src` once, XOR-folding the
    data into the int32 device tensor `out` (see lowbit_hbm_read_probe)."""
    nbytes = src.numel() * src.element_size()
    _check("lowbit_hbm_read_probe",
           lib().lowbit_hbm_read_probe(_ptr(src), nbytes, _ptr(out), _stream(stream)))


class Chain:
    """A planned chain of batch-1 products run as one persistent launch
    (lowbit_chain_*).  `stages` is a list of (fmt, N, K, pcodes, pscales, x, y,
    wait_prev[, epilogue]) with device tensors (epilogue EPI_NONE or
    EPI_SILU_MUL); rows > 1: every x is [rows][K] and every y [rows][N]
    (lowbit_chain_create_rows).  The tensors are kept referenced for the
    chain's lifetime."""

    def __init__(self, stages, x_dtype=BF16, y_dtype=F32, rows=1):
        self._keep = [t for st in stages for t in st[3:7]]
        arr = (GemvStage * len(stages))()
        for i, st in enumerate(stages):
            fmt, N, K, pc, ps, x, y, wait = st[:8]
            epi = st[8] if len(st) > 8 else EPI_NONE
            arr[i] = GemvStage(fmt, N, K, pc.data_ptr(), ps.data_ptr(), x.data_ptr(), y.data_ptr(),
                               int(wait), int(epi))
        h = ctypes.c_void_p()
        _check("lowbit_chain_create_rows",
               lib().lowbit_chain_create_rows(len(stages), arr, ctypes.c_int64(rows), x_dtype, y_dtype,
                                              ctypes.byref(h)))
        self._h = h

    def run(self, stream=None):
        _check("lowbit_chain_run", lib().lowbit_chain_run(self._h, _stream(stream)))

    def failed_waits(self):
        v = ctypes.c_int(0)
        _check("lowbit_chain_status", lib().lowbit_chain_status(self._h, ctypes.byref(v)))
        return v.value

    def close(self):
        if self._h:
            _check("lowbit_chain_destroy", lib().lowbit_chain_destroy(self._h))
            self._h = None
            self._keep = []

    def __del__(self):
        # at interpreter exit the HIP runtime may already be torn down: leave
        # the chain's memory to the process exit then
        if sys is None or sys.is_finalizing():
            return
        try:
            self.close()
        except Exception:
            pass
