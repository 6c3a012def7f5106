"""Counter-based random inputs, defined once and implemented twice.

Definition (all arithmetic on unsigned 32-bit words):

    mix(x)   = lowbias32: x ^= x>>16; x *= 0x7feb352d; x ^= x>>15;
               x *= 0x846ca68b; x ^= x>>16            (mod 2^32)
    k1       = mix(seed)
    k2       = mix(k1 ^ tensor_id)
    r(i)     = mix(mix(i ^ k2) + k1)                  (i < 2^32)

From r:
    binary code     c = 1 - 2 * (r >> 31)               Bernoulli(0.5) signs
    ternary code    c = (r mod 3) - 1                    {-1,0,+1}, ~1/3 each
    group scale     u = (r >> 8) / 2^24,  v = 0.01 + 0.09*u  (two fp64 ops),
                    s = fp16(fp32(v)), both roundings to nearest even
    normal          u1 = ((r(2i) >> 8) + 1) / 2^24, u2 = (r(2i+1) >> 8) / 2^24,
                    z = sqrt(-2 ln u1) cos(2 pi u2) in fp64, then fp32, then
                    bf16 (nearest even) where bf16 is used
    sign bit        b = r >> 31
    raw word        w = r(i)   (packed binary codes: every bit is a fair sign)

The host side uses numpy; codes and scales also have a device side written
with torch integer / fp64 tensor operations (no HIP code), so that multi-GB
weight sets can be filled on the GPU while the oracle regenerates any row on
the host bit-for-bit.  The multiply is split in 16-bit halves so that every
intermediate fits in a signed 64-bit integer on either side.
"""
import numpy as np

M32 = 0xFFFFFFFF
_C1 = 0x7FEB352D
_C2 = 0x846CA68B


def _mul32_np(x, c):
    lo = (x * np.uint64(c & 0xFFFF)) & np.uint64(M32)
    hi = ((x * np.uint64(c >> 16)) & np.uint64(0xFFFF)) << np.uint64(16)
    return (lo + hi) & np.uint64(M32)


def _mix_np(x):
    x = x ^ (x >> np.uint64(16))
    x = _mul32_np(x, _C1)
    x = x ^ (x >> np.uint64(15))
    x = _mul32_np(x, _C2)
    x = x ^ (x >> np.uint64(16))
    return x


def _keys(seed, tensor_id):
    k1 = int(_mix_np(np.array([seed & M32], dtype=np.uint64))[0])
    k2 = int(_mix_np(np.array([(k1 ^ (tensor_id & M32)) & M32], dtype=np.uint64))[0])
    return k1, k2


def rand_u32(seed, tensor_id, idx):
    """r(i) for an array of indices (host, numpy uint64 result)."""
    idx = np.asarray(idx, dtype=np.uint64)
    if idx.size and int(idx.max()) > M32:
        raise ValueError("index beyond 2^32 for one tensor id")
    k1, k2 = _keys(seed, tensor_id)
    x = _mix_np(idx ^ np.uint64(k2))
    return _mix_np((x + np.uint64(k1)) & np.uint64(M32))


def _row_idx(rows, ncols):
    rows = np.asarray(rows, dtype=np.uint64)
    cols = np.arange(ncols, dtype=np.uint64)
    return rows[:, None] * np.uint64(ncols) + cols[None, :]


def binary_codes(seed, tensor_id, N, K, rows=None):
    """int8 [len(rows)][K] codes in {-1,+1} (rows defaults to all N rows)."""
    rows = np.arange(N) if rows is None else rows
    r = rand_u32(seed, tensor_id, _row_idx(rows, K))
    return (1 - 2 * (r >> np.uint64(31)).astype(np.int64)).astype(np.int8)


def ternary_codes(seed, tensor_id, N, K, rows=None):
    rows = np.arange(N) if rows is None else rows
    r = rand_u32(seed, tensor_id, _row_idx(rows, K))
    return ((r % np.uint64(3)).astype(np.int64) - 1).astype(np.int8)


def group_scales(seed, tensor_id, N, G, rows=None):
    """fp16 bit patterns (uint16) [len(rows)][G], values in [0.01, 0.1]."""
    rows = np.arange(N) if rows is None else rows
    r = rand_u32(seed, tensor_id, _row_idx(rows, G))
    u = (r >> np.uint64(8)).astype(np.float64) / float(1 << 24)
    t = 0.09 * u
    v = 0.01 + t
    return v.astype(np.float32).astype(np.float16).view(np.uint16)


def f32_to_bf16_bits(a):
    """Round fp32 to bfloat16, nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_f32(seed, tensor_id, M, K):
    """N(0,1) samples as fp32 [M][K] (Box-Muller in fp64)."""
    n = M * K
    i = np.arange(n, dtype=np.uint64)
    r1 = rand_u32(seed, tensor_id, 2 * i)
    r2 = rand_u32(seed, tensor_id, 2 * i + np.uint64(1))
    u1 = ((r1 >> np.uint64(8)).astype(np.float64) + 1.0) / float(1 << 24)
    u2 = (r2 >> np.uint64(8)).astype(np.float64) / float(1 << 24)
    z = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)
    return z.astype(np.float32).reshape(M, K)


def normal_bf16(seed, tensor_id, M, K):
    """N(0,1) samples rounded to bf16, as uint16 bit patterns [M][K]."""
    return f32_to_bf16_bits(normal_f32(seed, tensor_id, M, K))


def sign_bits(seed, tensor_id, M, K):
    """Random sign activations, packed LSB-first: uint8 [M][K/8]."""
    r = rand_u32(seed, tensor_id, _row_idx(np.arange(M), K))
    b = (r >> np.uint64(31)).astype(np.uint8).reshape(M, K // 8, 8)
    w = np.zeros((M, K // 8), dtype=np.uint8)
    for j in range(8):
        w |= (b[:, :, j] << j).astype(np.uint8)
    return w


# ----------------------------------------------------------- device (torch)

def _mul32_t(x, c):
    lo = (x * (c & 0xFFFF)) & M32
    hi = ((x * (c >> 16)) & 0xFFFF) << 16
    return (lo + hi) & M32


def _mix_t(x):
    x = x ^ (x >> 16)
    x = _mul32_t(x, _C1)
    x = x ^ (x >> 15)
    x = _mul32_t(x, _C2)
    x = x ^ (x >> 16)
    return x


def _rand_t(seed, tensor_id, idx):
    k1, k2 = _keys(seed, tensor_id)
    x = _mix_t(idx ^ k2)
    return _mix_t((x + k1) & M32)


def device_codes(fmt_ternary, seed, tensor_id, N, K, device, chunk_rows=4096):
    """Fill int8 [N][K] codes on `device` with torch ops (same values as the
    host generators).  fmt_ternary selects the ternary mapping."""
    import torch
    out = torch.empty((N, K), dtype=torch.int8, device=device)
    if N * K > (1 << 32):
        raise ValueError("tensor too large for one tensor id")
    cols = torch.arange(K, dtype=torch.int64, device=device)
    for r0 in range(0, N, chunk_rows):
        r1 = min(N, r0 + chunk_rows)
        rows = torch.arange(r0, r1, dtype=torch.int64, device=device)
        idx = rows[:, None] * K + cols[None, :]
        r = _rand_t(seed, tensor_id, idx)
        if fmt_ternary:
            c = (r % 3) - 1
        else:
            c = 1 - 2 * (r >> 31)
        out[r0:r1] = c.to(torch.int8)
    return out


def device_scales(seed, tensor_id, N, G, device):
    """fp16 [N][G] group scales on `device` (returned as torch.float16)."""
    import torch
    idx = torch.arange(N * G, dtype=torch.int64, device=device)
    r = _rand_t(seed, tensor_id, idx)
    u = (r >> 8).to(torch.float64) / float(1 << 24)
    t = 0.09 * u
    v = 0.01 + t
    return v.to(torch.float32).to(torch.float16).reshape(N, G)


def device_u32(seed, tensor_id, n, device, chunk=1 << 26):
    """The raw words r(0) .. r(n - 1) on `device` as an int32 tensor (the
    same bits as rand_u32), n <= 2^32."""
    import torch
    if n > (1 << 32):
        raise ValueError("more words than one tensor id holds")
    out = torch.empty(n, dtype=torch.int32, device=device)
    for i0 in range(0, n, chunk):
        i1 = min(n, i0 + chunk)
        idx = torch.arange(i0, i1, dtype=torch.int64, device=device)
        r = _rand_t(seed, tensor_id, idx)
        out[i0:i1] = (r - ((r >> 31) << 32)).to(torch.int32)
    return out
