"""lowbit_pack / lowbit_unpack on the GPU against the oracle's packer:
byte-identical packing, exact round trips, invalid-code counting."""
import numpy as np
import pytest
import torch

import synth
from oracle import oracle as O
from ultra_bit_dit_amd import lowbit as lb

from helpers import SEED, codes_for

pytestmark = pytest.mark.gpu


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("fmt", [1, 2, 3])
@pytest.mark.parametrize("N,K", [(16, 128), (1, 128), (37, 384), (5, 1152), (33, 2048), (256, 1024)])
def test_pack_matches_oracle_bytes(fmt, N, K):
    print(f"pack fmt={fmt} N={N} K={K}", flush=True)
    codes = codes_for(fmt, SEED, 1, N, K)
    scales = synth.group_scales(SEED, 2, N, K // 128)
    pc_ref, ps_ref, bad_ref = O.pack(fmt, codes, scales)
    assert bad_ref == 0
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    pc, ps = lb.pack(fmt, dev(codes), dev(scales.view(np.int16)), bad=bad)
    torch.cuda.synchronize()
    assert np.array_equal(pc.cpu().numpy(), pc_ref)
    assert np.array_equal(ps.cpu().numpy().view(np.uint16), ps_ref)
    assert int(bad.item()) == 0
    c2, s2 = lb.unpack(fmt, N, K, pc, ps, bad=bad)
    torch.cuda.synchronize()
    assert np.array_equal(c2.cpu().numpy(), codes)
    assert np.array_equal(s2.cpu().numpy().view(np.uint16), scales)
    assert int(bad.item()) == 0


@pytest.mark.parametrize("fmt", [2, 3])
def test_pack_full_size_5120(fmt):
    """The 5120 x 5120 ternary matrix, codes generated on the device."""
    N = K = 5120
    print(f"pack full fmt={fmt}", flush=True)
    codes_t = synth.device_codes(True, SEED + 1, 11, N, K, "cuda")
    scales_t = synth.device_scales(SEED + 1, 12, N, K // 128, "cuda")
    codes = synth.ternary_codes(SEED + 1, 11, N, K)
    assert np.array_equal(codes_t.cpu().numpy(), codes)
    scales = synth.group_scales(SEED + 1, 12, N, K // 128)
    pc_ref, ps_ref, _ = O.pack(fmt, codes, scales)
    pc, ps = lb.pack(fmt, codes_t, scales_t)
    torch.cuda.synchronize()
    assert np.array_equal(pc.cpu().numpy(), pc_ref)
    assert np.array_equal(ps.cpu().numpy().view(np.uint16), ps_ref)


def test_invalid_codes_counted():
    N, K = 16, 256
    codes = synth.ternary_codes(SEED, 3, N, K)
    scales = synth.group_scales(SEED, 4, N, 2)
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    lb.pack(1, dev(codes), dev(scales.view(np.int16)), bad=bad)  # zeros are invalid for binary
    torch.cuda.synchronize()
    assert int(bad.item()) == O.pack(1, codes, scales)[2] == int((codes == 0).sum())
    c2 = codes.copy()
    c2[2, 3] = 5
    c2[7, 200] = -2
    for fmt in (2, 3):
        bad.zero_()
        lb.pack(fmt, dev(c2), dev(scales.view(np.int16)), bad=bad)
        torch.cuda.synchronize()
        assert int(bad.item()) == 2


def test_unpack_counts_reserved_patterns():
    N, K = 16, 1024
    z = np.zeros((N, K), np.int8)
    sc = np.zeros((N, 8), np.uint16)
    pc, ps, _ = O.pack(2, z, sc)
    pc[0] = 0x08
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    c2, _ = lb.unpack(2, N, K, dev(pc), dev(ps.view(np.int16)), bad=bad)
    torch.cuda.synchronize()
    assert int(bad.item()) == 1 and not c2.cpu().numpy().any()
    pc, ps, _ = O.pack(3, z, sc)
    pc[0] = 250
    pc[3072] = 90
    bad.zero_()
    c2, _ = lb.unpack(3, N, K, dev(pc), dev(ps.view(np.int16)), bad=bad)
    torch.cuda.synchronize()
    assert int(bad.item()) == 9 and not c2.cpu().numpy().any()


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 3 << 20, (64 << 20) + 112])
def test_hbm_read_probe_reads_every_byte(nbytes):
    """The streaming-read helper folds every 16-byte piece it reads into one
    XOR: equal to numpy's XOR of the same data (ragged tail included)."""
    print(f"read probe {nbytes} B", flush=True)
    rng = np.random.default_rng(nbytes)
    data = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    lb.hbm_read_probe(dev(data.view(np.int32)), out)
    torch.cuda.synchronize()
    assert int(out.item()) & 0xFFFFFFFF == int(np.bitwise_xor.reduce(data))
    with pytest.raises(lb.LowbitError) as e:
        lb.hbm_read_probe(dev(data.view(np.int32))[:3], out)
    assert e.value.status == lb.E_SHAPE
