"""The oracle's packer/unpacker against the written layout specification.

Pins: hand-worked byte positions, round trips (a bijection on valid codes),
exhaustive enumeration of every valid byte / field value, locality of each
16-row x 4-group block (what one wavefront reads as 1 KiB), reserved
patterns, and invalid-code counting.
"""
import itertools
import json
import os

import numpy as np
import pytest

import synth
from oracle import oracle as O

FMTS = (O.BINARY, O.TERNARY_2BIT, O.TERNARY_BASE3)


def zero_codes(fmt, N, K):
    return np.ones((N, K), np.int8) if fmt == O.BINARY else np.zeros((N, K), np.int8)


def test_handworked_positions(golden_dir):
    gold = json.load(open(os.path.join(golden_dir, "layout_handworked.json")))
    for case in gold["cases"]:
        fmt, N, K = case["fmt"], case["N"], case["K"]
        base = zero_codes(fmt, N, K)
        sc = np.zeros((N, K // 128), np.uint16)
        p0, _, _ = O.pack(fmt, base, sc)
        c = base.copy()
        for n, k, v in case["set"]:
            c[n, k] = v
        p1, _, bad = O.pack(fmt, c, sc)
        assert bad == 0
        diff = np.nonzero(p0 != p1)[0]
        got = [[int(i), int(p1[i])] for i in diff]
        assert got == case["expected"], (case["why"], got)
    for sc_case in gold["scale_cases"]:
        N, K, n, g = sc_case["N"], sc_case["K"], sc_case["n"], sc_case["g"]
        sc = np.zeros((N, K // 128), np.uint16)
        sc[n, g] = 0x3C00
        _, ps, _ = O.pack(O.BINARY, np.ones((N, K), np.int8), sc)
        assert np.nonzero(ps)[0].tolist() == [sc_case["index"]], sc_case["why"]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", [(16, 128), (37, 384), (5, 1152), (33, 2048)])
def test_round_trip_ragged(fmt, N, K):
    gen = synth.binary_codes if fmt == O.BINARY else synth.ternary_codes
    codes = gen(3, fmt, N, K)
    scales = synth.group_scales(3, 10 + fmt, N, K // 128)
    pc, ps, bad = O.pack(fmt, codes, scales)
    assert bad == 0
    assert (pc.size, 2 * ps.size) == O.packed_bytes(fmt, N, K)
    c2, s2, bad2 = O.unpack(fmt, N, K, pc, ps)
    assert bad2 == 0
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)


@pytest.mark.parametrize("fmt", FMTS)
def test_every_weight_has_its_own_position_inside_its_block(fmt):
    """Flipping one weight changes bytes only inside the block of its row-block
    and group range, in the 16-byte lane slice of its row."""
    N, K = 32, 1024
    G = K // 128
    base = zero_codes(fmt, N, K)
    sc = np.zeros((N, G), np.uint16)
    p0, _, _ = O.pack(fmt, base, sc)
    flip = -1 if fmt == O.BINARY else 1
    seen = set()
    rng = np.random.default_rng(0)
    for n in (0, 7, 16, 31):
        for k in sorted(set(range(0, 128)) | set(int(v) for v in rng.integers(0, K, 64))):
            c = base.copy()
            c[n, k] = flip
            p1, _, _ = O.pack(fmt, c, sc)
            d = np.nonzero(p0 != p1)[0]
            assert d.size == 1
            off = int(d[0])
            bitpos = (off, int(p0[off] ^ p1[off]))
            if fmt != O.TERNARY_BASE3:
                assert bin(bitpos[1]).count("1") == 1
                assert bitpos not in seen
                seen.add(bitpos)
            rb, g = n // 16, k // 128
            if fmt == O.BINARY:
                blk, per = 1024, 4  # 4 groups per 1 KiB block
            elif fmt == O.TERNARY_2BIT:
                blk, per = 1024, 2
            else:
                blk, per = 3328, 8
            nblk = -(-G // per)
            assert off // blk == rb * nblk + g // per
            inblk = off % blk
            lane = (inblk % 1024) // 16 if inblk < 3072 else (inblk - 3072) // 4
            assert lane % 16 == n % 16


def test_binary_all_256_byte_values():
    # the 8 weights that land in byte 0 of lane 0 / group 0, in every combination
    N, K = 16, 128
    weights = []
    for k in range(128):
        c = np.ones((N, K), np.int8)
        c[0, k] = -1
        pc, _, _ = O.pack(O.BINARY, c, np.zeros((N, 1), np.uint16))
        if pc[0] != 0:
            weights.append((k, int(pc[0])))
    assert sorted(v for _, v in weights) == [1 << b for b in range(8)]
    vals = set()
    for combo in itertools.product([1, -1], repeat=8):
        c = np.ones((N, K), np.int8)
        for (k, _), s in zip(weights, combo):
            c[0, k] = s
        pc, _, _ = O.pack(O.BINARY, c, np.zeros((N, 1), np.uint16))
        vals.add(int(pc[0]))
    assert vals == set(range(256))


def test_ternary2_all_81_byte_values_and_no_reserved():
    N, K = 16, 128
    ks = []
    for k in range(128):
        c = np.zeros((N, K), np.int8)
        c[0, k] = 1
        pc, _, _ = O.pack(O.TERNARY_2BIT, c, np.zeros((N, 1), np.uint16))
        if pc[0] != 0:
            ks.append(k)
    assert len(ks) == 4
    vals = set()
    for combo in itertools.product([-1, 0, 1], repeat=4):
        c = np.zeros((N, K), np.int8)
        for k, v in zip(ks, combo):
            c[0, k] = v
        pc, ps, _ = O.pack(O.TERNARY_2BIT, c, np.zeros((N, 1), np.uint16))
        b = int(pc[0])
        # the byte holds two nibbles; in each, bit pairs (z, s) are (1,3) and (0,2)
        for nib in (b & 15, b >> 4):
            for zb, sb in ((1, 3), (0, 2)):
                assert not ((nib >> sb) & 1 and not (nib >> zb) & 1)
        vals.add(b)
        c2, _, bad = O.unpack(O.TERNARY_2BIT, N, K, pc, ps)
        assert bad == 0 and np.array_equal(c2, c)
    assert len(vals) == 81


@pytest.mark.parametrize("slots,limit", [(range(0, 5), 243), (range(30, 32), 81)])
def test_base3_all_byte_values(slots, limit):
    """Every trit combination of a 5-trit byte (243) and of a 4-trit byte (81)
    is written as a distinct value below the limit and decodes back."""
    N, K = 16, 1024
    # quarter 0 slot i of group j: k = 128 j + KMAP(0, i)
    kmap0 = lambda i: 32 * (i >> 4) + (i & 15)
    if limit == 243:
        ks = [kmap0(i) for i in slots]  # group 0, slots 0..4 -> byte 0
        byte_off = 0
    else:
        ks = [kmap0(i) for i in slots] + [128 + kmap0(i) for i in slots]  # groups 0,1 -> byte 48
        byte_off = 3072
    vals = set()
    for combo in itertools.product([-1, 0, 1], repeat=len(ks)):
        c = np.zeros((N, K), np.int8)
        for k, v in zip(ks, combo):
            c[0, k] = v
        pc, ps, _ = O.pack(O.TERNARY_BASE3, c, np.zeros((N, 8), np.uint16))
        v = int(pc[byte_off])
        assert v < limit
        vals.add(v)
        c2, _, bad = O.unpack(O.TERNARY_BASE3, N, K, pc, ps)
        assert bad == 0 and np.array_equal(c2, c)
    assert len(vals) == limit


def test_reserved_and_out_of_range_packed_values_are_counted():
    N, K = 16, 1024
    c = np.zeros((N, K), np.int8)
    sc = np.zeros((N, 8), np.uint16)
    pc, ps, _ = O.pack(O.TERNARY_2BIT, c, sc)
    pc[0] = 0x08  # s = 1 with z = 0 in the (1,3) pair of nibble 0
    _, _, bad = O.unpack(O.TERNARY_2BIT, N, K, pc, ps)
    assert bad == 1
    pc, ps, _ = O.pack(O.TERNARY_BASE3, c, sc)
    pc[0] = 250  # >= 243: five weights decoded from an invalid byte
    pc[3072] = 90  # >= 81 in a 4-trit byte (4 weights)
    c2, _, bad = O.unpack(O.TERNARY_BASE3, N, K, pc, ps)
    assert bad == 9 and not c2.any()


def test_invalid_codes_are_counted_by_pack():
    N, K = 16, 256
    c = synth.ternary_codes(1, 1, N, K)
    sc = np.zeros((N, 2), np.uint16)
    assert O.pack(O.BINARY, c, sc)[2] == int((c == 0).sum())
    c2 = c.copy()
    c2[3, 5] = 2
    c2[4, 6] = -7
    assert O.pack(O.TERNARY_2BIT, c2, sc)[2] == 2
    assert O.pack(O.TERNARY_BASE3, c2, sc)[2] == 2
