"""The seeded input generators: host (numpy) and device-style (torch integer
ops) implementations of the same counter-based definition agree bit for bit,
and the value distributions are the intended ones."""
import numpy as np
import torch

import synth


def test_torch_and_numpy_generators_agree_on_cpu():
    for tern in (False, True):
        gen = synth.ternary_codes if tern else synth.binary_codes
        a = gen(1001, 7, 33, 640)
        b = synth.device_codes(tern, 1001, 7, 33, 640, "cpu", chunk_rows=5).numpy()
        assert np.array_equal(a, b)
    s1 = synth.group_scales(1001, 8, 33, 5)
    s2 = synth.device_scales(1001, 8, 33, 5, "cpu").numpy().view(np.uint16)
    assert np.array_equal(s1, s2)
    w1 = synth.rand_u32(1001, 9, np.arange(1000, dtype=np.uint64))
    w2 = synth.device_u32(1001, 9, 1000, "cpu", chunk=77).numpy().view(np.uint32)
    assert np.array_equal(np.asarray(w1, np.uint32), w2)


def test_row_subsets_regenerate_the_same_rows():
    full = synth.ternary_codes(5, 3, 50, 256)
    rows = np.array([0, 7, 49])
    assert np.array_equal(synth.ternary_codes(5, 3, 50, 256, rows=rows), full[rows])
    fs = synth.group_scales(5, 4, 50, 2)
    assert np.array_equal(synth.group_scales(5, 4, 50, 2, rows=rows), fs[rows])


def test_distributions():
    b = synth.binary_codes(1, 1, 256, 1024)
    assert set(np.unique(b)) == {-1, 1} and abs(b.mean()) < 0.01
    t = synth.ternary_codes(1, 2, 256, 1024)
    frac = np.bincount(t.ravel() + 1) / t.size
    assert np.all(np.abs(frac - 1 / 3) < 0.01)
    s = synth.group_scales(1, 3, 256, 64).view(np.float16).astype(np.float64)
    assert s.min() >= 0.00999 and s.max() <= 0.1001
    x = synth.bf16_bits_to_f32(synth.normal_bf16(1, 4, 64, 1024)).astype(np.float64)
    assert abs(x.mean()) < 0.02 and abs(x.std() - 1) < 0.02


def test_bf16_rounding_is_nearest_even():
    v = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    got = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(v))
    assert got.tolist() == [1.0, 1.0 + 4 * 2 ** -8, -1.0, 1.0 + 2 ** -7]
