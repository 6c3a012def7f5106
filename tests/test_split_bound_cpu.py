"""The staging bound behind the ternary bf16 split: three round-to-nearest-even
bf8 (e5m2) terms, each taking what the previous ones left scaled up by 2^3,
carry every bf16 value whose magnitude (after the block scaling that puts
the block maximum in [2^14, 2^15)) is at least 2^-13 exactly -- whether the
conversion keeps subnormal results or flushes them.  Staging flags any
smaller nonzero element for the exact recomputation.  Checked here over
every 8-bit significand at every exponent of that range, with an e5m2
rounding written from the format's definition (2 stored mantissa bits,
minimum normal exponent -14, subnormal step 2^-16)."""
import math

import pytest

MIN_EXACT_EXP = -13  # the bound the kernels use (2^-13)


def rne_e5m2(v, flush):
    if v == 0.0:
        return 0.0
    a = abs(v)
    e = math.floor(math.log2(a))
    if e < -14:
        if flush:
            return 0.0
        e = -14
    q = 2.0 ** (e - 2)
    f, d = divmod(a / q, 1.0)
    if d > 0.5 or (d == 0.5 and int(f) % 2 == 1):
        f += 1
    return math.copysign(f * q, v)


def residual(v, flush):
    tv = v
    for r in range(3):
        t = rne_e5m2(tv, flush)
        tv = (tv - t) * 8.0 if r < 2 else tv - t
    return tv


@pytest.mark.parametrize("flush", [False, True])
def test_three_bf8_terms_carry_bf16_exactly(flush):
    for e in range(MIN_EXACT_EXP, 15):
        for m in range(128, 256):
            for s in (1.0, -1.0):
                v = s * m * 2.0 ** (e - 7)
                assert residual(v, flush) == 0.0, (e, m, s)


def test_the_bound_is_needed():
    # one binade below the bound some values are no longer exact when the
    # conversion flushes subnormals (the flag is not a formality)
    e = MIN_EXACT_EXP - 1
    assert any(residual(m * 2.0 ** (e - 7), True) != 0.0 for m in range(128, 256))
