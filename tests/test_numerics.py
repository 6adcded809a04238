"""Host-side checks of the number formats the attention kernel relies on.

The fallback path of the attention kernel subtracts its running maximum m
inside the score product as one more K step: unit key columns against -m
split into three bfloat16 parts (each the round-to-nearest-even bfloat16 of
what the previous parts leave).  The sum of the three parts must equal the
float32 m exactly over the whole float32 range, so that no maximum is
rounded, however large the scores are.  The split is redone here in numpy
with bfloat16 rounding on the float32 bit patterns.
"""
import numpy as np

import workloads as W


def bf16_round(a32: np.ndarray) -> np.ndarray:
    return W.bf16_bits_to_f32(W.f32_to_bf16_bits(a32))


def split3(v: np.ndarray):
    v = v.astype(np.float32)
    hi = bf16_round(v)
    r1 = (v - hi).astype(np.float32)
    mid = bf16_round(r1)
    lo = bf16_round((r1 - mid).astype(np.float32))
    return hi, mid, lo


def test_three_bf16_parts_are_exact():
    rng = np.random.default_rng(0)
    mant = rng.uniform(1.0, 2.0, 200000)
    expo = rng.integers(-100, 120, mant.size)
    sign = rng.choice([-1.0, 1.0], mant.size)
    v = (sign * np.ldexp(mant, expo)).astype(np.float32)
    v = np.concatenate([v, np.float32([0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-30, 60.0, 16384.5])])
    hi, mid, lo = split3(v)
    # the parts are bfloat16 values ...
    for part in (hi, mid, lo):
        assert np.array_equal(bf16_round(part), part)
    # ... whose sum is v, in float64 and in float32 in either order
    assert np.array_equal(hi.astype(np.float64) + mid + lo, v.astype(np.float64))
    assert np.array_equal((hi + mid) + lo, v)
    assert np.array_equal(hi + (mid + lo), v)


def test_one_part_would_not_do():
    """A single bfloat16 maximum is off by up to half a bfloat16 step: 2^-9
    relative, which at |m| = 2^14 (log2 units) is 16, far past the threshold
    of 2^8 that bounds the probabilities."""
    v = np.float32([16384.0 + 31.0, 65536.0 + 255.0])
    one = bf16_round(v)
    assert (np.abs(one - v) >= 16.0).all()
