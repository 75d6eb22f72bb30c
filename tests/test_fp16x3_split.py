"""The arithmetic behind the opt-in fp16x3 MLP path, checked on the host with
NumPy (fp16 conversions round to nearest, as v_cvt_pk_f16_f32 does):

* two pieces h = fp16(x), l = fp16(x - h) carry x to within 2^-22 |x| for
  |x| in [2^-2, 2^15] (the normal range of both pieces), and to within an
  absolute 2^-25 below it (fp16's subnormal spacing is 2^-24);
* the three products kept (hh, hl, lh) are exact in fp32 and leave out at
  most ~2^-21 |a b| in the normal range;
* the wave rescaling 2^-j of a layer-2 input m >= 2^15 (j from the exponent
  of m) always lands below 2^15, and the constant-entry shift k keeps
  bound * 2^-k below 2^15.
"""
import math

import numpy as np


def split2(x):
    x = np.asarray(x, np.float32)
    h = x.astype(np.float16).astype(np.float32)
    l = (x - h).astype(np.float32).astype(np.float16).astype(np.float32)
    return h, l


def values(n, seed, lo, hi):
    rng = np.random.default_rng(seed)
    mag = 2.0 ** rng.uniform(lo, hi, n)
    return (np.where(rng.random(n) < 0.5, -1.0, 1.0) * mag).astype(np.float32)


def test_two_pieces_carry_22_bits_in_the_normal_range():
    x = values(200_000, 1, -2, 15)
    h, l = split2(x)
    err = np.abs(x.astype(np.float64) - h.astype(np.float64) - l.astype(np.float64))
    assert np.all(err <= 2.0 ** -22 * np.abs(x.astype(np.float64)))


def test_small_values_keep_an_absolute_floor():
    x = values(200_000, 2, -30, -2)
    h, l = split2(x)
    err = np.abs(x.astype(np.float64) - h.astype(np.float64) - l.astype(np.float64))
    assert np.all(err <= 2.0 ** -25 + 2.0 ** -22 * np.abs(x.astype(np.float64)))


def test_three_products_exact_in_fp32_and_the_rest_small():
    a, b = values(100_000, 3, -2, 8), values(100_000, 4, -2, 8)
    (ah, al), (bh, bl) = split2(a), split2(b)
    total = np.zeros(a.size)
    for p, q in ((ah, bh), (ah, bl), (al, bh)):
        p64 = p.astype(np.float64) * q.astype(np.float64)
        assert np.array_equal((p * q).astype(np.float32).astype(np.float64), p64)
        total += p64
    exact = a.astype(np.float64) * b.astype(np.float64)
    assert np.max(np.abs(total - exact) / np.abs(exact)) < 2.0 ** -20.5


def test_wave_rescaling_and_constant_shift_stay_below_2_15():
    for m in np.concatenate([2.0 ** np.linspace(15, 127.9, 4000), [32768.0, 65504.0, 1e30]]):
        _, ex = math.frexp(float(m))        # m < 2^ex
        j = ex - 15 if ex > 15 else 1
        assert j >= 1 and m * 2.0 ** -j < 32768.0
    for bound in 2.0 ** np.linspace(-5, 29, 3000):
        k = 0
        while bound * 2.0 ** -k >= 32768.0:
            k += 1
        assert bound * 2.0 ** -k < 32768.0 and (k == 0 or bound * 2.0 ** -(k - 1) >= 32768.0)
